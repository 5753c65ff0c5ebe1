// Streaming probes: the bandwidth of an access pattern on this device.
//
// Each probe moves exactly the bytes of one of the library's kernels -- the
// same arrays, element types, non-temporal/temporal cache policy and
// 4,096-element chunk per 256-lane workgroup -- but does trivial arithmetic.
// With the kernel's own lane width (4 elements per lane: a 64-bit access per
// BF16 stream, 128-bit per FP32 stream) it shows what the kernel's
// arithmetic costs; with 8 elements per lane (a 128-bit access per BF16
// stream, two 128-bit accesses per FP32 stream) it is the other design the
// width comparison weighs.  Measurement infrastructure only (built into
// libgro_probe.so, used by bench.py); not part of the gro_* ABI.
//
//   pattern 0 / 3, AdamW:       read acc (default policy; flags bit 0:
//                               non-temporal) and p, m, v
//                               (non-temporal); write p, m, v and a BF16 copy
//                               (non-temporal).  30 bytes per element; chunks
//                               in reverse order; 16 elements per lane.
//   pattern 1 / 4, window:      read k BF16 streams (non-temporal); write one
//                               FP32 stream (default policy; flags bit 0:
//                               non-temporal).  2k + 4 bytes
//                               per element; 8 elements per lane in flight
//                               per stream.
//   pattern 2 / 5, accumulate:  read one BF16 stream (non-temporal) and the
//                               FP32 stream; write the FP32 stream (flags
//                               bit 0: non-temporally).  10 bytes
//                               per element; 8 elements per lane in flight.
// Patterns 0-2 use 4 elements per lane access, 3-5 use 8.
//
// Reference streams, the same chunking and 4 elements per lane, default
// cache policy, to say what plain streaming reaches on this device at the
// same size:
//   pattern 6, read only:   read one FP32 stream (p); each workgroup writes
//                           its first wave's sum, one float (to m).  4 bytes
//                           per element.
//   pattern 7, write only:  write one FP32 stream (p).  4 bytes per element.
//   pattern 8, copy:        read one FP32 stream (acc), write another (p).
//                           8 bytes per element.
//
// Arguments: n elements (a multiple of 4,096); device pointers as the pattern
// needs them (unused ones may be NULL); for the window patterns `k` BF16
// stream pointers in `g`, k in 1..8, 12 or 16 (the window kernel reads window
// length x slots streams); `flags` the launch policy the kernels take on
// large accumulators: bit 0 moves the accumulator's stream (acc read by the
// AdamW pattern, the FP32 stream written by the window and accumulate
// patterns) with the non-temporal policy, bits 8-15 (0-16) cap the
// workgroups sharing a CU as the kernels do, with dynamic LDS that the probe
// does not use (0: no cap).  Returns 0, -1 for bad arguments, or a
// hipError_t.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

constexpr int kLanes = 256;
constexpr int kChunk = 4096;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// W BF16 elements per lane access: W / 2 32-bit words.
template <int W> struct Bf16Vec;
template <> struct Bf16Vec<4> { typedef u32x2 t; };
template <> struct Bf16Vec<8> { typedef u32x4 t; };

__device__ __forceinline__ f32x4 widen(uint32_t a, uint32_t b) {
  return f32x4{__uint_as_float(a << 16), __uint_as_float(a & 0xffff0000u), __uint_as_float(b << 16),
               __uint_as_float(b & 0xffff0000u)};
}
// The W elements of one access as W / 4 FP32 vectors.
__device__ __forceinline__ void widen_all(const u32x2 r, f32x4* t) { t[0] = widen(r.x, r.y); }
__device__ __forceinline__ void widen_all(const u32x4 r, f32x4* t) {
  t[0] = widen(r.x, r.y);
  t[1] = widen(r.z, r.w);
}
// Truncating FP32 -> BF16 of a vector pair's high halves (the probe's
// trivial stand-in for rounding).
__device__ __forceinline__ uint32_t hi2(float a, float b) {
  return __float_as_uint(a) >> 16 | (__float_as_uint(b) & 0xffff0000u);
}
template <int W>
__device__ __forceinline__ typename Bf16Vec<W>::t nt_load(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const typename Bf16Vec<W>::t*>(p));
}
__device__ __forceinline__ f32x4 load_nt(const float* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
}
__device__ __forceinline__ void store_nt(float* p, f32x4 x) {
  __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(p));
}
// The accumulator's stream: default policy, or non-temporal (NT).
template <bool NT>
__device__ __forceinline__ f32x4 load_acc(const float* p) {
  if constexpr (NT) return load_nt(p);
  else return *reinterpret_cast<const f32x4*>(p);
}
template <bool NT>
__device__ __forceinline__ void store_acc(float* p, f32x4 x) {
  if constexpr (NT) store_nt(p, x);
  else *reinterpret_cast<f32x4*>(p) = x;
}

struct Streams {
  const float* acc;
  float* p;
  float* m;
  float* v;
  uint16_t* pb;
  const uint16_t* g[16];
  int k;
};

// Lane accesses of W elements; U of them per lane and stream in flight.  A
// lane's access u covers elements base + W * (v0 + u * kLanes) .. + W - 1.
template <int W, bool NT>
__global__ __launch_bounds__(kLanes) void probe_adamw(const Streams s, int64_t n_chunks) {
  constexpr int U = 16 / W, H = W / 4;
  const int64_t base = (n_chunks - 1 - int64_t(blockIdx.x)) * kChunk;
  f32x4 a[U][H], p[U][H], m[U][H], v[U][H];
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int h = 0; h < H; ++h) {
      const int64_t e = base + W * (threadIdx.x + u * kLanes) + 4 * h;
      a[u][h] = load_acc<NT>(s.acc + e);
      p[u][h] = load_nt(s.p + e);
      m[u][h] = load_nt(s.m + e);
      v[u][h] = load_nt(s.v + e);
    }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    uint32_t b[W / 2];
#pragma unroll
    for (int h = 0; h < H; ++h) {
      const int64_t e = base + W * (threadIdx.x + u * kLanes) + 4 * h;
      p[u][h] = p[u][h] - a[u][h];
      m[u][h] = m[u][h] + a[u][h];
      v[u][h] = v[u][h] + a[u][h] * a[u][h];
      store_nt(s.p + e, p[u][h]);
      store_nt(s.m + e, m[u][h]);
      store_nt(s.v + e, v[u][h]);
      b[2 * h] = hi2(p[u][h].x, p[u][h].y);
      b[2 * h + 1] = hi2(p[u][h].z, p[u][h].w);
    }
    uint16_t* pb = s.pb + base + W * (threadIdx.x + u * kLanes);
    if constexpr (W == 4) __builtin_nontemporal_store(u32x2{b[0], b[1]}, reinterpret_cast<u32x2*>(pb));
    else __builtin_nontemporal_store(u32x4{b[0], b[1], b[2], b[3]}, reinterpret_cast<u32x4*>(pb));
  }
}

template <int K, int W, bool NT>
__global__ __launch_bounds__(kLanes) void probe_window(const Streams s) {
  constexpr int U = 8 / W, H = W / 4;
  const int64_t base = int64_t(blockIdx.x) * kChunk;
  for (int v0 = threadIdx.x; v0 < kChunk / W; v0 += U * kLanes) {
    typename Bf16Vec<W>::t r[K][U];
#pragma unroll
    for (int j = 0; j < K; ++j)
#pragma unroll
      for (int u = 0; u < U; ++u) r[j][u] = nt_load<W>(s.g[j] + base + W * (v0 + u * kLanes));
#pragma unroll
    for (int u = 0; u < U; ++u) {
      f32x4 t[H], x[H];
      widen_all(r[0][u], t);
#pragma unroll
      for (int j = 1; j < K; ++j) {
        widen_all(r[j][u], x);
#pragma unroll
        for (int h = 0; h < H; ++h) t[h] = t[h] + x[h];
      }
#pragma unroll
      for (int h = 0; h < H; ++h) store_acc<NT>(s.p + base + W * (v0 + u * kLanes) + 4 * h, t[h]);
    }
  }
}

template <int W, bool NT>
__global__ __launch_bounds__(kLanes) void probe_accumulate(const Streams s) {
  constexpr int U = 8 / W, H = W / 4;
  const int64_t base = int64_t(blockIdx.x) * kChunk;
  for (int v0 = threadIdx.x; v0 < kChunk / W; v0 += U * kLanes) {
    typename Bf16Vec<W>::t r[U];
    f32x4 old[U][H];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t e = base + W * (v0 + u * kLanes);
      r[u] = nt_load<W>(s.g[0] + e);
#pragma unroll
      for (int h = 0; h < H; ++h) old[u][h] = *reinterpret_cast<const f32x4*>(s.p + e + 4 * h);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      f32x4 t[H];
      widen_all(r[u], t);
#pragma unroll
      for (int h = 0; h < H; ++h) store_acc<NT>(s.p + base + W * (v0 + u * kLanes) + 4 * h, old[u][h] + t[h]);
    }
  }
}

// Reference streams: 16 elements per lane, all loads issued before use.
__global__ __launch_bounds__(kLanes) void probe_read(const Streams s) {
  const int64_t base = int64_t(blockIdx.x) * kChunk;
  f32x4 x[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) x[u] = *reinterpret_cast<const f32x4*>(s.p + base + 4 * (threadIdx.x + u * kLanes));
  f32x4 t = (x[0] + x[1]) + (x[2] + x[3]);
  float r = (t.x + t.y) + (t.z + t.w);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) r += __shfl_xor(r, m, 64);
  if (threadIdx.x == 0) s.m[blockIdx.x] = r;  // keeps the loads; 4 bytes written per 4,096 elements
}

__global__ __launch_bounds__(kLanes) void probe_write(const Streams s) {
  const int64_t base = int64_t(blockIdx.x) * kChunk;
  const float b = float(blockIdx.x);
#pragma unroll
  for (int u = 0; u < 4; ++u)
    *reinterpret_cast<f32x4*>(s.p + base + 4 * (threadIdx.x + u * kLanes)) = f32x4{b, b, b, b};
}

__global__ __launch_bounds__(kLanes) void probe_copy(const Streams s) {
  const int64_t base = int64_t(blockIdx.x) * kChunk;
  f32x4 x[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) x[u] = *reinterpret_cast<const f32x4*>(s.acc + base + 4 * (threadIdx.x + u * kLanes));
#pragma unroll
  for (int u = 0; u < 4; ++u) *reinterpret_cast<f32x4*>(s.p + base + 4 * (threadIdx.x + u * kLanes)) = x[u];
}

template <int W, bool NT>
hipError_t launch_window(int k, const dim3 grid, size_t lds, const Streams& s, hipStream_t st) {
  const dim3 block(kLanes);
  switch (k) {
    case 1: hipLaunchKernelGGL((probe_window<1, W, NT>), grid, block, lds, st, s); break;
    case 2: hipLaunchKernelGGL((probe_window<2, W, NT>), grid, block, lds, st, s); break;
    case 3: hipLaunchKernelGGL((probe_window<3, W, NT>), grid, block, lds, st, s); break;
    case 4: hipLaunchKernelGGL((probe_window<4, W, NT>), grid, block, lds, st, s); break;
    case 5: hipLaunchKernelGGL((probe_window<5, W, NT>), grid, block, lds, st, s); break;
    case 6: hipLaunchKernelGGL((probe_window<6, W, NT>), grid, block, lds, st, s); break;
    case 7: hipLaunchKernelGGL((probe_window<7, W, NT>), grid, block, lds, st, s); break;
    case 8: hipLaunchKernelGGL((probe_window<8, W, NT>), grid, block, lds, st, s); break;
    case 12: hipLaunchKernelGGL((probe_window<12, W, NT>), grid, block, lds, st, s); break;
    case 16: hipLaunchKernelGGL((probe_window<16, W, NT>), grid, block, lds, st, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipSuccess;
}

template <int W, bool NT>
void launch_adamw(const dim3 grid, size_t lds, const Streams& s, int64_t chunks, hipStream_t st) {
  hipLaunchKernelGGL((probe_adamw<W, NT>), grid, dim3(kLanes), lds, st, s, chunks);
}

template <int W, bool NT>
void launch_accumulate(const dim3 grid, size_t lds, const Streams& s, hipStream_t st) {
  hipLaunchKernelGGL((probe_accumulate<W, NT>), grid, dim3(kLanes), lds, st, s);
}

// Dynamic LDS that leaves room for at most `cap` workgroups on one gfx950
// CU (160 KiB of LDS), as the library's launches request it; 0: no cap.
size_t cap_lds(int cap) { return cap > 0 ? size_t(160 * 1024 / cap - 2048) : 0; }

}  // namespace

extern "C" int gro_probe_stream(int pattern, int64_t n, const float* acc, float* p, float* m, float* v,
                                uint16_t* pb, const uint16_t* const* g, int k, int flags, void* stream) {
  if (n <= 0 || n % kChunk != 0) return -1;
  const int64_t chunks = n / kChunk;
  if (chunks > 0x7fffffff) return -1;
  Streams s{};
  s.acc = acc;
  s.p = p;
  s.m = m;
  s.v = v;
  s.pb = pb;
  s.k = k;
  if (flags & ~0xff01) return -1;
  const int cap = (flags >> 8) & 0xff;
  if (cap > 16) return -1;
  const bool nt = (flags & 1) != 0;
  const size_t lds = cap_lds(cap);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid(static_cast<unsigned>(chunks)), block(kLanes);
  const bool wide = pattern >= 3;
  switch (pattern) {
    case 0:
    case 3:
      if (!acc || !p || !m || !v || !pb) return -1;
      if (wide) nt ? launch_adamw<8, true>(grid, lds, s, chunks, st) : launch_adamw<8, false>(grid, lds, s, chunks, st);
      else nt ? launch_adamw<4, true>(grid, lds, s, chunks, st) : launch_adamw<4, false>(grid, lds, s, chunks, st);
      break;
    case 1:
    case 4: {
      if (!p || !g || k < 1 || k > 16) return -1;
      if (!(k <= 8 || k == 12 || k == 16)) return -1;
      for (int j = 0; j < k; ++j) {
        if (!g[j]) return -1;
        s.g[j] = g[j];
      }
      const hipError_t e = wide ? (nt ? launch_window<8, true>(k, grid, lds, s, st)
                                      : launch_window<8, false>(k, grid, lds, s, st))
                                : (nt ? launch_window<4, true>(k, grid, lds, s, st)
                                      : launch_window<4, false>(k, grid, lds, s, st));
      if (e != hipSuccess) return -1;
      break;
    }
    case 2:
    case 5:
      if (!p || !g || !g[0]) return -1;
      s.g[0] = g[0];
      if (wide) nt ? launch_accumulate<8, true>(grid, lds, s, st) : launch_accumulate<8, false>(grid, lds, s, st);
      else nt ? launch_accumulate<4, true>(grid, lds, s, st) : launch_accumulate<4, false>(grid, lds, s, st);
      break;
    case 6:
      if (!p || !m) return -1;
      hipLaunchKernelGGL(probe_read, grid, block, lds, st, s);
      break;
    case 7:
      if (!p) return -1;
      hipLaunchKernelGGL(probe_write, grid, block, lds, st, s);
      break;
    case 8:
      if (!acc || !p) return -1;
      hipLaunchKernelGGL(probe_copy, grid, block, lds, st, s);
      break;
    default:
      return -1;
  }
  return static_cast<int>(hipGetLastError());
}
