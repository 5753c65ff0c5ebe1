// Streaming probes: what bandwidth an access pattern can reach on this device.
//
// Each probe moves exactly the bytes of one of the library's kernels -- the
// same arrays, element types, non-temporal/temporal cache policy, 4,096-element
// chunk per 256-lane workgroup and vectors per lane -- but does trivial
// arithmetic, so its bandwidth is the ceiling that kernel's access pattern can
// reach.  Measurement infrastructure only (built into libgro_probe.so, used by
// bench.py); not part of the gro_* ABI.
//
//   pattern 0, AdamW:       read acc (default policy) and p, m, v
//                           (non-temporal); write p, m, v and a BF16 copy
//                           (non-temporal).  30 bytes per element; chunks in
//                           reverse order, four vectors per lane.
//   pattern 1, window:      read k BF16 streams (non-temporal); write one FP32
//                           stream (default policy).  2k + 4 bytes per element.
//   pattern 2, accumulate:  read one BF16 stream (non-temporal) and the FP32
//                           stream; write the FP32 stream.  10 bytes per
//                           element.
//
// Arguments: n elements (a multiple of 4,096); device pointers as the pattern
// needs them (unused ones may be NULL); for pattern 1, `k` BF16 stream
// pointers in `g`, k in 1..8, 12 or 16 (the window kernel reads window length
// x slots streams).  Returns 0, -1 for bad arguments, or a hipError_t.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

constexpr int kLanes = 256;
constexpr int kChunk = 4096;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 load_nt(const float* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
}
__device__ __forceinline__ void store_nt(float* p, f32x4 x) {
  __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(p));
}
__device__ __forceinline__ f32x4 bf16x4_to_f32(u32x2 r) {
  return f32x4{__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u), __uint_as_float(r.y << 16),
               __uint_as_float(r.y & 0xffff0000u)};
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

__global__ __launch_bounds__(kLanes) void probe_adamw(const Streams s, int64_t n_chunks) {
  constexpr int kVec = 4;
  const int64_t base = (n_chunks - 1 - int64_t(blockIdx.x)) * kChunk;
  f32x4 a[kVec], p[kVec], m[kVec], v[kVec];
#pragma unroll
  for (int u = 0; u < kVec; ++u) {
    const int64_t e = base + 4 * (threadIdx.x + u * kLanes);
    a[u] = *reinterpret_cast<const f32x4*>(s.acc + e);
    p[u] = load_nt(s.p + e);
    m[u] = load_nt(s.m + e);
    v[u] = load_nt(s.v + e);
  }
#pragma unroll
  for (int u = 0; u < kVec; ++u) {
    const int64_t e = base + 4 * (threadIdx.x + u * kLanes);
    p[u] = p[u] - a[u];
    m[u] = m[u] + a[u];
    v[u] = v[u] + a[u] * a[u];
    store_nt(s.p + e, p[u]);
    store_nt(s.m + e, m[u]);
    store_nt(s.v + e, v[u]);
    const u32x2 b = {__float_as_uint(p[u].x) >> 16 | (__float_as_uint(p[u].y) & 0xffff0000u),
                     __float_as_uint(p[u].z) >> 16 | (__float_as_uint(p[u].w) & 0xffff0000u)};
    __builtin_nontemporal_store(b, reinterpret_cast<u32x2*>(s.pb + e));
  }
}

template <int K>
__global__ __launch_bounds__(kLanes) void probe_window(const Streams s) {
  constexpr int kVec = 2;
  const int64_t base = int64_t(blockIdx.x) * kChunk;
  for (int v0 = threadIdx.x; v0 < kChunk / 4; v0 += kVec * kLanes) {
    u32x2 r[K][kVec];
#pragma unroll
    for (int j = 0; j < K; ++j)
#pragma unroll
      for (int u = 0; u < kVec; ++u)
        r[j][u] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(s.g[j] + base + 4 * (v0 + u * kLanes)));
#pragma unroll
    for (int u = 0; u < kVec; ++u) {
      f32x4 t = bf16x4_to_f32(r[0][u]);
#pragma unroll
      for (int j = 1; j < K; ++j) t = t + bf16x4_to_f32(r[j][u]);
      *reinterpret_cast<f32x4*>(s.p + base + 4 * (v0 + u * kLanes)) = t;
    }
  }
}

__global__ __launch_bounds__(kLanes) void probe_accumulate(const Streams s) {
  constexpr int kVec = 2;
  const int64_t base = int64_t(blockIdx.x) * kChunk;
  for (int v0 = threadIdx.x; v0 < kChunk / 4; v0 += kVec * kLanes) {
    u32x2 r[kVec];
    f32x4 old[kVec];
#pragma unroll
    for (int u = 0; u < kVec; ++u) {
      const int64_t e = base + 4 * (v0 + u * kLanes);
      r[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(s.g[0] + e));
      old[u] = *reinterpret_cast<const f32x4*>(s.p + e);
    }
#pragma unroll
    for (int u = 0; u < kVec; ++u)
      *reinterpret_cast<f32x4*>(s.p + base + 4 * (v0 + u * kLanes)) = old[u] + bf16x4_to_f32(r[u]);
  }
}

}  // namespace

extern "C" int gro_probe_stream(int pattern, int64_t n, const float* acc, float* p, float* m, float* v,
                                uint16_t* pb, const uint16_t* const* g, int k, void* stream) {
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
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid(static_cast<unsigned>(chunks)), block(kLanes);
  switch (pattern) {
    case 0:
      if (!acc || !p || !m || !v || !pb) return -1;
      hipLaunchKernelGGL(probe_adamw, grid, block, 0, st, s, chunks);
      break;
    case 1:
      if (!p || !g || k < 1 || k > 16) return -1;
      for (int j = 0; j < k; ++j) {
        if (!g[j]) return -1;
        s.g[j] = g[j];
      }
      switch (k) {
        case 1: hipLaunchKernelGGL(probe_window<1>, grid, block, 0, st, s); break;
        case 2: hipLaunchKernelGGL(probe_window<2>, grid, block, 0, st, s); break;
        case 3: hipLaunchKernelGGL(probe_window<3>, grid, block, 0, st, s); break;
        case 4: hipLaunchKernelGGL(probe_window<4>, grid, block, 0, st, s); break;
        case 5: hipLaunchKernelGGL(probe_window<5>, grid, block, 0, st, s); break;
        case 6: hipLaunchKernelGGL(probe_window<6>, grid, block, 0, st, s); break;
        case 7: hipLaunchKernelGGL(probe_window<7>, grid, block, 0, st, s); break;
        case 8: hipLaunchKernelGGL(probe_window<8>, grid, block, 0, st, s); break;
        case 12: hipLaunchKernelGGL(probe_window<12>, grid, block, 0, st, s); break;
        case 16: hipLaunchKernelGGL(probe_window<16>, grid, block, 0, st, s); break;
        default: return -1;
      }
      break;
    case 2:
      if (!p || !g || !g[0]) return -1;
      s.g[0] = g[0];
      hipLaunchKernelGGL(probe_accumulate, grid, block, 0, st, s);
      break;
    default:
      return -1;
  }
  return static_cast<int>(hipGetLastError());
}
