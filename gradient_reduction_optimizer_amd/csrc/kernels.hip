// gfx950 (MI355X, CDNA4) kernels for the gradient-ownership hot path.
//
// Every pass is a multi-tensor walk over the plan's chunk table: one
// workgroup per chunk of up to kChunkElems elements, where a chunk lies
// inside one bucket and so has one owner class.  A lane owns 4-element
// vectors v = lane, lane + kBlock, lane + 2*kBlock, ... of its chunk, so
// every memory instruction of a wave covers one contiguous range: 1 KB of
// FP32 (a 128-bit access per lane) or 512 B of BF16 (64-bit per lane).
// kUnroll vectors per lane are loaded before any is consumed, to keep enough
// bytes in flight to cover HBM latency.  The path is bound by HBM bandwidth,
// not by a contraction, so there is no MFMA here.
//
// Arithmetic follows NeMo Automodel issue #3857, "refactor(distributed):
// establish shared native TP replica ownership" ("Why this needs separate
// work": Replicate averaged, Partial summed, Shard and already-reduced
// gradients left alone; "Preserved prototype and evidence": FP32 reduction,
// accumulation with partial windows, clipping, Adam updates).  Each
// floating-point step is one IEEE-rounded FP32 operation in a fixed order
// (the library is built without contraction), so results are reproducible
// bit for bit.
//
// Workgroup placement is XCD-aware: in the accumulate and norm passes chunk q
// runs in a workgroup whose index is congruent to q modulo 8, and the
// hardware deals workgroups to the eight XCDs round-robin, so a chunk visits
// the same XCD (and its L2) in each of them.  AdamW walks the chunks in
// reverse (see k_adamw).
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace gro {
namespace {

// Launch-shape knobs (compile-time; the chunking itself is fixed by the
// plan).  The norm's per-chunk summation order depends on kBlock, so a
// build has one fixed value.
#ifndef GRO_BLOCK
#define GRO_BLOCK 256
#endif
#ifndef GRO_UNROLL
#define GRO_UNROLL 2
#endif

constexpr int kBlock = GRO_BLOCK;      // lanes per workgroup (waves of 64)
constexpr int kWaves = kBlock / 64;
#ifndef GRO_UNROLL_ADAMW
// A full AdamW chunk in one sweep: 16 independent 16-byte loads per lane
// (120 VGPRs, 4 waves per SIMD) beat 8 loads at 5 waves per SIMD.
#define GRO_UNROLL_ADAMW 4
#endif
#ifndef GRO_ADAMW_MIN_BLOCKS
#define GRO_ADAMW_MIN_BLOCKS 1
#endif
#ifndef GRO_UNROLL_ACC
#define GRO_UNROLL_ACC GRO_UNROLL
#endif
#ifndef GRO_UNROLL_WIN
#define GRO_UNROLL_WIN GRO_UNROLL
#endif
// Window lengths up to this many microbatches issue every microbatch's loads
// at once (window_full_n); longer ones pipeline microbatch by microbatch.
#ifndef GRO_WIN_ALL_AT_ONCE
#define GRO_WIN_ALL_AT_ONCE 8
#endif
constexpr int kUnroll = GRO_UNROLL;    // 4-element vectors in flight per lane
constexpr int kUnrollWin = GRO_UNROLL_WIN;  // the same for the full-chunk window paths
static_assert((kChunkElems / 4) % (kUnrollWin * kBlock) == 0, "whole window sweeps per chunk");
constexpr int kUnrollAcc = GRO_UNROLL_ACC;  // the same for the one-microbatch full-chunk pass
static_assert((kChunkElems / 4) % (kUnrollAcc * kBlock) == 0, "whole accumulate sweeps per chunk");
constexpr int kUnrollAdam = GRO_UNROLL_ADAMW;
static_assert((kChunkElems / 4) % (kUnrollAdam * kBlock) == 0, "whole AdamW sweeps per chunk");
static_assert(kBlock % 64 == 0 && kBlock <= 1024, "whole wave64s");
static_assert(kChunkElems % (4 * kBlock) == 0, "chunks are whole workgroup tiles");

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// x / d for a positive integer d.  When d is a power of two its reciprocal
// is exact and x * (1/d) is the same correctly rounded value as x / d, so
// the multiply is used; otherwise an IEEE division.
struct Divisor {
  float d;
  float inv;
  int pow2;
};

__host__ __device__ inline Divisor make_divisor(int d) {
  Divisor r;
  r.d = float(d);
  r.inv = 1.0f / float(d);
  r.pow2 = (d & (d - 1)) == 0;
  return r;
}

__device__ __forceinline__ float divide(float x, const Divisor& q) {
  return q.pow2 ? x * q.inv : x / q.d;
}

// The same choice made at compile time, for the branch-free full-chunk paths:
// kNoDiv (nothing to divide), kMulInv (power-of-two divisor), kIeeeDiv.
enum DivMode { kNoDiv = 0, kMulInv = 1, kIeeeDiv = 2 };
__host__ __device__ inline int div_mode(const Divisor& q) { return q.pow2 ? kMulInv : kIeeeDiv; }
template <int M>
__device__ __forceinline__ float divide_m(float x, const Divisor& q) {
  if constexpr (M == kMulInv) return x * q.inv;
  else if constexpr (M == kIeeeDiv) return x / q.d;
  else return x;
}

// Four BF16 (two 32-bit words, element 0 in the low half) widened exactly.
__device__ __forceinline__ f32x4 widen4(const u32x2 r) {
  f32x4 x;
  x.x = __uint_as_float(r.x << 16);
  x.y = __uint_as_float(r.x & 0xffff0000u);
  x.z = __uint_as_float(r.y << 16);
  x.w = __uint_as_float(r.y & 0xffff0000u);
  return x;
}

__device__ __forceinline__ float widen1(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// FP32 -> BF16, round to nearest even, two per v_cvt_pk_bf16_f32:
// lo in bits 0..15, hi in 16..31.
__device__ __forceinline__ uint32_t bf16x2_bits(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
__device__ __forceinline__ uint16_t bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

__device__ __forceinline__ f32x4 ld4f(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ void st4f(float* p, const f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }
// Streaming variants with the non-temporal cache policy.  They are used for
// every stream a step touches once -- the gradient contributions and
// AdamW's p, m, v and BF16 copy -- so that these do not push the FP32
// accumulator out of the memory-side Infinity Cache between the pass that
// writes it and the AdamW pass that reads it, and so that AdamW leaves few
// dirty lines for the next step's first pass to drain.  The accumulator
// itself keeps the default policy.
__device__ __forceinline__ u32x2 ld2u_nt(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
}
__device__ __forceinline__ f32x4 ld4f_nt(const float* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
}
__device__ __forceinline__ void st4f_nt(float* p, const f32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p));
}
__device__ __forceinline__ void st2u_nt(uint16_t* p, const u32x2 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(p));
}
// An accumulator store with the policy fixed at compile time (a run-time
// choice between the two stores is merged into one plain store by the
// compiler).
template <bool NT>
__device__ __forceinline__ void st4f_acc(float* p, const f32x4 v) {
  if constexpr (NT) st4f_nt(p, v);
  else st4f(p, v);
}

// Sum over the workgroup in a fixed order: a wave64 butterfly (every lane
// ends with the same bits because IEEE addition commutes), then the wave
// totals in wave order.  Returned in every lane.
__device__ double block_sum(double x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  __shared__ double part[kWaves];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
  __syncthreads();
  double t = part[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) t += part[w];
  return t;
}

// Chunk index of this workgroup, placed so that q == blockIdx.x (mod 8).
__device__ __forceinline__ int64_t chunk_of_block(int64_t q_begin) {
  return q_begin - (q_begin & 7) + int64_t(blockIdx.x);
}

// The window pass's chunk placement: 0 as chunk_of_block; 1 gives each of
// the eight XCDs (workgroup index mod 8 under round-robin dispatch) one
// contiguous eighth of the range.
#ifndef GRO_WIN_MAP
#define GRO_WIN_MAP 0
#endif
__device__ __forceinline__ int64_t window_chunk_of_block(int64_t q_begin, int64_t q_end) {
  if (GRO_WIN_MAP == 0) return chunk_of_block(q_begin);
  const int64_t per = (q_end - q_begin + 7) >> 3;
  return q_begin + int64_t(blockIdx.x & 7) * per + int64_t(blockIdx.x >> 3);
}

__device__ __forceinline__ double sq(float x) {
  const double d = double(x);
  return d * d;
}

// ------------------------------------------------------ gradient inputs
// A bucket's gradient contributions are BF16 (widened exactly) or FP32 (used
// as they are); the element type is a template parameter of every path.
// Vector loads of contributions are non-temporal (each is read once a step).
struct Bf16In {
  typedef u32x2 raw_t;
  static __device__ __forceinline__ raw_t load(const void* base, int64_t e) {
    return ld2u_nt(static_cast<const uint16_t*>(base) + e);
  }
  static __device__ __forceinline__ f32x4 widen(const raw_t r) { return widen4(r); }
  static __device__ __forceinline__ float load1(const void* base, int64_t i) {
    return widen1(static_cast<const uint16_t*>(base)[i]);
  }
};
struct F32In {
  typedef f32x4 raw_t;
  static __device__ __forceinline__ raw_t load(const void* base, int64_t e) {
    return ld4f_nt(static_cast<const float*>(base) + e);
  }
  static __device__ __forceinline__ f32x4 widen(const raw_t r) { return r; }
  static __device__ __forceinline__ float load1(const void* base, int64_t i) {
    return static_cast<const float*>(base)[i];
  }
};

// ------------------------------------------------------------ accumulate
struct AccChunk {
  const void* g;       // the bucket's gradient buffer [slots][stride]
  int64_t off;         // this chunk's first element inside the bucket
  int64_t stride;      // slot stride (elements)
  float* acc;          // this chunk in the flat accumulator
  int len;
  int slots;
  bool mean;
  bool first;          // first microbatch of the window: overwrite
  bool fuse;           // also sum (acc/window)^2 for the norm
  Divisor rdiv;        // R, for MEAN
  Divisor wdiv;        // window length, for the norm
};

// One element's reduction: slots summed in slot order, then /R for MEAN.
// (The vector paths perform exactly these operations lane-wise.)
template <typename In>
__device__ __forceinline__ float reduce1(const AccChunk& c, int i) {
  float s = In::load1(c.g, c.off + i);
  for (int r = 1; r < c.slots; ++r) s = s + In::load1(c.g, int64_t(r) * c.stride + c.off + i);
  return c.mean ? divide(s, c.rdiv) : s;
}

// Ragged tail [4*nvec, len): handled by the lane that owns vector nvec, after
// its full vectors, so the lane's element order stays ascending.
template <typename In>
__device__ __forceinline__ double accumulate_tail(const AccChunk& c, int nvec) {
  double ss = 0.0;
  if ((c.len & 3) && int(threadIdx.x) == nvec % kBlock) {
    for (int i = nvec * 4; i < c.len; ++i) {
      float s = reduce1<In>(c, i);
      if (!c.first) s = c.acc[i] + s;
      c.acc[i] = s;
      if (c.fuse) ss += sq(divide(s, c.wdiv));
    }
  }
  return ss;
}

// Per element: widen the slots, sum them in slot order, divide by R for
// MEAN, then start or extend the accumulator.  Returns this lane's FP64 sum
// of (acc/window)^2 over its elements (0 unless fuse), in the lane's element
// order: its vectors in ascending order, each vector's elements in order,
// then the tail.  Any chunk length and slot count; runtime choices.
template <typename In>
__device__ double accumulate_generic(const AccChunk& c) {
  const int nvec = c.len >> 2;
  double ss = 0.0;
  for (int v0 = threadIdx.x; v0 < nvec; v0 += kUnroll * kBlock) {
    f32x4 red[kUnroll];
    f32x4 old[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int v = v0 + u * kBlock;
      if (v < nvec) {
        red[u] = In::widen(In::load(c.g, c.off + 4 * v));
        for (int r = 1; r < c.slots; ++r)
          red[u] = red[u] + In::widen(In::load(c.g, int64_t(r) * c.stride + c.off + 4 * v));
        if (!c.first) old[u] = ld4f(c.acc + 4 * v);
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int v = v0 + u * kBlock;
      if (v < nvec) {
        f32x4 s = red[u];
        if (c.mean) {
          s.x = divide(s.x, c.rdiv);
          s.y = divide(s.y, c.rdiv);
          s.z = divide(s.z, c.rdiv);
          s.w = divide(s.w, c.rdiv);
        }
        if (!c.first) s = old[u] + s;
        st4f(c.acc + 4 * v, s);
        if (c.fuse) {
          ss += sq(divide(s.x, c.wdiv));
          ss += sq(divide(s.y, c.wdiv));
          ss += sq(divide(s.z, c.wdiv));
          ss += sq(divide(s.w, c.wdiv));
        }
      }
    }
  }
  return ss + accumulate_tail<In>(c, nvec);
}

// A full chunk (len == kChunkElems) with every choice fixed at compile time:
// C slots, RM how the slot sum is divided (kNoDiv, or kMulInv for MEAN at
// R = 2), FIRST whether the window starts here, WM the window division for
// the fused norm (kNoDiv = no norm).  Same operations, same order as
// accumulate_generic, without bounds checks or per-element branches.
template <typename In, int C, int RM, bool FIRST, int WM, bool NT>
__device__ double accumulate_full(const AccChunk& c) {
  constexpr int nvec = kChunkElems / 4;
  double ss = 0.0;
#pragma unroll 1
  for (int v0 = threadIdx.x; v0 < nvec; v0 += kUnrollAcc * kBlock) {
    f32x4 red[kUnrollAcc];
    f32x4 old[kUnrollAcc];
#pragma unroll
    for (int u = 0; u < kUnrollAcc; ++u) {
      const int v = v0 + u * kBlock;
      typename In::raw_t raw[C];
#pragma unroll
      for (int r = 0; r < C; ++r) raw[r] = In::load(c.g, int64_t(r) * c.stride + c.off + 4 * v);
      if (!FIRST) old[u] = ld4f(c.acc + 4 * v);
      red[u] = In::widen(raw[0]);
#pragma unroll
      for (int r = 1; r < C; ++r) red[u] = red[u] + In::widen(raw[r]);
    }
#pragma unroll
    for (int u = 0; u < kUnrollAcc; ++u) {
      const int v = v0 + u * kBlock;
      f32x4 s = red[u];
      s.x = divide_m<RM>(s.x, c.rdiv);
      s.y = divide_m<RM>(s.y, c.rdiv);
      s.z = divide_m<RM>(s.z, c.rdiv);
      s.w = divide_m<RM>(s.w, c.rdiv);
      if (!FIRST) s = old[u] + s;
      st4f_acc<NT>(c.acc + 4 * v, s);
      if (WM != kNoDiv) {
        ss += sq(divide_m<WM>(s.x, c.wdiv));
        ss += sq(divide_m<WM>(s.y, c.wdiv));
        ss += sq(divide_m<WM>(s.z, c.wdiv));
        ss += sq(divide_m<WM>(s.w, c.wdiv));
      }
    }
  }
  return ss;
}

template <typename In, int C, int RM, bool NT>
__device__ double accumulate_full_dispatch(const AccChunk& c) {
  const int wm = c.fuse ? div_mode(c.wdiv) : kNoDiv;
  if (c.first) {
    if (wm == kNoDiv) return accumulate_full<In, C, RM, true, kNoDiv, NT>(c);
    if (wm == kMulInv) return accumulate_full<In, C, RM, true, kMulInv, NT>(c);
    return accumulate_full<In, C, RM, true, kIeeeDiv, NT>(c);
  }
  if (wm == kNoDiv) return accumulate_full<In, C, RM, false, kNoDiv, NT>(c);
  if (wm == kMulInv) return accumulate_full<In, C, RM, false, kMulInv, NT>(c);
  return accumulate_full<In, C, RM, false, kIeeeDiv, NT>(c);
}

template <typename In, bool NT>
__device__ double accumulate_chunk(const AccChunk& c) {
  if (c.len == kChunkElems && c.slots == 1 && !c.mean) return accumulate_full_dispatch<In, 1, kNoDiv, NT>(c);
  if (c.len == kChunkElems && c.slots == 2 && !c.mean) return accumulate_full_dispatch<In, 2, kNoDiv, NT>(c);
  if (c.len == kChunkElems && c.slots == 2 && c.rdiv.pow2) return accumulate_full_dispatch<In, 2, kMulInv, NT>(c);
  return accumulate_generic<In>(c);
}

// NT: full chunks store the accumulator non-temporally (one kernel per
// policy, chosen by the launcher).
template <bool NT>
__global__ __launch_bounds__(kBlock) void k_accumulate(const AccumulateLaunch P) {
  const int64_t q = chunk_of_block(P.q_begin);
  if (q < P.q_begin || q >= P.q_end) return;
  const ChunkDev ch = P.chunks[q];
  const BucketDev bk = P.buckets[ch.bucket];
  AccChunk c;
  c.g = P.grads[ch.bucket - P.b_first];
  c.off = ch.begin - bk.base;
  c.stride = bk.stride;
  c.acc = P.acc + ch.begin;
  c.len = ch.len;
  c.slots = bk.slots;
  c.mean = bk.owner == GRO_OWNER_MEAN;
  c.first = P.micro_index == 0;
  c.fuse = P.fuse_norm != 0;
  c.rdiv = make_divisor(P.R);
  c.wdiv = make_divisor(P.window > 0 ? P.window : 1);
  const double ss = bk.grad_fp32 ? accumulate_chunk<F32In, NT>(c) : accumulate_chunk<Bf16In, NT>(c);
  if (c.fuse) {
    const double t = block_sum(ss);
    if (threadIdx.x == 0) P.partials[q] = t;
  }
}

// ------------------------------------------------- accumulate a window
// Several microbatches of a window in one pass: for every element, the
// group's reductions are accumulated in registers in microbatch order --
// starting from red_0 when the group opens the window (`first`), else from
// the accumulator in memory -- the same operations as one accumulate pass per
// microbatch, and the accumulator is written once.  When the group closes the
// window (`fuse`) the norm partial is written too.
struct WinChunk {
  const WindowLaunch* P;
  int64_t off;         // chunk offset inside its bucket
  int64_t stride;
  int j;               // bucket index within the launch
  float* acc;
  int len;
  int slots;
  bool mean;
  bool first;          // the group starts the window: overwrite the accumulator
  bool fuse;           // the group ends the window: also sum (acc/window)^2
  Divisor rdiv;
  Divisor wdiv;
  __device__ const void* g(int k) const { return P->grads[k * P->n_buckets + j]; }
};

template <typename In>
__device__ __forceinline__ float win_reduce1(const WinChunk& c, int k, int i) {
  const void* g = c.g(k);
  float s = In::load1(g, c.off + i);
  for (int r = 1; r < c.slots; ++r) s = s + In::load1(g, int64_t(r) * c.stride + c.off + i);
  return c.mean ? divide(s, c.rdiv) : s;
}

// Any chunk, any slot count: runtime checks, same order.
template <typename In>
__device__ double window_generic(const WinChunk& c) {
  const int n = c.P->n_micro;
  const int nvec = c.len >> 2;
  double ss = 0.0;
  for (int v = threadIdx.x; v < nvec; v += kBlock) {
    f32x4 acc;
    if (!c.first) acc = ld4f(c.acc + 4 * v);
    for (int k = 0; k < n; ++k) {
      const void* g = c.g(k);
      f32x4 red = In::widen(In::load(g, c.off + 4 * v));
      for (int r = 1; r < c.slots; ++r) red = red + In::widen(In::load(g, int64_t(r) * c.stride + c.off + 4 * v));
      if (c.mean) {
        red.x = divide(red.x, c.rdiv);
        red.y = divide(red.y, c.rdiv);
        red.z = divide(red.z, c.rdiv);
        red.w = divide(red.w, c.rdiv);
      }
      acc = (c.first && k == 0) ? red : acc + red;
    }
    st4f(c.acc + 4 * v, acc);
    if (c.fuse) {
      ss += sq(divide(acc.x, c.wdiv));
      ss += sq(divide(acc.y, c.wdiv));
      ss += sq(divide(acc.z, c.wdiv));
      ss += sq(divide(acc.w, c.wdiv));
    }
  }
  if ((c.len & 3) && int(threadIdx.x) == nvec % kBlock) {
    for (int i = nvec * 4; i < c.len; ++i) {
      float a = c.first ? win_reduce1<In>(c, 0, i) : c.acc[i] + win_reduce1<In>(c, 0, i);
      for (int k = 1; k < n; ++k) a = a + win_reduce1<In>(c, k, i);
      c.acc[i] = a;
      if (c.fuse) ss += sq(divide(a, c.wdiv));
    }
  }
  return ss;
}

// A full chunk with C slots, the MEAN divisor mode RM, the window divisor
// mode WM (kNoDiv: no norm partial) and FIRST (the group opens the window)
// fixed at compile time, any number of microbatches.  Microbatch k+1's loads
// are issued before microbatch k's data is consumed.
template <typename In, int C, int RM, int WM, bool FIRST, bool NT>
__device__ double window_full(const WinChunk& c) {
  constexpr int nvec = kChunkElems / 4;
  const int n = c.P->n_micro;
  double ss = 0.0;
#pragma unroll 1
  for (int v0 = threadIdx.x; v0 < nvec; v0 += kUnrollWin * kBlock) {
    f32x4 acc[kUnrollWin];
    typename In::raw_t cur[kUnrollWin][C], nxt[kUnrollWin][C];
    {
      const void* g = c.g(0);
#pragma unroll
      for (int u = 0; u < kUnrollWin; ++u) {
#pragma unroll
        for (int r = 0; r < C; ++r) cur[u][r] = In::load(g, int64_t(r) * c.stride + c.off + 4 * (v0 + u * kBlock));
        if (!FIRST) acc[u] = ld4f(c.acc + 4 * (v0 + u * kBlock));
      }
    }
#pragma unroll 1
    for (int k = 0; k < n; ++k) {
      if (k + 1 < n) {
        const void* g = c.g(k + 1);
#pragma unroll
        for (int u = 0; u < kUnrollWin; ++u)
#pragma unroll
          for (int r = 0; r < C; ++r) nxt[u][r] = In::load(g, int64_t(r) * c.stride + c.off + 4 * (v0 + u * kBlock));
      }
#pragma unroll
      for (int u = 0; u < kUnrollWin; ++u) {
        f32x4 red = In::widen(cur[u][0]);
#pragma unroll
        for (int r = 1; r < C; ++r) red = red + In::widen(cur[u][r]);
        red.x = divide_m<RM>(red.x, c.rdiv);
        red.y = divide_m<RM>(red.y, c.rdiv);
        red.z = divide_m<RM>(red.z, c.rdiv);
        red.w = divide_m<RM>(red.w, c.rdiv);
        acc[u] = (FIRST && k == 0) ? red : acc[u] + red;
      }
#pragma unroll
      for (int u = 0; u < kUnrollWin; ++u)
#pragma unroll
        for (int r = 0; r < C; ++r) cur[u][r] = nxt[u][r];
    }
#pragma unroll
    for (int u = 0; u < kUnrollWin; ++u) {
      st4f_acc<NT>(c.acc + 4 * (v0 + u * kBlock), acc[u]);
      if (WM != kNoDiv) {
        ss += sq(divide_m<WM>(acc[u].x, c.wdiv));
        ss += sq(divide_m<WM>(acc[u].y, c.wdiv));
        ss += sq(divide_m<WM>(acc[u].z, c.wdiv));
        ss += sq(divide_m<WM>(acc[u].w, c.wdiv));
      }
    }
  }
  return ss;
}

// Common window lengths: every microbatch's loads are issued before any
// is consumed (N * C * kUnrollWin loads in flight per lane).
template <typename In, int C, int RM, int WM, int N, bool NT>
__device__ double window_full_n(const WinChunk& c) {
  constexpr int nvec = kChunkElems / 4;
  double ss = 0.0;
#pragma unroll 1
  for (int v0 = threadIdx.x; v0 < nvec; v0 += kUnrollWin * kBlock) {
    typename In::raw_t raw[N][kUnrollWin][C];
#pragma unroll
    for (int k = 0; k < N; ++k) {
      const void* g = c.g(k);
#pragma unroll
      for (int u = 0; u < kUnrollWin; ++u)
#pragma unroll
        for (int r = 0; r < C; ++r) raw[k][u][r] = In::load(g, int64_t(r) * c.stride + c.off + 4 * (v0 + u * kBlock));
    }
#pragma unroll
    for (int u = 0; u < kUnrollWin; ++u) {
      f32x4 acc;
#pragma unroll
      for (int k = 0; k < N; ++k) {
        f32x4 red = In::widen(raw[k][u][0]);
#pragma unroll
        for (int r = 1; r < C; ++r) red = red + In::widen(raw[k][u][r]);
        red.x = divide_m<RM>(red.x, c.rdiv);
        red.y = divide_m<RM>(red.y, c.rdiv);
        red.z = divide_m<RM>(red.z, c.rdiv);
        red.w = divide_m<RM>(red.w, c.rdiv);
        acc = k == 0 ? red : acc + red;
      }
      st4f_acc<NT>(c.acc + 4 * (v0 + u * kBlock), acc);
      ss += sq(divide_m<WM>(acc.x, c.wdiv));
      ss += sq(divide_m<WM>(acc.y, c.wdiv));
      ss += sq(divide_m<WM>(acc.z, c.wdiv));
      ss += sq(divide_m<WM>(acc.w, c.wdiv));
    }
  }
  return ss;
}

template <typename In, int C, int RM, int WM, bool NT>
__device__ double window_full_w(const WinChunk& c) {
  // FP32 contributions take twice the registers: keep them double-buffered.
  if (sizeof(typename In::raw_t) > 8) return window_full<In, C, RM, WM, true, NT>(c);
  const int n = c.P->n_micro;
  if (n > GRO_WIN_ALL_AT_ONCE) return window_full<In, C, RM, WM, true, NT>(c);
  switch (n) {
    case 2: return window_full_n<In, C, RM, WM, 2, NT>(c);
    case 3: return window_full_n<In, C, RM, WM, 3, NT>(c);
    case 4: return window_full_n<In, C, RM, WM, 4, NT>(c);
    case 8: return window_full_n<In, C, RM, WM, 8, NT>(c);
    default: return window_full<In, C, RM, WM, true, NT>(c);
  }
}

template <typename In, int C, int RM, bool NT>
__device__ double window_full_dispatch(const WinChunk& c) {
  if (c.first && c.fuse)  // a whole window in one pass
    return c.wdiv.pow2 ? window_full_w<In, C, RM, kMulInv, NT>(c) : window_full_w<In, C, RM, kIeeeDiv, NT>(c);
  // a group of microbatches inside a window
  if (!c.fuse)
    return c.first ? window_full<In, C, RM, kNoDiv, true, NT>(c) : window_full<In, C, RM, kNoDiv, false, NT>(c);
  return c.wdiv.pow2 ? window_full<In, C, RM, kMulInv, false, NT>(c) : window_full<In, C, RM, kIeeeDiv, false, NT>(c);
}

template <typename In, bool NT>
__device__ double window_chunk(const WinChunk& c) {
  if (c.len == kChunkElems && c.slots == 1 && !c.mean) return window_full_dispatch<In, 1, kNoDiv, NT>(c);
  if (c.len == kChunkElems && c.slots == 2 && !c.mean) return window_full_dispatch<In, 2, kNoDiv, NT>(c);
  if (c.len == kChunkElems && c.slots == 2 && c.rdiv.pow2) return window_full_dispatch<In, 2, kMulInv, NT>(c);
  return window_generic<In>(c);
}

template <bool NT>
__global__ __launch_bounds__(kBlock) void k_accumulate_window(const WindowLaunch P) {
  const int64_t q = window_chunk_of_block(P.q_begin, P.q_end);
  if (q < P.q_begin || q >= P.q_end) return;
  const ChunkDev ch = P.chunks[q];
  const BucketDev bk = P.buckets[ch.bucket];
  WinChunk c;
  c.P = &P;
  c.off = ch.begin - bk.base;
  c.stride = bk.stride;
  c.j = ch.bucket - P.b_first;
  c.acc = P.acc + ch.begin;
  c.len = ch.len;
  c.slots = bk.slots;
  c.mean = bk.owner == GRO_OWNER_MEAN;
  c.first = P.first != 0;
  c.fuse = P.fuse_norm != 0;
  c.rdiv = make_divisor(P.R);
  c.wdiv = make_divisor(P.window > 0 ? P.window : 1);
  const double ss = bk.grad_fp32 ? window_chunk<F32In, NT>(c) : window_chunk<Bf16In, NT>(c);
  if (c.fuse) {
    const double t = block_sum(ss);
    if (threadIdx.x == 0) P.partials[q] = t;
  }
}

// ------------------------------------------------------- norm, stage 1
// Lane's sum of (acc/window)^2 over its vectors of a full chunk.
template <int WM>
__device__ double sumsq_full(const float* acc, const Divisor& wdiv) {
  constexpr int nvec = kChunkElems / 4;
  double ss = 0.0;
#pragma unroll 1
  for (int v0 = threadIdx.x; v0 < nvec; v0 += kUnroll * kBlock) {
    f32x4 a[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) a[u] = ld4f(acc + 4 * (v0 + u * kBlock));
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      ss += sq(divide_m<WM>(a[u].x, wdiv));
      ss += sq(divide_m<WM>(a[u].y, wdiv));
      ss += sq(divide_m<WM>(a[u].z, wdiv));
      ss += sq(divide_m<WM>(a[u].w, wdiv));
    }
  }
  return ss;
}

// Same, any length, with the ragged tail.
__device__ double sumsq_generic(const float* acc, int len, const Divisor& wdiv) {
  const int nvec = len >> 2;
  double ss = 0.0;
  for (int v0 = threadIdx.x; v0 < nvec; v0 += kUnroll * kBlock) {
    f32x4 a[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int v = v0 + u * kBlock;
      if (v < nvec) a[u] = ld4f(acc + 4 * v);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int v = v0 + u * kBlock;
      if (v < nvec) {
        ss += sq(divide(a[u].x, wdiv));
        ss += sq(divide(a[u].y, wdiv));
        ss += sq(divide(a[u].z, wdiv));
        ss += sq(divide(a[u].w, wdiv));
      }
    }
  }
  if ((len & 3) && int(threadIdx.x) == nvec % kBlock) {
    for (int i = nvec * 4; i < len; ++i) ss += sq(divide(acc[i], wdiv));
  }
  return ss;
}

// Same lane/element order as the fused accumulate, so a chunk's partial is
// the same bits whichever kernel wrote it.
__global__ __launch_bounds__(kBlock) void k_norm_partials(const NormLaunch P) {
  const int64_t q = chunk_of_block(P.q_begin);
  if (q < P.q_begin || q >= P.q_end) return;
  const ChunkDev ch = P.chunks[q];
  const float* acc = P.acc + ch.begin;
  const Divisor wdiv = make_divisor(P.window);
  double ss;
  if (ch.len == kChunkElems)
    ss = wdiv.pow2 ? sumsq_full<kMulInv>(acc, wdiv) : sumsq_full<kIeeeDiv>(acc, wdiv);
  else
    ss = sumsq_generic(acc, ch.len, wdiv);
  const double t = block_sum(ss);
  if (threadIdx.x == 0) P.partials[q] = t;
}

// ------------------------------------------------------- norm, stage 2
// Two fixed-order levels, so the result never depends on launch shape or on
// which workgroup runs when:
//   group sum j = the kNormGroup partials from kNormGroup*j on: lane t adds
//                 partials kNormGroup*j + t + kBlock*i for i = 0, 1, ... in
//                 that order, then a butterfly and the wave totals in order;
//   total       = the group sums, lane t adding sums t, t + kBlock, ... in
//                 order, then a butterfly and the wave totals in order.
// One workgroup per group.  The workgroup that finishes last -- found with a
// completion counter, which it returns to zero -- adds the group sums and
// writes the norm.  The counter only says who is last; no atomic operation
// touches a sum.
constexpr int kGroupPerLane = int(kNormGroup / kBlock);
static_assert(kNormGroup % kBlock == 0, "whole lanes per group");

__device__ __forceinline__ void write_norm(double t, double* scalars) {
  scalars[kNormSq] = t;
  scalars[kNorm] = sqrt(t);
  scalars[kFinite] = __builtin_isfinite(t) ? 1.0 : 0.0;
}

__global__ __launch_bounds__(kBlock) void k_norm_final(const NormFinalLaunch P) {
  const int64_t J = norm_groups(P.n_chunks);
  if (J == 0) {  // nothing owned: the norm of no elements
    if (threadIdx.x == 0) write_norm(0.0, P.scalars);
    return;
  }
  const int64_t q0 = int64_t(blockIdx.x) * kNormGroup + threadIdx.x;
  double x[kGroupPerLane];
#pragma unroll
  for (int i = 0; i < kGroupPerLane; ++i) {  // all loads issued before any add
    const int64_t q = q0 + int64_t(i) * kBlock;
    x[i] = q < P.n_chunks ? P.partials[q] : 0.0;
  }
  double s = x[0];
#pragma unroll
  for (int i = 1; i < kGroupPerLane; ++i) s += x[i];
  const double sj = block_sum(s);
  __shared__ int last;
  if (threadIdx.x == 0) {
    P.group_sums[blockIdx.x] = sj;
    __threadfence();  // the group sum is visible before the count says so
    last = atomicAdd(P.counter, 1u) == uint32_t(J - 1);
  }
  __syncthreads();
  if (!last) return;
  __threadfence();    // and every other group's sum is visible here
  double t = 0.0;
  for (int64_t j = threadIdx.x; j < J; j += kBlock) t += P.group_sums[j];
  const double total = block_sum(t);
  if (threadIdx.x == 0) {
    write_norm(total, P.scalars);
    *P.counter = 0u;
  }
}

// ------------------------------------------------------- clip + AdamW
struct AdamScalars {
  Divisor wdiv;
  float coef, decay, b1, b2, omb1, omb2, step_size, sbc2, eps;
};

// g = acc/n; g^ = g*coef; p = p*decay; m = b1*m + (1-b1)*g^;
// v = b2*v + (1-b2)*(g^*g^); p = p - step_size*(m/(sqrt(v)/sqrt_bc2 + eps)).
template <int WM>
__device__ __forceinline__ void adamw_elem(float a, float& p, float& m, float& v, const AdamScalars& k) {
  const float g = WM == kNoDiv ? divide(a, k.wdiv) : divide_m<WM>(a, k.wdiv);
  const float gh = g * k.coef;
  p = p * k.decay;
  m = k.b1 * m + k.omb1 * gh;
  v = k.b2 * v + k.omb2 * (gh * gh);
  const float d = sqrtf(v) / k.sbc2 + k.eps;
  p = p - k.step_size * (m / d);
}

template <int WM>
__device__ __forceinline__ void adamw4(const f32x4 a, f32x4& p, f32x4& m, f32x4& v, const AdamScalars& k) {
  float pp[4] = {p.x, p.y, p.z, p.w}, mm[4] = {m.x, m.y, m.z, m.w}, vv[4] = {v.x, v.y, v.z, v.w};
  const float aa[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) adamw_elem<WM>(aa[e], pp[e], mm[e], vv[e], k);
  p = f32x4{pp[0], pp[1], pp[2], pp[3]};
  m = f32x4{mm[0], mm[1], mm[2], mm[3]};
  v = f32x4{vv[0], vv[1], vv[2], vv[3]};
}

struct AdamChunk {
  const float* acc;
  float* p;
  float* m;
  float* v;
  uint16_t* pb;   // BF16 copy, may be null
  int len;
};

__device__ __forceinline__ void store_bf16x4(uint16_t* pb, const f32x4 p) {
  st2u_nt(pb, u32x2{bf16x2_bits(p.x, p.y), bf16x2_bits(p.z, p.w)});
}

// The accumulator's load: the default policy, so that a step's last
// accumulate pass's final stretch is met in the Infinity Cache, or (NT) the
// non-temporal one, for accumulators that pass stored non-temporally.
template <bool NT>
__device__ __forceinline__ f32x4 ld4f_acc(const float* p) {
  if constexpr (NT) return ld4f_nt(p);
  else return ld4f(p);
}

// Any chunk: runtime window division, bounds checks, ragged tail.
template <bool NT>
__device__ void adamw_generic(const AdamChunk& c, const AdamScalars& k) {
  const int nvec = c.len >> 2;
  for (int v0 = threadIdx.x; v0 < nvec; v0 += kUnroll * kBlock) {
    f32x4 a[kUnroll], p[kUnroll], m[kUnroll], w[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int v = v0 + u * kBlock;
      if (v < nvec) {
        a[u] = ld4f_acc<NT>(c.acc + 4 * v);
        p[u] = ld4f_nt(c.p + 4 * v);
        m[u] = ld4f_nt(c.m + 4 * v);
        w[u] = ld4f_nt(c.v + 4 * v);
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int v = v0 + u * kBlock;
      if (v < nvec) {
        adamw4<kNoDiv>(a[u], p[u], m[u], w[u], k);
        st4f_nt(c.p + 4 * v, p[u]);
        st4f_nt(c.m + 4 * v, m[u]);
        st4f_nt(c.v + 4 * v, w[u]);
        if (c.pb) store_bf16x4(c.pb + 4 * v, p[u]);
      }
    }
  }
  if ((c.len & 3) && int(threadIdx.x) == nvec % kBlock) {
    for (int i = nvec * 4; i < c.len; ++i) {
      float p1 = c.p[i], m1 = c.m[i], v1 = c.v[i];
      adamw_elem<kNoDiv>(c.acc[i], p1, m1, v1, k);
      c.p[i] = p1;
      c.m[i] = m1;
      c.v[i] = v1;
      if (c.pb) c.pb[i] = bf16_bits(p1);
    }
  }
}

// A full chunk with the window division (WM) and the BF16 copy fixed at
// compile time: no bounds checks, no per-element branches.
template <int WM, bool BF16, bool NT>
__device__ void adamw_full(const AdamChunk& c, const AdamScalars& k) {
  constexpr int nvec = kChunkElems / 4;
#pragma unroll 1
  for (int v0 = threadIdx.x; v0 < nvec; v0 += kUnrollAdam * kBlock) {
    f32x4 a[kUnrollAdam], p[kUnrollAdam], m[kUnrollAdam], w[kUnrollAdam];
#pragma unroll
    for (int u = 0; u < kUnrollAdam; ++u) {
      const int v = v0 + u * kBlock;
      a[u] = ld4f_acc<NT>(c.acc + 4 * v);
      p[u] = ld4f_nt(c.p + 4 * v);
      m[u] = ld4f_nt(c.m + 4 * v);
      w[u] = ld4f_nt(c.v + 4 * v);
    }
#pragma unroll
    for (int u = 0; u < kUnrollAdam; ++u) {
      const int v = v0 + u * kBlock;
      adamw4<WM>(a[u], p[u], m[u], w[u], k);
      st4f_nt(c.p + 4 * v, p[u]);
      st4f_nt(c.m + 4 * v, m[u]);
      st4f_nt(c.v + 4 * v, w[u]);
      if (BF16) store_bf16x4(c.pb + 4 * v, p[u]);
    }
  }
}

// Chunks are visited last to first: the step's last accumulate pass has just
// written the accumulator front to back, so its final stretch is still in
// the MI355X's memory-side Infinity Cache when this pass starts.
#ifndef GRO_ADAMW_FORWARD
#define GRO_ADAMW_FORWARD 0
#endif
template <bool NT>
__global__ __launch_bounds__(kBlock, GRO_ADAMW_MIN_BLOCKS) void k_adamw(const AdamWLaunch P) {
  const int64_t q = GRO_ADAMW_FORWARD ? int64_t(blockIdx.x) : P.n_chunks - 1 - int64_t(blockIdx.x);
  if (q >= P.n_chunks) return;
  if (P.scalars[kFinite] == 0.0) return;  // non-finite norm: skip the step
  AdamScalars k;
  k.coef = 1.0f;
  if (P.clip_on) {
    const double r = P.max_norm / (P.scalars[kNorm] + 1e-6);
    k.coef = float(r < 1.0 ? r : 1.0);
  }
  const ChunkDev ch = P.chunks[q];
  const BucketDev bk = P.buckets[ch.bucket];
  k.wdiv = make_divisor(P.window);
  k.decay = bk.decayed ? P.decay : 1.0f;
  k.b1 = P.beta1;
  k.b2 = P.beta2;
  k.omb1 = P.one_minus_beta1;
  k.omb2 = P.one_minus_beta2;
  k.step_size = P.step_size;
  k.sbc2 = P.sqrt_bc2;
  k.eps = P.eps;

  AdamChunk c;
  c.acc = P.acc + ch.begin;
  c.p = P.master + ch.begin;
  c.m = P.m + ch.begin;
  c.v = P.v + ch.begin;
  c.pb = P.p_bf16 ? P.p_bf16 + ch.begin : nullptr;
  c.len = ch.len;
  if (c.len == kChunkElems) {
    const int wm = div_mode(k.wdiv);
    if (wm == kMulInv) {
      if (c.pb) adamw_full<kMulInv, true, NT>(c, k);
      else adamw_full<kMulInv, false, NT>(c, k);
    } else {
      if (c.pb) adamw_full<kIeeeDiv, true, NT>(c, k);
      else adamw_full<kIeeeDiv, false, NT>(c, k);
    }
  } else {
    adamw_generic<NT>(c, k);
  }
}

// ---------------------------------------------- replica-consistent init
// Philox4x64-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as
// easy as 1, 2, 3", SC 2011): ten rounds of two 64x64->128-bit multiplies
// with the key bumped by the Weyl constants between rounds.
struct U64x4 {
  uint64_t w[4];
};

__device__ __forceinline__ U64x4 philox4x64_10(U64x4 c, uint64_t k0, uint64_t k1) {
  constexpr uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  constexpr uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t hi0 = __umul64hi(M0, c.w[0]), lo0 = M0 * c.w[0];
    const uint64_t hi1 = __umul64hi(M1, c.w[2]), lo1 = M1 * c.w[2];
    U64x4 n;
    n.w[0] = hi1 ^ c.w[1] ^ k0;
    n.w[1] = lo1;
    n.w[2] = hi0 ^ c.w[3] ^ k1;
    n.w[3] = lo0;
    c = n;
    k0 += W0;
    k1 += W1;
  }
  return c;
}

// Element g of parameter pid: counter (g / 4, 0, 0, 0), key (seed, pid);
// output word g % 4, top 24 bits -> u = k * 2^-24 in [0, 1) (exact), value
// = offset + (2u - 1) * bound (2u - 1 is exact; one rounding each after).
__device__ __forceinline__ float init_value(uint64_t seed, const TensorDev& t, int64_t i) {
  const uint64_t g = uint64_t(t.index_base + i);
  U64x4 c;
  c.w[0] = g >> 2;
  c.w[1] = c.w[2] = c.w[3] = 0;
  const U64x4 o = philox4x64_10(c, seed, uint64_t(t.param_id));
  const float u = float(o.w[g & 3] >> 40) * 0x1p-24f;
  const float s = 2.0f * u - 1.0f;
  return t.offset + s * t.bound;
}

// One workgroup per chunk; each element finds its tensor by binary search
// over the flat offsets.  Elements of no updated tensor do not exist in a
// chunk, so every search succeeds.
__global__ __launch_bounds__(kBlock) void k_init_uniform(const InitLaunch P) {
  const int64_t q = int64_t(blockIdx.x);
  if (q >= P.n_chunks) return;
  const ChunkDev ch = P.chunks[q];
  for (int i = threadIdx.x; i < ch.len; i += kBlock) {
    const int64_t f = ch.begin + i;
    int lo = 0, hi = P.n_tensors - 1;
    while (lo < hi) {  // last tensor whose flat_offset <= f
      const int mid = (lo + hi + 1) >> 1;
      if (P.tensors[mid].flat_offset <= f) lo = mid; else hi = mid - 1;
    }
    const TensorDev t = P.tensors[lo];
    const float x = init_value(P.seed, t, f - t.flat_offset);
    P.master[f] = x;
    if (P.p_bf16) P.p_bf16[f] = bf16_bits(x);
  }
}

}  // namespace

// ------------------------------------------------------------ launchers
hipError_t launch_init_uniform(const InitLaunch& a, hipStream_t s) {
  if (a.n_chunks <= 0 || a.n_tensors <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_init_uniform, dim3(unsigned(a.n_chunks)), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

// LDS of one gfx950 CU.  A workgroup that requests a 1/cap share of it
// (less a margin for the kernels' own 32 bytes and the allocation granule)
// leaves room for cap workgroups and no more; the kernels do not touch it.
constexpr int64_t kLdsPerCu = 160 * 1024;
constexpr int64_t kLdsMargin = 2048;

size_t wg_cap_lds_bytes(int32_t cap, int32_t max_lds_per_block) {
  if (cap <= 0) return 0;
  const int64_t b = kLdsPerCu / cap - kLdsMargin;
  return (b > 0 && b + kLdsMargin / 2 <= max_lds_per_block) ? size_t(b) : 0;
}

hipError_t launch_accumulate(const AccumulateLaunch& a, size_t lds_bytes, hipStream_t s) {
  if (a.q_end <= a.q_begin) return hipSuccess;
  const int64_t blocks = (a.q_end - a.q_begin) + (a.q_begin & 7);
  if (a.acc_nt) hipLaunchKernelGGL(k_accumulate<true>, dim3(unsigned(blocks)), dim3(kBlock), lds_bytes, s, a);
  else hipLaunchKernelGGL(k_accumulate<false>, dim3(unsigned(blocks)), dim3(kBlock), lds_bytes, s, a);
  return hipGetLastError();
}

hipError_t launch_accumulate_window(const WindowLaunch& a, size_t lds_bytes, hipStream_t s) {
  if (a.q_end <= a.q_begin) return hipSuccess;
  const int64_t blocks = GRO_WIN_MAP == 0 ? (a.q_end - a.q_begin) + (a.q_begin & 7)
                                          : ((a.q_end - a.q_begin + 7) >> 3) * 8;
  if (a.acc_nt)
    hipLaunchKernelGGL(k_accumulate_window<true>, dim3(unsigned(blocks)), dim3(kBlock), lds_bytes, s, a);
  else
    hipLaunchKernelGGL(k_accumulate_window<false>, dim3(unsigned(blocks)), dim3(kBlock), lds_bytes, s, a);
  return hipGetLastError();
}

hipError_t launch_norm_partials(const NormLaunch& a, hipStream_t s) {
  if (a.q_end <= a.q_begin) return hipSuccess;
  const int64_t blocks = (a.q_end - a.q_begin) + (a.q_begin & 7);
  hipLaunchKernelGGL(k_norm_partials, dim3(unsigned(blocks)), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_norm_final(const NormFinalLaunch& a, hipStream_t s) {
  const int64_t groups = norm_groups(a.n_chunks);
  hipLaunchKernelGGL(k_norm_final, dim3(unsigned(groups > 0 ? groups : 1)), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_adamw(const AdamWLaunch& a, hipStream_t s) {
  if (a.n_chunks <= 0) return hipSuccess;
  if (a.acc_nt) hipLaunchKernelGGL(k_adamw<true>, dim3(unsigned(a.n_chunks)), dim3(kBlock), 0, s, a);
  else hipLaunchKernelGGL(k_adamw<false>, dim3(unsigned(a.n_chunks)), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

}  // namespace gro
