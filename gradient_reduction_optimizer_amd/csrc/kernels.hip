// gfx950 (MI355X, CDNA4) kernels for the gradient-ownership hot path.
//
// Every pass is a multi-tensor walk over the plan's chunk table: one
// 256-lane workgroup per chunk of up to kChunkElems elements, where a chunk
// lies inside one bucket and so has one owner class.  Lanes move 8 elements
// at a time with 128-bit loads and stores (8 BF16 or 4+4 FP32), two such
// vectors in flight per lane.  The path is bound by HBM bandwidth, not by a
// contraction, so there is no MFMA here.
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
// Workgroup placement is XCD-aware: chunk q always runs in a workgroup whose
// index is congruent to q modulo 8, and the hardware deals workgroups to the
// eight XCDs round-robin, so a chunk visits the same XCD (and its L2) in
// every pass of a step.
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace gro {
namespace {

constexpr int kBlock = 256;            // lanes per workgroup (4 waves of 64)
constexpr int kWaves = kBlock / 64;
constexpr int kUnroll = 2;             // 8-element vectors in flight per lane
constexpr int kFinalBlock = 1024;      // the norm's second stage
static_assert(kChunkElems % (8 * kBlock) == 0, "chunks are whole workgroup tiles");

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

__device__ __forceinline__ void widen8(const uint4 r, float (&x)[8]) {
  x[0] = __uint_as_float(r.x << 16);
  x[1] = __uint_as_float(r.x & 0xffff0000u);
  x[2] = __uint_as_float(r.y << 16);
  x[3] = __uint_as_float(r.y & 0xffff0000u);
  x[4] = __uint_as_float(r.z << 16);
  x[5] = __uint_as_float(r.z & 0xffff0000u);
  x[6] = __uint_as_float(r.w << 16);
  x[7] = __uint_as_float(r.w & 0xffff0000u);
}

__device__ __forceinline__ float widen1(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// FP32 -> BF16, round to nearest even (gfx950 converts in hardware).
__device__ __forceinline__ uint32_t bf16_bits(float x) {
  const __bf16 h = static_cast<__bf16>(x);
  return uint32_t(__builtin_bit_cast(uint16_t, h));
}

__device__ __forceinline__ uint4 ld4u(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ float4 ld4f(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ void st4f(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}

// Sum over the workgroup in a fixed order: a wave64 butterfly (every lane
// ends with the same bits because IEEE addition commutes), then the four
// wave totals in wave order.  Returned in every lane.
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

// ------------------------------------------------------------ accumulate
struct AccChunk {
  const uint16_t* g;   // slot 0 of this chunk in the bucket's gradient buffer
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

// Per element: widen the slots, sum them in slot order, divide by R for
// MEAN, then start or extend the accumulator.  Returns this lane's FP64 sum
// of (acc/window)^2 over its elements (0 unless fuse), taken in the lane's
// element order: vectors t, t+256, ... then, for the lane that owns vector
// len/8, the ragged tail.
template <int C>
__device__ double accumulate_chunk(const AccChunk& c) {
  const int nvec = c.len >> 3;
  double ss = 0.0;
  for (int v0 = threadIdx.x; v0 < nvec; v0 += kUnroll * kBlock) {
    uint4 raw[kUnroll][C];
    float4 old[kUnroll][2];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int v = v0 + u * kBlock;
      if (v < nvec) {
#pragma unroll
        for (int r = 0; r < C; ++r) raw[u][r] = ld4u(c.g + r * c.stride + 8 * v);
        if (!c.first) {
          old[u][0] = ld4f(c.acc + 8 * v);
          old[u][1] = ld4f(c.acc + 8 * v + 4);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int v = v0 + u * kBlock;
      if (v < nvec) {
        float s[8];
        widen8(raw[u][0], s);
#pragma unroll
        for (int r = 1; r < C; ++r) {
          float x[8];
          widen8(raw[u][r], x);
#pragma unroll
          for (int e = 0; e < 8; ++e) s[e] = s[e] + x[e];
        }
        if (c.mean) {
#pragma unroll
          for (int e = 0; e < 8; ++e) s[e] = divide(s[e], c.rdiv);
        }
        if (!c.first) {
          s[0] = old[u][0].x + s[0];
          s[1] = old[u][0].y + s[1];
          s[2] = old[u][0].z + s[2];
          s[3] = old[u][0].w + s[3];
          s[4] = old[u][1].x + s[4];
          s[5] = old[u][1].y + s[5];
          s[6] = old[u][1].z + s[6];
          s[7] = old[u][1].w + s[7];
        }
        st4f(c.acc + 8 * v, s[0], s[1], s[2], s[3]);
        st4f(c.acc + 8 * v + 4, s[4], s[5], s[6], s[7]);
        if (c.fuse) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const double gq = double(divide(s[e], c.wdiv));
            ss += gq * gq;
          }
        }
      }
    }
  }
  if ((c.len & 7) && int(threadIdx.x) == nvec % kBlock) {
    for (int i = nvec * 8; i < c.len; ++i) {
      float s = widen1(c.g[i]);
      for (int r = 1; r < c.slots; ++r) s = s + widen1(c.g[r * c.stride + i]);
      if (c.mean) s = divide(s, c.rdiv);
      if (!c.first) s = c.acc[i] + s;
      c.acc[i] = s;
      if (c.fuse) {
        const double gq = double(divide(s, c.wdiv));
        ss += gq * gq;
      }
    }
  }
  return ss;
}

// Any slot count (R other than 1 or 2): same arithmetic and element order,
// one vector at a time.
__device__ double accumulate_chunk_any(const AccChunk& c) {
  const int nvec = c.len >> 3;
  double ss = 0.0;
  for (int v = threadIdx.x; v < nvec; v += kBlock) {
    float s[8];
    widen8(ld4u(c.g + 8 * v), s);
    for (int r = 1; r < c.slots; ++r) {
      float x[8];
      widen8(ld4u(c.g + r * c.stride + 8 * v), x);
#pragma unroll
      for (int e = 0; e < 8; ++e) s[e] = s[e] + x[e];
    }
    if (c.mean) {
#pragma unroll
      for (int e = 0; e < 8; ++e) s[e] = divide(s[e], c.rdiv);
    }
    if (!c.first) {
      const float4 a0 = ld4f(c.acc + 8 * v), a1 = ld4f(c.acc + 8 * v + 4);
      s[0] = a0.x + s[0]; s[1] = a0.y + s[1]; s[2] = a0.z + s[2]; s[3] = a0.w + s[3];
      s[4] = a1.x + s[4]; s[5] = a1.y + s[5]; s[6] = a1.z + s[6]; s[7] = a1.w + s[7];
    }
    st4f(c.acc + 8 * v, s[0], s[1], s[2], s[3]);
    st4f(c.acc + 8 * v + 4, s[4], s[5], s[6], s[7]);
    if (c.fuse) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const double gq = double(divide(s[e], c.wdiv));
        ss += gq * gq;
      }
    }
  }
  if ((c.len & 7) && int(threadIdx.x) == nvec % kBlock) {
    for (int i = nvec * 8; i < c.len; ++i) {
      float s = widen1(c.g[i]);
      for (int r = 1; r < c.slots; ++r) s = s + widen1(c.g[r * c.stride + i]);
      if (c.mean) s = divide(s, c.rdiv);
      if (!c.first) s = c.acc[i] + s;
      c.acc[i] = s;
      if (c.fuse) {
        const double gq = double(divide(s, c.wdiv));
        ss += gq * gq;
      }
    }
  }
  return ss;
}

__global__ __launch_bounds__(kBlock) void k_accumulate(const AccumulateLaunch P) {
  const int64_t q = chunk_of_block(P.q_begin);
  if (q < P.q_begin || q >= P.q_end) return;
  const ChunkDev ch = P.chunks[q];
  const BucketDev bk = P.buckets[ch.bucket];
  AccChunk c;
  c.g = P.grads[ch.bucket - P.b_first] + (ch.begin - bk.base);
  c.stride = bk.stride;
  c.acc = P.acc + ch.begin;
  c.len = ch.len;
  c.slots = bk.slots;
  c.mean = bk.owner == GRO_OWNER_MEAN;
  c.first = P.micro_index == 0;
  c.fuse = P.fuse_norm != 0;
  c.rdiv = make_divisor(P.R);
  c.wdiv = make_divisor(P.window > 0 ? P.window : 1);
  double ss;
  if (c.slots == 1)
    ss = accumulate_chunk<1>(c);
  else if (c.slots == 2)
    ss = accumulate_chunk<2>(c);
  else
    ss = accumulate_chunk_any(c);
  if (c.fuse) {
    const double t = block_sum(ss);
    if (threadIdx.x == 0) P.partials[q] = t;
  }
}

// ------------------------------------------------------- norm, stage 1
// Same lane/element order as the fused accumulate, so a chunk's partial is
// the same bits whichever kernel wrote it.
__global__ __launch_bounds__(kBlock) void k_norm_partials(const NormLaunch P) {
  const int64_t q = chunk_of_block(P.q_begin);
  if (q < P.q_begin || q >= P.q_end) return;
  const ChunkDev ch = P.chunks[q];
  const float* acc = P.acc + ch.begin;
  const Divisor wdiv = make_divisor(P.window);
  const int nvec = ch.len >> 3;
  double ss = 0.0;
  for (int v0 = threadIdx.x; v0 < nvec; v0 += kUnroll * kBlock) {
    float4 a[kUnroll][2];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int v = v0 + u * kBlock;
      if (v < nvec) {
        a[u][0] = ld4f(acc + 8 * v);
        a[u][1] = ld4f(acc + 8 * v + 4);
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int v = v0 + u * kBlock;
      if (v < nvec) {
        const float s[8] = {a[u][0].x, a[u][0].y, a[u][0].z, a[u][0].w,
                            a[u][1].x, a[u][1].y, a[u][1].z, a[u][1].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const double gq = double(divide(s[e], wdiv));
          ss += gq * gq;
        }
      }
    }
  }
  if ((ch.len & 7) && int(threadIdx.x) == nvec % kBlock) {
    for (int i = nvec * 8; i < ch.len; ++i) {
      const double gq = double(divide(acc[i], wdiv));
      ss += gq * gq;
    }
  }
  const double t = block_sum(ss);
  if (threadIdx.x == 0) P.partials[q] = t;
}

// ------------------------------------------------------- norm, stage 2
// One workgroup: lane t sums partials t, t+1024, ... in order, then a fixed
// butterfly and the sixteen wave totals in order.  No atomics.
__global__ __launch_bounds__(kFinalBlock) void k_norm_final(const double* __restrict__ partials,
                                                            int64_t n, double* __restrict__ scalars) {
  double s = 0.0;
  for (int64_t i = threadIdx.x; i < n; i += kFinalBlock) s += partials[i];
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m, 64);
  __shared__ double part[kFinalBlock / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = part[0];
    for (int w = 1; w < kFinalBlock / 64; ++w) t += part[w];
    scalars[kNormSq] = t;
    scalars[kNorm] = sqrt(t);
    scalars[kFinite] = __builtin_isfinite(t) ? 1.0 : 0.0;
  }
}

// ------------------------------------------------------- clip + AdamW
struct AdamScalars {
  Divisor wdiv;
  float coef, decay, b1, b2, omb1, omb2, step_size, sbc2, eps;
};

__device__ __forceinline__ void adamw_elem(float a, float& p, float& m, float& v, const AdamScalars& k) {
  const float g = divide(a, k.wdiv);
  const float gh = g * k.coef;
  p = p * k.decay;
  m = k.b1 * m + k.omb1 * gh;
  v = k.b2 * v + k.omb2 * (gh * gh);
  const float d = sqrtf(v) / k.sbc2 + k.eps;
  p = p - k.step_size * (m / d);
}

__global__ __launch_bounds__(kBlock) void k_adamw(const AdamWLaunch P) {
  const int64_t q = int64_t(blockIdx.x);
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

  const float* acc = P.acc + ch.begin;
  float* pm = P.master + ch.begin;
  float* mm = P.m + ch.begin;
  float* vm = P.v + ch.begin;
  uint16_t* pb = P.p_bf16 ? P.p_bf16 + ch.begin : nullptr;
  const int nvec = ch.len >> 3;
  for (int v0 = threadIdx.x; v0 < nvec; v0 += kUnroll * kBlock) {
    float4 a[kUnroll][2], p[kUnroll][2], m[kUnroll][2], w[kUnroll][2];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int v = v0 + u * kBlock;
      if (v < nvec) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          a[u][h] = ld4f(acc + 8 * v + 4 * h);
          p[u][h] = ld4f(pm + 8 * v + 4 * h);
          m[u][h] = ld4f(mm + 8 * v + 4 * h);
          w[u][h] = ld4f(vm + 8 * v + 4 * h);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int v = v0 + u * kBlock;
      if (v < nvec) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          adamw_elem(a[u][h].x, p[u][h].x, m[u][h].x, w[u][h].x, k);
          adamw_elem(a[u][h].y, p[u][h].y, m[u][h].y, w[u][h].y, k);
          adamw_elem(a[u][h].z, p[u][h].z, m[u][h].z, w[u][h].z, k);
          adamw_elem(a[u][h].w, p[u][h].w, m[u][h].w, w[u][h].w, k);
          *reinterpret_cast<float4*>(pm + 8 * v + 4 * h) = p[u][h];
          *reinterpret_cast<float4*>(mm + 8 * v + 4 * h) = m[u][h];
          *reinterpret_cast<float4*>(vm + 8 * v + 4 * h) = w[u][h];
        }
        if (pb) {
          uint4 o;
          o.x = bf16_bits(p[u][0].x) | (bf16_bits(p[u][0].y) << 16);
          o.y = bf16_bits(p[u][0].z) | (bf16_bits(p[u][0].w) << 16);
          o.z = bf16_bits(p[u][1].x) | (bf16_bits(p[u][1].y) << 16);
          o.w = bf16_bits(p[u][1].z) | (bf16_bits(p[u][1].w) << 16);
          *reinterpret_cast<uint4*>(pb + 8 * v) = o;
        }
      }
    }
  }
  if ((ch.len & 7) && int(threadIdx.x) == nvec % kBlock) {
    for (int i = nvec * 8; i < ch.len; ++i) {
      float p1 = pm[i], m1 = mm[i], v1 = vm[i];
      adamw_elem(acc[i], p1, m1, v1, k);
      pm[i] = p1;
      mm[i] = m1;
      vm[i] = v1;
      if (pb) pb[i] = uint16_t(bf16_bits(p1));
    }
  }
}

}  // namespace

// ------------------------------------------------------------ launchers
hipError_t launch_accumulate(const AccumulateLaunch& a, hipStream_t s) {
  if (a.q_end <= a.q_begin) return hipSuccess;
  const int64_t blocks = (a.q_end - a.q_begin) + (a.q_begin & 7);
  hipLaunchKernelGGL(k_accumulate, dim3(unsigned(blocks)), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_norm_partials(const NormLaunch& a, hipStream_t s) {
  if (a.q_end <= a.q_begin) return hipSuccess;
  const int64_t blocks = (a.q_end - a.q_begin) + (a.q_begin & 7);
  hipLaunchKernelGGL(k_norm_partials, dim3(unsigned(blocks)), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_norm_final(const double* partials, int64_t n_chunks, double* scalars,
                             hipStream_t s) {
  hipLaunchKernelGGL(k_norm_final, dim3(1), dim3(kFinalBlock), 0, s, partials, n_chunks, scalars);
  return hipGetLastError();
}

hipError_t launch_adamw(const AdamWLaunch& a, hipStream_t s) {
  if (a.n_chunks <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_adamw, dim3(unsigned(a.n_chunks)), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

}  // namespace gro
