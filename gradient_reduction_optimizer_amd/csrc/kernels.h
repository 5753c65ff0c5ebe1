// Launchers for the gfx950 kernels (kernels.hip).  Internal to the library.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "plan.h"

namespace gro {

// Buckets whose gradient pointers travel in one launch's kernel arguments.
constexpr int kMaxBucketsPerLaunch = 64;

struct AccumulateLaunch {
  const ChunkDev* chunks;   // device chunk table
  const BucketDev* buckets; // device bucket table
  int64_t q_begin, q_end;   // chunk range [q_begin, q_end)
  int32_t b_first;          // bucket index of grads[0]
  int32_t n_grads;
  const void* grads[kMaxBucketsPerLaunch];  // BF16 or FP32 per bucket
  float* acc;
  double* partials;         // norm partials (written only when fuse_norm)
  int32_t R;
  int32_t micro_index;
  int32_t fuse_norm;
  int32_t window;           // microbatches in the window (used when fuse_norm)
  int32_t acc_nt;           // 1: store the accumulator with the non-temporal policy
};

// A whole accumulation window in one pass: grads[k * n_buckets + j] is
// microbatch k's buffer of bucket b_first + j, n_micro * n_buckets <= 64.
struct WindowLaunch {
  const ChunkDev* chunks;
  const BucketDev* buckets;
  int64_t q_begin, q_end;
  int32_t b_first;
  int32_t n_buckets;
  int32_t n_micro;          // microbatches in this group
  int32_t R;
  int32_t first;            // 1: the group opens the window (accumulator overwritten)
  int32_t fuse_norm;        // 1: the group closes the window (norm partials written)
  int32_t window;           // microbatches in the whole window (the norm's divisor)
  int32_t acc_nt;           // 1: store the accumulator with the non-temporal policy
  const void* grads[kMaxBucketsPerLaunch];
  float* acc;
  double* partials;
};

struct NormLaunch {
  const ChunkDev* chunks;
  const float* acc;
  double* partials;
  int64_t q_begin, q_end;
  int32_t window;
};

// The norm's second stage: group sums of the chunk partials, then their
// total, each in a fixed order.  `counter` is zero before and after.
struct NormFinalLaunch {
  const double* partials;
  int64_t n_chunks;
  double* group_sums;       // one per kNormGroup chunks
  uint32_t* counter;
  double* scalars;
};

struct AdamWLaunch {
  const ChunkDev* chunks;
  const BucketDev* buckets;
  int64_t n_chunks;
  const float* acc;
  float* master;
  float* m;
  float* v;
  uint16_t* p_bf16;         // may be null
  const double* scalars;    // norm written by the norm's second stage
  double max_norm;
  int32_t clip_on;
  int32_t window;
  float beta1, beta2, one_minus_beta1, one_minus_beta2;
  float step_size, sqrt_bc2, eps, decay;
  int32_t acc_nt;           // 1: load the accumulator with the non-temporal policy
};

struct InitLaunch {
  const ChunkDev* chunks;
  int64_t n_chunks;
  const TensorDev* tensors;   // sorted by flat offset
  int32_t n_tensors;
  uint64_t seed;
  float* master;
  uint16_t* p_bf16;           // may be null
};

// lds_bytes: dynamic LDS requested per workgroup, which caps the workgroups
// that share a CU (0: no cap; see wg_cap_lds_bytes).
hipError_t launch_accumulate(const AccumulateLaunch& a, size_t lds_bytes, hipStream_t s);
hipError_t launch_init_uniform(const InitLaunch& a, hipStream_t s);
hipError_t launch_accumulate_window(const WindowLaunch& a, size_t lds_bytes, hipStream_t s);
// Dynamic LDS that leaves room for at most `cap` workgroups of the
// accumulate passes on one CU (160 KiB of LDS each on gfx950), or 0 when
// cap <= 0 or the device allows no such allocation per workgroup.
size_t wg_cap_lds_bytes(int32_t cap, int32_t max_lds_per_block);
hipError_t launch_norm_partials(const NormLaunch& a, hipStream_t s);
hipError_t launch_norm_final(const NormFinalLaunch& a, hipStream_t s);
hipError_t launch_adamw(const AdamWLaunch& a, hipStream_t s);

}  // namespace gro
