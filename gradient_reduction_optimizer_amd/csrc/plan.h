// Internal host-side plan structures shared by the planner (plan.cpp, plain
// C++) and the HIP entry points (abi.hip).  Not part of the public ABI.
#pragma once

#include <cstdarg>
#include <cstdint>
#include <vector>

#include "gro.h"

namespace gro {

// Elements per chunk.  A chunk is one workgroup's unit of work in every pass
// and the granularity of the global norm's partial sums, so the norm's
// summation order is fixed by the plan, never by the launch shape.
#ifndef GRO_CHUNK_ELEMS
#define GRO_CHUNK_ELEMS 4096
#endif
constexpr int32_t kChunkElems = GRO_CHUNK_ELEMS;
// Bucket bases and slot strides are multiples of this many elements
// (256 B of FP32, 128 B of BF16) so every chunk starts 128-bit aligned.
constexpr int64_t kAlignElems = 64;
constexpr int64_t kMaxNumel = int64_t(1) << 46;

// Device-side tables, uploaded by gro_plan_bind.
struct ChunkDev {          // 16 B
  int64_t begin;           // flat index of the chunk's first element
  int32_t len;             // elements, 1..kChunkElems
  int32_t bucket;
};
struct BucketDev {         // 32 B
  int64_t base;            // flat index of the bucket's first element
  int64_t stride;          // slot stride of its BF16 gradient buffer
  int32_t owner;           // GRO_OWNER_*
  int32_t slots;
  int32_t decayed;
  int32_t grad_fp32;       // 1: FP32 gradient contributions, 0: BF16
};
// Per-tensor entry for gro_init_uniform (sorted by flat offset, updated
// tensors with at least one element).
struct TensorDev {         // 48 B
  int64_t flat_offset;
  int64_t numel;
  int64_t param_id;
  int64_t index_base;      // this rank's first element in the unsharded tensor
  float bound;
  float offset;
  int64_t reserved;
};
static_assert(sizeof(ChunkDev) == 16, "chunk table entry is 16 bytes");
static_assert(sizeof(TensorDev) == 48, "tensor table entry is 48 bytes");
static_assert(sizeof(BucketDev) == 32, "bucket table entry is 32 bytes");

// Device scalars written by the norm's second stage.
enum ScalarSlot { kNormSq = 0, kNorm = 1, kFinite = 2, kNumScalars = 8 };

// The norm's second stage sums the chunk partials in two fixed-order levels:
// groups of kNormGroup consecutive partials, then the group sums.
constexpr int64_t kNormGroup = 2048;
constexpr int64_t norm_groups(int64_t n_chunks) { return (n_chunks + kNormGroup - 1) / kNormGroup; }

struct WorkspaceLayout {
  uint64_t bucket_off = 0, chunk_off = 0, partial_off = 0, scalar_off = 0, tensor_off = 0;
  uint64_t group_off = 0;    // FP64 group sums, one per kNormGroup chunks
  uint64_t counter_off = 0;  // uint32 completion counters (zero between launches)
  uint64_t counter_bytes = 0;
  uint64_t total = 0;
};

inline int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

int set_error(int code, const char* fmt, ...);
void clear_error();

}  // namespace gro

struct gro_plan {
  int32_t R = 0;
  int64_t bucket_elems = 0;
  int64_t n_flat = 0;
  int64_t n_owned = 0;
  std::vector<gro_tensor_layout> tensors;
  std::vector<gro_bucket_info> buckets;
  std::vector<gro::BucketDev> bucket_dev;
  std::vector<gro::ChunkDev> chunks;
  std::vector<int32_t> shard_index;    // per tensor, as given (-1 unless Shard)
  std::vector<gro::TensorDev> init_table;  // host staging for gro_init_uniform
  gro::WorkspaceLayout ws;

  // Binding.
  char* d_ws = nullptr;
  bool bound = false;
  int device = -1;
  int32_t max_lds_per_block = 0;        // the bound device's limit (bytes)
  bool static_ws = false;               // bound to the library's static workspace
  uint64_t static_gen = 0;              // which binding of that workspace is this plan's

  // Window bookkeeping (host side, validated before any launch).
  std::vector<int32_t> count;          // microbatches accumulated per bucket
  std::vector<uint8_t> partials_ready; // norm partials written by the last accumulate
  const float* acc_ptr = nullptr;      // accumulator used in this window
  bool norm_done = false;               // a norm of the current window is on the device
  bool norm_valid = false;              // some norm has been computed since binding
  int32_t norm_window = 0;
  void* norm_stream = nullptr;
};
