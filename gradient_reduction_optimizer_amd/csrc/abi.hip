// C-ABI entry points that touch the device: binding, accumulate, norm,
// clip + AdamW.  All validation (arguments and the accumulation-window
// bookkeeping) happens on the host before the first launch, so a call that
// returns an error has enqueued nothing (Mixle "Distributed Transformer
// Training", section "Backend split": fail before fitting).
//
// Window semantics follow NeMo Automodel issue #3857, "refactor(distributed):
// establish shared native TP replica ownership", sections "Preserved prototype
// and evidence" and "Proposed scope and acceptance criteria": accumulation
// over 1, >1 and trailing (shorter) windows, each divided by the number of
// microbatches it actually holds; global norms; clipping on or off; Adam(W)
// updates.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <vector>

#include "kernels.h"
#include "plan.h"

using namespace gro;

// The library-owned workspace of gro_plan_bind_static: one copy per GPU,
// held until the process ends.  In host code `scratch` names a host-side
// shadow, not device memory; its device address comes from
// hipGetSymbolAddress (once per device, below) and only that address is
// ever handed to the runtime or to a kernel.
static __device__ __align__(256) unsigned char scratch[GRO_STATIC_WORKSPACE_BYTES];

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int hip_fail(hipError_t e, const char* what) {
  return set_error(GRO_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Device address of `scratch` on each device, looked up the first time a
// plan is bound to it on that device (with that device current).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
// Bumped by every gro_plan_bind_static on the device: a plan bound earlier
// no longer owns the array once another plan has been bound to it.
uint64_t g_scratch_gen[kMaxDevices] = {};

bool scratch_still_owned(const gro_plan* p) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  return p->device >= 0 && p->device < kMaxDevices && g_scratch_gen[p->device] == p->static_gen;
}

int scratch_address(int dev, char** out) {
  if (dev < 0 || dev >= kMaxDevices) return set_error(GRO_E_INVALID, "device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (ptr == nullptr || (reinterpret_cast<uintptr_t>(ptr) & 255u))
      return set_error(GRO_E_HIP, "static workspace has no 256-byte aligned device address");
    g_scratch_ptr[dev] = ptr;
  }
  *out = static_cast<char*>(g_scratch_ptr[dev]);
  return GRO_OK;
}

int check_bound(const gro_plan* p) {
  if (p == nullptr) return set_error(GRO_E_INVALID, "plan is NULL");
  if (!p->bound) return set_error(GRO_E_STATE, "plan is not bound to a workspace");
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev != p->device)
    return set_error(GRO_E_STATE, "plan is bound on device %d, current device is %d", p->device, dev);
  if (p->static_ws && !scratch_still_owned(p))
    return set_error(GRO_E_STATE, "the static workspace has been bound to another plan since; bind again");
  return GRO_OK;
}

const ChunkDev* dev_chunks(const gro_plan* p) {
  return reinterpret_cast<const ChunkDev*>(p->d_ws + p->ws.chunk_off);
}
const BucketDev* dev_buckets(const gro_plan* p) {
  return reinterpret_cast<const BucketDev*>(p->d_ws + p->ws.bucket_off);
}
double* dev_partials(const gro_plan* p) { return reinterpret_cast<double*>(p->d_ws + p->ws.partial_off); }
double* dev_scalars(const gro_plan* p) { return reinterpret_cast<double*>(p->d_ws + p->ws.scalar_off); }
double* dev_groups(const gro_plan* p) { return reinterpret_cast<double*>(p->d_ws + p->ws.group_off); }
uint32_t* dev_counters(const gro_plan* p) { return reinterpret_cast<uint32_t*>(p->d_ws + p->ws.counter_off); }

// One accumulator per window: a call that starts buckets [b0, b1) on
// another accumulator than the one buckets outside that range are already
// accumulating into is a bookkeeping error.
int check_window_acc(const gro_plan* p, int32_t b0, int32_t b1, const float* d_acc) {
  if (p->acc_ptr == nullptr || p->acc_ptr == d_acc) return GRO_OK;
  const int32_t nb = int32_t(p->buckets.size());
  for (int32_t b = 0; b < nb; ++b)
    if ((b < b0 || b >= b1) && p->count[size_t(b)] > 0)
      return set_error(GRO_E_STATE, "bucket %d of this window accumulates into another accumulator", b);
  return GRO_OK;
}

// Accumulator store policy of the window pass (GRO_WIN_ACC_NT) and of the
// per-microbatch pass (GRO_MB_ACC_NT), and its load policy in AdamW
// (GRO_ADAMW_ACC_NT).  The accumulator is read next by the following pass
// or by AdamW, which walks the chunks in reverse to meet the last-written
// ones in the 256 MB memory-side Infinity Cache.  That pays while the
// accumulator is about the cache's size; accumulators several times larger
// are stored and loaded non-temporally (they cannot stay in the cache and
// would otherwise churn it on their way to and from HBM), which measured
// faster.  Knobs: 0 never, 1 always, 2 when the accumulator is larger than
// GRO_ACC_NT_BYTES.
#ifndef GRO_WIN_ACC_NT
#define GRO_WIN_ACC_NT 2
#endif
#ifndef GRO_MB_ACC_NT
#define GRO_MB_ACC_NT 2
#endif
#ifndef GRO_ADAMW_ACC_NT
#define GRO_ADAMW_ACC_NT 2
#endif
#ifndef GRO_ACC_NT_BYTES
#define GRO_ACC_NT_BYTES (512ll << 20)
#endif
bool acc_nontemporal(const gro_plan* p, int knob) {
  if (knob == 2) return p->n_flat * int64_t(sizeof(float)) > GRO_ACC_NT_BYTES;
  return knob == 1;
}

// Workgroups per CU of the accumulate passes.  Far beyond the Infinity
// Cache each workgroup keeps every one of its input streams open in HBM at
// once; fewer workgroups sharing a CU measured faster there, the more so
// the more streams a pass reads: at most 2 per CU for a window pass of 12
// or more streams (8 microbatches of 2 slots), 3 for 5 to 11, and 3 for
// the per-microbatch pass.  On accumulators within a few times the cache
// (draft-67m-sized plans) and on window passes of 1-4 streams all of them
// stay, which measured faster.  The cap is a launch parameter, not a
// kernel argument: results are unchanged.
// Knobs: GRO_WG_CAP 0 never capped, 1 the rule above on every plan, 2 on
// accumulators larger than GRO_ACC_NT_BYTES; GRO_WIN_WG / GRO_MB_WG > 0
// force that cap on every window / per-microbatch pass, -1 none.
#ifndef GRO_WG_CAP
#define GRO_WG_CAP 2
#endif
#ifndef GRO_WIN_WG
#define GRO_WIN_WG 0
#endif
#ifndef GRO_MB_WG
#define GRO_MB_WG 0
#endif
bool wg_capped(const gro_plan* p) {
  if (GRO_WG_CAP == 2) return p->n_flat * int64_t(sizeof(float)) > GRO_ACC_NT_BYTES;
  return GRO_WG_CAP == 1;
}
size_t window_lds(const gro_plan* p, int32_t streams) {
  int32_t cap = GRO_WIN_WG;
  if (cap == 0) cap = !wg_capped(p) ? 0 : streams >= 12 ? 2 : streams >= 5 ? 3 : 0;
  return wg_cap_lds_bytes(cap, p->max_lds_per_block);
}
size_t micro_lds(const gro_plan* p) {
  int32_t cap = GRO_MB_WG;
  if (cap == 0) cap = wg_capped(p) ? 3 : 0;
  return wg_cap_lds_bytes(cap, p->max_lds_per_block);
}

void reset_window(gro_plan* p) {
  std::fill(p->count.begin(), p->count.end(), 0);
  std::fill(p->partials_ready.begin(), p->partials_ready.end(), 0);
  p->acc_ptr = nullptr;
  p->norm_done = false;
  p->norm_window = 0;
}

}  // namespace

namespace {

// Upload the plan's tables into `ws` on `stream`, clear the norm's
// completion counters (they must start at zero; every kernel that counts
// returns them to zero), wait, and mark the plan bound there.  Shared by
// gro_plan_bind and gro_plan_bind_static; for the static workspace the norm
// scalars are cleared too (the array keeps what the plan bound before left
// there) and the binding's generation is recorded.
int bind_to(gro_plan* p, char* ws, void* stream, bool is_static) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemsetAsync(ws + p->ws.counter_off, 0, p->ws.counter_bytes, s);
  if (e == hipSuccess && is_static)
    e = hipMemsetAsync(ws + p->ws.scalar_off, 0, kNumScalars * sizeof(double), s);
  if (e == hipSuccess && !p->bucket_dev.empty())
    e = hipMemcpyAsync(ws + p->ws.bucket_off, p->bucket_dev.data(),
                       p->bucket_dev.size() * sizeof(BucketDev), hipMemcpyHostToDevice, s);
  if (e == hipSuccess && !p->chunks.empty())
    e = hipMemcpyAsync(ws + p->ws.chunk_off, p->chunks.data(), p->chunks.size() * sizeof(ChunkDev),
                       hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "gro_plan_bind upload");
  int dev = -1;
  e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  int lds = 0;
  e = hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
  if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
  p->max_lds_per_block = lds;
  p->d_ws = ws;
  p->bound = true;
  p->device = dev;
  p->norm_valid = false;
  p->static_ws = is_static;
  if (is_static) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p->static_gen = ++g_scratch_gen[dev];
  }
  reset_window(p);
  return GRO_OK;
}

}  // namespace

extern "C" int gro_plan_bind(gro_plan* p, void* d_workspace, uint64_t bytes, void* stream) {
  clear_error();
  if (p == nullptr || d_workspace == nullptr) return set_error(GRO_E_INVALID, "NULL argument");
  if (reinterpret_cast<uintptr_t>(d_workspace) & 255u)
    return set_error(GRO_E_INVALID, "workspace must be 256-byte aligned");
  if (bytes < p->ws.total)
    return set_error(GRO_E_INVALID, "workspace has %llu bytes, plan needs %llu",
                     (unsigned long long)bytes, (unsigned long long)p->ws.total);
  return bind_to(p, static_cast<char*>(d_workspace), stream, false);
}

extern "C" int gro_plan_bind_static(gro_plan* p, void* stream) {
  clear_error();
  if (p == nullptr) return set_error(GRO_E_INVALID, "NULL argument");
  if (p->ws.total > uint64_t(GRO_STATIC_WORKSPACE_BYTES))
    return set_error(GRO_E_INVALID, "plan needs %llu workspace bytes, the static workspace holds %llu",
                     (unsigned long long)p->ws.total, (unsigned long long)GRO_STATIC_WORKSPACE_BYTES);
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  char* ws = nullptr;
  const int rc = scratch_address(dev, &ws);
  if (rc != GRO_OK) return rc;
  // The array may still be in use by the plan bound to it before, on any
  // stream: let all device work finish before overwriting its tables.
  const hipError_t se = hipDeviceSynchronize();
  if (se != hipSuccess) return hip_fail(se, "hipDeviceSynchronize");
  return bind_to(p, ws, stream, true);
}

extern "C" int gro_accumulate(gro_plan* p, int32_t b0, int32_t b1, const void* const* d_grad_buckets,
                              float* d_acc, int32_t micro_index, int32_t window_size, void* stream) {
  clear_error();
  int rc = check_bound(p);
  if (rc != GRO_OK) return rc;
  const int32_t nb = int32_t(p->buckets.size());
  if (b0 < 0 || b1 < b0 || b1 > nb)
    return set_error(GRO_E_INVALID, "bucket range [%d, %d) not within [0, %d)", b0, b1, nb);
  if (micro_index < 0) return set_error(GRO_E_INVALID, "micro_index < 0");
  if (window_size < 0) return set_error(GRO_E_INVALID, "window_size < 0");
  if (window_size > 0 && micro_index >= window_size)
    return set_error(GRO_E_INVALID, "micro_index %d outside a window of %d", micro_index, window_size);
  if (b1 == b0) return GRO_OK;
  if (d_grad_buckets == nullptr) return set_error(GRO_E_INVALID, "d_grad_buckets is NULL");
  if (d_acc == nullptr || !aligned16(d_acc))
    return set_error(GRO_E_INVALID, "d_acc must be a non-NULL 16-byte aligned device pointer");
  for (int32_t b = b0; b < b1; ++b) {
    const void* g = d_grad_buckets[b - b0];
    if (g == nullptr || !aligned16(g))
      return set_error(GRO_E_INVALID, "gradient buffer of bucket %d is NULL or not 16-byte aligned", b);
    if (micro_index != 0 && p->count[size_t(b)] != micro_index)
      return set_error(GRO_E_STATE, "bucket %d has accumulated %d microbatches, not %d", b,
                       p->count[size_t(b)], micro_index);
  }
  if (micro_index != 0 && p->acc_ptr != nullptr && p->acc_ptr != d_acc)
    return set_error(GRO_E_STATE, "a different accumulator than earlier in this window");
  rc = check_window_acc(p, b0, b1, d_acc);
  if (rc != GRO_OK) return rc;

  const bool fuse = window_size > 0 && micro_index == window_size - 1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int32_t lb = b0; lb < b1; lb += kMaxBucketsPerLaunch) {
    const int32_t le = (b1 - lb) < kMaxBucketsPerLaunch ? b1 : lb + kMaxBucketsPerLaunch;
    AccumulateLaunch a;
    std::memset(&a, 0, sizeof(a));
    a.chunks = dev_chunks(p);
    a.buckets = dev_buckets(p);
    a.q_begin = p->buckets[size_t(lb)].first_chunk;
    a.q_end = p->buckets[size_t(le - 1)].first_chunk + p->buckets[size_t(le - 1)].n_chunks;
    a.b_first = lb;
    a.n_grads = le - lb;
    for (int32_t b = lb; b < le; ++b) a.grads[b - lb] = d_grad_buckets[b - b0];
    a.acc = d_acc;
    a.partials = dev_partials(p);
    a.R = p->R;
    a.micro_index = micro_index;
    a.fuse_norm = fuse ? 1 : 0;
    a.window = window_size;
    a.acc_nt = acc_nontemporal(p, GRO_MB_ACC_NT) ? 1 : 0;
    const hipError_t e = launch_accumulate(a, micro_lds(p), s);
    if (e != hipSuccess) return hip_fail(e, "accumulate launch");
  }
  for (int32_t b = b0; b < b1; ++b) {
    p->count[size_t(b)] = micro_index + 1;
    p->partials_ready[size_t(b)] = fuse ? 1 : 0;
  }
  p->acc_ptr = d_acc;
  p->norm_done = false;
  return GRO_OK;
}

namespace {

// Microbatches first_micro .. first_micro+n-1 of a window of window_size
// (0 = length not known yet) for buckets [b0, b1), in one pass per bucket
// run.  Shared by gro_accumulate_window (a whole window) and
// gro_accumulate_microbatches (any group).
int accumulate_group(gro_plan* p, int32_t b0, int32_t b1, const void* const* d_grad_buckets, int32_t first_micro,
                     int32_t n, int32_t window_size, float* d_acc, void* stream) {
  int rc = check_bound(p);
  if (rc != GRO_OK) return rc;
  const int32_t nb = int32_t(p->buckets.size());
  if (b0 < 0 || b1 < b0 || b1 > nb)
    return set_error(GRO_E_INVALID, "bucket range [%d, %d) not within [0, %d)", b0, b1, nb);
  if (n < 1) return set_error(GRO_E_INVALID, "a group has at least one microbatch (n = %d)", n);
  if (n > kMaxBucketsPerLaunch)
    return set_error(GRO_E_INVALID, "group of %d microbatches exceeds %d", n, kMaxBucketsPerLaunch);
  if (first_micro < 0) return set_error(GRO_E_INVALID, "first_micro < 0");
  if (window_size < 0) return set_error(GRO_E_INVALID, "window_size < 0");
  if (window_size > 0 && int64_t(first_micro) + n > window_size)
    return set_error(GRO_E_INVALID, "microbatches %d..%d outside a window of %d", first_micro, first_micro + n - 1,
                     window_size);
  if (b1 == b0) return GRO_OK;
  if (d_grad_buckets == nullptr) return set_error(GRO_E_INVALID, "d_grad_buckets is NULL");
  if (d_acc == nullptr || !aligned16(d_acc))
    return set_error(GRO_E_INVALID, "d_acc must be a non-NULL 16-byte aligned device pointer");
  const int32_t span = b1 - b0;
  for (int32_t k = 0; k < n; ++k)
    for (int32_t j = 0; j < span; ++j) {
      const void* g = d_grad_buckets[int64_t(k) * span + j];
      if (g == nullptr || !aligned16(g))
        return set_error(GRO_E_INVALID, "microbatch %d buffer of bucket %d is NULL or not 16-byte aligned",
                         first_micro + k, b0 + j);
    }
  if (first_micro != 0) {
    for (int32_t b = b0; b < b1; ++b)
      if (p->count[size_t(b)] != first_micro)
        return set_error(GRO_E_STATE, "bucket %d has accumulated %d microbatches, not %d", b, p->count[size_t(b)],
                         first_micro);
    if (p->acc_ptr != nullptr && p->acc_ptr != d_acc)
      return set_error(GRO_E_STATE, "a different accumulator than earlier in this window");
  }
  rc = check_window_acc(p, b0, b1, d_acc);
  if (rc != GRO_OK) return rc;

  const bool fuse = window_size > 0 && first_micro + n == window_size;
  // Buckets of one launch: n * buckets <= kMaxBucketsPerLaunch pointers.
  const int32_t per = kMaxBucketsPerLaunch / n;
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int32_t lb = b0; lb < b1; lb += per) {
    const int32_t le = (b1 - lb) < per ? b1 : lb + per;
    WindowLaunch a;
    std::memset(&a, 0, sizeof(a));
    a.chunks = dev_chunks(p);
    a.buckets = dev_buckets(p);
    a.q_begin = p->buckets[size_t(lb)].first_chunk;
    a.q_end = p->buckets[size_t(le - 1)].first_chunk + p->buckets[size_t(le - 1)].n_chunks;
    a.b_first = lb;
    a.n_buckets = le - lb;
    a.n_micro = n;
    a.R = p->R;
    a.first = first_micro == 0 ? 1 : 0;
    a.fuse_norm = fuse ? 1 : 0;
    a.window = window_size;
    for (int32_t k = 0; k < n; ++k)
      for (int32_t b = lb; b < le; ++b)
        a.grads[k * (le - lb) + (b - lb)] = d_grad_buckets[int64_t(k) * span + (b - b0)];
    a.acc = d_acc;
    a.partials = dev_partials(p);
    a.acc_nt = acc_nontemporal(p, GRO_WIN_ACC_NT) ? 1 : 0;
    int32_t slots = 1;
    for (int32_t b = lb; b < le; ++b) slots = std::max(slots, p->bucket_dev[size_t(b)].slots);
    const int32_t streams = n * slots + (first_micro == 0 ? 0 : 1);
    const hipError_t e = launch_accumulate_window(a, window_lds(p, streams), s);
    if (e != hipSuccess) return hip_fail(e, "accumulate-window launch");
  }
  for (int32_t b = b0; b < b1; ++b) {
    p->count[size_t(b)] = first_micro + n;
    p->partials_ready[size_t(b)] = fuse ? 1 : 0;
  }
  p->acc_ptr = d_acc;
  p->norm_done = false;
  return GRO_OK;
}

}  // namespace

extern "C" int gro_accumulate_window(gro_plan* p, int32_t b0, int32_t b1, const void* const* d_grad_buckets,
                                     int32_t n, float* d_acc, void* stream) {
  clear_error();
  return accumulate_group(p, b0, b1, d_grad_buckets, 0, n, n, d_acc, stream);
}

extern "C" int gro_accumulate_microbatches(gro_plan* p, int32_t b0, int32_t b1,
                                           const void* const* d_grad_buckets, int32_t first_micro, int32_t n,
                                           int32_t window_size, float* d_acc, void* stream) {
  clear_error();
  return accumulate_group(p, b0, b1, d_grad_buckets, first_micro, n, window_size, d_acc, stream);
}

extern "C" int gro_reduce_norm(gro_plan* p, const float* d_acc, int32_t window_size, void* stream) {
  clear_error();
  int rc = check_bound(p);
  if (rc != GRO_OK) return rc;
  if (window_size < 1) return set_error(GRO_E_INVALID, "window_size must be >= 1");
  const int32_t nb = int32_t(p->buckets.size());
  if (nb > 0 && (d_acc == nullptr || !aligned16(d_acc)))
    return set_error(GRO_E_INVALID, "d_acc must be a non-NULL 16-byte aligned device pointer");
  for (int32_t b = 0; b < nb; ++b)
    if (p->count[size_t(b)] != window_size)
      return set_error(GRO_E_STATE, "bucket %d has accumulated %d microbatches, window is %d", b,
                       p->count[size_t(b)], window_size);
  if (nb > 0 && d_acc != p->acc_ptr)
    return set_error(GRO_E_STATE, "d_acc is not the accumulator of this window");

  hipStream_t s = static_cast<hipStream_t>(stream);
  // Stage 1 for runs of buckets whose partials the last accumulate did not write.
  int32_t b = 0;
  while (b < nb) {
    if (p->partials_ready[size_t(b)]) {
      ++b;
      continue;
    }
    int32_t e = b;
    while (e < nb && !p->partials_ready[size_t(e)]) ++e;
    NormLaunch a;
    a.chunks = dev_chunks(p);
    a.acc = d_acc;
    a.partials = dev_partials(p);
    a.q_begin = p->buckets[size_t(b)].first_chunk;
    a.q_end = p->buckets[size_t(e - 1)].first_chunk + p->buckets[size_t(e - 1)].n_chunks;
    a.window = window_size;
    const hipError_t err = launch_norm_partials(a, s);
    if (err != hipSuccess) return hip_fail(err, "norm stage-1 launch");
    b = e;
  }
  NormFinalLaunch f;
  f.partials = dev_partials(p);
  f.n_chunks = int64_t(p->chunks.size());
  f.group_sums = dev_groups(p);
  f.counter = dev_counters(p);
  f.scalars = dev_scalars(p);
  const hipError_t err = launch_norm_final(f, s);
  if (err != hipSuccess) return hip_fail(err, "norm stage-2 launch");
  std::fill(p->partials_ready.begin(), p->partials_ready.end(), 1);
  p->norm_done = true;
  p->norm_valid = true;
  p->norm_window = window_size;
  p->norm_stream = stream;
  return GRO_OK;
}

extern "C" int gro_init_uniform(gro_plan* p, uint64_t seed, const double* bounds, const double* offsets,
                                float* d_master, uint16_t* d_param_bf16, void* stream) {
  clear_error();
  int rc = check_bound(p);
  if (rc != GRO_OK) return rc;
  const size_t nt = p->tensors.size();
  if (nt > 0 && bounds == nullptr) return set_error(GRO_E_INVALID, "bounds is NULL");
  if (!p->buckets.empty() && (d_master == nullptr || !aligned16(d_master) ||
                              (d_param_bf16 != nullptr && !aligned16(d_param_bf16))))
    return set_error(GRO_E_INVALID, "master / BF16 pointers must be 16-byte aligned (master non-NULL)");
  std::vector<TensorDev>& tab = p->init_table;
  tab.clear();
  for (size_t i = 0; i < nt; ++i) {
    const gro_tensor_layout& t = p->tensors[i];
    const double b = bounds[i], o = offsets ? offsets[i] : 0.0;
    if (!(b >= 0.0) || !std::isfinite(b) || !std::isfinite(o))
      return set_error(GRO_E_INVALID, "tensor %zu: bound must be finite and >= 0, offset finite", i);
    if (!t.updated || t.numel == 0) continue;
    TensorDev d;
    d.flat_offset = t.flat_offset;
    d.numel = t.numel;
    d.param_id = t.param_id;
    d.index_base = t.owner == GRO_OWNER_LOCAL_SHARD ? int64_t(p->shard_index[i]) * t.numel : 0;
    d.bound = float(b);
    d.offset = float(o);
    d.reserved = 0;
    tab.push_back(d);
  }
  std::sort(tab.begin(), tab.end(),
            [](const TensorDev& a, const TensorDev& b) { return a.flat_offset < b.flat_offset; });
  if (tab.empty()) return GRO_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  TensorDev* dtab = reinterpret_cast<TensorDev*>(p->d_ws + p->ws.tensor_off);
  hipError_t e = hipMemcpyAsync(dtab, tab.data(), tab.size() * sizeof(TensorDev), hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return hip_fail(e, "init table upload");
  InitLaunch a;
  a.chunks = dev_chunks(p);
  a.n_chunks = int64_t(p->chunks.size());
  a.tensors = dtab;
  a.n_tensors = int32_t(tab.size());
  a.seed = seed;
  a.master = d_master;
  a.p_bf16 = d_param_bf16;
  e = launch_init_uniform(a, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "init launch");
  return GRO_OK;
}

extern "C" int gro_plan_get_norm(gro_plan* p, double* norm, double* norm_sq, int32_t* finite) {
  clear_error();
  int rc = check_bound(p);
  if (rc != GRO_OK) return rc;
  if (!p->norm_valid) return set_error(GRO_E_STATE, "no gro_reduce_norm since the plan was bound");
  hipStream_t s = static_cast<hipStream_t>(p->norm_stream);
  double host[kNumScalars];
  hipError_t e = hipStreamSynchronize(s);
  if (e == hipSuccess) e = hipMemcpy(host, dev_scalars(p), sizeof(host), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "reading the norm");
  if (norm) *norm = host[kNorm];
  if (norm_sq) *norm_sq = host[kNormSq];
  if (finite) *finite = host[kFinite] != 0.0 ? 1 : 0;
  return GRO_OK;
}

extern "C" int gro_clip_adamw(gro_plan* p, const float* d_acc, int32_t window_size, double max_norm,
                              const gro_adamw_hparams* hp, int64_t step, float* d_master, float* d_m,
                              float* d_v, uint16_t* d_param_bf16, void* stream) {
  clear_error();
  int rc = check_bound(p);
  if (rc != GRO_OK) return rc;
  if (hp == nullptr) return set_error(GRO_E_INVALID, "hp is NULL");
  if (step < 1) return set_error(GRO_E_INVALID, "step must be >= 1");
  if (window_size < 1) return set_error(GRO_E_INVALID, "window_size must be >= 1");
  if (std::isnan(max_norm)) return set_error(GRO_E_INVALID, "max_norm is NaN");
  if (!(hp->lr >= 0.0) || !std::isfinite(hp->lr) || !(hp->eps >= 0.0) || !std::isfinite(hp->eps) ||
      !(hp->weight_decay >= 0.0) || !std::isfinite(hp->weight_decay) || !(hp->beta1 >= 0.0) ||
      !(hp->beta1 < 1.0) || !(hp->beta2 >= 0.0) || !(hp->beta2 < 1.0))
    return set_error(GRO_E_INVALID, "hyper-parameters out of range (lr, eps, wd >= 0; 0 <= beta < 1)");
  const bool any = !p->buckets.empty();
  if (any) {
    if (d_acc == nullptr || !aligned16(d_acc) || d_master == nullptr || !aligned16(d_master) ||
        d_m == nullptr || !aligned16(d_m) || d_v == nullptr || !aligned16(d_v) ||
        (d_param_bf16 != nullptr && !aligned16(d_param_bf16)))
      return set_error(GRO_E_INVALID, "state pointers must be non-NULL and 16-byte aligned");
    if (d_acc != p->acc_ptr) return set_error(GRO_E_STATE, "d_acc is not the accumulator of this window");
  }
  if (!p->norm_done || p->norm_window != window_size)
    return set_error(GRO_E_STATE, "gro_reduce_norm of this window (size %d) has not run", window_size);

  // Per-step scalars in FP64 from the hyper-parameters as given, each rounded
  // once to FP32.
  const double bc1 = 1.0 - std::pow(hp->beta1, double(step));
  const double bc2 = 1.0 - std::pow(hp->beta2, double(step));
  AdamWLaunch a;
  std::memset(&a, 0, sizeof(a));
  a.chunks = dev_chunks(p);
  a.buckets = dev_buckets(p);
  a.n_chunks = int64_t(p->chunks.size());
  a.acc = d_acc;
  a.master = d_master;
  a.m = d_m;
  a.v = d_v;
  a.p_bf16 = d_param_bf16;
  a.scalars = dev_scalars(p);
  a.max_norm = max_norm;
  a.clip_on = (max_norm > 0.0 && !std::isinf(max_norm)) ? 1 : 0;
  a.window = window_size;
  a.beta1 = float(hp->beta1);
  a.beta2 = float(hp->beta2);
  a.one_minus_beta1 = float(1.0 - hp->beta1);
  a.one_minus_beta2 = float(1.0 - hp->beta2);
  a.step_size = float(hp->lr / bc1);
  a.sqrt_bc2 = float(std::sqrt(bc2));
  a.eps = float(hp->eps);
  a.decay = float(1.0 - hp->lr * hp->weight_decay);
  a.acc_nt = acc_nontemporal(p, GRO_ADAMW_ACC_NT) ? 1 : 0;
  const hipError_t e = launch_adamw(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "clip+AdamW launch");
  reset_window(p);
  return GRO_OK;
}
