// Host planner: ownership of every parameter from its placement, then the
// flat/bucket/chunk layout the kernels walk.  Plain C++ (no HIP), so it is
// exercised on any host.
//
// Ownership follows NeMo Automodel issue #3857, "refactor(distributed):
// establish shared native TP replica ownership", section "Why this needs
// separate work" (Replicate -> average over the R TP ranks, Partial -> sum,
// Shard -> local, already reduced -> not reduced again) and section
// "Proposed scope and acceptance criteria" (exactly one reduction owner per
// parameter; unsupported compositions rejected).  Mixle "Distributed
// Transformer Training", section "Backend split": rejection happens before
// any work is done.
//
// Buckets hold one owner class, one decay setting and one gradient type
// each, so every chunk of a bucket runs the same arithmetic; tensors are packed densely inside a
// bucket and only a tensor larger than the capacity is split.
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <unordered_set>

#include "plan.h"

namespace gro {

static thread_local std::string g_last_error;

int set_error(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

void clear_error() { g_last_error.clear(); }

namespace {

int classify(const gro_tensor_desc& d, int32_t R, gro_tensor_layout* lay) {
  std::memset(lay, 0, sizeof(*lay));
  lay->param_id = d.param_id;
  if (d.ndim < 0 || d.ndim > GRO_MAX_NDIM)
    return set_error(GRO_E_INVALID, "param_id %lld: ndim %d not in [0, %d]",
                     (long long)d.param_id, d.ndim, GRO_MAX_NDIM);
  if (d.ndim > 0 && d.shape == nullptr)
    return set_error(GRO_E_INVALID, "param_id %lld: shape is NULL", (long long)d.param_id);
  int64_t numel = 1;
  for (int k = 0; k < d.ndim; ++k) {
    const int64_t s = d.shape[k];
    if (s < 0)
      return set_error(GRO_E_INVALID, "param_id %lld: negative dimension", (long long)d.param_id);
    if (s != 0 && numel > kMaxNumel / s)
      return set_error(GRO_E_INVALID, "param_id %lld: too many elements", (long long)d.param_id);
    numel *= s;
  }
  lay->numel = numel;
  if (d.flags & ~(GRO_NO_DECAY | GRO_FROZEN | GRO_FP32_GRAD))
    return set_error(GRO_E_PLACEMENT, "param_id %lld: unknown flags 0x%x",
                     (long long)d.param_id, d.flags);
  switch (d.placement) {
    case GRO_SHARD:
      if (d.shard_index < 0 || d.shard_index >= R)
        return set_error(GRO_E_PLACEMENT, "param_id %lld: shard_index %d not in [0, %d)",
                         (long long)d.param_id, d.shard_index, R);
      break;
    case GRO_REPLICATE:
    case GRO_PARTIAL:
    case GRO_REDUCED:
      if (d.shard_index != -1)
        return set_error(GRO_E_PLACEMENT, "param_id %lld: shard_index must be -1 unless Shard",
                         (long long)d.param_id);
      break;
    default:
      return set_error(GRO_E_PLACEMENT, "param_id %lld: unknown placement %d",
                       (long long)d.param_id, d.placement);
  }
  lay->flat_offset = -1;
  lay->first_bucket = -1;
  if (d.flags & GRO_FROZEN) {
    lay->owner = GRO_OWNER_EXCLUDED;
    return GRO_OK;
  }
  switch (d.placement) {
    case GRO_REPLICATE: lay->owner = GRO_OWNER_MEAN; lay->slots = R; lay->divisor = R; break;
    case GRO_PARTIAL: lay->owner = GRO_OWNER_SUM; lay->slots = R; lay->divisor = 1; break;
    case GRO_SHARD: lay->owner = GRO_OWNER_LOCAL_SHARD; lay->slots = 1; lay->divisor = 1; break;
    default: lay->owner = GRO_OWNER_LOCAL_REDUCED; lay->slots = 1; lay->divisor = 1; break;
  }
  lay->in_norm = 1;
  lay->updated = 1;
  lay->decayed = (d.flags & GRO_NO_DECAY) ? 0 : 1;
  lay->grad_dtype = (d.flags & GRO_FP32_GRAD) ? GRO_GRAD_FP32 : GRO_GRAD_BF16;
  return GRO_OK;
}

void open_bucket(gro_plan* p, int64_t base, int32_t owner, int32_t slots, int32_t decayed,
                 int32_t grad_dtype) {
  gro_bucket_info b;
  std::memset(&b, 0, sizeof(b));
  b.flat_base = base;
  b.owner = owner;
  b.slots = slots;
  b.decayed = decayed;
  b.grad_dtype = grad_dtype;
  p->buckets.push_back(b);
}

}  // namespace
}  // namespace gro

using namespace gro;

extern "C" int gro_plan_create(const gro_tensor_desc* tensors, int32_t n_tensors, int32_t R,
                               int64_t bucket_elems, gro_plan** out) {
  clear_error();
  if (out == nullptr) return set_error(GRO_E_INVALID, "out is NULL");
  *out = nullptr;
  if (R < 1) return set_error(GRO_E_INVALID, "R must be >= 1 (got %d)", R);
  if (n_tensors < 0) return set_error(GRO_E_INVALID, "n_tensors < 0");
  if (n_tensors > 0 && tensors == nullptr) return set_error(GRO_E_INVALID, "tensors is NULL");
  if (bucket_elems < kAlignElems)
    return set_error(GRO_E_INVALID, "bucket_elems must be >= %lld", (long long)kAlignElems);

  gro_plan* p = new (std::nothrow) gro_plan();
  if (p == nullptr) return set_error(GRO_E_INVALID, "out of host memory");
  p->R = R;
  p->bucket_elems = bucket_elems;
  p->tensors.resize(size_t(n_tensors));

  std::unordered_set<int64_t> seen;
  seen.reserve(size_t(n_tensors) * 2 + 1);
  for (int32_t i = 0; i < n_tensors; ++i) {
    if (!seen.insert(tensors[i].param_id).second) {
      delete p;
      return set_error(GRO_E_DUPLICATE, "param_id %lld has a second owner",
                       (long long)tensors[i].param_id);
    }
    p->shard_index.push_back(tensors[i].shard_index);
    const int rc = classify(tensors[i], R, &p->tensors[size_t(i)]);
    if (rc != GRO_OK) {
      delete p;
      return rc;
    }
  }

  // Layout.  Groups in a fixed order of (owner, decay); descriptor order
  // inside a group.  `split` is the capacity rounded down to the alignment,
  // so the pieces of a split tensor stay contiguous in the flat arrays.
  const int64_t split = bucket_elems / kAlignElems * kAlignElems;
  int64_t pos = 0;  // end of the last bucket
  const int32_t owners[4] = {GRO_OWNER_MEAN, GRO_OWNER_SUM, GRO_OWNER_LOCAL_SHARD,
                             GRO_OWNER_LOCAL_REDUCED};
  for (int32_t owner : owners) {
    for (int32_t decayed = 1; decayed >= 0; --decayed) {
     for (int32_t dtype = GRO_GRAD_BF16; dtype <= GRO_GRAD_FP32; ++dtype) {
      bool open = false;  // a bucket of this group accepts more tensors
      for (auto& t : p->tensors) {
        if (t.owner != owner || t.decayed != decayed || t.grad_dtype != dtype || t.numel == 0 ||
            !t.updated)
          continue;
        if (t.numel <= bucket_elems) {
          if (!open || p->buckets.back().len + t.numel > bucket_elems) {
            open_bucket(p, align_up(pos, kAlignElems), owner, t.slots, decayed, dtype);
            open = true;
          }
          gro_bucket_info& b = p->buckets.back();
          t.flat_offset = b.flat_base + b.len;
          t.first_bucket = int32_t(p->buckets.size() - 1);
          t.n_buckets = 1;
          b.len += t.numel;
          pos = b.flat_base + b.len;
        } else {
          int64_t left = t.numel;
          const int64_t base = align_up(pos, kAlignElems);
          t.flat_offset = base;
          t.first_bucket = int32_t(p->buckets.size());
          t.n_buckets = 0;
          while (left > 0) {
            const int64_t piece = left < split ? left : split;
            open_bucket(p, align_up(pos, kAlignElems), owner, t.slots, decayed, dtype);
            p->buckets.back().len = piece;
            pos = p->buckets.back().flat_base + piece;
            left -= piece;
            ++t.n_buckets;
          }
          open = true;  // the last piece's bucket may take following tensors
        }
      }
     }
    }
  }
  p->n_flat = align_up(pos, kAlignElems);
  if (p->n_flat / kChunkElems + int64_t(p->buckets.size()) + 8 > int64_t(INT32_MAX)) {
    delete p;
    return set_error(GRO_E_INVALID, "plan too large: more chunks than one launch grid addresses");
  }

  // Chunks and device tables.
  for (size_t b = 0; b < p->buckets.size(); ++b) {
    gro_bucket_info& bk = p->buckets[b];
    bk.slot_stride = align_up(bk.len, kAlignElems);
    bk.first_chunk = int64_t(p->chunks.size());
    for (int64_t off = 0; off < bk.len; off += kChunkElems) {
      ChunkDev c;
      c.begin = bk.flat_base + off;
      c.len = int32_t((bk.len - off) < kChunkElems ? (bk.len - off) : kChunkElems);
      c.bucket = int32_t(b);
      p->chunks.push_back(c);
    }
    bk.n_chunks = int64_t(p->chunks.size()) - bk.first_chunk;
    p->n_owned += bk.len;
    BucketDev d;
    d.base = bk.flat_base;
    d.stride = bk.slot_stride;
    d.owner = bk.owner;
    d.slots = bk.slots;
    d.decayed = bk.decayed;
    d.grad_fp32 = bk.grad_dtype == GRO_GRAD_FP32 ? 1 : 0;
    p->bucket_dev.push_back(d);
  }

  WorkspaceLayout& ws = p->ws;
  uint64_t off = 0;
  ws.scalar_off = off;
  off += 256;
  ws.bucket_off = off;
  off = uint64_t(align_up(int64_t(off + p->bucket_dev.size() * sizeof(BucketDev)), 256));
  ws.chunk_off = off;
  off = uint64_t(align_up(int64_t(off + p->chunks.size() * sizeof(ChunkDev)), 256));
  ws.partial_off = off;
  off = uint64_t(align_up(int64_t(off + p->chunks.size() * sizeof(double)), 256));
  ws.tensor_off = off;
  off = uint64_t(align_up(int64_t(off + p->tensors.size() * sizeof(TensorDev)), 256));
  const int64_t groups = norm_groups(int64_t(p->chunks.size()));
  ws.group_off = off;
  off = uint64_t(align_up(int64_t(off + uint64_t(groups) * sizeof(double)), 256));
  ws.counter_off = off;
  ws.counter_bytes = uint64_t(align_up(int64_t((groups + 1) * sizeof(uint32_t)), 256));
  off += ws.counter_bytes;
  ws.total = off;

  p->count.assign(p->buckets.size(), 0);
  p->partials_ready.assign(p->buckets.size(), 0);
  *out = p;
  return GRO_OK;
}

extern "C" void gro_plan_destroy(gro_plan* plan) { delete plan; }

extern "C" int gro_plan_get_info(const gro_plan* p, gro_plan_info* info) {
  clear_error();
  if (p == nullptr || info == nullptr) return set_error(GRO_E_INVALID, "NULL argument");
  std::memset(info, 0, sizeof(*info));
  info->R = p->R;
  info->n_tensors = int32_t(p->tensors.size());
  info->n_buckets = int32_t(p->buckets.size());
  info->chunk_elems = kChunkElems;
  info->n_chunks = int64_t(p->chunks.size());
  info->n_flat = p->n_flat;
  info->n_owned = p->n_owned;
  info->bucket_elems = p->bucket_elems;
  info->workspace_bytes = p->ws.total;
  return GRO_OK;
}

extern "C" int gro_plan_tensor(const gro_plan* p, int32_t i, gro_tensor_layout* out) {
  clear_error();
  if (p == nullptr || out == nullptr) return set_error(GRO_E_INVALID, "NULL argument");
  if (i < 0 || size_t(i) >= p->tensors.size())
    return set_error(GRO_E_INVALID, "tensor index %d out of range", i);
  *out = p->tensors[size_t(i)];
  return GRO_OK;
}

extern "C" int gro_plan_bucket(const gro_plan* p, int32_t b, gro_bucket_info* out) {
  clear_error();
  if (p == nullptr || out == nullptr) return set_error(GRO_E_INVALID, "NULL argument");
  if (b < 0 || size_t(b) >= p->buckets.size())
    return set_error(GRO_E_INVALID, "bucket index %d out of range", b);
  *out = p->buckets[size_t(b)];
  return GRO_OK;
}

extern "C" const char* gro_last_error(void) { return g_last_error.c_str(); }
