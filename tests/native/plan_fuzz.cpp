// Host fuzz driver for the planner (gro_plan_create / get_info / tensor /
// bucket / destroy), built with AddressSanitizer and UndefinedBehavior-
// Sanitizer by tests/test_plan_sanitizers.py.  Random descriptor sets; for
// each accepted plan it checks the layout invariants (disjoint, aligned,
// capacity-bounded buckets; chunks partitioning every bucket; every updated
// element in exactly one tensor span; a workspace large enough for every
// device table) and that rejected plans return a GRO_E_* code with a
// message.  Exit status 0 = all checks held.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "gro.h"

#define CHECK(cond)                                                         \
  do {                                                                      \
    if (!(cond)) {                                                          \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      std::exit(1);                                                         \
    }                                                                       \
  } while (0)

int main(int argc, char** argv) {
  const int trials = argc > 1 ? std::atoi(argv[1]) : 2000;
  std::mt19937_64 rng(1234);
  int accepted = 0, rejected = 0;
  for (int trial = 0; trial < trials; ++trial) {
    const bool bad = rng() % 2 == 0;                     // half the trials may hold one mistake
    const int32_t R = bad && rng() % 6 == 0 ? 0 : int32_t(1 + rng() % 8);
    const int32_t n = int32_t(rng() % 40);
    std::vector<std::vector<int64_t>> shapes(static_cast<size_t>(n));
    std::vector<gro_tensor_desc> d(static_cast<size_t>(n));
    for (int32_t i = 0; i < n; ++i) {
      const int nd = int(rng() % 4);
      for (int k = 0; k < nd; ++k)
        shapes[size_t(i)].push_back(int64_t(rng() % 90) - (bad && rng() % 200 == 0 ? 100 : 0));
      d[size_t(i)].param_id = (bad && rng() % 40 == 0 && i > 0) ? d[size_t(i - 1)].param_id : int64_t(rng() >> 3);
      d[size_t(i)].shape = shapes[size_t(i)].empty() ? nullptr : shapes[size_t(i)].data();
      d[size_t(i)].ndim = nd;
      d[size_t(i)].placement = bad && rng() % 40 == 0 ? 4 : int32_t(rng() % 4);   // 4 is unknown
      d[size_t(i)].shard_index = d[size_t(i)].placement == GRO_SHARD
                                     ? (bad && rng() % 40 == 0 ? R : int32_t(rng() % (R > 0 ? R : 1)))
                                     : -1;
      d[size_t(i)].flags = bad && rng() % 40 == 0 ? 8u : uint32_t(rng() % 8);     // 8 is unknown
    }
    const int64_t cap = int64_t(std::vector<int64_t>{32, 64, 100, 1000, 1 << 20}[rng() % 5]);
    gro_plan* p = nullptr;
    const int rc = gro_plan_create(d.empty() ? nullptr : d.data(), n, R, cap, &p);
    if (rc != GRO_OK) {
      CHECK(p == nullptr);
      CHECK(rc == GRO_E_INVALID || rc == GRO_E_PLACEMENT || rc == GRO_E_DUPLICATE);
      CHECK(std::strlen(gro_last_error()) > 0);
      ++rejected;
      continue;
    }
    ++accepted;
    gro_plan_info info;
    CHECK(gro_plan_get_info(p, &info) == GRO_OK);
    CHECK(info.n_tensors == n && info.R == R);
    std::vector<uint8_t> owner(static_cast<size_t>(info.n_flat), 0);
    int64_t end = 0, q = 0, owned = 0;
    for (int32_t b = 0; b < info.n_buckets; ++b) {
      gro_bucket_info bk;
      CHECK(gro_plan_bucket(p, b, &bk) == GRO_OK);
      CHECK(bk.flat_base % 64 == 0 && bk.flat_base >= end && bk.len > 0 && bk.len <= cap);
      CHECK(bk.slot_stride % 64 == 0 && bk.slot_stride >= bk.len);
      CHECK(bk.first_chunk == q && bk.n_chunks == (bk.len + info.chunk_elems - 1) / info.chunk_elems);
      q += bk.n_chunks;
      end = bk.flat_base + bk.len;
      owned += bk.len;
      CHECK(end <= info.n_flat);
    }
    CHECK(q == info.n_chunks && owned == info.n_owned);
    // the device workspace holds the scalars, the bucket and chunk tables,
    // one FP64 partial per chunk, the init table, one FP64 sum per group of
    // 2,048 partials and a uint32 counter per group plus one
    const uint64_t groups = uint64_t((info.n_chunks + 2047) / 2048);
    CHECK(info.workspace_bytes % 256 == 0);
    CHECK(info.workspace_bytes >= 256 + 32 * uint64_t(info.n_buckets) + 24 * uint64_t(info.n_chunks) +
                                      48 * uint64_t(info.n_tensors) + 8 * groups + 4 * (groups + 1));
    int64_t spans = 0;
    for (int32_t i = 0; i < n; ++i) {
      gro_tensor_layout t;
      CHECK(gro_plan_tensor(p, i, &t) == GRO_OK);
      if (!t.updated || t.numel == 0) {
        CHECK(t.flat_offset == -1 && t.n_buckets == 0);
        continue;
      }
      CHECK(t.flat_offset >= 0 && t.flat_offset + t.numel <= info.n_flat);
      for (int64_t k = 0; k < t.numel; ++k) {
        CHECK(owner[size_t(t.flat_offset + k)] == 0);
        owner[size_t(t.flat_offset + k)] = 1;
      }
      spans += t.numel;
    }
    CHECK(spans == info.n_owned);
    gro_tensor_layout t;
    CHECK(gro_plan_tensor(p, n, &t) == GRO_E_INVALID);
    gro_bucket_info bk;
    CHECK(gro_plan_bucket(p, info.n_buckets, &bk) == GRO_E_INVALID);
    gro_plan_destroy(p);
  }
  std::printf("trials %d accepted %d rejected %d\n", trials, accepted, rejected);
  return accepted > 0 && rejected > 0 ? 0 : 2;
}
