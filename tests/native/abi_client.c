/*
 * A plain C client of the C ABI (include/gro.h): no Python, no torch.  It
 * allocates every device buffer with hipMalloc, reads a plan and its inputs
 * from a binary file, runs `steps` optimizer windows (use_window_call 0: one
 * gro_accumulate per microbatch; 1: one gro_accumulate_window per window; 2:
 * gro_accumulate_microbatches for the first half of each window, then for the
 * rest), and writes the norm
 * of every window and the final master, m, v and BF16 copy to an output file.
 * tests/test_gpu_c_client.py writes the input, runs this program and checks
 * the output against the CPU oracle.
 *
 * Input file (little-endian):
 *   int32 n_tensors, R, steps, window, use_window_call; int64 bucket_elems;
 *   double lr, beta1, beta2, eps, weight_decay, max_norm;
 *   per tensor: int64 param_id, numel; int32 placement, shard_index; uint32 flags;
 *   per tensor (updated, in descriptor order): float master[numel];
 *   per step, per microbatch, per tensor (not frozen), per slot: uint16 bf16[numel]
 * Output file: double norm[steps]; int32 finite[steps];
 *   per tensor (updated): float master[numel], m[numel], v[numel]; uint16 bf16[numel]
 * With a third argument (a seed), the master read from the input is replaced
 * by gro_init_uniform(seed, bound 0.02 for every tensor, offset 0) before
 * the first window.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "gro.h"

#define DIE(...) do { fprintf(stderr, __VA_ARGS__); fprintf(stderr, "\n"); exit(1); } while (0)
#define HIPCHK(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) DIE("%s: %s", #x, hipGetErrorString(e_)); } while (0)
#define GROCHK(x) do { int r_ = (x); if (r_ != GRO_OK) DIE("%s: %d %s", #x, r_, gro_last_error()); } while (0)

static void rd(FILE* f, void* p, size_t n) { if (fread(p, 1, n, f) != n) DIE("short read"); }
static void wr(FILE* f, const void* p, size_t n) { if (fwrite(p, 1, n, f) != n) DIE("short write"); }

int main(int argc, char** argv) {
  if (argc != 3 && argc != 4) DIE("usage: %s input output [init_seed]", argv[0]);
  FILE* in = fopen(argv[1], "rb");
  if (!in) DIE("cannot open %s", argv[1]);
  int32_t hdr[5];
  int64_t bucket_elems;
  double hpv[6];
  rd(in, hdr, sizeof(hdr));
  rd(in, &bucket_elems, sizeof(bucket_elems));
  rd(in, hpv, sizeof(hpv));
  const int32_t nt = hdr[0], R = hdr[1], steps = hdr[2], window = hdr[3], use_window = hdr[4];
  gro_tensor_desc* d = calloc((size_t)(nt > 0 ? nt : 1), sizeof(gro_tensor_desc));
  int64_t* numel = calloc((size_t)(nt > 0 ? nt : 1), sizeof(int64_t));
  for (int32_t i = 0; i < nt; ++i) {
    rd(in, &d[i].param_id, 8);
    rd(in, &numel[i], 8);
    rd(in, &d[i].placement, 4);
    rd(in, &d[i].shard_index, 4);
    rd(in, &d[i].flags, 4);
    d[i].ndim = 1;
    d[i].shape = &numel[i];
  }
  gro_plan* plan = NULL;
  GROCHK(gro_plan_create(d, nt, R, bucket_elems, &plan));
  gro_plan_info info;
  GROCHK(gro_plan_get_info(plan, &info));
  const size_t nflat = (size_t)(info.n_flat > 0 ? info.n_flat : 1);

  void* ws = NULL;
  float *acc, *master, *m, *v;
  uint16_t* p16;
  HIPCHK(hipMalloc(&ws, info.workspace_bytes));
  HIPCHK(hipMalloc((void**)&acc, nflat * 4));
  HIPCHK(hipMalloc((void**)&master, nflat * 4));
  HIPCHK(hipMalloc((void**)&m, nflat * 4));
  HIPCHK(hipMalloc((void**)&v, nflat * 4));
  HIPCHK(hipMalloc((void**)&p16, nflat * 2));
  HIPCHK(hipMemset(m, 0, nflat * 4));
  HIPCHK(hipMemset(v, 0, nflat * 4));
  hipStream_t s;
  HIPCHK(hipStreamCreate(&s));
  GROCHK(gro_plan_bind(plan, ws, info.workspace_bytes, s));

  gro_tensor_layout* lay = calloc((size_t)(nt > 0 ? nt : 1), sizeof(gro_tensor_layout));
  for (int32_t i = 0; i < nt; ++i) GROCHK(gro_plan_tensor(plan, i, &lay[i]));
  gro_bucket_info* bk = calloc((size_t)(info.n_buckets > 0 ? info.n_buckets : 1), sizeof(gro_bucket_info));
  for (int32_t b = 0; b < info.n_buckets; ++b) GROCHK(gro_plan_bucket(plan, b, &bk[b]));

  for (int32_t i = 0; i < nt; ++i) {
    if (!lay[i].updated || lay[i].numel == 0) continue;
    float* h = malloc((size_t)lay[i].numel * 4);
    rd(in, h, (size_t)lay[i].numel * 4);
    HIPCHK(hipMemcpy(master + lay[i].flat_offset, h, (size_t)lay[i].numel * 4, hipMemcpyHostToDevice));
    free(h);
  }
  if (argc == 4) {
    double* bounds = calloc((size_t)(nt > 0 ? nt : 1), sizeof(double));
    for (int32_t i = 0; i < nt; ++i) bounds[i] = 0.02;
    GROCHK(gro_init_uniform(plan, strtoull(argv[3], NULL, 10), bounds, NULL, master, NULL, s));
    free(bounds);
  }
  /* one set of bucket buffers per microbatch of a window */
  const int nb = info.n_buckets;
  void** bufs = calloc((size_t)(window * (nb > 0 ? nb : 1)), sizeof(void*));
  for (int k = 0; k < window; ++k)
    for (int b = 0; b < nb; ++b) HIPCHK(hipMalloc(&bufs[k * nb + b], (size_t)(bk[b].slots * bk[b].slot_stride) * 2));
  gro_adamw_hparams hp = {hpv[0], hpv[1], hpv[2], hpv[3], hpv[4]};
  const double max_norm = hpv[5];
  double* norms = calloc((size_t)(steps > 0 ? steps : 1), sizeof(double));
  int32_t* fin = calloc((size_t)(steps > 0 ? steps : 1), sizeof(int32_t));
  for (int32_t t = 0; t < steps; ++t) {
    for (int k = 0; k < window; ++k) {
      for (int32_t i = 0; i < nt; ++i) {
        if (lay[i].owner == GRO_OWNER_EXCLUDED) continue;
        uint16_t* h = malloc((size_t)(lay[i].numel > 0 ? lay[i].numel : 1) * 2);
        for (int r = 0; r < lay[i].slots; ++r) {
          rd(in, h, (size_t)lay[i].numel * 2);
          /* scatter the tensor's elements over the buckets it spans */
          for (int b = lay[i].first_bucket; b >= 0 && b < lay[i].first_bucket + lay[i].n_buckets; ++b) {
            int64_t lo = lay[i].flat_offset > bk[b].flat_base ? lay[i].flat_offset : bk[b].flat_base;
            int64_t hi = lay[i].flat_offset + lay[i].numel < bk[b].flat_base + bk[b].len
                             ? lay[i].flat_offset + lay[i].numel : bk[b].flat_base + bk[b].len;
            if (hi <= lo) continue;
            uint16_t* dst = (uint16_t*)bufs[k * nb + b] + (size_t)r * bk[b].slot_stride + (lo - bk[b].flat_base);
            HIPCHK(hipMemcpy(dst, h + (lo - lay[i].flat_offset), (size_t)(hi - lo) * 2, hipMemcpyHostToDevice));
          }
        }
        free(h);
      }
      if (!use_window) GROCHK(gro_accumulate(plan, 0, nb, (const void* const*)&bufs[k * nb], acc, k, window, s));
    }
    if (use_window == 1) GROCHK(gro_accumulate_window(plan, 0, nb, (const void* const*)bufs, window, acc, s));
    if (use_window == 2) {
      const int half = window / 2 > 0 ? window / 2 : 1;
      GROCHK(gro_accumulate_microbatches(plan, 0, nb, (const void* const*)bufs, 0, half, window, acc, s));
      if (window > half)
        GROCHK(gro_accumulate_microbatches(plan, 0, nb, (const void* const*)&bufs[half * nb], half, window - half,
                                           window, acc, s));
    }
    GROCHK(gro_reduce_norm(plan, acc, window, s));
    GROCHK(gro_plan_get_norm(plan, &norms[t], NULL, &fin[t]));
    GROCHK(gro_clip_adamw(plan, acc, window, max_norm, &hp, (int64_t)t + 1, master, m, v, p16, s));
  }
  HIPCHK(hipStreamSynchronize(s));
  fclose(in);

  FILE* out = fopen(argv[2], "wb");
  if (!out) DIE("cannot open %s", argv[2]);
  wr(out, norms, (size_t)steps * 8);
  wr(out, fin, (size_t)steps * 4);
  for (int32_t i = 0; i < nt; ++i) {
    if (!lay[i].updated || lay[i].numel == 0) continue;
    const size_t n = (size_t)lay[i].numel;
    float* h = malloc(n * 4);
    float* arrs[3] = {master, m, v};
    for (int a = 0; a < 3; ++a) {
      HIPCHK(hipMemcpy(h, arrs[a] + lay[i].flat_offset, n * 4, hipMemcpyDeviceToHost));
      wr(out, h, n * 4);
    }
    HIPCHK(hipMemcpy(h, p16 + lay[i].flat_offset, n * 2, hipMemcpyDeviceToHost));
    wr(out, h, n * 2);
    free(h);
  }
  fclose(out);
  for (int k = 0; k < window * nb; ++k) HIPCHK(hipFree(bufs[k]));
  HIPCHK(hipFree(ws));
  HIPCHK(hipFree(acc));
  HIPCHK(hipFree(master));
  HIPCHK(hipFree(m));
  HIPCHK(hipFree(v));
  HIPCHK(hipFree(p16));
  HIPCHK(hipStreamDestroy(s));
  gro_plan_destroy(plan);
  printf("c client: %d steps of window %d, %s\n", steps, window,
         use_window == 1 ? "window call" : use_window == 2 ? "two groups" : "per microbatch");
  return 0;
}
