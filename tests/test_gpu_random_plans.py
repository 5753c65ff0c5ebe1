"""Randomised GPU parity: seeded random parameter sets -- tensor count,
sizes (1 to ~50K elements, many ragged), placements, frozen / no-decay /
FP32-gradient flags, R, bucket capacity -- run through random window
sequences with one of the call styles, compared with the oracle bit for
bit.  Catches layout and tail cases that the hand-written workloads miss."""
import sys

import numpy as np
import pytest
import torch

from gradient_reduction_optimizer_amd import synth
from gpu_harness import assert_parity, run_parity

pytestmark = pytest.mark.gpu

SEEDS = list(range(48))


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _need_gpu(gpu):
    torch.cuda.synchronize()
    yield
    torch.cuda.synchronize()


def random_workload(seed: int):
    rng = np.random.default_rng(1000 + seed)
    R = int(rng.choice([1, 2, 3, 4]))
    n_t = int(rng.integers(1, 31))
    tensors = []
    for i in range(n_t):
        placement = str(rng.choice(synth.PLACEMENTS))
        if rng.random() < 0.3:
            shape = (int(rng.integers(1, 65)), int(rng.integers(1, 700)))
        else:
            shape = (int(np.clip(np.exp(rng.normal(7.0, 2.5)), 1, 50000)),)
        t = synth.TensorSpec(param_id=int(rng.integers(0, 1 << 40)) * 64 + i, name=f"t{i}", shape=shape,
                             placement=placement,
                             shard_index=int(rng.integers(0, R)) if placement == "shard" else -1,
                             frozen=bool(rng.random() < 0.08), no_decay=bool(rng.random() < 0.2),
                             fp32_grad=bool(rng.random() < 0.2))
        tensors.append(t)
    cap = int(rng.choice([64, 1000, 4096, 30000, 1 << 20]))
    windows = [int(x) for x in rng.integers(1, 6, size=int(rng.integers(1, 4)))]
    w = synth.Workload(f"random-{seed}", tensors, R=R, windows=windows, sigma=1e-2, seed=500 + seed,
                       bucket_elems=cap, max_norm=float(rng.choice([1.0, 0.0, 1e-3, 50.0])))
    style = str(rng.choice(["window", "microbatch", "unfused"]))
    return w, style


@pytest.mark.parametrize("seed", SEEDS)
def test_random_plan_matches_oracle(seed):
    w, style = random_workload(seed)
    log(f"case random seed={seed}: {len(w.tensors)} tensors, {w.numel} elements, R={w.R}, "
        f"cap={w.bucket_elems}, windows={w.windows}, style={style}, max_norm={w.max_norm}")
    c, cmps, norms = run_parity(w, w.windows, window_call=style == "window", fuse=style != "unfused",
                                log=log)
    assert_parity(cmps, norms)
    for k in cmps.values():
        assert k.n_diff_bits == 0, str(k)
