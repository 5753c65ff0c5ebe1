"""GPU parity: the HIP path through the C ABI against the CPU oracle, element
by element, on the same seeded inputs.

Tolerances: FP32 states and the norm within 1e-6 relative (floor 1e-6 of
the tensor's RMS), the BF16 copy within 1e-2 relative, the ownership table
bit-exact.  Both sides execute the same FP32 operations in the same order,
so the expected outcome is bit-identical states; the count of differing
elements is printed and, for the small cases, required to be zero.
"""
import math
import sys
from types import SimpleNamespace

import numpy as np
import pytest
import torch

import oracle.method as M
from gradient_reduction_optimizer_amd import binding as B
from gradient_reduction_optimizer_amd import synth
from gradient_reduction_optimizer_amd.buffers import DeviceState, Plan
from gpu_harness import (BF16_RTOL, FP32_RTOL, Case, Compare, assert_parity, bits16, host,
                         run_parity)

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _spec(pid, shape, placement, shard_index=None, frozen=False, no_decay=False):
    if shard_index is None:
        shard_index = 0 if placement == "shard" else -1
    return synth.TensorSpec(pid, f"t{pid}", tuple(shape), placement, shard_index=shard_index,
                            frozen=frozen, no_decay=no_decay)


def ragged_workload(R=2, seed=7, bucket_elems=25_000_000, sizes=None, fp32_every=0):
    """Odd-sized tensors of every placement spanning several chunks, plus a
    frozen and a no-decay tensor."""
    rng = np.random.default_rng(seed)
    if sizes is None:
        sizes = [1, 7, 8, 9, 63, 65, 1000, 4095, 4096, 4097, 8193, 16383, 16384, 16385, 40000, 70001,
                 3 * 16384 + 5]
    tensors = []
    for i, n in enumerate(sizes):
        pl = synth.PLACEMENTS[i % 4]
        tensors.append(_spec(i, (n,), pl, shard_index=(i % R) if pl == "shard" else -1,
                             no_decay=(i % 5 == 3)))
        tensors[-1].fp32_grad = bool(fp32_every) and i % fp32_every == 1
    tensors.append(_spec(len(sizes), (33, 17), "replicate", frozen=True))
    tensors.append(_spec(len(sizes) + 1, (0, 4), "partial"))
    return synth.Workload("ragged", tensors, R=R, windows=[3], sigma=1e-2, seed=seed,
                          bucket_elems=bucket_elems)


@pytest.fixture(autouse=True)
def _need_gpu(gpu):
    torch.cuda.synchronize()
    yield
    torch.cuda.synchronize()


# --------------------------------------------------------------- tiny sets
@pytest.mark.parametrize("name", ["tiny", "tiny-literal"])
def test_tiny_parity_bit_exact(name):
    w = synth.WORKLOADS[name]()
    log(f"case {name} windows [1, 3, 2]")
    _, cmps, norms = run_parity(w, [1, 3, 2], log=log)
    assert_parity(cmps, norms)
    for k in cmps.values():
        assert k.n_diff_bits == 0, str(k)


def test_tiny_small_buckets_split_tensors():
    w = synth.tiny(bucket_elems=4096)
    log("case tiny bucket_elems=4096")
    c, cmps, norms = run_parity(w, [2, 1], log=log)
    assert c.plan.info["n_buckets"] > 8
    assert_parity(cmps, norms)
    for k in cmps.values():
        assert k.n_diff_bits == 0, str(k)


@pytest.mark.parametrize("R", [1, 2, 3, 4, 8, 16])
def test_ragged_sizes_every_R(R):
    w = ragged_workload(R=R)
    log(f"case ragged R={R}")
    _, cmps, norms = run_parity(w, [3, 4, 1], log=log)
    assert_parity(cmps, norms)
    for k in cmps.values():
        assert k.n_diff_bits == 0, str(k)


@pytest.mark.parametrize("R", [2, 3])
@pytest.mark.parametrize("window_call", [False, True])
def test_subnormal_contributions(R, window_call):
    """Subnormal BF16 and FP32 contributions: the kernels' FP32 arithmetic
    keeps subnormals (no flush to zero), as the oracle's numpy does -- the
    sums, means, accumulation, the FP64 norm and m come out bit-identical
    (v underflows to zero on both sides)."""
    w = ragged_workload(R=R, fp32_every=4)
    w.values = "subnormal"
    log(f"case subnormal contributions R={R} window_call={window_call}")
    c, cmps, norms = run_parity(w, [2, 3], window_call=window_call, log=log)
    assert_parity(cmps, norms)
    for k in cmps.values():
        assert k.n_diff_bits == 0, str(k)
    tiny = (c.st.acc != 0) & (c.st.acc.abs() < torch.finfo(torch.float32).tiny)
    assert int(tiny.sum()) > 1000
    assert 0.0 < norms[-1][0] < 1e-30


def test_large_step_counts():
    """Bias corrections at step counts from 1 to 2^40 (beta^t underflows to 0
    long before): the FP64 host scalars and the kernels follow the oracle."""
    w = ragged_workload(R=2)
    steps = [1, 2, 1000, 10 ** 6, 2 ** 31 + 7, 2 ** 40]
    log(f"case step counts {steps}")
    _, cmps, norms = run_parity(w, [2] * len(steps), step_numbers=steps, log=log)
    assert_parity(cmps, norms)
    for k in cmps.values():
        assert k.n_diff_bits == 0, str(k)


def test_more_than_64_buckets_per_call():
    w = ragged_workload(bucket_elems=64, sizes=[5000, 3, 64, 129, 777])
    log("case ragged bucket_elems=64 (many launches per call)")
    c, cmps, norms = run_parity(w, [2], log=log)
    assert c.plan.info["n_buckets"] > 64
    assert_parity(cmps, norms)


def test_unfused_and_per_bucket_calls_give_identical_bits():
    w = ragged_workload(bucket_elems=20000)
    log("case fused vs unfused vs per-bucket calls")
    ca, _, na = run_parity(w, [3, 2], fuse=True, log=log)
    cb, _, nb_ = run_parity(w, [3, 2], fuse=False, log=log)
    nbk = ca.plan.info["n_buckets"]
    cc, _, nc = run_parity(w, [3, 2], fuse=True, bucket_order=list(range(nbk))[::-1], log=log)
    for x in (cb, cc):
        for arr in ("acc", "master", "m", "v"):
            assert torch.equal(getattr(ca.st, arr).view(torch.int32), getattr(x.st, arr).view(torch.int32)), arr
        assert torch.equal(ca.st.p_bf16.view(torch.int16), x.st.p_bf16.view(torch.int16))
    assert [n[0] for n in na] == [n[0] for n in nb_] == [n[0] for n in nc]


@pytest.mark.parametrize("R", [1, 2, 3])
def test_window_call_matches_oracle_and_microbatch_calls(R):
    """gro_accumulate_window gives the oracle's results and the same bits as
    one gro_accumulate per microbatch, for full, trailing and single windows."""
    w = ragged_workload(R=R, bucket_elems=30000)
    log(f"case window call R={R}")
    ca, cmps, na = run_parity(w, [3, 4, 1, 8], window_call=True, log=log)
    assert_parity(cmps, na)
    for k in cmps.values():
        assert k.n_diff_bits == 0, str(k)
    cb, _, nb_ = run_parity(w, [3, 4, 1, 8], window_call=False, log=log)
    for arr in ("acc", "master", "m", "v"):
        assert torch.equal(getattr(ca.st, arr).view(torch.int32), getattr(cb.st, arr).view(torch.int32)), arr
    assert [n[0] for n in na] == [n[0] for n in nb_]


@pytest.mark.parametrize("window_call", [False, True])
def test_poisoned_padding_is_never_read_or_written(window_call):
    """NaN in every padding element -- the gradient buffers past each
    bucket's length, and the flat-array gaps between buckets -- changes no
    result (the oracle never sees it) and is still there afterwards."""
    w = ragged_workload(R=2, bucket_elems=30000, fp32_every=4)
    log(f"case poisoned padding, window_call={window_call}")
    c, cmps, norms = run_parity(w, [3, 1, 2], window_call=window_call, poison=True, log=log)
    assert c.flat_gaps(), "the layout has no gaps to poison"
    assert_parity(cmps, norms)
    for k in cmps.values():
        assert k.n_diff_bits == 0, str(k)
    assert c.flat_gaps_untouched()


@pytest.mark.parametrize("R", [1, 2, 3])
@pytest.mark.parametrize("announce", [True, False])
def test_microbatch_groups_match_oracle_and_per_microbatch_calls(R, announce):
    """gro_accumulate_microbatches over groups of a window (3+1+4 of 8, 2+1 of a
    trailing 3, 5 of 5, 1 of 1), with and without the window length
    announced: the oracle's results, and the same bits as one gro_accumulate
    per microbatch."""
    w = ragged_workload(R=R, bucket_elems=30000, fp32_every=4)
    windows, groups = [8, 3, 5, 1], [[3, 1, 4], [2, 1], [5], [1]]
    log(f"case microbatch groups R={R} announce={announce}")
    ca, cmps, na = run_parity(w, windows, groups=groups, announce=announce, log=log)
    assert_parity(cmps, na)
    for k in cmps.values():
        assert k.n_diff_bits == 0, str(k)
    cb, _, nb_ = run_parity(w, windows, log=log)
    for arr in ("acc", "master", "m", "v"):
        assert torch.equal(getattr(ca.st, arr).view(torch.int32), getattr(cb.st, arr).view(torch.int32)), arr
    assert [n[0] for n in na] == [n[0] for n in nb_]


def test_call_styles_mixed_within_one_window():
    """One window of 6 built from gro_accumulate (microbatch 0), a group
    (1-3), gro_accumulate (4) and a group of one that closes it (5) gives the
    same bits as six gro_accumulate calls; a group that does not continue
    where the buckets stand, or runs past the window, is rejected."""
    w = ragged_workload(R=2, bucket_elems=30000)
    ca, cb = Case(w), Case(w)
    n = 6
    micro = [ca.draw(1, k) for k in range(n)]
    for k in range(n):
        cb.gpu_accumulate(micro[k], k, n)
    nb = ca.plan.info["n_buckets"]
    while len(ca.window_bufs) < n:
        ca.window_bufs.append(ca.st.grad_buffers())
    for k in range(n):
        for i, g in enumerate(micro[k]):
            if g is not None:
                ca.st.pack(ca.window_bufs[k], i, g)
    h, s, acc = ca.plan.handle, ca.stream, ca.st.acc.data_ptr()
    ptrs = lambda k0, g: [ca.window_bufs[k][b].data_ptr() for k in range(k0, k0 + g) for b in range(nb)]
    B.gro_accumulate(h, 0, nb, [b.data_ptr() for b in ca.window_bufs[0]], acc, 0, n, s)
    with pytest.raises(B.GroError) as e:                 # skips microbatch 1
        B.gro_accumulate_microbatches(h, 0, nb, ptrs(2, 2), 2, 2, n, acc, s)
    assert e.value.kind == "state"
    with pytest.raises(B.GroError) as e:                 # runs past the window
        B.gro_accumulate_microbatches(h, 0, nb, ptrs(1, 5) + ptrs(5, 1), 1, 6, n, acc, s)
    assert e.value.kind == "invalid"
    B.gro_accumulate_microbatches(h, 0, nb, ptrs(1, 3), 1, 3, n, acc, s)
    B.gro_accumulate(h, 0, nb, [b.data_ptr() for b in ca.window_bufs[4]], acc, 4, n, s)
    B.gro_accumulate_microbatches(h, 0, nb, ptrs(5, 1), 5, 1, n, acc, s)
    na = ca.gpu_finish(n, 1, w.max_norm)
    nb_ = cb.gpu_finish(n, 1, w.max_norm)
    assert na[0] == nb_[0]
    for arr in ("acc", "master", "m", "v"):
        assert torch.equal(getattr(ca.st, arr).view(torch.int32), getattr(cb.st, arr).view(torch.int32)), arr


def test_window_call_longest_windows():
    """The longest window one call takes (64 microbatches, one bucket per
    launch), then windows of 5 and 17 (the double-buffered path), with BF16
    and FP32 contributions mixed: oracle results, and the same bits as one
    gro_accumulate per microbatch."""
    w = ragged_workload(R=2, bucket_elems=30000, fp32_every=3)
    windows = [64, 5, 17]
    log(f"case window call windows {windows}")
    ca, cmps, na = run_parity(w, windows, window_call=True, log=log)
    assert_parity(cmps, na)
    for k in cmps.values():
        assert k.n_diff_bits == 0, str(k)
    cb, _, nb_ = run_parity(w, windows, window_call=False, log=log)
    for arr in ("acc", "master", "m", "v"):
        assert torch.equal(getattr(ca.st, arr).view(torch.int32), getattr(cb.st, arr).view(torch.int32)), arr
    assert [n[0] for n in na] == [n[0] for n in nb_]


def test_window_call_tiny_and_many_buckets():
    for w in (synth.tiny(), synth.tiny(bucket_elems=4096)):
        log(f"case window call {w.name} cap={w.bucket_elems}")
        c, cmps, norms = run_parity(w, [2, 5], window_call=True, log=log)
        assert_parity(cmps, norms)
        for k in cmps.values():
            assert k.n_diff_bits == 0, str(k)


@pytest.mark.parametrize("R", [1, 2, 3])
@pytest.mark.parametrize("window_call", [False, True])
def test_fp32_gradient_contributions(R, window_call):
    """Tensors whose contributions arrive in FP32 (their own buckets) next to
    BF16 ones, per-microbatch and window calls."""
    w = ragged_workload(R=R, fp32_every=2, bucket_elems=30000)
    assert any(t.fp32_grad for t in w.tensors) and not all(t.fp32_grad for t in w.tensors)
    log(f"case fp32 contributions R={R} window_call={window_call}")
    c, cmps, norms = run_parity(w, [3, 2, 8], window_call=window_call, log=log)
    assert any(bk["grad_dtype"] == B.GRO_GRAD_FP32 for bk in c.plan.buckets)
    assert_parity(cmps, norms)
    for k in cmps.values():
        assert k.n_diff_bits == 0, str(k)


def test_unused_parameters_are_still_decayed_and_updated():
    """An unused parameter contributes zero gradients (DDP semantics): it is
    in the norm (adding 0), decayed and stepped like any other."""
    w = ragged_workload()
    zero = [i for i, t in enumerate(w.tensors) if not t.frozen and t.numel > 100][:3]
    log(f"case unused parameters {zero}")
    c, cmps, norms = run_parity(w, [2, 3], zero_tensors=zero, log=log)
    assert_parity(cmps, norms)
    for k in cmps.values():
        assert k.n_diff_bits == 0, str(k)
    m = host(c.st.m)
    for i in zero:
        off = c.plan.tensors[i]["flat_offset"]
        assert not np.any(m[off:off + w.tensors[i].numel])   # m stays 0 for a zero gradient


@pytest.mark.parametrize("max_norm", [0.0, float("inf"), -1.0, 1e-3, 1e9])
def test_clip_settings(max_norm):
    w = synth.tiny()
    log(f"case tiny max_norm={max_norm}")
    _, cmps, norms = run_parity(w, [2], max_norm=max_norm, log=log)
    assert_parity(cmps, norms)


def test_repeat_runs_are_bit_identical():
    w = synth.tiny(literal=True)
    a, _, na = run_parity(w, [2, 3], log=log)
    b, _, nb_ = run_parity(w, [2, 3], log=log)
    assert [x[0] for x in na] == [x[0] for x in nb_]
    for arr in ("acc", "master", "m", "v"):
        assert torch.equal(getattr(a.st, arr).view(torch.int32), getattr(b.st, arr).view(torch.int32))


# ----------------------------------------------------------- edge cases
def test_nonfinite_gradient_skips_the_step():
    w = ragged_workload()
    c = Case(w)
    before = {k: getattr(c.st, k).clone() for k in ("master", "m", "v", "p_bf16")}
    g = c.draw(1, 0)
    i = next(j for j, x in enumerate(g) if x is not None and x[0].numel() > 100)
    g[i][0][37] = float("nan")
    c.gpu_accumulate(g, 0, 1)
    norm, norm_sq, finite = c.gpu_finish(1, 1, 1.0)
    log(f"nan case: norm={norm} finite={finite}")
    assert not finite and math.isnan(norm)
    for k, t in before.items():
        assert torch.equal(getattr(c.st, k).view(torch.int16 if k == "p_bf16" else torch.int32),
                           t.view(torch.int16 if k == "p_bf16" else torch.int32)), k
    # the next window works normally
    g = c.draw(2, 0)
    c.gpu_accumulate(g, 0, 1)
    norm, _, finite = c.gpu_finish(1, 1, 1.0)
    assert finite and math.isfinite(norm)
    # an infinity is reported the same way
    g = c.draw(3, 0)
    g[i][0][5] = float("inf")
    c.gpu_accumulate(g, 0, 1)
    norm, _, finite = c.gpu_finish(1, 2, 1.0)
    assert not finite


def test_empty_and_all_frozen_plans():
    for tensors in ([], [_spec(1, (100,), "replicate", frozen=True), _spec(2, (0,), "shard")]):
        plan = Plan(tensors, 2, 1 << 20)
        st = DeviceState(plan)
        s = torch.cuda.current_stream().cuda_stream
        B.gro_accumulate(plan.handle, 0, 0, [], st.acc.data_ptr(), 0, 1, s)
        B.gro_reduce_norm(plan.handle, st.acc.data_ptr(), 1, s)
        norm, sq, finite = B.gro_plan_get_norm(plan.handle)
        assert norm == 0.0 and sq == 0.0 and finite
        B.gro_clip_adamw(plan.handle, st.acc.data_ptr(), 1, 1.0,
                         dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01), 1,
                         st.master.data_ptr(), st.m.data_ptr(), st.v.data_ptr(), st.p_bf16.data_ptr(), s)
        torch.cuda.synchronize()


def test_bf16_copy_rounding_edge_classes():
    """With lr = 0 and no decay the update leaves p unchanged, so the BF16
    copy is RNE(p) for arbitrary FP32 bit patterns fed in as the master."""
    hi = np.arange(0, 65536, 7, dtype=np.uint32) << np.uint32(16)
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32)
    pats = (hi[:, None] | lows[None, :]).ravel()
    pats = np.concatenate([pats, np.array([0x7F7FFFFF, 0xFF7FFFFF, 0x7F7F8000, 0x00008000,
                                           0x7F800000, 0xFF800000, 0x7FC00000, 0x00000001], np.uint32)])
    x = pats.view(np.float32)
    n = x.size
    w = synth.Workload("bf16-edges", [_spec(0, (n,), "reduced")], R=1, windows=[1], sigma=0.0, seed=0,
                       bucket_elems=1 << 24, lr=0.0, weight_decay=0.0)
    plan = Plan(w.tensors, 1, w.bucket_elems)
    st = DeviceState(plan)
    st.flat_view(st.master, 0).copy_(torch.from_numpy(x.copy()))
    bufs = st.grad_buffers()  # zero gradients
    s = torch.cuda.current_stream().cuda_stream
    B.gro_accumulate(plan.handle, 0, 1, [bufs[0].data_ptr()], st.acc.data_ptr(), 0, 1, s)
    B.gro_reduce_norm(plan.handle, st.acc.data_ptr(), 1, s)
    B.gro_clip_adamw(plan.handle, st.acc.data_ptr(), 1, 0.0, w.hparams, 1, st.master.data_ptr(),
                     st.m.data_ptr(), st.v.data_ptr(), st.p_bf16.data_ptr(), s)
    got = bits16(st.flat_view(st.p_bf16, 0))
    want = M.f32_to_bf16(x)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.isnan(M.bf16_to_f32(got[nan])).all()
    master = host(st.flat_view(st.master, 0))
    fin = np.isfinite(x)
    assert np.array_equal(master[fin].view(np.uint32), x[fin].view(np.uint32))


def test_window_bookkeeping_errors():
    w = synth.tiny()
    c = Case(w)
    s = c.stream
    nb = c.plan.info["n_buckets"]
    ptrs = [b.data_ptr() for b in c.bufs]
    h = c.plan.handle
    acc = c.st.acc.data_ptr()
    with pytest.raises(B.GroError) as e:      # no norm computed yet
        B.gro_plan_get_norm(h)
    assert e.value.kind == "state"
    with pytest.raises(B.GroError) as e:      # skipping microbatch 0
        B.gro_accumulate(h, 0, nb, ptrs, acc, 1, 2, s)
    assert e.value.kind == "state"
    B.gro_accumulate(h, 0, nb, ptrs, acc, 0, 2, s)
    with pytest.raises(B.GroError) as e:      # window not complete
        B.gro_reduce_norm(h, acc, 2, s)
    assert e.value.kind == "state"
    with pytest.raises(B.GroError) as e:      # clip before norm
        B.gro_clip_adamw(h, acc, 1, 1.0, w.hparams, 1, c.st.master.data_ptr(), c.st.m.data_ptr(),
                         c.st.v.data_ptr(), 0, s)
    assert e.value.kind == "state"
    with pytest.raises(B.GroError) as e:      # misaligned pointer
        B.gro_accumulate(h, 0, nb, ptrs, acc + 4, 1, 2, s)
    assert e.value.kind == "invalid"
    B.gro_accumulate(h, 0, nb, ptrs, acc, 1, 2, s)
    with pytest.raises(B.GroError) as e:      # window-size mismatch
        B.gro_reduce_norm(h, acc, 3, s)
    assert e.value.kind == "state"
    B.gro_reduce_norm(h, acc, 2, s)
    with pytest.raises(B.GroError) as e:      # bad step
        B.gro_clip_adamw(h, acc, 2, 1.0, w.hparams, 0, c.st.master.data_ptr(), c.st.m.data_ptr(),
                         c.st.v.data_ptr(), 0, s)
    assert e.value.kind == "invalid"
    with pytest.raises(B.GroError) as e:      # NaN max_norm
        B.gro_clip_adamw(h, acc, 2, float("nan"), w.hparams, 1, c.st.master.data_ptr(), c.st.m.data_ptr(),
                         c.st.v.data_ptr(), 0, s)
    assert e.value.kind == "invalid"
    B.gro_clip_adamw(h, acc, 2, 1.0, w.hparams, 1, c.st.master.data_ptr(), c.st.m.data_ptr(),
                     c.st.v.data_ptr(), 0, s)
    with pytest.raises(B.GroError) as e:      # the window was consumed
        B.gro_reduce_norm(h, acc, 2, s)
    assert e.value.kind == "state"
    # one accumulator per window
    assert nb >= 2
    acc2 = torch.zeros_like(c.st.acc)
    B.gro_accumulate(h, 0, 1, ptrs[:1], acc, 0, 1, s)
    for call in (lambda: B.gro_accumulate(h, 1, nb, ptrs[1:], acc2.data_ptr(), 0, 1, s),
                 lambda: B.gro_accumulate_window(h, 1, nb, ptrs[1:], 1, acc2.data_ptr(), s)):
        with pytest.raises(B.GroError) as e:
            call()
        assert e.value.kind == "state"
    B.gro_accumulate_window(h, 1, nb, ptrs[1:], 1, acc, s)
    B.gro_reduce_norm(h, acc, 1, s)
    torch.cuda.synchronize()


def test_two_plans_on_two_streams_from_two_threads():
    """Distinct plans may be driven from distinct host threads on distinct
    streams at the same time; both runs still match the oracle bit for bit."""
    import threading
    results, failures = {}, {}

    def run(name, w, window_call):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                _, cmps, norms = run_parity(w, [3, 2, 4], window_call=window_call, log=lambda m: None)
            torch.cuda.synchronize()
            results[name] = (cmps, norms)
        except Exception as e:  # surfaced below
            failures[name] = repr(e)

    ws = {"a": (ragged_workload(R=2, seed=21), False), "b": (ragged_workload(R=3, seed=22, fp32_every=3), True)}
    threads = [threading.Thread(target=run, args=(k, w, wc)) for k, (w, wc) in ws.items()]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not failures, failures
    for name, (cmps, norms) in results.items():
        log(f"thread {name}: " + "; ".join(str(k) for k in cmps.values()))
        assert_parity(cmps, norms)
        for k in cmps.values():
            assert k.n_diff_bits == 0, (name, str(k))


def test_rebinding_moves_the_tables_and_resets_the_window():
    """gro_plan_bind may be repeated: the tables move to the new workspace,
    an unfinished window is dropped (its bookkeeping reset), and results
    equal a run that was bound there from the start.  A workspace that is
    too small or misaligned is rejected."""
    w = ragged_workload(R=2, bucket_elems=30000)
    c = Case(w)
    h, s = c.plan.handle, c.stream
    nb = c.plan.info["n_buckets"]
    ptrs = [b.data_ptr() for b in c.bufs]
    need = int(c.plan.info["workspace_bytes"])
    ws2 = torch.zeros(need + 512, dtype=torch.uint8, device="cuda")
    base = (ws2.data_ptr() + 255) // 256 * 256
    for bad_ptr, bad_bytes in ((base, need - 8), (base + 16, need)):
        with pytest.raises(B.GroError) as e:
            B.gro_plan_bind(h, bad_ptr, bad_bytes, s)
        assert e.value.kind == "invalid"
    B.gro_accumulate(h, 0, nb, ptrs, c.st.acc.data_ptr(), 0, 2, s)     # a window left unfinished
    B.gro_plan_bind(h, base, need, s)
    c.st.workspace_keepalive = ws2
    with pytest.raises(B.GroError) as e:                                # its bookkeeping is gone
        B.gro_reduce_norm(h, c.st.acc.data_ptr(), 2, s)
    assert e.value.kind == "state"
    with pytest.raises(B.GroError) as e:                                # and no norm is readable
        B.gro_plan_get_norm(h)
    assert e.value.kind == "state"
    # full windows on the new workspace match the oracle
    cmps = {k: Compare(k) for k in ("acc", "master", "m", "v", "p_bf16")}
    for step, n in enumerate([2, 3], start=1):
        grads_host = []
        for k in range(n):
            g = c.draw(step, k)
            c.gpu_accumulate(g, k, n)
            grads_host.append([None if x is None else [synth.host_values(t) for t in x] for x in g])
        norm, _, finite = c.gpu_finish(n, step, w.max_norm)
        res = c.oracle_window(grads_host, step, w.max_norm)
        c.compare_acc(res, cmps["acc"])
        c.compare_states(res, cmps)
        assert finite and abs(norm - res.norm) <= FP32_RTOL * res.norm
    for k in cmps.values():
        assert k.ok and k.n_diff_bits == 0, str(k)


def test_two_hundred_steps_stay_bit_identical():
    """A long run: 200 optimizer steps (windows of 1 to 4 microbatches, one
    call per microbatch) on the literal tiny set; the states still match
    the oracle bit for bit at every step, so nothing drifts as m and v grow
    and the bias corrections approach 1."""
    w = synth.tiny(literal=True)
    rng = np.random.default_rng(5)
    windows = [int(x) for x in rng.integers(1, 5, size=200)]
    log(f"case 200 steps, {sum(windows)} microbatches")
    _, cmps, norms = run_parity(w, windows, log=lambda m: None)
    assert_parity(cmps, norms)
    for k in cmps.values():
        assert k.n_diff_bits == 0, str(k)
