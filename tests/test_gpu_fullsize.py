"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark uses (whole-plan accumulate calls with the fused norm partials).

Every element is compared with the CPU oracle on the same seeded inputs:
67M draft model (whole set and the TP2 half share, window 4), the 1B-class
FSDP flat shard (windows 8 then a trailing 3), the 4000-tensor hybrid/MoE
set (window 2), and a two-bucket sub-plan of the 8B share (2 x 64M elements,
window 8, weight decay 0.1).  The whole 8B share (1e9 elements) does not fit
the oracle's host arrays; it is run in full and checked on sampled elements
against the oracle and on every element against closed forms and plain torch
FP32 ops.
"""
import math
import sys
import time

import numpy as np
import pytest
import torch

import oracle.method as M
from gradient_reduction_optimizer_amd import binding as B
from gradient_reduction_optimizer_amd import synth
from gradient_reduction_optimizer_amd.buffers import DeviceState, Plan
from gpu_harness import BF16_RTOL, FP32_RTOL, Compare, assert_parity, bits16, host, run_parity

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _need_gpu(gpu):
    torch.cuda.synchronize()
    yield
    torch.cuda.empty_cache()


CASES = {
    "draft-67m": lambda: synth.draft_67m(),
    "draft-67m-tp2-half": lambda: synth.draft_67m(half_share=True),
    "dense-1b-fsdp8-shard": lambda: synth.dense_1b_shard(),
    "hybrid-moe-4000": lambda: synth.hybrid_moe(),
    "dense-8b-share-2-buckets": lambda: synth.dense_8b_share(numel=128_000_000),
}


@pytest.mark.parametrize("name", list(CASES))
def test_full_size_parity(name):
    w = CASES[name]()
    t0 = time.time()
    log(f"case {name}: {w.numel} elements, windows {w.windows}, R={w.R}")
    c, cmps, norms = run_parity(w, w.windows, log=log)
    log(f"case {name} done in {time.time() - t0:.1f} s, {c.plan.info['n_buckets']} buckets, "
        f"{c.plan.info['n_chunks']} chunks")
    assert_parity(cmps, norms)


@pytest.mark.parametrize("name", ["draft-67m", "dense-1b-fsdp8-shard", "hybrid-moe-4000"])
def test_full_size_parity_window_call(name):
    """The one-call-per-window entry point at full size."""
    w = CASES[name]()
    t0 = time.time()
    log(f"case {name} (window call): {w.numel} elements, windows {w.windows}")
    c, cmps, norms = run_parity(w, w.windows, window_call=True, log=log)
    log(f"case {name} (window call) done in {time.time() - t0:.1f} s")
    assert_parity(cmps, norms)


@pytest.mark.parametrize("name,groups", [("draft-67m", [[2, 2]]), ("dense-1b-fsdp8-shard", [[4, 4], [2, 1]])])
def test_full_size_parity_microbatch_groups(name, groups):
    """gro_accumulate_microbatches in groups at full size."""
    w = CASES[name]()
    t0 = time.time()
    log(f"case {name} (groups {groups}): {w.numel} elements, windows {w.windows}")
    c, cmps, norms = run_parity(w, w.windows, groups=groups, log=log)
    log(f"case {name} (groups) done in {time.time() - t0:.1f} s")
    assert_parity(cmps, norms)


# ------------------------------------------------ the whole 1e9-element share
def _sample_positions(plan, n_random=20000, seed=11):
    """Positions in the single flat tensor to compare with the oracle:
    random ones plus the first and last three elements of every bucket.
    Returns (positions in tensor order, [(bucket, device index of the
    bucket offsets, indices into positions)])."""
    N = plan.tensors[0]["numel"]
    rng = np.random.default_rng(seed)
    pos = set(int(p) for p in rng.integers(0, N, n_random))
    segs = plan.segments(0)
    for _, _, toff, cnt in segs:
        pos.update(toff + d for d in (0, 1, 2, cnt - 3, cnt - 2, cnt - 1))
    pos = np.array(sorted(p for p in pos if 0 <= p < N), dtype=np.int64)
    per = []
    for b, boff, toff, cnt in segs:
        sel = np.nonzero((pos >= toff) & (pos < toff + cnt))[0]
        per.append((b, torch.from_numpy(pos[sel] - toff + boff).cuda(), sel))
    return pos, per


def _gather_bucketed(plan, flat, per):
    """Host copy of a flat (acc/master/m/v/p_bf16) array at the sample positions."""
    parts = []
    for b, idx, _ in per:
        base = plan.buckets[b]["flat_base"]
        parts.append(flat[base:base + plan.buckets[b]["len"]].index_select(0, idx))
    t = torch.cat(parts)
    return bits16(t) if t.dtype == torch.bfloat16 else host(t)


@pytest.mark.parametrize("mode", ["window", "microbatch"])
def test_dense_8b_full_share_sampled(mode):
    """The 8B config's whole 1e9-element share (16 buckets of 64M, windows 8
    then a trailing 3, weight decay 0.1) in the launch configuration the
    benchmark uses.  Every accumulator element is compared bit for bit with
    plain torch FP32 ops on the same inputs; ~20,000 sampled elements of
    acc, master, m, v and the BF16 copy are compared with the oracle, which
    takes the clip coefficient from a norm computed by torch (FP64) from
    those inputs -- the oracle cannot hold the full share in host memory;
    the GPU norm is compared with that torch norm (within the FP32
    tolerance: torch divides by a non-power-of-two window as a multiply by
    the reciprocal); after the first window every m and v element is
    checked against its closed form (m = (1-b1)g^, v = (1-b2)g^2), and every
    BF16 copy against torch's cast of the master."""
    _flat_share_sampled(synth.dense_8b_share(), [8, 3], mode)


def test_flat_share_beyond_32_bit_offsets():
    """One bucket of 2^31 + 2^20 + 3 elements (a ragged last chunk): element
    offsets inside the bucket and in the flat arrays pass 2^31, so every
    index computation must be 64-bit.  Same checks as the 8B share, windows
    2 then 1; the sample includes both ends of the bucket."""
    numel = 2 ** 31 + 2 ** 20 + 3
    _flat_share_sampled(synth.dense_8b_share(numel=numel, bucket_elems=numel), [2, 1], "window")


def _flat_share_sampled(w, windows, mode):
    log(f"case {w.name} full ({mode}): {w.numel} elements, windows {windows}")
    plan = Plan(w.tensors, w.R, w.bucket_elems)
    st = DeviceState(plan, "cuda")
    s = torch.cuda.current_stream().cuda_stream
    owner = M.assign_owners(w.tensors, w.R)[0]
    assert owner.owner == M.MEAN and owner.slots == 2 and owner.decayed
    nb = plan.info["n_buckets"]
    pos, per = _sample_positions(plan)
    for b, bk in enumerate(plan.buckets):
        st.master[bk["flat_base"]:bk["flat_base"] + bk["len"]].copy_(synth.bucket_master(w, b, bk["len"], "cuda"))
    p_h = _gather_bucketed(plan, st.master, per)
    m_h = np.zeros_like(p_h)
    v_h = np.zeros_like(p_h)
    acc_ref = torch.zeros_like(st.acc)
    cmps = {k: Compare(k) for k in ("acc", "master", "m", "v", "p_bf16")}

    def fill(bufs, step, k):
        """Draw microbatch k into bufs; update acc_ref; return the sampled
        contributions [slot0 bits, slot1 bits]."""
        samp = [[], []]
        for (b, idx, _), bk in zip(per, plan.buckets):
            L = bk["len"]
            g = synth.bucket_grads_bf16(w, step, k, b, bk["slots"], L, "cuda")
            bufs[b][:, :L].copy_(g)
            red = (g[0].float() + g[1].float()) / 2.0
            dst = acc_ref[bk["flat_base"]:bk["flat_base"] + L]
            if k == 0:
                dst.copy_(red)
            else:
                dst.add_(red)
            for r in range(2):
                samp[r].append(bits16(bufs[b][r].index_select(0, idx)))
        return [np.concatenate(x) for x in samp]

    for step, n in enumerate(windows, start=1):
        t0 = time.time()
        acc_h = None
        if mode == "window":
            sets = [st.grad_buffers() for _ in range(n)]
            for k in range(n):
                sl = fill(sets[k], step, k)
                acc_h = M.accumulate(acc_h, M.reduce_contributions(owner, w.R, sl), k)
            ptrs = [sets[k][b].data_ptr() for k in range(n) for b in range(nb)]
            B.gro_accumulate_window(plan.handle, 0, nb, ptrs, n, st.acc.data_ptr(), s)
        else:
            bufs = st.grad_buffers()
            for k in range(n):
                sl = fill(bufs, step, k)
                acc_h = M.accumulate(acc_h, M.reduce_contributions(owner, w.R, sl), k)
                B.gro_accumulate(plan.handle, 0, nb, [x.data_ptr() for x in bufs], st.acc.data_ptr(), k, n, s)
        B.gro_reduce_norm(plan.handle, st.acc.data_ptr(), n, s)
        norm, _, finite = B.gro_plan_get_norm(plan.handle)
        assert finite
        assert torch.equal(st.acc.view(torch.int32), acc_ref.view(torch.int32)), "accumulator"
        g_ref = acc_ref / float(n)
        norm_ref = math.sqrt(math.fsum(g_ref[i:i + (1 << 26)].double().square().sum().item()
                                       for i in range(0, g_ref.numel(), 1 << 26)))
        del g_ref
        assert abs(norm - norm_ref) <= FP32_RTOL * norm_ref, (norm, norm_ref)
        hp = w.hparams
        B.gro_clip_adamw(plan.handle, st.acc.data_ptr(), n, w.max_norm, hp, step, st.master.data_ptr(),
                         st.m.data_ptr(), st.v.data_ptr(), st.p_bf16.data_ptr(), s)
        # the oracle on the sampled elements
        coef, stepped = M.clip_coefficient(norm_ref, w.max_norm)
        assert stepped and coef < 1.0
        sc = M.adamw_scalars(hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"], step)
        g_h = M.window_gradient(acc_h, n)
        p_h, m_h, v_h, pb_h = M.adamw_update(g_h, coef, p_h, m_h, v_h, sc, owner.decayed)
        cmps["acc"].add(_gather_bucketed(plan, st.acc, per), acc_h, FP32_RTOL)
        cmps["master"].add(_gather_bucketed(plan, st.master, per), p_h, FP32_RTOL)
        cmps["m"].add(_gather_bucketed(plan, st.m, per), m_h, FP32_RTOL)
        cmps["v"].add(_gather_bucketed(plan, st.v, per), v_h, FP32_RTOL)
        cmps["p_bf16"].add(_gather_bucketed(plan, st.p_bf16, per), pb_h, BF16_RTOL)
        # properties over every element
        assert torch.equal(st.p_bf16.view(torch.int16), st.master.to(torch.bfloat16).view(torch.int16))
        if step == 1:
            coef_gpu = float(np.float32(min(1.0, w.max_norm / (norm + 1e-6))))
            gh = (st.acc / float(n)) * coef_gpu          # n = 8: the division is exact
            m_cf = torch.zeros_like(gh).mul_(float(sc.beta1)).add_(gh * float(sc.one_minus_beta1))
            assert torch.equal(st.m.view(torch.int32), m_cf.view(torch.int32)), "m after the first window"
            del m_cf
            v_cf = torch.zeros_like(gh).mul_(float(sc.beta2)).add_((gh * gh) * float(sc.one_minus_beta2))
            assert torch.equal(st.v.view(torch.int32), v_cf.view(torch.int32)), "v after the first window"
            del v_cf, gh
        if mode == "window":
            del sets
        else:
            del bufs
        torch.cuda.empty_cache()
        log(f"step {step} (window {n}) checked in {time.time() - t0:.1f} s: norm gpu={norm!r} torch={norm_ref!r}")
    for k in cmps.values():
        log(str(k))
    for k in cmps.values():
        assert k.ok, str(k)
    assert cmps["acc"].n_diff_bits == 0
    assert len(pos) == cmps["acc"].n // 2
