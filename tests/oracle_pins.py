"""Pins for the CPU oracle: each ties an oracle function to something other
than itself (closed forms, brute-force gradients of tiny sharded layers,
library routines, exact rational arithmetic, a hand-written table).

Each pin takes the oracle's ``method`` module and raises AssertionError on a
mismatch, so the same pins also run against deliberately broken copies of
the oracle (tests/test_oracle_mutants.py) to show they catch mistakes.

Page keys: P1 = NeMo Automodel issue #3857, "refactor(distributed):
establish shared native TP replica ownership".
"""
from __future__ import annotations

import math
import os
from fractions import Fraction
from types import SimpleNamespace

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
F32 = np.float32


def spec(pid, shape, placement, shard_index=None, frozen=False, no_decay=False):
    if shard_index is None:
        shard_index = 0 if placement == "shard" else -1
    return SimpleNamespace(param_id=pid, shape=tuple(shape), placement=placement,
                           shard_index=shard_index, frozen=frozen, no_decay=no_decay)


def bf16_bits_of(x) -> np.ndarray:
    """BF16 bits of float64/float32 values via torch's own cast (library)."""
    t = torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_value(bits) -> np.ndarray:
    """Value of BF16 bits via torch (library), as float64."""
    t = torch.from_numpy(np.asarray(bits, dtype=np.uint16).view(np.int16).copy()).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def rms(x) -> float:
    x = np.asarray(x, dtype=np.float64)
    return float(np.sqrt(np.mean(x * x))) if x.size else 0.0


def rel_close(a, b, rtol, floor=0.0):
    """|a - b| <= rtol * max(|b|, floor), elementwise.  ``floor`` is an
    absolute magnitude (the tensor's scale) so that results that cancel to
    near zero are judged against the size of the terms that produced them."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    tol = rtol * np.maximum(np.abs(b), floor)
    return bool(np.all(np.abs(a - b) <= tol))


# ----------------------------------------------------------- ownership
def read_golden_ownership():
    rows = []
    with open(os.path.join(GOLDEN, "tiny_ownership.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            pid, name, placement, owner, slots, div, innorm, upd, dec = line.split()
            rows.append(dict(param_id=int(pid), name=name, placement=placement, owner=owner,
                             slots=int(slots), divisor=int(div), in_norm=bool(int(innorm)),
                             updated=bool(int(upd)), decayed=bool(int(dec))))
    return rows


def pin_ownership_table(M):
    """The oracle's owners for the tiny tensor list equal the hand table."""
    gold = read_golden_ownership()
    specs = [spec(g["param_id"], (4,), g["placement"]) for g in gold]
    got = M.assign_owners(specs, 2)
    assert len(got) == len(gold)
    for o, g in zip(got, gold):
        assert (o.param_id, o.owner, o.slots, o.divisor, o.in_norm, o.updated, o.decayed) == \
            (g["param_id"], g["owner"], g["slots"], g["divisor"], g["in_norm"], g["updated"], g["decayed"]), (o, g)


def pin_ownership_rejections(M):
    """One owner per parameter; bad compositions fail before any data."""
    def kind(specs, R=2):
        try:
            M.assign_owners(specs, R)
        except M.Rejected as e:
            return e.kind
        return None
    assert kind([spec(1, (3,), "shard"), spec(1, (3,), "replicate")]) == "duplicate"
    assert kind([spec(1, (3,), "replicate")], R=0) == "invalid"
    assert kind([spec(1, (3,), "shard", shard_index=2)]) == "placement"
    assert kind([spec(1, (3,), "shard", shard_index=-1)]) == "placement"
    assert kind([spec(1, (3,), "partial", shard_index=0)]) == "placement"
    assert kind([spec(1, (3,), "sharded")]) == "placement"
    assert kind([spec(1, (3, -1), "replicate")]) == "invalid"
    assert kind([spec(1, (0,), "replicate"), spec(2, (5,), "shard", shard_index=1)]) is None
    fro = M.assign_owners([spec(7, (3,), "replicate", frozen=True),
                           spec(8, (3,), "partial", no_decay=True)], 2)
    assert (fro[0].owner, fro[0].slots, fro[0].in_norm, fro[0].updated, fro[0].decayed) == \
        ("excluded", 0, False, False, False)
    assert (fro[1].owner, fro[1].updated, fro[1].decayed) == ("sum", True, False)


# ---------------------------------------------- O2: replicate -> mean
def pin_identical_replicas_average_to_replica(M):
    """R identical complete gradients average to exactly that gradient
    (while R*|x| stays below the FP32 overflow threshold)."""
    rng = np.random.default_rng(11)
    x = bf16_bits_of(rng.standard_normal(4096) * 1e-2)
    specials = np.array([0x0000, 0x8000, 0x0001, 0x807F, 0x7A7F, 0xFA7F, 0x3F80, 0x0080],
                        dtype=np.uint16)
    x = np.concatenate([x, specials])
    for R in (1, 2, 3, 4, 5, 7, 8, 16):
        o = M.assign_owners([spec(0, x.shape, "replicate")], R)[0]
        red = M.reduce_contributions(o, R, [x.copy() for _ in range(R)])
        want = bf16_value(x).astype(np.float32)
        assert np.array_equal(red.view(np.uint32), want.view(np.uint32)), f"R={R}"


# ---------------------------------------------- O2: partial -> sum
def _fd_grad(loss, w, delta=1e-3):
    """Central finite differences in FP64 (exact up to rounding for a loss
    linear in w)."""
    g = np.zeros_like(w)
    for j in range(w.size):
        e = np.zeros_like(w)
        e.flat[j] = delta
        g.flat[j] = (loss(w + e) - loss(w - e)) / (2 * delta)
    return g


def _head_sharded_qk_norm_case(seed=5):
    """Q/K RMSNorm with one weight w[64] shared by 8 heads; heads split 4/4
    over two TP ranks.  Loss <C, y>.  Returns (full_grad, [partial_r])."""
    rng = np.random.default_rng(seed)
    T, H, D = 3, 8, 64
    x = rng.standard_normal((T, H, D))
    C = rng.standard_normal((T, H, D))
    w0 = 1.0 + 0.1 * rng.standard_normal(D)

    def loss(w, heads=slice(None)):
        xs = x[:, heads]
        rms = np.sqrt(np.mean(xs * xs, axis=-1, keepdims=True) + 1e-6)
        return float(np.sum(C[:, heads] * (w * xs / rms)))

    full = _fd_grad(loss, w0)
    parts = [_fd_grad(lambda w, r=r: loss(w, slice(4 * r, 4 * r + 4)), w0) for r in range(2)]
    return full, parts


def _sequence_sharded_linear_case(seed=6):
    """y = x W^T with W replicated; 10 tokens split 5/5 over two ranks.
    Loss <C, y>.  Returns (full_grad, [partial_r])."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((10, 6))
    C = rng.standard_normal((10, 4))
    W0 = rng.standard_normal((4, 6)) * 0.3

    def loss(W, rows=slice(None)):
        return float(np.sum(C[rows] * (x[rows] @ W.T)))

    full = _fd_grad(loss, W0)
    parts = [_fd_grad(lambda W, r=r: loss(W, slice(5 * r, 5 * r + 5)), W0) for r in range(2)]
    return full.ravel(), [p.ravel() for p in parts]


def pin_partial_contributions_sum_to_full_gradient(M):
    """Summing BF16-rounded partial gradients of head- and sequence-sharded
    layers gives the unsharded layer's gradient (P1 "Why this needs
    separate work"); averaging them instead is off by a factor of R, the
    lost-sum failure P1 describes for a backend that does not resolve the
    Partial placement."""
    for full, parts in (_head_sharded_qk_norm_case(), _sequence_sharded_linear_case()):
        bits = [bf16_bits_of(p) for p in parts]
        o = M.assign_owners([spec(0, full.shape, "partial")], 2)[0]
        red = M.reduce_contributions(o, 2, bits).astype(np.float64)
        bound = sum(np.abs(p) for p in parts) * 2.0 ** -8 + 1e-9
        assert np.all(np.abs(red - full) <= bound), np.max(np.abs(red - full) / bound)
        # the averaging reading must fail this check
        mean_reading = (bf16_value(bits[0]) + bf16_value(bits[1])) / 2
        assert not np.all(np.abs(mean_reading - full) <= bound)


def pin_rank_order(M):
    """Contributions are added in rank order 0, 1, ..., R-1 (FP32 addition is
    not associative): 1 + 2^-24 rounds to 1 (a tie, to even) and again with
    the second 2^-24, while 2^-24 + 2^-24 + 1 is exactly 1 + 2^-23."""
    rows = M.assign_owners([spec(0, (1,), "partial")], 3)
    bits = lambda v: M.f32_to_bf16(np.array([v], dtype=np.float32))
    s = M.reduce_contributions(rows[0], 3, [bits(1.0), bits(2.0 ** -24), bits(2.0 ** -24)])
    assert s[0] == np.float32(1.0)
    s = M.reduce_contributions(rows[0], 3, [bits(2.0 ** -24), bits(2.0 ** -24), bits(1.0)])
    assert s[0] == np.float32(1.0 + 2.0 ** -23)


def pin_redundant_compute_is_averaged(M):
    """Every TP rank computing the full gradient redundantly: Replicate
    recovers it exactly, a Partial-style sum would double it."""
    full, _ = _sequence_sharded_linear_case(seed=9)
    bits = bf16_bits_of(full)
    o = M.assign_owners([spec(0, full.shape, "replicate")], 2)[0]
    red = M.reduce_contributions(o, 2, [bits, bits.copy()])
    assert np.array_equal(red.astype(np.float64), bf16_value(bits))


# ---------------------------------------------- O2: local owners
def pin_local_owners_left_alone(M):
    """Shard and pre-reduced gradients are used as they are: with one
    microbatch the accumulator is the widened gradient, bit for bit, and
    the inputs are not written."""
    rng = np.random.default_rng(12)
    x = bf16_bits_of(rng.standard_normal(3001) * 3e-3)
    keep = x.copy()
    for placement in ("shard", "reduced"):
        o = M.assign_owners([spec(0, x.shape, placement)], 2)[0]
        assert o.slots == 1
        acc = M.accumulate(None, M.reduce_contributions(o, 2, [x]), 0)
        g = M.window_gradient(acc, 1)
        want = bf16_value(keep).astype(np.float32)
        assert np.array_equal(g.view(np.uint32), want.view(np.uint32))
        assert np.array_equal(x, keep)


# ---------------------------------------------- O2/O3: windows
def pin_windows(M):
    """A window of n identical microbatches has the single microbatch's
    gradient (exact: n*x needs at most 8+3 bits); a window of distinct
    microbatches is their mean within FP32 rounding of exact rational
    arithmetic, for n = 1, 3 (trailing) and 8."""
    rng = np.random.default_rng(13)
    specs = [spec(0, (257,), "replicate"), spec(1, (129,), "partial"), spec(2, (300,), "shard")]
    owners = M.assign_owners(specs, 2)
    base = [[bf16_bits_of(rng.standard_normal(s.shape) * 1e-2) for _ in range(o.slots)]
            for s, o in zip(specs, owners)]
    single = [M.window_gradient(M.accumulate(None, M.reduce_contributions(o, 2, b), 0), 1)
              for o, b in zip(owners, base)]
    for n in (3, 8):
        for i, o in enumerate(owners):
            acc = None
            for k in range(n):
                acc = M.accumulate(acc, M.reduce_contributions(o, 2, base[i]), k)
            g = M.window_gradient(acc, n)
            assert np.array_equal(g.view(np.uint32), single[i].view(np.uint32)), (n, i)
    # distinct microbatches against exact rationals
    for n in (1, 3, 8):
        o = owners[0]
        draws = [[bf16_bits_of(rng.standard_normal(64) * 1e-2) for _ in range(2)] for _ in range(n)]
        acc = None
        for k in range(n):
            acc = M.accumulate(acc, M.reduce_contributions(o, 2, draws[k]), k)
        g = M.window_gradient(acc, n)
        for j in range(64):
            exact = sum((Fraction(float(bf16_value(draws[k][0][j:j + 1])[0])) +
                         Fraction(float(bf16_value(draws[k][1][j:j + 1])[0]))) / 2 for k in range(n)) / n
            mag = sum(abs(float(bf16_value(draws[k][r][j:j + 1])[0])) for k in range(n) for r in range(2))
            err = abs(Fraction(float(g[j])) - exact)
            assert err <= Fraction(2 * (n + 2)) * Fraction(2.0 ** -24) * Fraction(mag) + Fraction(1, 10 ** 40), (n, j)


# ---------------------------------------------- O4: norm
def pin_norm(M):
    """Closed form, exact rational sum, and torch's FP64 vector norm."""
    a = np.full(1024, 0.75, dtype=np.float32)
    norm, sq = M.global_norm([a])
    assert norm == 24.0 and sq == 576.0
    b = np.full(1000, -3.0, dtype=np.float32)
    norm, sq = M.global_norm([b, np.zeros(24, dtype=np.float32)])
    assert sq == 9000.0 and abs(norm - 3.0 * math.sqrt(1000)) <= 1e-15 * norm
    rng = np.random.default_rng(14)
    parts = [(rng.standard_normal(n) * 10.0 ** rng.uniform(-6, 2)).astype(np.float32)
             for n in (1, 17, 300, 4096)]
    norm, sq = M.global_norm(parts)
    exact = sum(Fraction(float(x)) ** 2 for p in parts for x in p)
    assert sq == float(exact)
    ref = torch.linalg.vector_norm(torch.from_numpy(np.concatenate(parts).astype(np.float64))).item()
    assert abs(norm - ref) <= 1e-12 * ref
    bad = parts[1].copy()
    bad[3] = np.inf
    assert not math.isfinite(M.global_norm([parts[0], bad])[0])
    bad[3] = np.nan
    assert math.isnan(M.global_norm([bad])[0])


# ---------------------------------------------- O5: clipping
def pin_clip(M):
    rng = np.random.default_rng(15)
    g = (rng.standard_normal(5000) * 0.05).astype(np.float32)   # norm ~ 3.5
    norm, _ = M.global_norm([g])
    for max_norm in (1.0, 0.25, 2.0):
        coef, stepped = M.clip_coefficient(norm, max_norm)
        assert stepped and coef < 1
        clipped = g * coef
        cn, _ = M.global_norm([clipped])
        assert cn <= max_norm * (1 + 2.0 ** -22), (cn, max_norm)
        # torch.nn.utils.clip_grad_norm_ (FP32 tensors) as a library case
        p = torch.nn.Parameter(torch.zeros(g.size, dtype=torch.float32))
        p.grad = torch.from_numpy(g.copy())
        tn = torch.nn.utils.clip_grad_norm_([p], max_norm).item()
        assert abs(tn - norm) <= 1e-6 * norm
        assert rel_close(clipped, p.grad.numpy(), 1e-6, floor=rms(clipped))
    # a tiny norm, where clip_grad_norm_'s 1e-6 in the denominator is
    # visible in FP32 (norm ~ 1e-3: a relative 1e-3 change of the coefficient)
    small = (g * np.float32(3e-4)).astype(np.float32)
    sn, _ = M.global_norm([small])
    coef, stepped = M.clip_coefficient(sn, 1e-4)
    p = torch.nn.Parameter(torch.zeros(small.size, dtype=torch.float32))
    p.grad = torch.from_numpy(small.copy())
    torch.nn.utils.clip_grad_norm_([p], 1e-4)
    assert rel_close(small * coef, p.grad.numpy(), 1e-6, floor=rms(small * coef))
    # below the threshold, and clipping off, leave g untouched
    coef, stepped = M.clip_coefficient(norm, norm + 1.0)
    assert coef == 1.0 and stepped
    for off in (0.0, -1.0, float("inf")):
        coef, stepped = M.clip_coefficient(norm, off)
        assert coef == 1.0 and stepped
    coef, stepped = M.clip_coefficient(float("nan"), 1.0)
    assert not stepped
    coef, stepped = M.clip_coefficient(float("inf"), 1.0)
    assert not stepped


# ---------------------------------------------- O6: AdamW
def pin_adamw_first_step(M):
    """t=1, m=v=0: p1 = p0*(1-lr*wd) - lr*g^/(|g^|+eps); g = 0 leaves p*decay."""
    rng = np.random.default_rng(16)
    g = (rng.standard_normal(4096) * 1e-2).astype(np.float32)
    g[:5] = [0.0, 1e-30, -1e-12, 3.0, -0.5]
    p0 = (rng.standard_normal(4096) * 0.02).astype(np.float32)
    z = np.zeros_like(p0)
    lr, wd, eps = 1e-3, 0.01, 1e-8
    for coef in (1.0, 0.3):
        sc = M.adamw_scalars(lr, 0.9, 0.999, eps, wd, 1)
        p1, m1, v1, _ = M.adamw_update(g, F32(coef), p0, z, z, sc, True)
        gh = g.astype(np.float64) * np.float64(F32(coef))
        want = p0.astype(np.float64) * (1 - lr * wd) - lr * gh / (np.abs(gh) + eps)
        assert rel_close(p1, want, 1e-6, floor=rms(want))
        assert rel_close(m1, 0.1 * gh, 1e-6, floor=1e-30)
        assert rel_close(v1, 0.001 * gh * gh, 1e-6, floor=1e-30)
    sc = M.adamw_scalars(lr, 0.9, 0.999, eps, wd, 1)
    p1, m1, v1, _ = M.adamw_update(np.zeros_like(p0), F32(1), p0, z, z, sc, True)
    assert np.array_equal(p1, p0 * sc.decay)
    p1, _, _, _ = M.adamw_update(np.zeros_like(p0), F32(1), p0, z, z, sc, False)
    assert np.array_equal(p1, p0)


def pin_adamw_matches_torch(M):
    """R=1, one microbatch, pre-reduced, clipping off: the oracle's window
    steps equal torch.optim.AdamW (FP32, CPU, single-tensor loop) over 6
    steps, for a decayed and a no-decay tensor."""
    rng = np.random.default_rng(17)
    specs = [spec(0, (777,), "reduced"), spec(1, (300,), "reduced", no_decay=True)]
    owners = M.assign_owners(specs, 1)
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    master = {i: (rng.standard_normal(s.shape) * 0.02).astype(np.float32) for i, s in enumerate(specs)}
    m = {i: np.zeros(s.shape, np.float32) for i, s in enumerate(specs)}
    v = {i: np.zeros(s.shape, np.float32) for i, s in enumerate(specs)}
    params = [torch.nn.Parameter(torch.from_numpy(master[i].copy())) for i in range(2)]
    opt = torch.optim.AdamW([{"params": [params[0]], "weight_decay": 0.01},
                             {"params": [params[1]], "weight_decay": 0.0}],
                            lr=1e-3, betas=(0.9, 0.999), eps=1e-8, foreach=False)
    for step in range(1, 7):
        grads = [[bf16_bits_of(rng.standard_normal(s.shape) * 1e-2)] for s in specs]
        res = M.optimizer_window(owners, 1, [grads], master, m, v, hp, 0.0, step)
        master, m, v = res.master, res.m, res.v
        for i in range(2):
            params[i].grad = torch.from_numpy(bf16_value(grads[i][0]).astype(np.float32))
        opt.step()
        for i in range(2):
            st = opt.state[params[i]]
            ref_p, ref_m, ref_v = (params[i].detach().numpy(), st["exp_avg"].numpy(),
                                   st["exp_avg_sq"].numpy())
            assert rel_close(master[i], ref_p, 1e-6, floor=rms(ref_p)), (step, i)
            assert rel_close(m[i], ref_m, 1e-6, floor=rms(ref_m)), (step, i)
            assert rel_close(v[i], ref_v, 1e-6, floor=rms(ref_v)), (step, i)


def pin_clip_then_adamw_matches_torch(M):
    """Clipping on, window of 2, Replicate at R=2 with identical replicas:
    equals torch clip_grad_norm_ then AdamW on the mean gradient."""
    rng = np.random.default_rng(18)
    specs = [spec(0, (2000,), "replicate"), spec(1, (64,), "shard")]
    owners = M.assign_owners(specs, 2)
    hp = dict(lr=2e-3, beta1=0.8, beta2=0.99, eps=1e-6, weight_decay=0.1)
    master = {i: (rng.standard_normal(s.shape) * 0.02).astype(np.float32) for i, s in enumerate(specs)}
    zeros = {i: np.zeros(s.shape, np.float32) for i, s in enumerate(specs)}
    micro = []
    for k in range(2):
        row = []
        for s, o in zip(specs, owners):
            b = bf16_bits_of(rng.standard_normal(s.shape) * 0.05)
            row.append([b] * o.slots)
        micro.append(row)
    res = M.optimizer_window(owners, 2, micro, master, zeros, zeros, hp, 0.5, 1)
    params = [torch.nn.Parameter(torch.from_numpy(master[i].copy())) for i in range(2)]
    for i in range(2):
        params[i].grad = torch.from_numpy(
            ((bf16_value(micro[0][i][0]) + bf16_value(micro[1][i][0])) / 2).astype(np.float32))
    total = torch.nn.utils.clip_grad_norm_(params, 0.5).item()
    assert abs(total - res.norm) <= 1e-6 * res.norm
    opt = torch.optim.AdamW(params, lr=2e-3, betas=(0.8, 0.99), eps=1e-6, weight_decay=0.1, foreach=False)
    opt.step()
    for i in range(2):
        ref = params[i].detach().numpy()
        assert rel_close(res.master[i], ref, 1e-6, floor=rms(ref))


# ---------------------------------------------- BF16 conversions
def pin_bf16(M):
    """Widening and RNE narrowing agree with torch's bfloat16 casts on every
    BF16 pattern, every rounding edge class and 1M random FP32 patterns."""
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    w = M.bf16_to_f32(allbits)
    ref = bf16_value(allbits).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(w), nan)
    assert np.array_equal(w[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    hi = np.arange(65536, dtype=np.uint32) << np.uint32(16)
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xC000, 0xFFFF], dtype=np.uint32)
    edge = (hi[:, None] | lows[None, :]).ravel()
    rand = np.random.default_rng(19).integers(0, 2 ** 32, size=1_000_000, dtype=np.uint64).astype(np.uint32)
    for pats in (edge, rand):
        x = pats.view(np.float32)
        got = M.f32_to_bf16(x)
        want = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        xn = np.isnan(x)
        gn = np.isnan(M.bf16_to_f32(got))
        assert np.array_equal(gn, xn)
        assert np.array_equal(got[~xn], want[~xn])


# ---------------------------------------------- FP32 contributions
def pin_fp32_contributions(M):
    """FP32 contributions (P1 acceptance matrix: BF16/FP32): partial sums of
    the head- and sequence-sharded layers match the unsharded gradient within
    FP32 rounding; two identical FP32 replicas average to the replica exactly;
    a local FP32 gradient passes through bit for bit."""
    for full, parts in (_head_sharded_qk_norm_case(), _sequence_sharded_linear_case()):
        f32 = [p.astype(np.float32) for p in parts]
        o = M.assign_owners([spec(0, full.shape, "partial")], 2)[0]
        red = M.reduce_contributions(o, 2, f32).astype(np.float64)
        bound = sum(np.abs(p) for p in parts) * 2.0 ** -22 + 1e-12
        assert np.all(np.abs(red - full) <= bound), np.max(np.abs(red - full) / bound)
    rng = np.random.default_rng(21)
    x = (rng.standard_normal(5000) * 1e-2).astype(np.float32)
    x[:4] = [0.0, -0.0, 1e-40, -1.5e38]  # |x| below half the FP32 maximum: x + x is exact
    o = M.assign_owners([spec(0, x.shape, "replicate")], 2)[0]
    red = M.reduce_contributions(o, 2, [x, x.copy()])
    assert np.array_equal(red.view(np.uint32), x.view(np.uint32))
    for placement in ("shard", "reduced"):
        o = M.assign_owners([spec(0, x.shape, placement)], 2)[0]
        red = M.reduce_contributions(o, 2, [x])
        assert np.array_equal(red.view(np.uint32), x.view(np.uint32))
    # FP32 values are not rounded to BF16 on the way in
    y = np.array([1.0 + 2.0 ** -20], dtype=np.float32)
    o = M.assign_owners([spec(0, y.shape, "shard")], 2)[0]
    assert M.reduce_contributions(o, 2, [y])[0] == y[0]


# ---------------------------------------------- N3 initialisation
def pin_philox_matches_numpy(M):
    """Philox4x64-10 equals numpy's Philox bit generator (which advances the
    256-bit counter by one before each block)."""
    rng = np.random.default_rng(22)
    for _ in range(20):
        c = [int(x) for x in rng.integers(1, 2 ** 63, size=4)]
        k = [int(x) for x in rng.integers(0, 2 ** 63, size=2)]
        bg = np.random.Philox(key=np.array(k, dtype=np.uint64),
                              counter=np.array([c[0] - 1] + c[1:], dtype=np.uint64))
        assert [int(x) for x in bg.random_raw(4)] == M.philox4x64_10(c, k)


def pin_init_uniform(M):
    """Values lie in [offset - bound, offset + bound), on the 2^-24 grid of
    the unit interval; bound 0 gives exactly the offset; moments of 20,000
    draws match U(-b, b); different param_ids give different streams."""
    idx = np.arange(20000)
    x = M.init_uniform(7, 11, 0, idx, 0.5, 0.0).astype(np.float64)
    assert np.all(x >= -0.5) and np.all(x < 0.5)
    u = (x / 0.5 + 1) / 2
    assert np.all(u * 2 ** 24 == np.round(u * 2 ** 24))
    assert abs(x.mean()) < 4 * 0.5 / np.sqrt(3 * 20000)
    assert abs(x.var() - 0.25 / 3) < 0.01
    ones = M.init_uniform(7, 3, 5, np.arange(100), 0.0, 1.0)
    assert np.all(ones == 1.0)
    y = M.init_uniform(7, 12, 0, idx[:1000], 0.5, 0.0)
    assert np.count_nonzero(y == x[:1000].astype(np.float32)) < 5
    # the index is the unsharded one: shard r of length n starts at r*n
    full = M.init_uniform(9, 4, 0, np.arange(64), 0.1, 0.0)
    assert np.array_equal(M.init_uniform(9, 4, 32, np.arange(32), 0.1, 0.0), full[32:])
    # element g takes the top 24 bits of word g % 4 of block g // 4, drawn
    # here with numpy's Philox (key (seed, param_id); it steps its 256-bit
    # counter by one before each block, so block b comes from counter b - 1,
    # and block 0 from the all-ones counter)
    g = np.array([0, 1, 2, 3, 4, 5, 6, 7, 401, 402, 403, 404, 99999], dtype=np.int64)
    want = []
    ones = 2 ** 64 - 1
    for e in g:
        blk = int(e) >> 2
        ctr = [blk - 1, 0, 0, 0] if blk > 0 else [ones, ones, ones, ones]
        bg = np.random.Philox(key=np.array([7, 11], dtype=np.uint64), counter=np.array(ctr, dtype=np.uint64))
        word = int(bg.random_raw(4)[int(e) & 3])
        want.append(np.float32(2.0) * (np.float32(word >> 40) * np.float32(2.0 ** -24)) - np.float32(1.0))
    got = M.init_uniform(7, 11, 0, g, 1.0, 0.0)
    assert np.array_equal(got, np.array(want, dtype=np.float32))


PINS = [
    pin_ownership_table,
    pin_ownership_rejections,
    pin_identical_replicas_average_to_replica,
    pin_partial_contributions_sum_to_full_gradient,
    pin_redundant_compute_is_averaged,
    pin_rank_order,
    pin_local_owners_left_alone,
    pin_windows,
    pin_norm,
    pin_clip,
    pin_adamw_first_step,
    pin_adamw_matches_torch,
    pin_clip_then_adamw_matches_torch,
    pin_bf16,
    pin_fp32_contributions,
    pin_philox_matches_numpy,
    pin_init_uniform,
]
