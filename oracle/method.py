"""Step-by-step CPU statement of the gradient-ownership hot path.

TEST INFRASTRUCTURE ONLY (see the package docstring).  numpy float32 arrays
are used for every per-element FP32 operation: each ufunc rounds once, no
operations are fused, denormals are kept.  BF16 values travel as uint16 bit
patterns.

Page keys used in citations:
  P1 = NeMo Automodel issue #3857, "refactor(distributed): establish shared
       native TP replica ownership"
  P3 = Cosmos 3 training framework, "distributed parallel"
  P4 = Mixle v0.8.1, "Distributed Transformer Training"
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence

import numpy as np

F32 = np.float32

# Owner classes.  One per parameter (P1, "Proposed scope and acceptance
# criteria": each parameter's gradient is reduced by a single owner).
MEAN = "mean"                    # Replicate: complete gradients, averaged
SUM = "sum"                      # Partial: partial contributions, summed
LOCAL_SHARD = "local_shard"      # Shard: owned outright, never synchronised
LOCAL_REDUCED = "local_reduced"  # already reduced by another owner
EXCLUDED = "excluded"            # frozen: no gradient, not updated

OWNERS = (MEAN, SUM, LOCAL_SHARD, LOCAL_REDUCED, EXCLUDED)


class Rejected(ValueError):
    """A plan the method refuses; ``kind`` is invalid/placement/duplicate."""

    def __init__(self, kind: str, msg: str):
        super().__init__(f"{kind}: {msg}")
        self.kind = kind


@dataclasses.dataclass
class Owner:
    param_id: int
    owner: str
    slots: int       # rank contributions read per microbatch
    divisor: int     # what the slot sum is divided by (1 = not divided)
    in_norm: bool
    updated: bool
    decayed: bool


# --------------------------------------------------------------- O1 owners
def assign_owners(tensors: Sequence, R: int) -> List[Owner]:
    """Ownership of every parameter, from its placement tag.

    P1 "Why this needs separate work": replication alone does not say what a
    local gradient means --
      * redundant full computation gives complete gradients, averaged over
        the R tensor-parallel ranks            -> MEAN, R slots, divide by R
      * head/sequence-sharded computation gives partial contributions to a
        replicated parameter, which are summed  -> SUM, R slots
      * TP/EP/model-owned local shards are not synchronised as replicas
                                                -> LOCAL_SHARD, 1 slot
      * a gradient an existing FSDP/DDP/DTensor reduction already reduced is
        not reduced again                       -> LOCAL_REDUCED, 1 slot
    P1 "Proposed scope and acceptance criteria": one owner per parameter,
    unsupported compositions rejected, no double reduction; frozen
    parameters are outside the update (EXCLUDED).
    P4 "Backend split": an unsupported request fails before fitting, so
    every check happens here, before any data is touched.

    ``tensors`` items need attributes param_id, shape, placement,
    shard_index, frozen, no_decay.
    """
    if int(R) < 1:
        raise Rejected("invalid", f"R must be >= 1, got {R}")
    seen = set()
    rows: List[Owner] = []
    for t in tensors:
        pid = int(t.param_id)
        if pid in seen:
            raise Rejected("duplicate", f"param_id {pid} has a second owner")
        seen.add(pid)
        if any(int(d) < 0 for d in t.shape):
            raise Rejected("invalid", f"param_id {pid}: negative dimension")
        if t.placement == "shard":
            if not (0 <= int(t.shard_index) < R):
                raise Rejected("placement", f"param_id {pid}: shard_index {t.shard_index} not in [0, {R})")
        elif t.placement in ("replicate", "partial", "reduced"):
            if int(t.shard_index) != -1:
                raise Rejected("placement", f"param_id {pid}: shard_index given for a non-Shard tensor")
        else:
            raise Rejected("placement", f"param_id {pid}: unknown placement {t.placement!r}")

        if t.frozen:
            rows.append(Owner(pid, EXCLUDED, 0, 0, False, False, False))
            continue
        if t.placement == "replicate":
            owner, slots, divisor = MEAN, R, R
        elif t.placement == "partial":
            owner, slots, divisor = SUM, R, 1
        elif t.placement == "shard":
            owner, slots, divisor = LOCAL_SHARD, 1, 1
        else:
            owner, slots, divisor = LOCAL_REDUCED, 1, 1
        rows.append(Owner(pid, owner, slots, divisor, True, True, not t.no_decay))
    return rows


# -------------------------------------------------------------------- BF16
def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen BF16 bit patterns to FP32 (exact: BF16 is FP32's top half)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(F32)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """FP32 -> BF16 by IEEE 754 round-to-nearest, ties to even.

    Keep the top 16 bits; round up when the dropped 16 bits exceed half an
    ulp, or equal it and the kept part is odd.  A carry into the exponent is
    the correct result (it reaches infinity from the largest finite values).
    NaN stays NaN (quiet bit set, sign kept).
    """
    b = np.ascontiguousarray(x, dtype=F32).view(np.uint32)
    upper = b >> np.uint32(16)
    lower = b & np.uint32(0xFFFF)
    up = (lower > 0x8000) | ((lower == 0x8000) & ((upper & np.uint32(1)) == 1))
    out = upper + up.astype(np.uint32)
    nan = (b & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    out = np.where(nan, upper | np.uint32(0x0040), out)
    return out.astype(np.uint16)


def as_f32(x: np.ndarray) -> np.ndarray:
    """A gradient contribution as FP32: BF16 bits widened, FP32 as is."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return bf16_to_f32(x)
    if x.dtype == np.float32:
        return x
    raise TypeError(f"gradient contributions are BF16 bits (uint16) or float32, not {x.dtype}")


# ---------------------------------------------------- O2 reduce, accumulate
def reduce_contributions(owner: Owner, R: int, slots: Sequence[np.ndarray]) -> np.ndarray:
    """One microbatch's reduced FP32 gradient for one parameter.

    The ``owner.slots`` contributions -- BF16 bit patterns (uint16 arrays),
    widened exactly, or FP32 arrays, used as they are (P1 "Proposed scope
    and acceptance criteria": BF16/FP32) -- are summed in FP32 in rank order
    0..c-1 (P1 "Preserved prototype and evidence": FP32 reduction).  MEAN then divides by R (the average over TP ranks, P1 "Why
    this needs separate work"); SUM keeps the sum; a LOCAL owner's single
    contribution is used as it is.
    """
    if owner.owner == EXCLUDED:
        raise ValueError("an excluded parameter has no gradient")
    if len(slots) != owner.slots:
        raise ValueError(f"expected {owner.slots} contributions, got {len(slots)}")
    s = as_f32(slots[0])
    for r in range(1, owner.slots):
        s = s + as_f32(slots[r])
    if owner.owner == MEAN:
        s = s / F32(R)
    return s


def accumulate(acc: Optional[np.ndarray], red: np.ndarray, micro_index: int) -> np.ndarray:
    """FP32 gradient accumulation across a window's microbatches.

    The first microbatch of a window starts the accumulator; later ones add
    (P1 "Preserved prototype and evidence" and "Proposed scope and
    acceptance criteria": accumulation over 1, >1 and trailing windows).
    """
    if micro_index == 0:
        return red.astype(F32, copy=True)
    return acc + red


def window_gradient(acc: np.ndarray, n: int) -> np.ndarray:
    """The window's gradient: accumulator / n, n = microbatches actually in
    this window (a trailing window of 3 divides by 3)."""
    return acc / F32(n)


# ----------------------------------------------------------------- O4 norm
def global_norm(grads: Sequence[np.ndarray]):
    """Global L2 norm over every owned element (P1: "global norms").

    Squares of FP32 values are exact in FP64; their sum is rounded once
    (``math.fsum``), then the FP64 square root is taken.
    Returns (norm, norm_squared).
    """
    sq = [np.square(np.asarray(g, dtype=np.float64)) for g in grads]
    if not all(np.isfinite(s).all() for s in sq):
        bad = float("nan") if any(np.isnan(s).any() for s in sq) else float("inf")
        return bad, bad
    total = math.fsum(x for s in sq for x in s)
    return math.sqrt(total), total


# ----------------------------------------------------------- O5 clip coef
def clip_coefficient(norm: float, max_norm: float):
    """Clip coefficient and whether the step is taken.

    Clipping on/off (P1 "Proposed scope and acceptance criteria"): on when
    max_norm is finite and > 0.  coef = min(1, max_norm / (norm + 1e-6)) in
    FP64, then rounded to FP32.  A non-finite norm skips the update.
    Returns (coef as float32, step_taken).
    """
    if not math.isfinite(norm):
        return F32(1.0), False
    mx = float(max_norm)
    if not (mx > 0.0) or math.isinf(mx):
        return F32(1.0), True
    return F32(min(1.0, mx / (norm + 1e-6))), True


# ---------------------------------------------------------------- O6 AdamW
@dataclasses.dataclass
class AdamWScalars:
    beta1: np.float32
    beta2: np.float32
    one_minus_beta1: np.float32
    one_minus_beta2: np.float32
    step_size: np.float32       # lr / (1 - beta1^t)
    sqrt_bc2: np.float32        # sqrt(1 - beta2^t)
    eps: np.float32
    decay: np.float32           # 1 - lr * weight_decay


def adamw_scalars(lr, beta1, beta2, eps, weight_decay, step: int) -> AdamWScalars:
    """Per-step scalars: computed in FP64 from the hyper-parameters as given
    (FP64 values), each rounded once to FP32.  ``step`` counts updates from 1."""
    if step < 1:
        raise ValueError("step counts from 1")
    lr, b1, b2, eps, wd = (float(x) for x in (lr, beta1, beta2, eps, weight_decay))
    bc1 = 1.0 - b1 ** step
    bc2 = 1.0 - b2 ** step
    return AdamWScalars(F32(b1), F32(b2), F32(1.0 - b1), F32(1.0 - b2),
                        F32(lr / bc1), F32(math.sqrt(bc2)), F32(eps),
                        F32(1.0 - lr * wd))


def adamw_update(g: np.ndarray, coef, p: np.ndarray, m: np.ndarray, v: np.ndarray,
                 sc: AdamWScalars, decayed: bool):
    """Clip + AdamW (decoupled weight decay, bias-corrected) on one tensor.

    The pages name Adam/AdamW as the update (P1 "Preserved prototype and
    evidence": the restored state matched the following Adam step; P4
    "Optimizer and checkpoint semantics": Adam and AdamW remain explicit
    options) without a formula;
    this is the standard decoupled form:
        g^ = g * coef
        p  = p * (1 - lr*wd)
        m  = beta1*m + (1-beta1)*g^
        v  = beta2*v + (1-beta2)*g^*g^
        p  = p - (lr/bc1) * m / (sqrt(v)/sqrt(bc2) + eps)
    Every operation is one FP32 rounding, evaluated left to right.
    Returns (p, m, v, p_bf16_bits).
    """
    gh = g * F32(coef)
    p = p * (sc.decay if decayed else F32(1.0))
    m = sc.beta1 * m + sc.one_minus_beta1 * gh
    v = sc.beta2 * v + sc.one_minus_beta2 * (gh * gh)
    d = np.sqrt(v) / sc.sqrt_bc2 + sc.eps
    p = p - sc.step_size * (m / d)
    return p, m, v, f32_to_bf16(p)


# ------------------------------------------------------------- N3 init
_MASK64 = (1 << 64) - 1
_PHILOX_M = (0xD2E7470EE14C6C93, 0xCA5A826395121157)
_PHILOX_W = (0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B)


def philox4x64_10(counter, key):
    """Philox4x64-10 of Salmon, Moraes, Dror and Shaw ("Parallel random
    numbers: as easy as 1, 2, 3", SC 2011), in Python integers: ten rounds;
    each multiplies words 0 and 2 by the two round constants (128-bit
    products), mixes the high halves with the other words and the key, and
    bumps the key by the Weyl constants."""
    c = [int(x) & _MASK64 for x in counter]
    k = [int(x) & _MASK64 for x in key]
    for _ in range(10):
        p0 = _PHILOX_M[0] * c[0]
        p1 = _PHILOX_M[1] * c[2]
        c = [(p1 >> 64) ^ c[1] ^ k[0], p1 & _MASK64, (p0 >> 64) ^ c[3] ^ k[1], p0 & _MASK64]
        k = [(k[0] + _PHILOX_W[0]) & _MASK64, (k[1] + _PHILOX_W[1]) & _MASK64]
    return c


def init_uniform(seed: int, param_id: int, index_base: int, indices, bound: float, offset: float) -> np.ndarray:
    """Replica-consistent initial values of the given element indices of one
    parameter (P1 "Why this needs separate work": initialisation after
    parallelisation must not depend on rank-specific training RNG).

    Element g (its index in the unsharded parameter, index_base + i) draws
    word g % 4 of Philox4x64-10 with counter (g // 4, 0, 0, 0) and key
    (seed, param_id); its top 24 bits give u = k * 2^-24 in [0, 1); the value
    is offset + (2u - 1) * bound in FP32 (bound, offset rounded to FP32).
    Pure Python: meant for small or sampled index sets.
    """
    b, o = F32(bound), F32(offset)
    out = np.empty(len(indices), dtype=F32)
    cache = {}
    for j, i in enumerate(indices):
        g = int(index_base) + int(i)
        blk = cache.get(g >> 2)
        if blk is None:
            blk = cache[g >> 2] = philox4x64_10((g >> 2, 0, 0, 0), (seed, param_id))
        u = F32(blk[g & 3] >> 40) * F32(2.0 ** -24)
        s = F32(2.0) * u - F32(1.0)
        out[j] = o + s * b
    return out


# ----------------------------------------------------------- whole window
@dataclasses.dataclass
class WindowResult:
    acc: Dict[int, np.ndarray]       # per tensor index, FP32 accumulator
    norm: float
    norm_sq: float
    coef: np.float32
    stepped: bool
    master: Dict[int, np.ndarray]
    m: Dict[int, np.ndarray]
    v: Dict[int, np.ndarray]
    p_bf16: Dict[int, np.ndarray]


def optimizer_window(owners: Sequence[Owner], R: int, micro_grads, master, m, v,
                     hparams: dict, max_norm: float, step: int) -> WindowResult:
    """One optimizer step over a window of ``len(micro_grads)`` microbatches.

    ``micro_grads[k][i]`` is the list of BF16 (uint16) contributions of
    tensor i in microbatch k (one array per slot).  ``master``, ``m``, ``v``
    map tensor index -> FP32 array and are not modified; new arrays are
    returned.  Reduce per microbatch, then accumulate; scale by the window
    length; global norm; clip coefficient; AdamW on every updated tensor.
    """
    n = len(micro_grads)
    if n < 1:
        raise ValueError("a window has at least one microbatch")
    acc: Dict[int, np.ndarray] = {}
    for k in range(n):
        for i, o in enumerate(owners):
            if o.owner == EXCLUDED:
                continue
            red = reduce_contributions(o, R, micro_grads[k][i])
            acc[i] = accumulate(acc.get(i), red, k)
    g = {i: window_gradient(a, n) for i, a in acc.items()}
    norm, norm_sq = global_norm([g[i] for i, o in enumerate(owners) if o.in_norm])
    coef, stepped = clip_coefficient(norm, max_norm)
    sc = adamw_scalars(step=step, **hparams)
    new_p, new_m, new_v, p16 = {}, {}, {}, {}
    for i, o in enumerate(owners):
        if not o.updated:
            continue
        if stepped:
            new_p[i], new_m[i], new_v[i], p16[i] = adamw_update(
                g[i], coef, master[i], m[i], v[i], sc, o.decayed)
        else:
            new_p[i], new_m[i], new_v[i] = master[i].copy(), m[i].copy(), v[i].copy()
            p16[i] = None
    return WindowResult(acc, norm, norm_sq, coef, stepped, new_p, new_m, new_v, p16)


__all__ = [
    "MEAN", "SUM", "LOCAL_SHARD", "LOCAL_REDUCED", "EXCLUDED", "OWNERS",
    "Rejected", "Owner", "assign_owners", "bf16_to_f32", "f32_to_bf16", "as_f32",
    "reduce_contributions", "accumulate", "window_gradient", "global_norm",
    "clip_coefficient", "AdamWScalars", "adamw_scalars", "adamw_update",
    "WindowResult", "optimizer_window", "philox4x64_10", "init_uniform",
]
