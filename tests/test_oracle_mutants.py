"""Plant plausible mistakes in the CPU oracle and check that the pins catch
each one.  Every mutant replaces one oracle function (on the CPU only) and
at least one pin must then fail."""
import numpy as np
import pytest

import oracle.method as M
from oracle_pins import PINS

F32 = np.float32
_orig = {name: getattr(M, name) for name in (
    "assign_owners", "reduce_contributions", "accumulate", "window_gradient",
    "global_norm", "clip_coefficient", "adamw_scalars", "adamw_update", "f32_to_bf16",
    "bf16_to_f32", "as_f32", "philox4x64_10", "init_uniform")}


def _partial_as_replicate(tensors, R):
    rows = _orig["assign_owners"](tensors, R)
    for o in rows:
        if o.owner == M.SUM:
            o.owner, o.divisor = M.MEAN, R
    return rows


def _mean_not_divided(owner, R, slots):
    s = M.bf16_to_f32(slots[0])
    for r in range(1, owner.slots):
        s = s + M.bf16_to_f32(slots[r])
    return s


def _sum_divided(owner, R, slots):
    s = _orig["reduce_contributions"](owner, R, slots)
    return s / F32(R) if owner.owner == M.SUM else s


def _mean_uses_first_slot(owner, R, slots):
    return M.bf16_to_f32(slots[0]) if owner.owner == M.MEAN else _orig["reduce_contributions"](owner, R, slots)


def _local_scaled(owner, R, slots):
    s = _orig["reduce_contributions"](owner, R, slots)
    return s / F32(R) if owner.owner in (M.LOCAL_SHARD, M.LOCAL_REDUCED) else s


def _accumulate_overwrites(acc, red, k):
    return red.astype(F32, copy=True)


def _window_not_divided(acc, n):
    return acc.copy()


def _window_divided_by_full_length(acc, n):
    return acc / F32(8)


def _norm_of_abs_sum(grads):
    import math
    t = math.fsum(float(abs(x)) for g in grads for x in np.asarray(g, np.float64))
    return t, t * t


def _norm_sq_not_rooted(grads):
    n, sq = _orig["global_norm"](grads)
    return sq, sq


def _clip_unclamped(norm, max_norm):
    import math
    if not math.isfinite(norm):
        return F32(1), False
    if not (max_norm > 0) or math.isinf(max_norm):
        return F32(1), True
    return F32(max_norm / (norm + 1e-6)), True


def _clip_inverted(norm, max_norm):
    import math
    if not math.isfinite(norm):
        return F32(1), False
    if not (max_norm > 0) or math.isinf(max_norm):
        return F32(1), True
    return F32(min(1.0, (norm + 1e-6) / max_norm)), True


def _clip_never_skips(norm, max_norm):
    c, _ = _orig["clip_coefficient"](norm if norm == norm and abs(norm) != float("inf") else 0.0, max_norm)
    return c, True


def _no_bias_correction(lr, beta1, beta2, eps, weight_decay, step):
    sc = _orig["adamw_scalars"](lr, beta1, beta2, eps, weight_decay, step)
    sc.step_size, sc.sqrt_bc2 = F32(lr), F32(1.0)
    return sc


def _decay_wd_only(lr, beta1, beta2, eps, weight_decay, step):
    sc = _orig["adamw_scalars"](lr, beta1, beta2, eps, weight_decay, step)
    sc.decay = F32(1.0 - weight_decay)
    return sc


def _betas_swapped(lr, beta1, beta2, eps, weight_decay, step):
    return _orig["adamw_scalars"](lr, beta2, beta1, eps, weight_decay, step)


def _eps_inside_sqrt(g, coef, p, m, v, sc, decayed):
    gh = g * F32(coef)
    p = p * (sc.decay if decayed else F32(1.0))
    m = sc.beta1 * m + sc.one_minus_beta1 * gh
    v = sc.beta2 * v + sc.one_minus_beta2 * (gh * gh)
    d = np.sqrt(v + sc.eps) / sc.sqrt_bc2
    p = p - sc.step_size * (m / d)
    return p, m, v, M.f32_to_bf16(p)


def _sign_flipped(g, coef, p, m, v, sc, decayed):
    p1, m1, v1, _ = _orig["adamw_update"](g, coef, p, m, v, sc, decayed)
    p1 = p * (sc.decay if decayed else F32(1.0)) + (p * (sc.decay if decayed else F32(1.0)) - p1)
    return p1, m1, v1, M.f32_to_bf16(p1)


def _clip_ignored(g, coef, p, m, v, sc, decayed):
    return _orig["adamw_update"](g, F32(1.0), p, m, v, sc, decayed)


def _decay_after_update(g, coef, p, m, v, sc, decayed):
    p1, m1, v1, _ = _orig["adamw_update"](g, coef, p, m, v, sc, False)
    p1 = p1 * (sc.decay if decayed else F32(1.0))
    return p1, m1, v1, M.f32_to_bf16(p1)


def _decay_ignores_flag(g, coef, p, m, v, sc, decayed):
    return _orig["adamw_update"](g, coef, p, m, v, sc, True)


def _truncate_bf16(x):
    return (np.ascontiguousarray(x, dtype=F32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _ties_away(x):
    b = np.ascontiguousarray(x, dtype=F32).view(np.uint32)
    out = (b + np.uint32(0x8000)) >> np.uint32(16)
    return out.astype(np.uint16)


def _fp32_through_bf16(x):
    x = np.asarray(x)
    if x.dtype == np.float32:
        return M.bf16_to_f32(M.f32_to_bf16(x))
    return _orig["as_f32"](x)


def _philox_nine_rounds(counter, key):
    c = [int(x) for x in counter]
    k = [int(x) for x in key]
    MASK = (1 << 64) - 1
    for _ in range(9):
        p0 = 0xD2E7470EE14C6C93 * c[0]
        p1 = 0xCA5A826395121157 * c[2]
        c = [(p1 >> 64) ^ c[1] ^ k[0], p1 & MASK, (p0 >> 64) ^ c[3] ^ k[1], p0 & MASK]
        k = [(k[0] + 0x9E3779B97F4A7C15) & MASK, (k[1] + 0xBB67AE8584CAA73B) & MASK]
    return c


def _init_ignores_shard_offset(seed, param_id, index_base, indices, bound, offset):
    return _orig["init_uniform"](seed, param_id, 0, indices, bound, offset)


def _clip_without_eps(norm, max_norm):
    import math
    if not math.isfinite(norm):
        return F32(1), False
    if not (max_norm > 0) or math.isinf(max_norm):
        return F32(1), True
    return F32(min(1.0, max_norm / norm)) if norm > 0 else F32(1), True


def _v_unclipped(g, coef, p, m, v, sc, decayed):
    gh = g * F32(coef)
    p = p * (sc.decay if decayed else F32(1.0))
    m = sc.beta1 * m + sc.one_minus_beta1 * gh
    v = sc.beta2 * v + sc.one_minus_beta2 * (g * g)
    d = np.sqrt(v) / sc.sqrt_bc2 + sc.eps
    p = p - sc.step_size * (m / d)
    return p, m, v, M.f32_to_bf16(p)


def _m_unclipped(g, coef, p, m, v, sc, decayed):
    gh = g * F32(coef)
    p = p * (sc.decay if decayed else F32(1.0))
    m = sc.beta1 * m + sc.one_minus_beta1 * g
    v = sc.beta2 * v + sc.one_minus_beta2 * (gh * gh)
    d = np.sqrt(v) / sc.sqrt_bc2 + sc.eps
    p = p - sc.step_size * (m / d)
    return p, m, v, M.f32_to_bf16(p)


def _philox_key_fixed(counter, key):
    c = [int(x) for x in counter]
    k = [int(x) for x in key]
    MASK = (1 << 64) - 1
    for _ in range(10):
        p0 = 0xD2E7470EE14C6C93 * c[0]
        p1 = 0xCA5A826395121157 * c[2]
        c = [(p1 >> 64) ^ c[1] ^ k[0], p1 & MASK, (p0 >> 64) ^ c[3] ^ k[1], p0 & MASK]
    return c


def _philox_multipliers_swapped(counter, key):
    c = [int(x) for x in counter]
    k = [int(x) for x in key]
    MASK = (1 << 64) - 1
    for _ in range(10):
        p0 = 0xCA5A826395121157 * c[0]
        p1 = 0xD2E7470EE14C6C93 * c[2]
        c = [(p1 >> 64) ^ c[1] ^ k[0], p1 & MASK, (p0 >> 64) ^ c[3] ^ k[1], p0 & MASK]
        k = [(k[0] + 0x9E3779B97F4A7C15) & MASK, (k[1] + 0xBB67AE8584CAA73B) & MASK]
    return c


def _eps_before_bias_correction(g, coef, p, m, v, sc, decayed):
    gh = g * F32(coef)
    p = p * (sc.decay if decayed else F32(1.0))
    m = sc.beta1 * m + sc.one_minus_beta1 * gh
    v = sc.beta2 * v + sc.one_minus_beta2 * (gh * gh)
    d = (np.sqrt(v) + sc.eps) / sc.sqrt_bc2
    p = p - sc.step_size * (m / d)
    return p, m, v, M.f32_to_bf16(p)


def _no_second_moment_correction(lr, beta1, beta2, eps, weight_decay, step):
    sc = _orig["adamw_scalars"](lr, beta1, beta2, eps, weight_decay, step)
    sc.sqrt_bc2 = F32(1.0)
    return sc


def _step_off_by_one(lr, beta1, beta2, eps, weight_decay, step):
    return _orig["adamw_scalars"](lr, beta1, beta2, eps, weight_decay, step + 1)


def _frozen_not_excluded(tensors, R):
    import copy
    thawed = []
    for t in tensors:
        t = copy.copy(t)
        if getattr(t, "frozen", False):
            t.frozen = False
        thawed.append(t)
    return _orig["assign_owners"](thawed, R)


def _slots_summed_last_first(owner, R, slots):
    s = M.as_f32(slots[owner.slots - 1])
    for r in range(owner.slots - 2, -1, -1):
        s = s + M.as_f32(slots[r])
    if owner.owner == M.MEAN:
        s = s / F32(R)
    return s


def _init_wrong_word(seed, param_id, index_base, indices, bound, offset):
    b, o = F32(bound), F32(offset)
    out = np.empty(len(indices), dtype=F32)
    for j, i in enumerate(indices):
        g = int(index_base) + int(i)
        blk = M.philox4x64_10((g >> 2, 0, 0, 0), (seed, param_id))
        u = F32(blk[(g + 1) & 3] >> 40) * F32(2.0 ** -24)
        out[j] = o + (F32(2.0) * u - F32(1.0)) * b
    return out


def _init_low_bits(seed, param_id, index_base, indices, bound, offset):
    b, o = F32(bound), F32(offset)
    out = np.empty(len(indices), dtype=F32)
    for j, i in enumerate(indices):
        g = int(index_base) + int(i)
        blk = M.philox4x64_10((g >> 2, 0, 0, 0), (seed, param_id))
        u = F32(blk[g & 3] & 0xFFFFFF) * F32(2.0 ** -24)
        out[j] = o + (F32(2.0) * u - F32(1.0)) * b
    return out


def _init_one_sided(seed, param_id, index_base, indices, bound, offset):
    v = _orig["init_uniform"](seed, param_id, index_base, indices, bound, offset)
    # offset + u * bound instead of offset + (2u - 1) * bound
    return (F32(offset) + (v - F32(offset) + F32(bound)) / F32(2.0)).astype(F32)


def _widen_wrong_shift(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(15)).view(F32)


MUTANTS = {
    "partial_treated_as_replicate": ("assign_owners", _partial_as_replicate),
    "mean_not_divided": ("reduce_contributions", _mean_not_divided),
    "sum_divided_by_R": ("reduce_contributions", _sum_divided),
    "mean_reads_one_slot": ("reduce_contributions", _mean_uses_first_slot),
    "local_scaled": ("reduce_contributions", _local_scaled),
    "accumulate_overwrites": ("accumulate", _accumulate_overwrites),
    "window_not_divided": ("window_gradient", _window_not_divided),
    "trailing_window_divided_by_full": ("window_gradient", _window_divided_by_full_length),
    "norm_l1": ("global_norm", _norm_of_abs_sum),
    "norm_not_rooted": ("global_norm", _norm_sq_not_rooted),
    "clip_unclamped": ("clip_coefficient", _clip_unclamped),
    "clip_inverted": ("clip_coefficient", _clip_inverted),
    "clip_never_skips": ("clip_coefficient", _clip_never_skips),
    "no_bias_correction": ("adamw_scalars", _no_bias_correction),
    "decay_missing_lr": ("adamw_scalars", _decay_wd_only),
    "betas_swapped": ("adamw_scalars", _betas_swapped),
    "eps_inside_sqrt": ("adamw_update", _eps_inside_sqrt),
    "update_sign_flipped": ("adamw_update", _sign_flipped),
    "clip_coef_ignored": ("adamw_update", _clip_ignored),
    "decay_after_update": ("adamw_update", _decay_after_update),
    "decay_ignores_opt_out": ("adamw_update", _decay_ignores_flag),
    "bf16_truncates": ("f32_to_bf16", _truncate_bf16),
    "bf16_ties_away": ("f32_to_bf16", _ties_away),
    "widen_wrong_shift": ("bf16_to_f32", _widen_wrong_shift),
    "fp32_rounded_to_bf16": ("as_f32", _fp32_through_bf16),
    "philox_nine_rounds": ("philox4x64_10", _philox_nine_rounds),
    "init_ignores_shard_offset": ("init_uniform", _init_ignores_shard_offset),
    "clip_without_eps": ("clip_coefficient", _clip_without_eps),
    "v_from_unclipped_gradient": ("adamw_update", _v_unclipped),
    "eps_before_bias_correction": ("adamw_update", _eps_before_bias_correction),
    "no_second_moment_correction": ("adamw_scalars", _no_second_moment_correction),
    "step_off_by_one": ("adamw_scalars", _step_off_by_one),
    "frozen_not_excluded": ("assign_owners", _frozen_not_excluded),
    "slots_summed_last_first": ("reduce_contributions", _slots_summed_last_first),
    "init_wrong_word": ("init_uniform", _init_wrong_word),
    "init_low_bits": ("init_uniform", _init_low_bits),
    "init_one_sided": ("init_uniform", _init_one_sided),
    "m_from_unclipped_gradient": ("adamw_update", _m_unclipped),
    "philox_key_not_bumped": ("philox4x64_10", _philox_key_fixed),
    "philox_multipliers_swapped": ("philox4x64_10", _philox_multipliers_swapped),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_some_pin_catches_mutant(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(M, attr, fn)
    caught = []
    for pin in PINS:
        try:
            pin(M)
        except (AssertionError, ValueError, TypeError, M.Rejected):
            caught.append(pin.__name__)
            break
    assert caught, f"mutant {name} passed every pin"
