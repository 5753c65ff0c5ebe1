"""Shared helpers for the GPU parity tests: draw inputs, run the HIP path
through the C ABI, run the oracle on the same bits, compare.

Inputs come from the seeded generator (gradient_reduction_optimizer_amd.synth)
on the GPU and are copied to the host for the oracle; expected values come
only from the oracle.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

import oracle.method as M
from gradient_reduction_optimizer_amd import binding as B
from gradient_reduction_optimizer_amd import synth
from gradient_reduction_optimizer_amd.buffers import DeviceState, Plan

FP32_RTOL = 1e-6   # FP32 states (acc, master, m, v) and the norm
BF16_RTOL = 1e-2   # BF16 parameter copy


def bits16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16).copy()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().copy()


@dataclasses.dataclass
class Compare:
    name: str
    n: int = 0
    n_diff_bits: int = 0
    max_rel: float = 0.0
    ok: bool = True

    def add(self, got: np.ndarray, want: np.ndarray, rtol: float, floor_scale: Optional[float] = None):
        got = np.asarray(got)
        want = np.asarray(want)
        assert got.shape == want.shape, (self.name, got.shape, want.shape)
        if got.size == 0:
            return
        self.n += got.size
        if got.dtype == np.float32:
            self.n_diff_bits += int(np.count_nonzero(got.view(np.uint32) != want.view(np.uint32)))
        else:
            self.n_diff_bits += int(np.count_nonzero(got != want))
        g = got.astype(np.float64) if got.dtype != np.uint16 else M.bf16_to_f32(got).astype(np.float64)
        w = want.astype(np.float64) if want.dtype != np.uint16 else M.bf16_to_f32(want).astype(np.float64)
        both_nan = np.isnan(g) & np.isnan(w)
        if floor_scale is None:
            floor_scale = float(np.sqrt(np.mean(w[np.isfinite(w)] ** 2))) if np.isfinite(w).any() else 0.0
        tol = rtol * np.maximum(np.abs(w), rtol * floor_scale)
        err = np.abs(g - w)
        bad = ~both_nan & ~(err <= tol)
        if bad.any():
            self.ok = False
        with np.errstate(divide="ignore", invalid="ignore"):
            rel = np.where(both_nan, 0.0, err / np.maximum(np.abs(w), 1e-300))
        self.max_rel = max(self.max_rel, float(np.nanmax(rel)))

    def __str__(self):
        return f"{self.name}: n={self.n} bit-diff={self.n_diff_bits} max_rel={self.max_rel:.3e} ok={self.ok}"


class Case:
    """One workload run through both the GPU path and the oracle."""

    def __init__(self, w: synth.Workload, device="cuda", R: Optional[int] = None, poison: bool = False):
        self.w = w
        self.R = w.R if R is None else R
        self.device = device
        self.poison = poison
        self.plan = Plan(w.tensors, self.R, w.bucket_elems)
        self.owners = M.assign_owners(w.tensors, self.R)
        self.st = DeviceState(self.plan, device)
        self.stream = torch.cuda.current_stream().cuda_stream
        # FP32 master from the generator, identical on both sides.
        self.master_h: Dict[int, np.ndarray] = {}
        self.m_h: Dict[int, np.ndarray] = {}
        self.v_h: Dict[int, np.ndarray] = {}
        for i, o in enumerate(self.owners):
            if not o.updated:
                continue
            if w.tensors[i].numel == 0:
                self.master_h[i] = self.m_h[i] = self.v_h[i] = np.zeros(0, np.float32)
                continue
            p = synth.master_init(w, i, device=device)
            self.st.flat_view(self.st.master, i).copy_(p)
            self.master_h[i] = host(p)
            self.m_h[i] = np.zeros(w.tensors[i].numel, np.float32)
            self.v_h[i] = np.zeros(w.tensors[i].numel, np.float32)
        self.bufs = self.st.grad_buffers()
        self.window_bufs = []
        if poison:
            self.poison_flat_gaps()
            self.poison_grad_padding(self.bufs)
        torch.cuda.synchronize()

    # ------------------------------------------------- poisoned padding
    def flat_gaps(self):
        """[lo, hi) ranges of the flat arrays that no bucket covers."""
        spans = sorted((bk["flat_base"], bk["flat_base"] + bk["len"]) for bk in self.plan.buckets)
        gaps, at = [], 0
        for lo, hi in spans:
            if lo > at:
                gaps.append((at, lo))
            at = max(at, hi)
        if self.st.acc.numel() > at:
            gaps.append((at, self.st.acc.numel()))
        return gaps

    def poison_flat_gaps(self):
        for lo, hi in self.flat_gaps():
            for arr in (self.st.acc, self.st.master, self.st.m, self.st.v):
                arr[lo:hi].fill_(float("nan"))
            self.st.p_bf16[lo:hi].fill_(float("nan"))

    def poison_grad_padding(self, bufs):
        """NaN in every bucket buffer element past the bucket's length."""
        for b, bk in enumerate(self.plan.buckets):
            bufs[b][:, bk["len"]:].fill_(float("nan"))

    def flat_gaps_untouched(self) -> bool:
        for lo, hi in self.flat_gaps():
            for arr in (self.st.acc, self.st.master, self.st.m, self.st.v, self.st.p_bf16):
                if not bool(torch.isnan(arr[lo:hi]).all()):
                    return False
        return True

    def draw(self, step: int, k: int):
        """Per-tensor per-slot BF16 gradients of microbatch k of step."""
        out = []
        for i, o in enumerate(self.owners):
            if o.owner == M.EXCLUDED:
                out.append(None)
                continue
            if self.w.tensors[i].numel == 0:
                dt = torch.float32 if self.w.tensors[i].fp32_grad else torch.bfloat16
                out.append([torch.zeros(0, dtype=dt, device=self.device)] * o.slots)
                continue
            out.append([synth.grad_contribution(self.w, i, 1000 * step + k, r, device=self.device)
                        for r in range(o.slots)])
        return out

    # ---------------------------------------------------------- GPU side
    def gpu_accumulate(self, grads, k: int, n: int, fuse: bool = True, bucket_order=None):
        for i, g in enumerate(grads):
            if g is not None:
                self.st.pack(self.bufs, i, g)
        nb = self.plan.info["n_buckets"]
        ptrs = [b.data_ptr() for b in self.bufs]
        if bucket_order is None:
            B.gro_accumulate(self.plan.handle, 0, nb, ptrs, self.st.acc.data_ptr(), k,
                             n if fuse else 0, self.stream)
        else:
            for b in bucket_order:
                B.gro_accumulate(self.plan.handle, b, b + 1, [ptrs[b]], self.st.acc.data_ptr(), k,
                                 n if fuse else 0, self.stream)

    def gpu_accumulate_window(self, grads_per_micro, n: int):
        """Pack each microbatch into its own bucket-buffer set, then reduce and
        accumulate the whole window in one call."""
        while len(self.window_bufs) < n:
            self.window_bufs.append(self.st.grad_buffers())
            if self.poison:
                self.poison_grad_padding(self.window_bufs[-1])
        for k in range(n):
            for i, g in enumerate(grads_per_micro[k]):
                if g is not None:
                    self.st.pack(self.window_bufs[k], i, g)
        nb = self.plan.info["n_buckets"]
        ptrs = [self.window_bufs[k][b].data_ptr() for k in range(n) for b in range(nb)]
        B.gro_accumulate_window(self.plan.handle, 0, nb, ptrs, n, self.st.acc.data_ptr(), self.stream)

    def gpu_accumulate_groups(self, grads_per_micro, n: int, groups: Sequence[int], announce: bool = True):
        """Pack the window's microbatches, then call gro_accumulate_microbatches
        once per group (sizes `groups`, summing to n); `announce` passes the
        window length (else 0, and gro_reduce_norm computes the partials)."""
        assert sum(groups) == n
        while len(self.window_bufs) < n:
            self.window_bufs.append(self.st.grad_buffers())
            if self.poison:
                self.poison_grad_padding(self.window_bufs[-1])
        for k in range(n):
            for i, g in enumerate(grads_per_micro[k]):
                if g is not None:
                    self.st.pack(self.window_bufs[k], i, g)
        nb = self.plan.info["n_buckets"]
        k0 = 0
        for g in groups:
            ptrs = [self.window_bufs[k][b].data_ptr() for k in range(k0, k0 + g) for b in range(nb)]
            B.gro_accumulate_microbatches(self.plan.handle, 0, nb, ptrs, k0, g, n if announce else 0,
                                          self.st.acc.data_ptr(), self.stream)
            k0 += g

    def gpu_finish(self, n: int, step: int, max_norm: float, with_bf16=True):
        B.gro_reduce_norm(self.plan.handle, self.st.acc.data_ptr(), n, self.stream)
        norm, norm_sq, finite = B.gro_plan_get_norm(self.plan.handle)
        B.gro_clip_adamw(self.plan.handle, self.st.acc.data_ptr(), n, max_norm, self.w.hparams, step,
                         self.st.master.data_ptr(), self.st.m.data_ptr(), self.st.v.data_ptr(),
                         self.st.p_bf16.data_ptr() if with_bf16 else 0, self.stream)
        return norm, norm_sq, finite

    # ------------------------------------------------------- oracle side
    def oracle_window(self, grads_host, step: int, max_norm: float):
        res = M.optimizer_window(self.owners, self.R, grads_host, self.master_h, self.m_h, self.v_h,
                                 self.w.hparams, max_norm, step)
        self.master_h, self.m_h, self.v_h = res.master, res.m, res.v
        return res

    # -------------------------------------------------------- comparison
    def compare_acc(self, res, cmp: Compare):
        acc = host(self.st.acc)
        for i, a in res.acc.items():
            off = self.plan.tensors[i]["flat_offset"]
            cmp.add(acc[off:off + a.size], a, FP32_RTOL)

    def compare_states(self, res, cmps: Dict[str, Compare], check_bf16=True):
        master, m, v = host(self.st.master), host(self.st.m), host(self.st.v)
        p16 = bits16(self.st.p_bf16)
        for i in res.master:
            off = self.plan.tensors[i]["flat_offset"]
            n = res.master[i].size
            cmps["master"].add(master[off:off + n], res.master[i], FP32_RTOL)
            cmps["m"].add(m[off:off + n], res.m[i], FP32_RTOL)
            cmps["v"].add(v[off:off + n], res.v[i], FP32_RTOL)
            if check_bf16 and res.p_bf16[i] is not None:
                cmps["p_bf16"].add(p16[off:off + n], res.p_bf16[i], BF16_RTOL)


def run_parity(w: synth.Workload, windows: Sequence[int], max_norm: Optional[float] = None,
               fuse: bool = True, R: Optional[int] = None, bucket_order=None, window_call: bool = False,
               log=print, zero_tensors=(), poison: bool = False, step_numbers: Optional[Sequence[int]] = None,
               groups: Optional[Sequence[Sequence[int]]] = None, announce: bool = True):
    """Run len(windows) optimizer steps on both sides and compare after each.
    window_call: use gro_accumulate_window (one call per window) instead of
    one gro_accumulate per microbatch.  poison: NaN in every padding element
    of the flat arrays and the gradient buffers before the first step.
    step_numbers: the optimizer step count t of each window (default 1, 2, ...).
    groups: per window, the group sizes for gro_accumulate_microbatches
    (announce: pass the window length to it)."""
    c = Case(w, R=R, poison=poison)
    max_norm = w.max_norm if max_norm is None else max_norm
    cmps = {k: Compare(k) for k in ("acc", "master", "m", "v", "p_bf16")}
    norms = []
    steps = list(step_numbers) if step_numbers is not None else list(range(1, len(windows) + 1))
    assert len(steps) == len(windows)
    for step, n in zip(steps, windows):
        grads_host = []
        micro = []
        for k in range(n):
            g = c.draw(step, k)
            for i in zero_tensors:  # an unused parameter: zero contributions
                g[i] = [torch.zeros_like(x) for x in g[i]]
            if window_call or groups is not None:
                micro.append(g)
            else:
                c.gpu_accumulate(g, k, n, fuse=fuse, bucket_order=bucket_order)
            grads_host.append([None if x is None else [synth.host_values(s) for s in x] for x in g])
        if groups is not None:
            c.gpu_accumulate_groups(micro, n, groups[len(norms)], announce=announce)
        elif window_call:
            c.gpu_accumulate_window(micro, n)
        norm, norm_sq, finite = c.gpu_finish(n, step, max_norm)
        res = c.oracle_window(grads_host, step, max_norm)
        c.compare_acc(res, cmps["acc"])
        c.compare_states(res, cmps)
        norms.append((norm, res.norm, finite, res.stepped))
    for k in cmps.values():
        log(str(k))
    for got, want, finite, stepped in norms:
        log(f"norm gpu={got!r} oracle={want!r} rel={abs(got - want) / max(abs(want), 1e-300):.3e}")
    return c, cmps, norms


def assert_parity(cmps, norms):
    for k in cmps.values():
        assert k.ok, str(k)
    for got, want, finite, stepped in norms:
        assert finite == stepped
        if math.isfinite(want):
            assert abs(got - want) <= FP32_RTOL * abs(want), (got, want)
