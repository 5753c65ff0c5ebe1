"""Device-memory plumbing around a plan: PyTorch allocates the buffers the
C ABI asks for, and copies per-tensor gradients into the bucket buffers.

Nothing here computes any part of the path; it only allocates and moves
bytes (the kernels in libgro.so do the work).
"""
from __future__ import annotations

from typing import Dict, List, Sequence, Tuple

from . import binding as B


class Plan:
    """Owns a plan handle and caches its info, tensor rows and buckets."""

    def __init__(self, tensors: Sequence, R: int, bucket_elems: int):
        self.handle = B.gro_plan_create(tensors, R, bucket_elems)
        self.R = int(R)
        # this rank's shard index per tensor, as registered (-1 unless Shard)
        self.shard_index = [int(B._attr(t, "shard_index", -1)) for t in tensors]
        self.info = B.gro_plan_get_info(self.handle)
        self.tensors = [B.gro_plan_tensor(self.handle, i) for i in range(self.info["n_tensors"])]
        self.buckets = [B.gro_plan_bucket(self.handle, b) for b in range(self.info["n_buckets"])]

    def close(self) -> None:
        if self.handle:
            B.gro_plan_destroy(self.handle)
            self.handle = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def segments(self, i: int) -> List[Tuple[int, int, int, int]]:
        """Where tensor i's elements sit in the bucket buffers:
        [(bucket, offset in bucket, offset in tensor, count)]."""
        t = self.tensors[i]
        out = []
        if t["n_buckets"] <= 0:
            return out
        start, end = t["flat_offset"], t["flat_offset"] + t["numel"]
        for b in range(t["first_bucket"], t["first_bucket"] + t["n_buckets"]):
            bk = self.buckets[b]
            lo, hi = max(start, bk["flat_base"]), min(end, bk["flat_base"] + bk["len"])
            if hi > lo:
                out.append((b, lo - bk["flat_base"], lo - start, hi - lo))
        return out


class DeviceState:
    """FP32 accumulator / master / m / v, the BF16 parameter copy and the
    workspace for one plan, allocated with torch on ``device`` and bound.
    With ``static_workspace`` no workspace is allocated: the plan is bound
    to the library's own per-GPU workspace (gro_plan_bind_static)."""

    def __init__(self, plan: Plan, device="cuda", with_bf16: bool = True, stream=None,
                 static_workspace: bool = False):
        import torch
        self.plan = plan
        self.device = torch.device(device)
        n = max(int(plan.info["n_flat"]), 1)
        f32 = dict(dtype=torch.float32, device=self.device)
        self.acc = torch.zeros(n, **f32)
        self.master = torch.zeros(n, **f32)
        self.m = torch.zeros(n, **f32)
        self.v = torch.zeros(n, **f32)
        self.p_bf16 = torch.zeros(n, dtype=torch.bfloat16, device=self.device) if with_bf16 else None
        self.stream = stream if stream is not None else torch.cuda.current_stream(self.device)
        if static_workspace:
            self.workspace, self.ws_ptr, self.ws_bytes = None, None, 0
            B.gro_plan_bind_static(plan.handle, self.stream.cuda_stream)
            return
        nbytes = int(plan.info["workspace_bytes"])
        self.workspace = torch.zeros(nbytes + 256, dtype=torch.uint8, device=self.device)
        base = self.workspace.data_ptr()
        self.ws_ptr = (base + 255) // 256 * 256
        self.ws_bytes = nbytes
        B.gro_plan_bind(plan.handle, self.ws_ptr, nbytes, self.stream.cuda_stream)

    def grad_buffers(self) -> List:
        """One [slots, slot_stride] buffer per bucket (zeros), BF16 or FP32
        as the bucket's gradient type says."""
        import torch
        return [torch.zeros((bk["slots"], bk["slot_stride"]),
                            dtype=torch.float32 if bk["grad_dtype"] == B.GRO_GRAD_FP32 else torch.bfloat16,
                            device=self.device)
                for bk in self.plan.buckets]

    def pack(self, bufs: List, i: int, slot_grads: Sequence) -> None:
        """Copy tensor i's per-slot gradients (1-D, length numel, the
        bucket's type) into the bucket buffers."""
        for b, dst, src, cnt in self.plan.segments(i):
            for r, g in enumerate(slot_grads):
                bufs[b][r, dst:dst + cnt].copy_(g[src:src + cnt], non_blocking=True)

    def flat_view(self, arr, i: int):
        """Tensor i's slice of a flat array (acc, master, m, v, p_bf16)."""
        t = self.plan.tensors[i]
        off = t["flat_offset"]
        return arr[off:off + t["numel"]] if off >= 0 else arr[:0]
