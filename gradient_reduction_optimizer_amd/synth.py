"""Seeded synthetic workloads: tensor lists, placements and input values.

This module only *describes and draws inputs*.  It holds none of the
method's arithmetic (no reduction, no accumulation, no norm, no optimizer
step, no BF16 rounding routine of its own): BF16 values come from
``torch.Tensor.to(torch.bfloat16)``.  Both the CPU oracle's callers and the
GPU path's callers draw their inputs here, so the two sides see the same
bits.

Placements are plain strings ("replicate", "partial", "shard", "reduced");
each side maps them to its own representation.

The workloads stand in for the parameter sets the TP-replica-ownership issue
(NeMo Automodel #3857, "refactor(distributed): establish shared native TP
replica ownership") talks about: a synthetic 67M-parameter BF16 draft model
(section "Preserved prototype and evidence"), a dense model's FSDP flat shard
with hybrid-replica averaging (Cosmos 3 "distributed parallel" page, the
dp_replicate axis), and a hybrid/MoE-like many-tensor set with EP-local
experts (issue section "Proposed scope and acceptance criteria").
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence, Tuple

import numpy as np

PLACEMENTS = ("replicate", "partial", "shard", "reduced")


@dataclasses.dataclass
class TensorSpec:
    """One parameter as seen by this GPU: stable id, local shape, placement."""
    param_id: int
    name: str
    shape: Tuple[int, ...]
    placement: str
    shard_index: int = -1
    frozen: bool = False
    no_decay: bool = False
    fp32_grad: bool = False       # contributions arrive in FP32 instead of BF16

    @property
    def numel(self) -> int:
        return int(np.prod(self.shape, dtype=np.int64)) if len(self.shape) else 1


@dataclasses.dataclass
class Workload:
    name: str
    tensors: List[TensorSpec]
    R: int
    windows: List[int]            # microbatches per accumulation window, in order
    sigma: float                  # standard deviation of the BF16 gradient draws
    seed: int
    bucket_elems: int
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.01
    max_norm: float = 1.0
    master_sigma: float = 0.02
    values: str = "normal"        # "subnormal": contributions are random subnormal patterns

    @property
    def numel(self) -> int:
        return sum(t.numel for t in self.tensors)

    @property
    def hparams(self) -> dict:
        return dict(lr=self.lr, beta1=self.beta1, beta2=self.beta2,
                    eps=self.eps, weight_decay=self.weight_decay)


def _spec(tid: int, name: str, shape, placement: str, **kw) -> TensorSpec:
    shard_index = kw.pop("shard_index", 0 if placement == "shard" else -1)
    return TensorSpec(tid, name, tuple(int(s) for s in shape), placement,
                      shard_index=shard_index, **kw)


# ---------------------------------------------------------------- workloads
def tiny(literal: bool = False, bucket_elems: int = 25_000_000) -> Workload:
    """Ten tensors of mixed placement, R=2, one microbatch.

    The stated total (~100K) and the stated shape [1024,256] disagree; the
    default swaps that tensor for [256,64] (96,409 elements), ``literal``
    keeps [1024,256] (342,169 elements).
    """
    shapes = [
        ("proj_shard", (256, 256), "shard"),
        ("rmsnorm_a", (256,), "replicate"),
        ("mlp_shard", (1024, 256) if literal else (256, 64), "shard"),
        ("q_norm", (64,), "partial"),
        ("k_norm", (64,), "partial"),
        ("seq_sharded_linear", (64, 64), "partial"),
        ("rmsnorm_b", (256,), "replicate"),
        ("ddp_reduced", (32, 256), "reduced"),
        ("odd_replicated", (1000,), "replicate"),
        ("odd_shard", (17, 33), "shard"),
    ]
    tensors = [_spec(i, n, s, p) for i, (n, s, p) in enumerate(shapes)]
    return Workload("tiny-literal" if literal else "tiny", tensors, R=2,
                    windows=[1], sigma=1e-2, seed=0, bucket_elems=bucket_elems)


def draft_67m(half_share: bool = False, bucket_elems: int = 25_000_000) -> Workload:
    """4-layer hidden-1024 draft model with a 16384x1024 embedding, TP2 plan.

    Projections and the embedding are Shard, RMSNorm weights Replicate, Q/K
    norm weights (head_dim 64) Partial.  ``half_share`` halves every Shard
    tensor (the TP2 rank's local share); the default treats the whole
    67,118,592-element set as this GPU's share.
    """
    h = 1024
    div = 2 if half_share else 1
    tensors: List[TensorSpec] = []

    def add(name, shape, placement):
        tensors.append(_spec(len(tensors), name, shape, placement))

    add("embed", (16384 // div, h), "shard")
    for layer in range(4):
        p = f"layers.{layer}."
        add(p + "attn_norm", (h,), "replicate")
        add(p + "qkv", (3 * h // div, h), "shard")
        add(p + "q_norm", (64,), "partial")
        add(p + "k_norm", (64,), "partial")
        add(p + "o", (h, h // div), "shard")
        add(p + "mlp_norm", (h,), "replicate")
        add(p + "up", (4 * h // div, h), "shard")
        add(p + "down", (h, 4 * h // div), "shard")
    add("final_norm", (h,), "replicate")
    name = "draft-67m-tp2-half" if half_share else "draft-67m"
    return Workload(name, tensors, R=2, windows=[4], sigma=1e-2, seed=1,
                    bucket_elems=bucket_elems)


def dense_1b_shard(bucket_elems: int = 25_000_000, windows=(8, 3)) -> Workload:
    """One GPU's 1/8 FSDP flat shard of a 1B-class dense model.

    hidden 2048, 24 layers, vocab 32000, non-gated 4x MLP, untied head:
    1,339,131,904 parameters / 8 = 167,391,488 elements, averaged across
    R=2 hybrid replicas.
    """
    per_layer = 4 * 2048 * 2048 + 2 * 2048 * 8192 + 2 * 2048
    total = 24 * per_layer + 2 * 32000 * 2048 + 2048
    assert total % 8 == 0
    t = [_spec(0, "fsdp_flat_shard", (total // 8,), "replicate")]
    return Workload("dense-1b-fsdp8-shard", t, R=2, windows=list(windows),
                    sigma=1e-3, seed=2, bucket_elems=bucket_elems)


def hybrid_moe(n_tensors: int = 4000, target: int = 300_000_000,
               bucket_elems: int = 25_000_000) -> Workload:
    """Many-small-tensor set: lognormal sizes in [64, 4M], ~300M total.

    By size rank: the smallest 25% are norms (two Replicate for each Partial,
    standing for attention norms), the next 5% routers (Replicate), the
    largest 70% EP-local experts (Shard).
    """
    rng = np.random.default_rng(3)
    raw = np.exp(rng.normal(9.3, 2.0, size=n_tensors))
    sizes = np.clip(np.round(raw), 64, 4_194_304)
    sizes = np.clip(np.round(sizes * (target / sizes.sum())), 64, 4_194_304).astype(np.int64)
    order = np.argsort(sizes, kind="stable")
    role = np.empty(n_tensors, dtype=object)
    n_norm = n_tensors // 4
    n_router = n_tensors // 20
    for rank, idx in enumerate(order):
        if rank < n_norm:
            role[idx] = "partial" if rank % 3 == 2 else "replicate"
        elif rank < n_norm + n_router:
            role[idx] = "replicate"
        else:
            role[idx] = "shard"
    tensors = [_spec(i, f"t{i}", (int(sizes[i]),), role[i]) for i in range(n_tensors)]
    return Workload("hybrid-moe-4000", tensors, R=2, windows=[2], sigma=1e-2,
                    seed=3, bucket_elems=bucket_elems)


def dense_8b_share(numel: int = 1_000_000_000, bucket_elems: int = 64_000_000) -> Workload:
    """One GPU's 1B-element FSDP shard of an 8B dense model (Replicate, R=2)."""
    t = [_spec(0, "fsdp_flat_shard", (numel,), "replicate")]
    return Workload("dense-8b-share", t, R=2, windows=[8], sigma=1e-3, seed=4,
                    bucket_elems=bucket_elems, weight_decay=0.1)


WORKLOADS = {
    "tiny": tiny,
    "tiny-literal": lambda **kw: tiny(literal=True, **kw),
    "draft-67m": draft_67m,
    "draft-67m-tp2-half": lambda **kw: draft_67m(half_share=True, **kw),
    "dense-1b-fsdp8-shard": dense_1b_shard,
    "hybrid-moe-4000": hybrid_moe,
    "dense-8b-share": dense_8b_share,
}


# ------------------------------------------------------------------ values
def stream_seed(*ids: int) -> int:
    """A 63-bit seed for one independent stream, from integer ids."""
    state = np.random.SeedSequence([int(i) & 0xFFFFFFFF for i in ids]).generate_state(2, np.uint32)
    return int((int(state[0]) << 31) ^ int(state[1])) & ((1 << 63) - 1)


_GRAD, _MASTER, _BUCKET_GRAD, _BUCKET_MASTER = 1, 2, 3, 4


def _normal(numel: int, sigma: float, seed: int, device):
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    x = torch.randn(numel, generator=gen, device=device, dtype=torch.float32)
    return x.mul_(float(np.float32(sigma)))


def grad_bf16(w: Workload, tensor_index: int, micro: int, slot: int,
              device="cpu", numel: Optional[int] = None):
    """BF16 gradient contribution of rank-slot ``slot`` in microbatch ``micro``.

    Returned as a 1-D ``torch.bfloat16`` tensor on ``device``.  Values:
    float32 normals times sigma, rounded by torch's float->bfloat16 cast.
    """
    import torch
    n = w.tensors[tensor_index].numel if numel is None else numel
    seed = stream_seed(w.seed, _GRAD, tensor_index, micro, slot)
    if w.values == "subnormal":
        return _subnormal(n, seed, torch.int16, device).view(torch.bfloat16)
    return _normal(n, w.sigma, seed, device).to(torch.bfloat16)


def grad_contribution(w: Workload, tensor_index: int, micro: int, slot: int, device="cpu"):
    """Gradient contribution in the tensor's own type: BF16 as grad_bf16,
    or the FP32 normals themselves for an fp32_grad tensor."""
    import torch
    t = w.tensors[tensor_index]
    if not t.fp32_grad:
        return grad_bf16(w, tensor_index, micro, slot, device=device)
    seed = stream_seed(w.seed, _GRAD, tensor_index, micro, slot)
    if w.values == "subnormal":
        return _subnormal(t.numel, seed, torch.int32, device).view(torch.float32)
    return _normal(t.numel, w.sigma, seed, device)


def _subnormal(numel: int, seed: int, itype, device):
    """Random subnormal bit patterns (exponent field 0, random sign and
    nonzero mantissa) as a signed-integer tensor of the format's width."""
    import torch
    rng = np.random.default_rng(seed)
    if itype == torch.int16:      # BF16: 7 mantissa bits
        bits = rng.integers(1, 1 << 7, size=numel, dtype=np.uint32) | (rng.integers(0, 2, size=numel, dtype=np.uint32) << 15)
        arr = bits.astype(np.uint16).view(np.int16)
    else:                         # FP32: 23 mantissa bits
        bits = rng.integers(1, 1 << 23, size=numel, dtype=np.uint32) | (rng.integers(0, 2, size=numel, dtype=np.uint32) << 31)
        arr = bits.view(np.int32)
    return torch.from_numpy(arr.copy()).to(device)


def bucket_grads_bf16(w: Workload, step: int, micro: int, bucket: int, slots: int, length: int,
                      device="cpu"):
    """BF16 contributions for a whole bucket at once, [slots, length]: for
    workloads too large to draw tensor by tensor (the 1e9-element share).
    float32 normals times sigma, rounded by torch's float->bfloat16 cast."""
    import torch
    seed = stream_seed(w.seed, _BUCKET_GRAD, step, micro, bucket)
    return _normal(slots * length, w.sigma, seed, device).view(slots, length).to(torch.bfloat16)


def bucket_master(w: Workload, bucket: int, length: int, device="cpu"):
    """FP32 master weights ~ N(0, master_sigma) for a whole bucket (1-D)."""
    return _normal(length, w.master_sigma, stream_seed(w.seed, _BUCKET_MASTER, bucket), device)


def host_values(t) -> np.ndarray:
    """Host copy for the oracle: uint16 bits for BF16, float32 otherwise."""
    import torch
    if t.dtype == torch.bfloat16:
        return bf16_bits(t)
    return t.detach().cpu().numpy().astype(np.float32, copy=True)


def master_init(w: Workload, tensor_index: int, device="cpu"):
    """FP32 master weights ~ N(0, master_sigma) for one tensor (1-D)."""
    seed = stream_seed(w.seed, _MASTER, tensor_index)
    return _normal(w.tensors[tensor_index].numel, w.master_sigma, seed, device)


def bf16_bits(t) -> np.ndarray:
    """Host uint16 view of a torch.bfloat16 tensor's bits."""
    import torch
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
