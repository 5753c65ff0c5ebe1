"""ctypes binding of libgro.so: the C-ABI calls under the same names.

Argument marshalling only -- every step of the path runs in the library's
HIP kernels.  Device pointers and streams are plain integers (for instance
``tensor.data_ptr()`` and ``torch.cuda.current_stream().cuda_stream``).
There is no fallback: if the library is not built, the first call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Iterable, List, Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgro.so")

# ---- constants (mirror include/gro.h) ----
GRO_OK = 0
GRO_E_INVALID = -1
GRO_E_PLACEMENT = -2
GRO_E_DUPLICATE = -3
GRO_E_STATE = -4
GRO_E_HIP = -5
ERROR_NAMES = {GRO_E_INVALID: "invalid", GRO_E_PLACEMENT: "placement",
               GRO_E_DUPLICATE: "duplicate", GRO_E_STATE: "state", GRO_E_HIP: "hip"}

GRO_REPLICATE, GRO_PARTIAL, GRO_SHARD, GRO_REDUCED = 0, 1, 2, 3
PLACEMENT_CODES = {"replicate": GRO_REPLICATE, "partial": GRO_PARTIAL,
                   "shard": GRO_SHARD, "reduced": GRO_REDUCED}
GRO_NO_DECAY, GRO_FROZEN, GRO_FP32_GRAD = 1, 2, 4
GRO_GRAD_BF16, GRO_GRAD_FP32 = 0, 1
GRO_OWNER_MEAN, GRO_OWNER_SUM, GRO_OWNER_LOCAL_SHARD, GRO_OWNER_LOCAL_REDUCED, GRO_OWNER_EXCLUDED = range(5)
OWNER_NAMES = ("mean", "sum", "local_shard", "local_reduced", "excluded")
GRO_MAX_NDIM = 8
GRO_STATIC_WORKSPACE_BYTES = 16777216

EXPORTS = ("gro_plan_create", "gro_plan_destroy", "gro_plan_get_info", "gro_plan_tensor",
           "gro_plan_bucket", "gro_plan_bind", "gro_plan_bind_static", "gro_accumulate", "gro_accumulate_window",
           "gro_accumulate_microbatches",
           "gro_reduce_norm", "gro_plan_get_norm", "gro_clip_adamw", "gro_init_uniform",
           "gro_last_error")


class gro_tensor_desc(ctypes.Structure):
    _fields_ = [("param_id", ctypes.c_int64), ("shape", ctypes.POINTER(ctypes.c_int64)),
                ("ndim", ctypes.c_int32), ("placement", ctypes.c_int32),
                ("shard_index", ctypes.c_int32), ("flags", ctypes.c_uint32)]


class gro_plan_info(ctypes.Structure):
    _fields_ = [("R", ctypes.c_int32), ("n_tensors", ctypes.c_int32), ("n_buckets", ctypes.c_int32),
                ("chunk_elems", ctypes.c_int32), ("n_chunks", ctypes.c_int64),
                ("n_flat", ctypes.c_int64), ("n_owned", ctypes.c_int64),
                ("bucket_elems", ctypes.c_int64), ("workspace_bytes", ctypes.c_uint64)]


class gro_tensor_layout(ctypes.Structure):
    _fields_ = [("param_id", ctypes.c_int64), ("numel", ctypes.c_int64), ("flat_offset", ctypes.c_int64),
                ("owner", ctypes.c_int32), ("slots", ctypes.c_int32), ("divisor", ctypes.c_int32),
                ("in_norm", ctypes.c_int32), ("updated", ctypes.c_int32), ("decayed", ctypes.c_int32),
                ("first_bucket", ctypes.c_int32), ("n_buckets", ctypes.c_int32),
                ("grad_dtype", ctypes.c_int32)]


class gro_bucket_info(ctypes.Structure):
    _fields_ = [("flat_base", ctypes.c_int64), ("len", ctypes.c_int64), ("slot_stride", ctypes.c_int64),
                ("first_chunk", ctypes.c_int64), ("n_chunks", ctypes.c_int64),
                ("owner", ctypes.c_int32), ("slots", ctypes.c_int32), ("decayed", ctypes.c_int32),
                ("grad_dtype", ctypes.c_int32)]


class gro_adamw_hparams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double), ("beta2", ctypes.c_double),
                ("eps", ctypes.c_double), ("weight_decay", ctypes.c_double)]


class GroError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{ERROR_NAMES.get(code, code)}: {msg}")
        self.code = code
        self.kind = ERROR_NAMES.get(code, str(code))


_lib: Optional[ctypes.CDLL] = None


def load() -> ctypes.CDLL:
    """Load libgro.so.  If the in-tree library has not been built yet and
    hipcc is available, build it first; otherwise raise."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from . import build as _build
        if os.path.abspath(LIB_PATH) == os.path.abspath(_build.LIB) and os.path.exists(_build.HIPCC):
            _build.build()
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m gradient_reduction_optimizer_amd.build`")
    # PyTorch ships its own HIP runtime under the same library name.  Load it
    # first, so that libgro.so binds to the runtime PyTorch uses: with the
    # system one loaded first, two runtimes would own the device in one
    # process and device calls fail.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, U64, D = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_double
    L.gro_plan_create.argtypes = [ctypes.POINTER(gro_tensor_desc), I32, I32, I64, ctypes.POINTER(P)]
    L.gro_plan_destroy.argtypes = [P]
    L.gro_plan_destroy.restype = None
    L.gro_plan_get_info.argtypes = [P, ctypes.POINTER(gro_plan_info)]
    L.gro_plan_tensor.argtypes = [P, I32, ctypes.POINTER(gro_tensor_layout)]
    L.gro_plan_bucket.argtypes = [P, I32, ctypes.POINTER(gro_bucket_info)]
    L.gro_plan_bind.argtypes = [P, P, U64, P]
    L.gro_plan_bind_static.argtypes = [P, P]
    L.gro_accumulate.argtypes = [P, I32, I32, ctypes.POINTER(P), P, I32, I32, P]
    L.gro_accumulate_window.argtypes = [P, I32, I32, ctypes.POINTER(P), I32, P, P]
    L.gro_accumulate_microbatches.argtypes = [P, I32, I32, ctypes.POINTER(P), I32, I32, I32, P, P]
    L.gro_reduce_norm.argtypes = [P, P, I32, P]
    L.gro_plan_get_norm.argtypes = [P, ctypes.POINTER(D), ctypes.POINTER(D), ctypes.POINTER(I32)]
    L.gro_clip_adamw.argtypes = [P, P, I32, D, ctypes.POINTER(gro_adamw_hparams), I64, P, P, P, P, P]
    L.gro_init_uniform.argtypes = [P, ctypes.c_uint64, ctypes.POINTER(D), ctypes.POINTER(D), P, P, P]
    L.gro_last_error.argtypes = []
    L.gro_last_error.restype = ctypes.c_char_p
    for name in EXPORTS:
        if name not in ("gro_plan_destroy", "gro_last_error"):
            getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def _check(rc: int) -> None:
    if rc != GRO_OK:
        raise GroError(rc, gro_last_error())


def gro_last_error() -> str:
    return load().gro_last_error().decode()


def _attr(t, name, default=None):
    if isinstance(t, dict):
        return t.get(name, default)
    return getattr(t, name, default)


def gro_plan_create(tensors: Sequence, R: int, bucket_elems: int) -> int:
    """``tensors``: objects or dicts with param_id, shape, placement (a
    GRO_* code or "replicate"/"partial"/"shard"/"reduced"), shard_index,
    and optional frozen / no_decay / fp32_grad.  Returns the plan handle."""
    n = len(tensors)
    descs = (gro_tensor_desc * max(n, 1))()
    keep = []
    for i, t in enumerate(tensors):
        shape = tuple(int(s) for s in _attr(t, "shape"))
        arr = (ctypes.c_int64 * max(len(shape), 1))(*shape)
        keep.append(arr)
        pl = _attr(t, "placement")
        pl = PLACEMENT_CODES.get(pl, pl) if isinstance(pl, str) else int(pl)
        if isinstance(pl, str):
            pl = 99  # unknown name: let the library reject it
        flags = (GRO_FROZEN if _attr(t, "frozen", False) else 0) | \
                (GRO_NO_DECAY if _attr(t, "no_decay", False) else 0) | \
                (GRO_FP32_GRAD if _attr(t, "fp32_grad", False) else 0) | int(_attr(t, "flags", 0) or 0)
        descs[i] = gro_tensor_desc(int(_attr(t, "param_id")), ctypes.cast(arr, ctypes.POINTER(ctypes.c_int64)),
                                   len(shape), int(pl), int(_attr(t, "shard_index", -1)), flags)
    out = ctypes.c_void_p()
    _check(load().gro_plan_create(descs if n else None, n, int(R), int(bucket_elems), ctypes.byref(out)))
    return int(out.value)


def gro_plan_destroy(plan: int) -> None:
    if plan:
        load().gro_plan_destroy(ctypes.c_void_p(plan))


def _struct_dict(s) -> dict:
    return {name: getattr(s, name) for name, _ in s._fields_}


def gro_plan_get_info(plan: int) -> dict:
    info = gro_plan_info()
    _check(load().gro_plan_get_info(ctypes.c_void_p(plan), ctypes.byref(info)))
    return _struct_dict(info)


def gro_plan_tensor(plan: int, i: int) -> dict:
    lay = gro_tensor_layout()
    _check(load().gro_plan_tensor(ctypes.c_void_p(plan), int(i), ctypes.byref(lay)))
    return _struct_dict(lay)


def gro_plan_bucket(plan: int, b: int) -> dict:
    bk = gro_bucket_info()
    _check(load().gro_plan_bucket(ctypes.c_void_p(plan), int(b), ctypes.byref(bk)))
    return _struct_dict(bk)


def gro_plan_bind(plan: int, d_workspace: int, nbytes: int, stream: int = 0) -> None:
    _check(load().gro_plan_bind(ctypes.c_void_p(plan), ctypes.c_void_p(d_workspace), int(nbytes),
                                ctypes.c_void_p(stream)))


def gro_plan_bind_static(plan: int, stream: int = 0) -> None:
    """Bind to the library's own per-GPU workspace (no allocation)."""
    _check(load().gro_plan_bind_static(ctypes.c_void_p(plan), ctypes.c_void_p(stream)))


def _pointer_array(ptrs: Sequence[int], expected: int, what: str):
    """A C array of the given device pointers.  `expected` is how many the
    library will read (0 when it rejects the call's other arguments before
    reading any); a list of another length must never reach it."""
    if expected and len(ptrs) != expected:
        raise ValueError(f"{what}: {len(ptrs)} pointers given, the call reads {expected}")
    return (ctypes.c_void_p * max(len(ptrs), 1))(*[ctypes.c_void_p(int(p)) for p in ptrs])


# A window or group call takes at most this many microbatches (include/gro.h).
GRO_MAX_GROUP = 64


def _reads(plan: int, b0: int, b1: int, n: int = 1) -> int:
    """Pointers the library reads for buckets [b0, b1) and n microbatches:
    n * (b1 - b0) for a valid range and group size, else 0 (the library then
    rejects the call, or does nothing, before reading a pointer)."""
    nb = gro_plan_get_info(plan)["n_buckets"]
    if not (0 <= int(b0) < int(b1) <= nb and 1 <= int(n) <= GRO_MAX_GROUP):
        return 0
    return int(n) * (int(b1) - int(b0))


def gro_accumulate(plan: int, b0: int, b1: int, d_grad_buckets: Sequence[int], d_acc: int,
                   micro_index: int, window_size: int = 0, stream: int = 0) -> None:
    ptrs = _pointer_array(d_grad_buckets, _reads(plan, b0, b1), "gro_accumulate")
    _check(load().gro_accumulate(ctypes.c_void_p(plan), int(b0), int(b1), ptrs, ctypes.c_void_p(d_acc),
                                 int(micro_index), int(window_size), ctypes.c_void_p(stream)))


def gro_accumulate_window(plan: int, b0: int, b1: int, d_grad_buckets: Sequence[int], n: int, d_acc: int,
                          stream: int = 0) -> None:
    """d_grad_buckets: n*(b1-b0) pointers, microbatch-major."""
    ptrs = _pointer_array(d_grad_buckets, _reads(plan, b0, b1, n), "gro_accumulate_window")
    _check(load().gro_accumulate_window(ctypes.c_void_p(plan), int(b0), int(b1), ptrs, int(n),
                                        ctypes.c_void_p(d_acc), ctypes.c_void_p(stream)))


def gro_accumulate_microbatches(plan: int, b0: int, b1: int, d_grad_buckets: Sequence[int], first_micro: int,
                                n: int, window_size: int, d_acc: int, stream: int = 0) -> None:
    """Microbatches first_micro..first_micro+n-1 of a window; d_grad_buckets:
    n*(b1-b0) pointers, microbatch-major."""
    ptrs = _pointer_array(d_grad_buckets, _reads(plan, b0, b1, n), "gro_accumulate_microbatches")
    _check(load().gro_accumulate_microbatches(ctypes.c_void_p(plan), int(b0), int(b1), ptrs, int(first_micro),
                                              int(n), int(window_size), ctypes.c_void_p(d_acc),
                                              ctypes.c_void_p(stream)))


def gro_reduce_norm(plan: int, d_acc: int, window_size: int, stream: int = 0) -> None:
    _check(load().gro_reduce_norm(ctypes.c_void_p(plan), ctypes.c_void_p(d_acc), int(window_size),
                                  ctypes.c_void_p(stream)))


def gro_plan_get_norm(plan: int):
    """Returns (norm, norm_sq, finite)."""
    n, sq, f = ctypes.c_double(), ctypes.c_double(), ctypes.c_int32()
    _check(load().gro_plan_get_norm(ctypes.c_void_p(plan), ctypes.byref(n), ctypes.byref(sq), ctypes.byref(f)))
    return n.value, sq.value, bool(f.value)


def gro_clip_adamw(plan: int, d_acc: int, window_size: int, max_norm: float, hp: dict, step: int,
                   d_master: int, d_m: int, d_v: int, d_param_bf16: int = 0, stream: int = 0) -> None:
    h = gro_adamw_hparams(float(hp["lr"]), float(hp["beta1"]), float(hp["beta2"]), float(hp["eps"]),
                          float(hp["weight_decay"]))
    _check(load().gro_clip_adamw(ctypes.c_void_p(plan), ctypes.c_void_p(d_acc), int(window_size),
                                 float(max_norm), ctypes.byref(h), int(step), ctypes.c_void_p(d_master),
                                 ctypes.c_void_p(d_m), ctypes.c_void_p(d_v),
                                 ctypes.c_void_p(d_param_bf16 or 0), ctypes.c_void_p(stream)))


def gro_init_uniform(plan: int, seed: int, bounds: Sequence[float], offsets: Optional[Sequence[float]],
                     d_master: int, d_param_bf16: int = 0, stream: int = 0) -> None:
    """bounds/offsets: one value per tensor, in descriptor order (the library
    reads the plan's n_tensors entries of each)."""
    nt = gro_plan_get_info(plan)["n_tensors"]
    if len(bounds) != nt or (offsets is not None and len(offsets) != nt):
        raise ValueError(f"gro_init_uniform: bounds/offsets need {nt} entries each, got {len(bounds)}"
                         f"{'' if offsets is None else ' / ' + str(len(offsets))}")
    n = max(nt, 1)
    b = (ctypes.c_double * n)(*[float(x) for x in bounds])
    o = None if offsets is None else (ctypes.c_double * n)(*[float(x) for x in offsets])
    _check(load().gro_init_uniform(ctypes.c_void_p(plan), ctypes.c_uint64(int(seed) & ((1 << 64) - 1)), b, o,
                                   ctypes.c_void_p(d_master), ctypes.c_void_p(d_param_bf16 or 0),
                                   ctypes.c_void_p(stream)))
