"""The streaming probes that bench.py uses to measure what each kernel's
access pattern can reach: they must move the bytes they claim to (each
output element is the trivial function of its inputs) and reject bad
arguments."""
import ctypes
import os

import pytest
import torch

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "gradient_reduction_optimizer_amd", "libgro_probe.so")
V = ctypes.c_void_p


@pytest.fixture(scope="module")
def lib(gpu):
    lib = ctypes.CDLL(LIB)
    lib.gro_probe_stream.argtypes = [ctypes.c_int, ctypes.c_int64, V, V, V, V, V, V, ctypes.c_int, ctypes.c_int, V]
    lib.gro_probe_stream.restype = ctypes.c_int
    return lib


def _rand(n, seed, dtype=torch.float32):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return torch.randn(n, generator=g, device="cuda").to(dtype)


@pytest.mark.parametrize("flags", [0, 1 | (2 << 8)], ids=["default", "nontemporal-acc-cap2"])
@pytest.mark.parametrize("wide", [False, True])
def test_probe_patterns_compute_what_they_read(lib, wide, flags):
    """Patterns 0-2 (4 elements per lane access) and 3-5 (8 per lane), with
    the default launch and with the large-plan one (the accumulator's stream
    non-temporal, at most 2 workgroups per CU)."""
    off = 3 if wide else 0
    n = 3 * 4096
    s = torch.cuda.current_stream().cuda_stream
    gs = [_rand(n, 10 + j, torch.bfloat16) for j in range(3)]
    gp = (V * 3)(*[x.data_ptr() for x in gs])
    out = torch.zeros(n, device="cuda")
    assert lib.gro_probe_stream(1 + off, n, None, out.data_ptr(), None, None, None, gp, 3, flags, s) == 0
    torch.cuda.synchronize()
    want = (gs[0].float() + gs[1].float()) + gs[2].float()
    assert torch.equal(out, want)
    old = out.clone()
    assert lib.gro_probe_stream(2 + off, n, None, out.data_ptr(), None, None, None, gp, 1, flags, s) == 0
    torch.cuda.synchronize()
    assert torch.equal(out, old + gs[0].float())
    a, p, m, v = (_rand(n, 20 + j) for j in range(4))
    pb = torch.zeros(n, dtype=torch.bfloat16, device="cuda")
    p0, m0, v0 = p.clone(), m.clone(), v.clone()
    assert lib.gro_probe_stream(0 + off, n, a.data_ptr(), p.data_ptr(), m.data_ptr(), v.data_ptr(), pb.data_ptr(),
                                None, 0, flags, s) == 0
    torch.cuda.synchronize()
    assert torch.equal(p, p0 - a) and torch.equal(m, m0 + a) and torch.equal(v, v0 + a * a)
    assert torch.equal(pb.view(torch.int16), (p.view(torch.int32) >> 16).to(torch.int16))


def test_reference_streams_compute_what_they_read(lib):
    """Patterns 6-8: read-only (one sum per workgroup), write-only, copy."""
    n = 3 * 4096
    s = torch.cuda.current_stream().cuda_stream
    src, dst, sums = _rand(n, 31), torch.zeros(n, device="cuda"), torch.zeros(n, device="cuda")
    assert lib.gro_probe_stream(8, n, src.data_ptr(), dst.data_ptr(), None, None, None, None, 0, 0, s) == 0
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    assert lib.gro_probe_stream(7, n, None, dst.data_ptr(), None, None, None, None, 0, 0, s) == 0
    torch.cuda.synchronize()
    assert torch.equal(dst, torch.arange(3, device="cuda").float().repeat_interleave(4096))
    x = torch.ones(n, device="cuda")
    assert lib.gro_probe_stream(6, n, None, x.data_ptr(), sums.data_ptr(), None, None, None, 0, 0, s) == 0
    torch.cuda.synchronize()
    # each workgroup's first wave: 64 lanes x 16 elements
    assert torch.equal(sums[:3], torch.full((3,), 1024.0, device="cuda"))
    assert lib.gro_probe_stream(6, n, None, x.data_ptr(), None, None, None, None, 0, 0, s) == -1


def test_probe_rejects_bad_arguments(lib):
    s = torch.cuda.current_stream().cuda_stream
    out = torch.zeros(8192, device="cuda")
    g = torch.zeros(8192, dtype=torch.bfloat16, device="cuda")
    gp = (V * 1)(g.data_ptr())
    assert lib.gro_probe_stream(1, 4000, None, out.data_ptr(), None, None, None, gp, 1, 0, s) == -1  # not whole chunks
    assert lib.gro_probe_stream(1, 8192, None, out.data_ptr(), None, None, None, gp, 9, 0, s) == -1  # k not built
    assert lib.gro_probe_stream(1, 8192, None, out.data_ptr(), None, None, None, gp, 17, 0, s) == -1
    assert lib.gro_probe_stream(0, 8192, None, out.data_ptr(), None, None, None, None, 0, 0, s) == -1  # missing arrays
    assert lib.gro_probe_stream(4, 8192, None, out.data_ptr(), None, None, None, gp, 9, 0, s) == -1  # k not built
    assert lib.gro_probe_stream(9, 8192, None, out.data_ptr(), None, None, None, gp, 1, 0, s) == -1  # no such pattern
    assert lib.gro_probe_stream(1, 8192, None, out.data_ptr(), None, None, None, gp, 1, 2, s) == -1  # unknown flag
    assert lib.gro_probe_stream(1, 8192, None, out.data_ptr(), None, None, None, gp, 1, 17 << 8, s) == -1  # cap
