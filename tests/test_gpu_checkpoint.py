"""GPU: a checkpoint of the owned state restored into a different layout and
a different ownership gives the same next AdamW update, bit for bit, as the
uninterrupted run."""
import sys

import numpy as np
import pytest
import torch

from gradient_reduction_optimizer_amd import binding as B
from gradient_reduction_optimizer_amd import synth
from gradient_reduction_optimizer_amd.buffers import DeviceState, Plan
from gradient_reduction_optimizer_amd.checkpoint import load_state, save_state

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)


@pytest.fixture(autouse=True)
def _need_gpu(gpu):
    torch.cuda.synchronize()
    yield
    torch.cuda.synchronize()


def _grad(pid, numel, step, k, r, sigma=1e-2):
    """Seeded BF16 gradient of one parameter, keyed by param_id (no -0.0)."""
    gen = torch.Generator(device="cuda").manual_seed(synth.stream_seed(77, pid, step, k, r))
    g = (torch.randn(numel, generator=gen, device="cuda") * sigma).to(torch.bfloat16)
    return torch.where(g == 0, torch.zeros_like(g), g)  # canonical +0


class Run:
    def __init__(self, tensors, R, cap, hp, max_norm):
        self.plan = Plan(tensors, R, cap)
        self.st = DeviceState(self.plan)
        self.bufs = self.st.grad_buffers()
        self.pos = {int(t.param_id): i for i, t in enumerate(tensors)}
        self.tensors = tensors
        self.hp, self.max_norm = hp, max_norm
        self.s = torch.cuda.current_stream().cuda_stream

    def init_master(self, seed):
        for i, t in enumerate(self.tensors):
            row = self.plan.tensors[i]
            if row["updated"] and row["numel"]:
                gen = torch.Generator(device="cuda").manual_seed(synth.stream_seed(seed, int(t.param_id)))
                self.st.flat_view(self.st.master, i).copy_(torch.randn(row["numel"], generator=gen, device="cuda") * 0.02)

    def step(self, step, n, legacy_pids=()):
        """One window; a parameter in legacy_pids gets its full gradient in
        slot 0 (pre-reduced); otherwise Partial parameters get (g, 0)."""
        nb = self.plan.info["n_buckets"]
        ptrs = [b.data_ptr() for b in self.bufs]
        for k in range(n):
            for i, t in enumerate(self.tensors):
                row = self.plan.tensors[i]
                if not row["updated"]:
                    continue
                g = _grad(int(t.param_id), row["numel"], step, k, 0)
                slots = [g] + [torch.zeros_like(g) if t.placement == "partial" else g
                               for _ in range(row["slots"] - 1)]
                self.st.pack(self.bufs, i, slots)
            B.gro_accumulate(self.plan.handle, 0, nb, ptrs, self.st.acc.data_ptr(), k, n, self.s)
        B.gro_reduce_norm(self.plan.handle, self.st.acc.data_ptr(), n, self.s)
        B.gro_clip_adamw(self.plan.handle, self.st.acc.data_ptr(), n, self.max_norm, self.hp, step,
                         self.st.master.data_ptr(), self.st.m.data_ptr(), self.st.v.data_ptr(),
                         self.st.p_bf16.data_ptr(), self.s)

    def by_pid(self):
        out = {}
        for i, t in enumerate(self.tensors):
            if self.plan.tensors[i]["updated"]:
                out[int(t.param_id)] = [self.st.flat_view(a, i).clone() for a in
                                        (self.st.master, self.st.m, self.st.v, self.st.p_bf16)]
        return out


def test_restore_into_new_layout_and_ownership_matches_next_update(tmp_path):
    w = synth.tiny(literal=True)
    # legacy ownership: Q/K norms and the sequence-sharded linear arrive pre-reduced
    legacy = [synth.TensorSpec(t.param_id, t.name, t.shape, "reduced" if t.placement == "partial" else t.placement,
                               shard_index=t.shard_index) for t in w.tensors]
    a = Run(legacy, w.R, w.bucket_elems, w.hparams, w.max_norm)
    a.init_master(5)
    a.step(1, 2)
    a.step(2, 3)
    save_state(a.plan, a.st.master, a.st.m, a.st.v, step=2, directory=str(tmp_path))
    a.step(3, 4)
    ref = a.by_pid()
    # native ownership (Partial), reversed registration order, small buckets
    b = Run(list(reversed(w.tensors)), w.R, 5000, w.hparams, w.max_norm)
    step = load_state(b.plan, b.st.master, b.st.m, b.st.v, str(tmp_path))
    assert step == 2
    b.step(step + 1, 4)
    got = b.by_pid()
    torch.cuda.synchronize()
    assert ref.keys() == got.keys()
    for pid in ref:
        for name, x, y in zip(("master", "m", "v", "p_bf16"), ref[pid], got[pid]):
            same = torch.equal(x.view(torch.int16), y.view(torch.int16))
            assert same, (pid, name)
    log(f"restored {len(ref)} parameters; next update bit-identical")
