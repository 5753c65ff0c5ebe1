"""GPU: gro_plan_bind_static, the binding for callers that cannot allocate
device memory, gives bit for bit the results of gro_plan_bind on a
caller-allocated workspace -- on two plans bound one after the other to the
same static array, the second smaller than the first -- and a plan whose
array was taken over by another plan is rejected until it binds again."""
import pytest
import torch

from gradient_reduction_optimizer_amd import binding as B
from gradient_reduction_optimizer_amd import synth
from gradient_reduction_optimizer_amd.buffers import DeviceState, Plan

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)


@pytest.fixture(autouse=True)
def _need_gpu(gpu):
    torch.cuda.synchronize()
    yield
    torch.cuda.synchronize()


class Side:
    """One plan of a workload with its own states, bound to a caller
    workspace (static=False) or to the library's static one."""

    def __init__(self, w, static: bool):
        self.w = w
        self.plan = Plan(w.tensors, w.R, w.bucket_elems)
        self.st = DeviceState(self.plan, "cuda", static_workspace=static)
        self.bufs = self.st.grad_buffers()
        self.s = self.st.stream.cuda_stream
        for i, row in enumerate(self.plan.tensors):
            if row["updated"] and row["numel"]:
                self.st.flat_view(self.st.master, i).copy_(synth.master_init(w, i, device="cuda"))

    def bind_static(self):
        B.gro_plan_bind_static(self.plan.handle, self.s)

    def step(self, step: int, n: int, window_call: bool):
        """One window of n microbatches, norm, clip + AdamW; returns the norm."""
        nb = self.plan.info["n_buckets"]
        acc = self.st.acc.data_ptr()
        sets = []
        for k in range(n):
            bufs = self.st.grad_buffers() if window_call else self.bufs
            for i, row in enumerate(self.plan.tensors):
                if row["owner"] != B.GRO_OWNER_EXCLUDED and row["numel"]:
                    g = [synth.grad_contribution(self.w, i, 1000 * step + k, r, device="cuda")
                         for r in range(row["slots"])]
                    self.st.pack(bufs, i, g)
            if window_call:
                sets.append(bufs)
            else:
                B.gro_accumulate(self.plan.handle, 0, nb, [b.data_ptr() for b in bufs], acc, k, n, self.s)
        if window_call:
            B.gro_accumulate_window(self.plan.handle, 0, nb, [b.data_ptr() for bs in sets for b in bs], n,
                                    acc, self.s)
        B.gro_reduce_norm(self.plan.handle, acc, n, self.s)
        norm, _, finite = B.gro_plan_get_norm(self.plan.handle)
        B.gro_clip_adamw(self.plan.handle, acc, n, self.w.max_norm, self.w.hparams, step,
                         self.st.master.data_ptr(), self.st.m.data_ptr(), self.st.v.data_ptr(),
                         self.st.p_bf16.data_ptr(), self.s)
        torch.cuda.synchronize()
        assert finite
        return norm


def assert_same(a: Side, b: Side, what: str):
    for name in ("acc", "master", "m", "v"):
        x, y = getattr(a.st, name), getattr(b.st, name)
        assert torch.equal(x.view(torch.int32), y.view(torch.int32)), (what, name)
    assert torch.equal(a.st.p_bf16.view(torch.int16), b.st.p_bf16.view(torch.int16)), (what, "p_bf16")
    log(f"{what}: acc, master, m, v and the BF16 copy bit-identical ({a.st.acc.numel()} elements)")


def test_static_binding_matches_caller_workspace_on_two_plans_in_a_row():
    big, small = synth.draft_67m(half_share=True), synth.tiny()
    assert small.numel < big.numel
    a_ws, a_st = Side(big, False), Side(big, True)
    log(f"plan 1: {big.name}, {a_st.plan.info['workspace_bytes']} workspace bytes, static")
    na, ns = a_ws.step(1, 4, window_call=False), a_st.step(1, 4, window_call=False)
    assert na == ns, (na, ns)
    assert_same(a_ws, a_st, f"{big.name} step 1")

    b_ws, b_st = Side(small, False), Side(small, True)  # rebinds the static array to the smaller plan
    log(f"plan 2: {small.name}, {b_st.plan.info['workspace_bytes']} workspace bytes, static")
    na, ns = b_ws.step(1, 3, window_call=True), b_st.step(1, 3, window_call=True)
    assert na == ns, (na, ns)
    assert_same(b_ws, b_st, f"{small.name} step 1")

    # the first plan lost the array to the second: rejected before any work
    with pytest.raises(B.GroError) as e:
        B.gro_reduce_norm(a_st.plan.handle, a_st.st.acc.data_ptr(), 4, a_st.s)
    assert e.value.kind == "state"
    a_st.bind_static()       # takes it back; the second plan is now the stale one
    na, ns = a_ws.step(2, 2, window_call=True), a_st.step(2, 2, window_call=True)
    assert na == ns, (na, ns)
    assert_same(a_ws, a_st, f"{big.name} step 2 after rebinding")
    with pytest.raises(B.GroError) as e:
        B.gro_plan_get_norm(b_st.plan.handle)
    assert e.value.kind == "state"


def test_static_binding_rejects_a_plan_larger_than_the_array():
    # one tensor of 3e9 elements: ~732,000 chunks, over the 16 MiB array
    t = [synth.TensorSpec(0, "flat", (3_000_000_000,), "shard", shard_index=0)]
    plan = Plan(t, 2, 64_000_000)
    assert plan.info["workspace_bytes"] > B.GRO_STATIC_WORKSPACE_BYTES
    with pytest.raises(B.GroError) as e:
        B.gro_plan_bind_static(plan.handle, 0)
    assert e.value.kind == "invalid"
