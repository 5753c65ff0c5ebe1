"""GPU: one optimizer step captured in a HIP graph and replayed gives bit for
bit the results of the same calls issued eagerly.

A step is the window's accumulate calls (one window call, or one call per
microbatch), gro_reduce_norm and gro_clip_adamw.  None of them allocates,
synchronizes or records a memory fill: the tables are uploaded and the
norm's completion counter is cleared when the plan is bound, before the
capture, and the last workgroup of the norm's second stage returns the
counter to zero, so every replay starts from the state the previous one
left.  Two plans of the same parameters run side by side on the same
gradient buffers: one eagerly, one by replaying the captured step.  Every
replay is compared with the eager step it corresponds to, with new
gradients, eager work and device synchronizations between the replays.
The captured step's step count stays fixed (it is a kernel argument), so the
eager side repeats the same count.  The graph side is bound either to a
caller workspace or to the library's static workspace (gro_plan_bind_static,
made for callers such as this one that cannot allocate while capturing)."""
import numpy as np
import pytest
import torch

from gradient_reduction_optimizer_amd import binding as B
from gradient_reduction_optimizer_amd import synth
from gradient_reduction_optimizer_amd.buffers import DeviceState, Plan

pytestmark = pytest.mark.gpu

STEP = 7       # the AdamW step count of every step here (t = 7)
WINDOW = 3     # microbatches per window
REPLAYS = 3


def log(msg):
    print(msg, flush=True)


@pytest.fixture(autouse=True)
def _need_gpu(gpu):
    torch.cuda.synchronize()
    yield
    torch.cuda.synchronize()


class Side:
    """One plan of the workload with its own states, on the shared gradient
    buffers (one set per microbatch)."""

    def __init__(self, w, grads, static: bool):
        self.w = w
        self.plan = Plan(w.tensors, w.R, w.bucket_elems)
        self.st = DeviceState(self.plan, "cuda", static_workspace=static)
        self.grads = grads
        for i, row in enumerate(self.plan.tensors):
            if row["updated"] and row["numel"]:
                self.st.flat_view(self.st.master, i).copy_(synth.master_init(w, i, device="cuda"))

    def step(self, stream: int, window_call: bool):
        h, nb, acc = self.plan.handle, self.plan.info["n_buckets"], self.st.acc.data_ptr()
        ptrs = [[b.data_ptr() for b in bufs] for bufs in self.grads]
        if window_call:
            B.gro_accumulate_window(h, 0, nb, [p for row in ptrs for p in row], WINDOW, acc, stream)
        else:
            for k in range(WINDOW):
                B.gro_accumulate(h, 0, nb, ptrs[k], acc, k, WINDOW, stream)
        B.gro_reduce_norm(h, acc, WINDOW, stream)
        B.gro_clip_adamw(h, acc, WINDOW, self.w.max_norm, self.w.hparams, STEP, self.st.master.data_ptr(),
                         self.st.m.data_ptr(), self.st.v.data_ptr(), self.st.p_bf16.data_ptr(), stream)

    def states(self):
        torch.cuda.synchronize()
        out = [x.cpu().numpy().view(np.uint32).copy() for x in (self.st.master, self.st.m, self.st.v)]
        out.append(self.st.p_bf16.cpu().view(torch.int16).numpy().view(np.uint16).copy())
        return out


def buffers(plan):
    """One set of bucket buffers, as DeviceState.grad_buffers lays them out."""
    return [torch.zeros((bk["slots"], bk["slot_stride"]),
                        dtype=torch.float32 if bk["grad_dtype"] == B.GRO_GRAD_FP32 else torch.bfloat16, device="cuda")
            for bk in plan.buckets]


def fill(w, plan, grads, rnd):
    """New seeded gradients in every microbatch's buffers (the same buffers
    the graph captured)."""
    for k, bufs in enumerate(grads):
        for b in bufs:
            b.zero_()
        for i, row in enumerate(plan.tensors):
            if row["owner"] != B.GRO_OWNER_EXCLUDED and row["numel"]:
                g = [synth.grad_contribution(w, i, 1000 * rnd + k, r, device="cuda") for r in range(row["slots"])]
                for bk, dst, src, cnt in plan.segments(i):
                    for r, x in enumerate(g):
                        bufs[bk][r, dst:dst + cnt].copy_(x[src:src + cnt])


@pytest.mark.parametrize("static", [False, True], ids=["workspace", "static"])
@pytest.mark.parametrize("window_call", [True, False], ids=["window_call", "microbatch_calls"])
def test_graph_replays_match_eager_steps(window_call, static):
    w = synth.tiny(literal=True)
    log(f"case graph replay: {w.name}, window {WINDOW}, window_call={window_call}, static={static}")
    probe = Plan(w.tensors, w.R, w.bucket_elems)
    grads = [buffers(probe) for _ in range(WINDOW)]
    eager = Side(w, grads, static=False)
    graph = Side(w, grads, static=static)
    assert eager.plan.info["n_buckets"] == graph.plan.info["n_buckets"]
    fill(w, probe, grads, 0)
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        graph.step(side.cuda_stream, window_call)
    torch.cuda.synchronize()
    # capture recorded the work without running it: the states are untouched
    assert all(np.array_equal(x, y) for x, y in zip(graph.states(), eager.states()))

    s = torch.cuda.current_stream().cuda_stream
    for rnd in range(REPLAYS):
        if rnd:
            fill(w, probe, grads, rnd)
        eager.step(s, window_call)
        want_norm = B.gro_plan_get_norm(eager.plan.handle)[0]
        g.replay()
        torch.cuda.synchronize()
        got_norm = B.gro_plan_get_norm(graph.plan.handle)[0]
        assert got_norm == want_norm, (rnd, got_norm, want_norm)
        for name, x, y in zip(("master", "m", "v", "p_bf16"), graph.states(), eager.states()):
            diff = int(np.count_nonzero(x != y))
            assert diff == 0, f"replay {rnd}: {name}: {diff} of {x.size} elements differ"
        log(f"replay {rnd}: norm {got_norm:.9g}, master/m/v/BF16 copy bit-identical to the eager step")
    del g
    torch.cuda.synchronize()
