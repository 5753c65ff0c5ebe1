"""GPU: checkpoint and restore of the owned state (NeMo Automodel issue #3857,
"refactor(distributed): establish shared native TP replica ownership",
section "Preserved prototype and evidence": a restore from legacy ownership
into native ownership was exact and then matched the next Adam update;
section "Proposed scope and acceptance criteria": checkpoint compatibility,
exact restored state, continued optimizer updates).

Legacy ownership here is the old helper's view: the Partial parameters (Q/K
norms, the sequence-sharded linear) arrive already reduced, one slot.  Native
ownership registers them as Partial over R slots, rank 0 holding the whole
contribution and the other ranks zero, so both views describe the same
gradient.  The oracle runs the same windows on the same input bits and
supplies every expected value: the saved state, the restored state and the
updates after the restore, compared bit for bit."""
import numpy as np
import pytest
import torch

import oracle.method as M
from gradient_reduction_optimizer_amd import binding as B
from gradient_reduction_optimizer_amd import synth
from gradient_reduction_optimizer_amd.buffers import DeviceState, Plan
from gradient_reduction_optimizer_amd.checkpoint import load_state, save_state

pytestmark = pytest.mark.gpu

FP32_RTOL = 1e-6


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


def legacy_of(tensors):
    """The same parameters as the legacy helper saw them: Partial ones pre-reduced."""
    return [synth.TensorSpec(t.param_id, t.name, t.shape, "reduced" if t.placement == "partial" else t.placement,
                             shard_index=t.shard_index) for t in tensors]


def slots_of(t, n_slots, g):
    """Per-slot contributions carrying the gradient g: Partial -> (g, 0, ...),
    Replicate -> R copies, a one-slot owner -> (g,)."""
    return [g] + [torch.zeros_like(g) if t.placement == "partial" else g for _ in range(n_slots - 1)]


class Run:
    """The HIP path through the C ABI on one plan."""

    def __init__(self, tensors, R, cap, hp, max_norm):
        self.plan = Plan(tensors, R, cap)
        self.st = DeviceState(self.plan)
        self.bufs = self.st.grad_buffers()
        self.tensors = tensors
        self.hp, self.max_norm = hp, max_norm
        self.s = torch.cuda.current_stream().cuda_stream

    def init_master(self, seed):
        for i, t in enumerate(self.tensors):
            row = self.plan.tensors[i]
            if row["updated"] and row["numel"]:
                gen = torch.Generator(device="cuda").manual_seed(synth.stream_seed(seed, int(t.param_id)))
                self.st.flat_view(self.st.master, i).copy_(torch.randn(row["numel"], generator=gen, device="cuda") * 0.02)

    def draw(self, step, n):
        """The window's gradients, keyed by param_id: [microbatch] -> {pid: BF16 tensor}."""
        return [{int(t.param_id): _grad(int(t.param_id), self.plan.tensors[i]["numel"], step, k, 0)
                 for i, t in enumerate(self.tensors) if self.plan.tensors[i]["updated"]} for k in range(n)]

    def step(self, step, grads):
        n = len(grads)
        nb = self.plan.info["n_buckets"]
        ptrs = [b.data_ptr() for b in self.bufs]
        for k in range(n):
            for i, t in enumerate(self.tensors):
                row = self.plan.tensors[i]
                if row["updated"]:
                    self.st.pack(self.bufs, i, slots_of(t, row["slots"], grads[k][int(t.param_id)]))
            B.gro_accumulate(self.plan.handle, 0, nb, ptrs, self.st.acc.data_ptr(), k, n, self.s)
        B.gro_reduce_norm(self.plan.handle, self.st.acc.data_ptr(), n, self.s)
        norm, _, _ = B.gro_plan_get_norm(self.plan.handle)
        B.gro_clip_adamw(self.plan.handle, self.st.acc.data_ptr(), n, self.max_norm, self.hp, step,
                         self.st.master.data_ptr(), self.st.m.data_ptr(), self.st.v.data_ptr(),
                         self.st.p_bf16.data_ptr(), self.s)
        return norm

    def by_pid(self):
        """{pid: [master, m, v (float32), p_bf16 (uint16 bits)]} on the host."""
        torch.cuda.synchronize()
        out = {}
        for i, t in enumerate(self.tensors):
            if self.plan.tensors[i]["updated"]:
                a = [self.st.flat_view(x, i).cpu().numpy().copy() for x in (self.st.master, self.st.m, self.st.v)]
                a.append(self.st.flat_view(self.st.p_bf16, i).cpu().view(torch.int16).numpy().view(np.uint16).copy())
                out[int(t.param_id)] = a
        return out


class OracleRun:
    """The oracle on the same parameters, states keyed by param_id between
    windows (so that it, too, can change ownership at a restore)."""

    def __init__(self, tensors, R, hp, max_norm, master_by_pid):
        self.R, self.hp, self.max_norm = R, hp, max_norm
        self.set_tensors(tensors)
        self.state = {pid: [np.asarray(p, np.float32).copy(), np.zeros_like(p), np.zeros_like(p), None]
                      for pid, p in master_by_pid.items()}

    def set_tensors(self, tensors):
        self.tensors = tensors
        self.owners = M.assign_owners(tensors, self.R)

    def step(self, step, grads):
        micro = []
        for gk in grads:
            row = []
            for t, o in zip(self.tensors, self.owners):
                if o.owner == M.EXCLUDED:
                    row.append(None)
                    continue
                g = synth.host_values(gk[int(t.param_id)])
                row.append([g] + [np.zeros_like(g) if t.placement == "partial" else g for _ in range(o.slots - 1)])
            micro.append(row)
        idx = {int(t.param_id): i for i, t in enumerate(self.tensors)}
        take = lambda j: {idx[pid]: st[j] for pid, st in self.state.items() if pid in idx}
        res = M.optimizer_window(self.owners, self.R, micro, take(0), take(1), take(2), self.hp, self.max_norm, step)
        assert res.stepped
        for pid, i in idx.items():
            if i in res.master:
                self.state[pid] = [res.master[i], res.m[i], res.v[i], res.p_bf16[i]]
        return res.norm


def assert_states_equal(got, want, what, with_bf16=True):
    """Bit for bit, per param_id; counts the compared elements."""
    assert got.keys() == want.keys(), what
    n = 0
    for pid in want:
        names = ("master", "m", "v", "p_bf16") if with_bf16 else ("master", "m", "v")
        for j, name in enumerate(names):
            x, y = got[pid][j], want[pid][j]
            if x.dtype == np.float32:
                x, y = x.view(np.uint32), np.asarray(y, np.float32).view(np.uint32)
            diff = int(np.count_nonzero(x != y))
            assert diff == 0, f"{what}: param {pid} {name}: {diff} of {x.size} elements differ"
            n += x.size
    log(f"{what}: {len(want)} parameters, {n} values bit-identical to the oracle")


def check_norm(got, want, what):
    assert abs(got - want) <= FP32_RTOL * abs(want), (what, got, want)


def saved_state(directory, pids):
    """What the checkpoint files hold, read back with safetensors."""
    from safetensors.numpy import load_file
    st = load_file(f"{directory}/state.safetensors")
    return {pid: [st[f"{name}/{pid}"] for name in ("master", "m", "v")] for pid in pids}


def run_legacy_save_restore_native(w, cap_native, windows_before, window_after, tmp_path, seed):
    """Windows under legacy ownership, save, restore into native ownership
    (reversed registration order, bucket capacity cap_native), one window
    after: every stage against the oracle.  Returns the GPU runs."""
    legacy = legacy_of(w.tensors)
    a = Run(legacy, w.R, w.bucket_elems, w.hparams, w.max_norm)
    a.init_master(seed)
    o = OracleRun(legacy, w.R, w.hparams, w.max_norm, {pid: s[0] for pid, s in a.by_pid().items()})
    step = 0
    for n in windows_before:
        step += 1
        grads = a.draw(step, n)
        check_norm(a.step(step, grads), o.step(step, grads), f"legacy window {step}")
    assert_states_equal(a.by_pid(), o.state, f"legacy ownership after {step} windows")
    save_state(a.plan, a.st.master, a.st.m, a.st.v, step=step, directory=str(tmp_path))
    assert_states_equal(saved_state(str(tmp_path), o.state.keys()), o.state, "saved checkpoint", with_bf16=False)

    native = list(reversed(w.tensors))
    b = Run(native, w.R, cap_native, w.hparams, w.max_norm)
    assert b.plan.info["n_buckets"] != a.plan.info["n_buckets"]
    restored = load_state(b.plan, b.st.master, b.st.m, b.st.v, str(tmp_path))
    assert restored == step
    assert_states_equal(b.by_pid(), o.state, "restored into native ownership", with_bf16=False)
    o.set_tensors(native)
    step += 1
    grads = b.draw(step, window_after)
    check_norm(b.step(step, grads), o.step(step, grads), f"native window {step}")
    assert_states_equal(b.by_pid(), o.state, f"native ownership, first update after the restore")
    return a, b, step, grads


def test_restore_into_new_layout_and_ownership_matches_the_oracle(tmp_path):
    w = synth.tiny(literal=True)
    a, b, step, grads = run_legacy_save_restore_native(w, 5000, [2, 3], 4, tmp_path, seed=5)
    # the uninterrupted legacy run takes the same update, bit for bit
    a.step(step, grads)
    ref, got = a.by_pid(), b.by_pid()
    for pid in ref:
        for x, y in zip(ref[pid], got[pid]):
            assert np.array_equal(x.view(np.uint16 if x.dtype == np.uint16 else np.uint32),
                                  y.view(np.uint16 if y.dtype == np.uint16 else np.uint32)), pid
    log("the uninterrupted legacy run takes the same next update")


def test_full_size_draft_67m_save_and_restore(tmp_path):
    """The 67M draft set at full size: one window of 4 under legacy ownership,
    save, restore into native ownership with 4M-element buckets, then one
    more window, each against the oracle on every element."""
    w = synth.draft_67m()
    run_legacy_save_restore_native(w, 4_000_000, [4], 4, tmp_path, seed=6)
