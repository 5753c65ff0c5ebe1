"""Random call sequences against the accumulation-window bookkeeping.

A plain Python model of the documented rules (include/gro.h) predicts, for
every call, whether it succeeds or fails and with which error kind; the
library must agree on each of ~3,000 seeded calls -- valid windows, skipped
or repeated microbatches, mixed call styles, a second accumulator, a wrong
window length, clip before norm, rebinding.  Every rejected call is
rejected on the host before any launch; the accepted ones run their
kernels on small buffers."""
import numpy as np
import pytest
import torch

from gradient_reduction_optimizer_amd import binding as B
from gradient_reduction_optimizer_amd import synth
from gradient_reduction_optimizer_amd.buffers import DeviceState, Plan

pytestmark = pytest.mark.gpu

OK, INVALID, STATE = "ok", "invalid", "state"


class Model:
    """The bookkeeping the header documents, per plan."""

    def __init__(self, nb):
        self.nb = nb
        self.bind()

    def bind(self):
        self.norm_valid = False
        self.reset()

    def reset(self):
        self.count = [0] * self.nb
        self.acc = None
        self.norm_done = False
        self.norm_window = 0

    def _other_active(self, b0, b1, acc):
        return self.acc is not None and self.acc != acc and any(
            self.count[b] > 0 for b in range(self.nb) if b < b0 or b >= b1)

    def accumulate(self, b0, b1, k, W, acc):
        if b0 < 0 or b1 < b0 or b1 > self.nb or k < 0 or W < 0 or (W > 0 and k >= W):
            return INVALID
        if b1 == b0:
            return OK
        if k != 0 and any(self.count[b] != k for b in range(b0, b1)):
            return STATE
        if k != 0 and self.acc is not None and self.acc != acc:
            return STATE
        if self._other_active(b0, b1, acc):
            return STATE
        for b in range(b0, b1):
            self.count[b] = k + 1
        self.acc, self.norm_done = acc, False
        return OK

    def window(self, b0, b1, n, acc):
        return self.group(b0, b1, 0, n, n, acc)

    def group(self, b0, b1, k0, n, W, acc):
        if b0 < 0 or b1 < b0 or b1 > self.nb or n < 1 or n > 64 or k0 < 0 or W < 0 or (W > 0 and k0 + n > W):
            return INVALID
        if b1 == b0:
            return OK
        if k0 != 0 and any(self.count[b] != k0 for b in range(b0, b1)):
            return STATE
        if k0 != 0 and self.acc is not None and self.acc != acc:
            return STATE
        if self._other_active(b0, b1, acc):
            return STATE
        for b in range(b0, b1):
            self.count[b] = k0 + n
        self.acc, self.norm_done = acc, False
        return OK

    def reduce_norm(self, W, acc):
        if W < 1:
            return INVALID
        if any(c != W for c in self.count) or (self.nb > 0 and acc != self.acc):
            return STATE
        self.norm_done, self.norm_valid, self.norm_window = True, True, W
        return OK

    def clip(self, W, acc, step):
        if step < 1 or W < 1:
            return INVALID
        if self.nb > 0 and acc != self.acc:
            return STATE
        if not self.norm_done or self.norm_window != W:
            return STATE
        self.reset()
        return OK

    def get_norm(self):
        return OK if self.norm_valid else STATE


def outcome(fn):
    try:
        fn()
        return OK
    except B.GroError as e:
        return e.kind


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_random_call_sequences_follow_the_documented_rules(gpu, seed):
    w = synth.tiny(bucket_elems=4096)
    plan = Plan(w.tensors, w.R, w.bucket_elems)
    st = DeviceState(plan, "cuda")
    s = torch.cuda.current_stream().cuda_stream
    nb = plan.info["n_buckets"]
    assert nb >= 4
    sets = [st.grad_buffers() for _ in range(4)]         # up to 4 resident microbatches
    accs = [st.acc, torch.zeros_like(st.acc)]
    ws = torch.zeros(int(plan.info["workspace_bytes"]) + 256, dtype=torch.uint8, device="cuda")
    ws_ptr = (ws.data_ptr() + 255) // 256 * 256
    model = Model(nb)
    rng = np.random.default_rng(100 + seed)
    counts = {}
    step = 1
    W_cur = 2
    for i in range(1000):
        op = str(rng.choice(["acc", "acc", "acc", "win", "grp", "grp", "norm", "norm", "clip", "clip", "get", "bind"]))
        a = int(rng.choice([0, 0, 0, 1]))                  # mostly the same accumulator
        acc = accs[a].data_ptr()
        W = int(rng.choice([1, 2, 3, 4]))
        if rng.random() < 0.6:
            # the next call of a well-formed window, so that whole windows complete
            a, acc, W = 0, accs[0].data_ptr(), W_cur
            if model.norm_done:
                op = "clip"
            elif all(c == W for c in model.count):
                op = "norm"
            else:
                op = "acc" if rng.random() < 0.6 else "grp"
        if op == "clip" and rng.random() < 0.5:
            W_cur = int(rng.choice([1, 2, 3, 4]))
        if op in ("acc", "win", "grp"):
            b0 = int(rng.integers(-1, nb + 1)) if rng.random() < 0.05 else int(rng.integers(0, nb))
            b1 = b0 + int(rng.integers(0, nb - max(b0, 0) + 1)) if b0 >= 0 else nb
            if rng.random() < 0.1:
                b0, b1 = 0, nb
            if rng.random() < 0.03:
                b1 = nb + 1
            span = max(b1 - b0, 0)
            if op == "acc":
                if W == W_cur and a == 0 and rng.random() < 0.7:
                    b0, b1 = 0, nb                          # the whole plan, next microbatch
                k = int(rng.choice([0, 1, 2, 3, -1])) if rng.random() < 0.2 else min(
                    model.count[max(min(b0, nb - 1), 0)], W - 1)
                ptrs = [sets[0][min(max(b, 0), nb - 1)].data_ptr() for b in range(b0, b1)]
                want = model.accumulate(b0, b1, k, W, a)
                got = outcome(lambda: B.gro_accumulate(plan.handle, b0, b1, ptrs, acc, k, W, s))
            elif op == "grp":
                if W == W_cur and a == 0 and rng.random() < 0.7:
                    b0, b1 = 0, nb
                k0 = int(rng.choice([0, 1, 2, 3, -1])) if rng.random() < 0.2 else min(
                    model.count[max(min(b0, nb - 1), 0)], W - 1)
                n = int(rng.integers(1, 4)) if rng.random() < 0.9 else int(rng.choice([0, 65]))
                Wg = W if rng.random() < 0.9 else 0
                ptrs = [sets[(k0 + kk) % 4][min(max(b, 0), nb - 1)].data_ptr()
                        for kk in range(n if 1 <= n <= 64 else 1) for b in range(b0, b1)]
                want = model.group(b0, b1, k0, n, Wg, a)
                got = outcome(lambda: B.gro_accumulate_microbatches(plan.handle, b0, b1, ptrs, k0, n, Wg, acc, s))
            else:
                n = int(rng.choice([1, 2, 3, 4, 0, 65])) if rng.random() < 0.1 else W
                ptrs = [sets[kk % 4][min(max(b, 0), nb - 1)].data_ptr() for kk in range(max(n, 0) if n <= 64 else 1)
                        for b in range(b0, b1)]
                if n > 64 or n < 1:
                    ptrs = ptrs or [sets[0][0].data_ptr()] * max(span, 1)
                want = model.window(b0, b1, n, a)
                got = outcome(lambda: B.gro_accumulate_window(plan.handle, b0, b1, ptrs, n, acc, s))
        elif op == "norm":
            Wn = W if rng.random() < 0.8 else int(rng.choice([0, 5]))
            want = model.reduce_norm(Wn, a)
            got = outcome(lambda: B.gro_reduce_norm(plan.handle, acc, Wn, s))
        elif op == "clip":
            t = step if rng.random() < 0.95 else 0
            Wc = model.norm_window if (model.norm_done and rng.random() < 0.8) else W
            want = model.clip(Wc, a, t)
            got = outcome(lambda: B.gro_clip_adamw(plan.handle, acc, Wc, 1.0, w.hparams, t, st.master.data_ptr(),
                                                   st.m.data_ptr(), st.v.data_ptr(), st.p_bf16.data_ptr(), s))
            if got == OK:
                step += 1
        elif op == "get":
            want = model.get_norm()
            got = outcome(lambda: B.gro_plan_get_norm(plan.handle))
        else:
            model.bind()
            target = ws_ptr if rng.random() < 0.5 else st.ws_ptr
            want = OK
            got = outcome(lambda: B.gro_plan_bind(plan.handle, target, int(plan.info["workspace_bytes"]), s))
        assert got == want, (i, op, got, want, B.gro_last_error())
        counts[(op, got)] = counts.get((op, got), 0) + 1
    torch.cuda.synchronize()
    print(sorted(counts.items()))
    # the walk exercised both outcomes of the main calls
    for op in ("acc", "grp", "norm", "clip"):
        assert counts.get((op, OK), 0) > 10 and counts.get((op, STATE), 0) > 10, (op, counts)
