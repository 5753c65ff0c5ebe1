"""Checkpoint/restore of the owned state on the host (CPU tensors): exact
round trip by param_id across different layouts and placements, manifest
gating, coverage checks."""
import os

import numpy as np
import pytest
import torch

from gradient_reduction_optimizer_amd import synth
from gradient_reduction_optimizer_amd.buffers import Plan
from gradient_reduction_optimizer_amd.checkpoint import CheckpointError, load_state, save_state


def _states(plan, seed):
    g = torch.Generator().manual_seed(seed)
    n = max(plan.info["n_flat"], 1)
    return [torch.randn(n, generator=g) for _ in range(3)]


def _by_pid(plan, arrs):
    out = {}
    for row in plan.tensors:
        if row["updated"]:
            off = row["flat_offset"]
            out[row["param_id"]] = [a[off:off + row["numel"]].clone() for a in arrs] if row["numel"] else \
                [torch.zeros(0)] * 3
    return out


def test_round_trip_into_another_layout(tmp_path):
    w = synth.tiny()
    a = Plan(w.tensors, w.R, w.bucket_elems)
    # registration order reversed and a small bucket capacity: other buckets, other flat offsets
    b = Plan(list(reversed(w.tensors)), w.R, 1000)
    off_a = {r["param_id"]: r["flat_offset"] for r in a.tensors}
    off_b = {r["param_id"]: r["flat_offset"] for r in b.tensors}
    assert off_a != off_b and a.info["n_buckets"] != b.info["n_buckets"]
    sa = _states(a, 1)
    save_state(a, *sa, step=7, directory=str(tmp_path))
    assert os.path.exists(tmp_path / "_SUCCESS")
    sb = [torch.zeros(max(b.info["n_flat"], 1)) for _ in range(3)]
    assert load_state(b, *sb, directory=str(tmp_path)) == 7
    pa, pb = _by_pid(a, sa), _by_pid(b, sb)
    assert pa.keys() == pb.keys()
    for pid in pa:
        for x, y in zip(pa[pid], pb[pid]):
            assert torch.equal(x.view(torch.int32), y.view(torch.int32))


def test_restore_into_new_ownership(tmp_path):
    """Legacy ownership (Q/K norms already reduced by a helper) restored into
    native ownership (Partial): states are keyed by param_id, not placement."""
    w = synth.tiny()
    legacy = [synth.TensorSpec(t.param_id, t.name, t.shape, "reduced" if t.placement == "partial" else t.placement,
                               shard_index=t.shard_index) for t in w.tensors]
    a = Plan(legacy, w.R, w.bucket_elems)
    b = Plan(w.tensors, w.R, w.bucket_elems)
    sa = _states(a, 2)
    save_state(a, *sa, step=3, directory=str(tmp_path))
    sb = [torch.zeros(max(b.info["n_flat"], 1)) for _ in range(3)]
    load_state(b, *sb, directory=str(tmp_path))
    pa, pb = _by_pid(a, sa), _by_pid(b, sb)
    for pid in pa:
        for x, y in zip(pa[pid], pb[pid]):
            assert torch.equal(x, y)


def test_manifest_gates_loading(tmp_path):
    w = synth.tiny()
    a = Plan(w.tensors, w.R, w.bucket_elems)
    sa = _states(a, 3)
    save_state(a, *sa, step=1, directory=str(tmp_path))
    os.remove(tmp_path / "_SUCCESS")
    with pytest.raises(CheckpointError):
        load_state(a, *sa, directory=str(tmp_path))
    # a new save removes a stale manifest before writing anything
    (tmp_path / "_SUCCESS").write_text("stale")
    save_state(a, *sa, step=2, directory=str(tmp_path))
    assert load_state(a, *[torch.zeros_like(x) for x in sa], directory=str(tmp_path)) == 2


def test_coverage_and_size_checks(tmp_path):
    w = synth.tiny()
    a = Plan(w.tensors[:5], w.R, w.bucket_elems)
    save_state(a, *_states(a, 4), step=1, directory=str(tmp_path))
    full = Plan(w.tensors, w.R, w.bucket_elems)
    with pytest.raises(CheckpointError, match="lacks"):
        load_state(full, *_states(full, 5), directory=str(tmp_path))
    grown = [synth.TensorSpec(t.param_id, t.name, (t.numel + 1,), t.placement, shard_index=t.shard_index)
             for t in w.tensors[:5]]
    g = Plan(grown, w.R, w.bucket_elems)
    with pytest.raises(CheckpointError, match="elements"):
        load_state(g, *_states(g, 6), directory=str(tmp_path))
    # frozen parameters are not saved and not required
    fro = [synth.TensorSpec(t.param_id, t.name, t.shape, t.placement, shard_index=t.shard_index,
                            frozen=(i == 0)) for i, t in enumerate(w.tensors[:5])]
    f = Plan(fro, w.R, w.bucket_elems)
    assert load_state(f, *_states(f, 7), directory=str(tmp_path)) == 1


def test_shard_state_restores_only_into_the_same_shard(tmp_path):
    """A Shard parameter's state is that shard's: restoring it into a plan
    that holds another shard index, another R, or the parameter as a
    replicated tensor is refused; ownership changes among Replicate, Partial
    and already-reduced stay allowed (the test above)."""
    w = synth.tiny()
    a = Plan(w.tensors, w.R, w.bucket_elems)
    save_state(a, *_states(a, 8), step=4, directory=str(tmp_path))
    shards = [i for i, t in enumerate(w.tensors) if t.placement == "shard"]
    assert shards

    def with_change(i, **kw):
        t = w.tensors[i]
        f = dict(placement=t.placement, shard_index=t.shard_index)
        f.update(kw)
        return [synth.TensorSpec(u.param_id, u.name, u.shape, f["placement"], shard_index=f["shard_index"])
                if j == i else u for j, u in enumerate(w.tensors)]

    i = shards[0]
    other = (w.tensors[i].shard_index + 1) % w.R
    for tensors, R in ((with_change(i, shard_index=other), w.R),
                       (with_change(i, placement="replicate", shard_index=-1), w.R),
                       (w.tensors, w.R + 1)):
        p = Plan(tensors, R, w.bucket_elems)
        with pytest.raises(CheckpointError):
            load_state(p, *_states(p, 9), directory=str(tmp_path))
    # a replicated tensor saved as such does not restore into a shard either
    j = next(k for k, t in enumerate(w.tensors) if t.placement == "replicate")
    b = Plan(with_change(j, placement="shard", shard_index=0), w.R, w.bucket_elems)
    with pytest.raises(CheckpointError):
        load_state(b, *_states(b, 10), directory=str(tmp_path))
    assert load_state(a, *_states(a, 11), directory=str(tmp_path)) == 4
