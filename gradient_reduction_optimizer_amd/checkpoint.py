"""Checkpoint and restore of the owned optimizer state, keyed by param_id.

What is saved is what the optimizer owns for every updated parameter: the
FP32 master shard, the FP32 Adam moments m and v, and the step count, plus
each parameter's shape and ownership row.  Entries are keyed by the stable
param_id, never by flat offset, so a checkpoint restores into a plan with a
different bucket capacity (a different flat layout) or different placements
(for example a parameter that was "reduced" by an earlier owner and is now
"partial"), as long as every updated param_id has the same number of
elements.  This follows NeMo Automodel issue #3857, "refactor(distributed):
establish shared native TP replica ownership", section "Preserved prototype
and evidence" (restore from legacy ownership into native ownership exactly,
then match the next Adam update) and section "Proposed scope and acceptance
criteria" (checkpoint compatibility, exact restored state, continued
updates); and Mixle "Distributed Transformer Training", section "Optimizer
and checkpoint semantics" (a save counts as complete, and may be loaded,
once its success marker exists).

Layout of a checkpoint directory:
    state.safetensors   master/<param_id>, m/<param_id>, v/<param_id> (FP32)
    meta.json           step, R, per-parameter numel/owner/shard_index/decayed
    _SUCCESS            written last; its presence marks a complete save

A rank-local shard's state belongs to that shard only: a parameter saved or
restored as a Shard must be a Shard on both sides, with the same shard index
and the same R (ownership may change freely among Replicate, Partial and
already-reduced, whose state is the whole parameter's).

This is host plumbing around the plan's layout (torch copies), not part of
the per-step path.  The arrays may live on any torch device.
"""
from __future__ import annotations

import json
import os
import tempfile
from typing import Dict

from . import binding as B

MANIFEST = "_SUCCESS"
STATE_FILE = "state.safetensors"
META_FILE = "meta.json"
FORMAT = "gro-owned-state-v2"


class CheckpointError(RuntimeError):
    pass


def _slice(arr, row):
    off = row["flat_offset"]
    return arr[off:off + row["numel"]]


def save_state(plan, master, m, v, step: int, directory: str) -> None:
    """Write the owned state of every updated parameter of ``plan``.

    ``master``, ``m``, ``v``: flat FP32 torch tensors laid out as the plan
    says.  ``step``: optimizer steps taken so far.  The success manifest is
    written only after the state and metadata files are complete; an
    existing manifest is removed first so that a failed save is never
    mistaken for a complete one.
    """
    import torch
    from safetensors.torch import save_file

    os.makedirs(directory, exist_ok=True)
    manifest = os.path.join(directory, MANIFEST)
    if os.path.exists(manifest):
        os.remove(manifest)
    tensors: Dict[str, "torch.Tensor"] = {}
    params = []
    for i, row in enumerate(plan.tensors):
        if not row["updated"]:
            continue
        pid = int(row["param_id"])
        for name, arr in (("master", master), ("m", m), ("v", v)):
            tensors[f"{name}/{pid}"] = _slice(arr, row).detach().to("cpu", copy=True).contiguous() \
                if row["numel"] else torch.zeros(0, dtype=torch.float32)
        params.append({"param_id": pid, "numel": int(row["numel"]), "owner": B.OWNER_NAMES[row["owner"]],
                       "shard_index": int(plan.shard_index[i]), "decayed": bool(row["decayed"])})
    meta = {"format": FORMAT, "step": int(step), "R": int(plan.R), "params": params}
    for fname, writer in ((STATE_FILE, lambda p: save_file(tensors, p)),
                          (META_FILE, lambda p: open(p, "w").write(json.dumps(meta, indent=1)))):
        fd, tmp = tempfile.mkstemp(dir=directory, prefix=".tmp-")
        os.close(fd)
        writer(tmp)
        os.replace(tmp, os.path.join(directory, fname))
    with open(manifest, "w") as f:
        f.write(json.dumps({"format": FORMAT, "files": [STATE_FILE, META_FILE]}))


def load_state(plan, master, m, v, directory: str) -> int:
    """Restore the owned state into ``plan``'s layout; returns the step.

    Every updated parameter of ``plan`` must be present in the checkpoint
    with the same number of elements; the checkpoint may hold parameters
    the plan does not update (they are ignored).  Raises CheckpointError
    when the manifest is missing or the checkpoint does not cover the plan.
    """
    from safetensors.torch import load_file

    if not os.path.exists(os.path.join(directory, MANIFEST)):
        raise CheckpointError(f"{directory}: no {MANIFEST} manifest, the save did not complete")
    with open(os.path.join(directory, META_FILE)) as f:
        meta = json.load(f)
    if meta.get("format") != FORMAT:
        raise CheckpointError(f"{directory}: unknown format {meta.get('format')!r}")
    saved = {p["param_id"]: p for p in meta["params"]}
    state = load_file(os.path.join(directory, STATE_FILE))
    missing = [int(r["param_id"]) for r in plan.tensors if r["updated"] and int(r["param_id"]) not in saved]
    if missing:
        raise CheckpointError(f"checkpoint lacks updated parameters {missing[:8]}")
    shard = B.OWNER_NAMES[B.GRO_OWNER_LOCAL_SHARD]
    for i, row in enumerate(plan.tensors):
        if not row["updated"]:
            continue
        pid = int(row["param_id"])
        sv = saved[pid]
        if sv["numel"] != row["numel"]:
            raise CheckpointError(f"param_id {pid}: {sv['numel']} elements saved, plan has {row['numel']}")
        owner = B.OWNER_NAMES[row["owner"]]
        if (sv["owner"] == shard) != (owner == shard):
            raise CheckpointError(f"param_id {pid}: saved as {sv['owner']}, the plan owns it as {owner}; "
                                  "a shard's state is not the whole parameter's")
        if owner == shard and (sv["shard_index"] != plan.shard_index[i] or int(meta["R"]) != plan.R):
            raise CheckpointError(f"param_id {pid}: shard {sv['shard_index']} of R={meta['R']} saved, "
                                  f"the plan holds shard {plan.shard_index[i]} of R={plan.R}")
    for row in plan.tensors:
        if not row["updated"] or row["numel"] == 0:
            continue
        pid = int(row["param_id"])
        for name, arr in (("master", master), ("m", m), ("v", v)):
            _slice(arr, row).copy_(state[f"{name}/{pid}"])
    return int(meta["step"])
