"""Checkpoint and resume of one rank's optimizer shard.

The shard state is the checkpoint unit of a ZeRO rank: its fp32 master,
exp_avg and exp_avg_sq partitions plus the step scalars (applied steps, loss
scaler).  save() writes them as three .npy files and one JSON file in a
directory; load() restores them into a ShardAdam built over the same shard
size.  Because every step is deterministic, k steps, save, load and k more
steps give the same bits as 2k uninterrupted steps.
"""
import json
import os

import numpy as np
import torch

_ARRAYS = ("master", "exp_avg", "exp_avg_sq")
_SCALER = ("scale", "min_scale", "backoff", "growth", "growth_interval", "good_steps")


def state_dict(opt) -> dict:
    """Host copies of the shard and its scalars (waits for queued steps)."""
    skipped = 0
    if opt.state is not None:
        skipped = opt.read_state().skipped          # refreshes opt.t and opt.scaler
    torch.cuda.current_stream().synchronize()
    d = {k: getattr(opt, k).cpu().numpy() for k in _ARRAYS}
    d["t"] = int(opt.t)
    d["skipped"] = int(skipped)
    d["scaler"] = {k: getattr(opt.scaler.s, k) for k in _SCALER}
    d["hyper"] = dict(opt.hyper)
    return d


def load_state_dict(opt, d: dict) -> None:
    """Restore a state_dict into opt (same shard size and dtypes)."""
    from . import LossScaler, StepState
    for k in _ARRAYS:
        src = np.ascontiguousarray(d[k])
        dst = getattr(opt, k)
        if src.dtype != np.float32 or src.shape != (dst.numel(),):
            raise ValueError(f"{k}: expected float32[{dst.numel()}], got {src.dtype}{list(src.shape)}")
        dst.copy_(torch.from_numpy(src))
    opt.t = int(d["t"])
    opt.scaler = LossScaler(**d["scaler"])
    opt.hyper = dict(d["hyper"])
    if opt.state is not None:
        opt.state = StepState(opt.scaler, opt.t, opt.master.device)
        if d.get("skipped"):
            st = opt.state.read()
            st.skipped = int(d["skipped"])
            opt.state.tensor.copy_(torch.frombuffer(bytearray(bytes(st)), dtype=torch.uint8))
    opt._graph, opt._graph_key = None, None          # recordings refer to the old state buffer
    torch.cuda.current_stream().synchronize()


def save(opt, directory: str) -> None:
    os.makedirs(directory, exist_ok=True)
    d = state_dict(opt)
    for k in _ARRAYS:
        np.save(os.path.join(directory, f"{k}.npy"), d[k])
    meta = {k: d[k] for k in ("t", "skipped", "scaler", "hyper")}
    with open(os.path.join(directory, "scalars.json"), "w") as f:
        json.dump(meta, f, indent=1)


def load(opt, directory: str) -> None:
    d = {k: np.load(os.path.join(directory, f"{k}.npy"), allow_pickle=False) for k in _ARRAYS}
    with open(os.path.join(directory, "scalars.json")) as f:
        d.update(json.load(f))
    load_state_dict(opt, d)
