"""Seeded synthetic inputs as a function of *global* flat position.

Every value depends only on (seed, workload id, array id, step, global index):
the flat index space is cut into fixed chunks of 2**24 elements and chunk c of
array a at step s is drawn from numpy's PCG64 seeded with
SeedSequence([seed, wid, a, s, c]).  Because values are tied to global
positions, the N_d ranks' shards of one workload are slices of one flat
buffer, and any element can be regenerated without drawing the whole shard.

Elements at or beyond the model's real parameter count (the padding tail of
the flat buffer) are zero in every array.

This module draws random numbers and converts them to storage formats; it
computes no step of the optimizer.  16-bit gradients are returned as raw
uint16 bit patterns (fp16 via numpy's cast, bf16 via torch's CPU cast).
"""
from concurrent.futures import ThreadPoolExecutor
import os
from typing import Optional, Tuple

import numpy as np

from .configs import Dist, Workload, real_total

CHUNK = 1 << 24
SEED = 0
ARRAY_IDS = {"master": 0, "exp_avg": 1, "exp_avg_sq": 2, "grad": 3, "inf_pos": 4}


def _rng(wid: int, array: str, step: int, chunk: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([SEED, wid, ARRAY_IDS[array], step, chunk]))


def _draw_f32(dist: Dist, rng: np.random.Generator, n: int, scale: float = 1.0) -> np.ndarray:
    out = np.empty(n, np.float32)
    if dist.kind == "zero":
        out.fill(0.0)
    elif dist.kind == "normal":
        rng.standard_normal(n, dtype=np.float32, out=out)
        np.multiply(out, np.float32(dist.a * scale), out=out)
    elif dist.kind == "uniform":
        rng.random(n, dtype=np.float32, out=out)
        np.multiply(out, np.float32((dist.b - dist.a) * scale), out=out)
        np.add(out, np.float32(dist.a * scale), out=out)
    else:
        raise ValueError(dist.kind)
    return out


def to_bits16(x: np.ndarray, fmt: str) -> np.ndarray:
    """float32 -> raw 16-bit patterns of fp16 ('f16') or bf16 ('bf16')."""
    if fmt == "f16":
        return x.astype(np.float16).view(np.uint16)
    if fmt == "bf16":
        import torch
        return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    raise ValueError(fmt)


def _chunk_values(w: Workload, array: str, step: int, c: int, loss_scale: float) -> np.ndarray:
    """Full chunk c of one array (float32, or uint16 bits for 'grad')."""
    if array == "grad":
        x = _draw_f32(w.grad, _rng(w.wid, "grad", step, c), CHUNK, scale=loss_scale)
        return to_bits16(x, w.grad_dtype)
    dist = {"master": w.master, "exp_avg": w.exp_avg, "exp_avg_sq": w.exp_avg_sq}[array]
    # optimizer state is drawn once (step 0); only gradients change per step
    return _draw_f32(dist, _rng(w.wid, array, 0, c), CHUNK)


def fill(w: Workload, array: str, begin: int, count: int, step: int = 0,
         loss_scale: Optional[float] = None, out: Optional[np.ndarray] = None,
         threads: int = 0) -> np.ndarray:
    """Values of `array` at global flat indices [begin, begin+count).

    array: 'master' | 'exp_avg' | 'exp_avg_sq' (float32) or 'grad' (uint16
    bits of w.grad_dtype).  `step` selects the gradient draw; `loss_scale`
    defaults to the workload's.  Positions >= the real parameter count are 0.
    """
    ls = w.loss_scale if loss_scale is None else loss_scale
    dt = np.uint16 if array == "grad" else np.float32
    if out is None:
        out = np.empty(count, dt)
    assert out.shape == (count,) and out.dtype == dt
    if count == 0:
        return out
    valid_end = real_total(w)
    c0, c1 = begin // CHUNK, (begin + count - 1) // CHUNK

    def one(c: int) -> None:
        lo, hi = max(begin, c * CHUNK), min(begin + count, (c + 1) * CHUNK)
        if lo >= valid_end:
            out[lo - begin:hi - begin] = 0
            return
        vals = _chunk_values(w, array, step, c, ls)
        out[lo - begin:hi - begin] = vals[lo - c * CHUNK:hi - c * CHUNK]
        if hi > valid_end:
            out[valid_end - begin:hi - begin] = 0

    nthreads = threads or min(16, os.cpu_count() or 1)
    if c1 > c0 and nthreads > 1:
        with ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(one, range(c0, c1 + 1)))
    else:
        for c in range(c0, c1 + 1):
            one(c)
    return out


def inf_positions(w: Workload, shard_numel: int, step: int) -> np.ndarray:
    """Shard-relative positions that receive +inf at an injection step:
    floor(inf_fraction * shard_numel) distinct positions, uniform."""
    k = int(w.inf_fraction * shard_numel)
    rng = _rng(w.wid, "inf_pos", step, 0)
    return np.sort(rng.choice(shard_numel, size=k, replace=False))


POS_INF_BITS = {"f16": 0x7C00, "bf16": 0x7F80}


def grad_for_step(w: Workload, begin: int, count: int, iteration: int, loss_scale: float,
                  threads: int = 0) -> np.ndarray:
    """Gradient shard bits for a trajectory iteration (1-based), with +inf
    injected at the workload's injection iterations."""
    g = fill(w, "grad", begin, count, step=iteration, loss_scale=loss_scale, threads=threads)
    if iteration in w.inf_steps:
        g[inf_positions(w, count, iteration)] = POS_INF_BITS[w.grad_dtype]
    return g


def sample_indices(n: int, k: int, seed: int = 1234, edges: int = 8) -> np.ndarray:
    """k sorted distinct shard-relative indices in [0, n) including the first
    and last `edges` positions (ragged tails live there)."""
    if n == 0:
        return np.zeros(0, np.int64)
    rng = np.random.default_rng(seed)
    pick = set(range(min(edges, n))) | set(range(max(0, n - edges), n))
    if k > len(pick):
        pick |= set(rng.integers(0, n, size=k - len(pick)).tolist())
    return np.array(sorted(pick), dtype=np.int64)


def shard_inputs(w: Workload, begin: int, count: int, step: Optional[int] = None,
                 threads: int = 0) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """(master, exp_avg, exp_avg_sq, grad_bits) for one contiguous range; the
    gradient draw defaults to the workload's own step index."""
    step = w.step if step is None else step
    return (fill(w, "master", begin, count, threads=threads),
            fill(w, "exp_avg", begin, count, threads=threads),
            fill(w, "exp_avg_sq", begin, count, threads=threads),
            fill(w, "grad", begin, count, step=step, threads=threads))
