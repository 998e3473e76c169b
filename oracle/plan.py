"""Flat-buffer partition plan (oracle).

[ZeRO method entry, description]: the model states are partitioned across the
data-parallel processes instead of replicated.  [Explainer, History, "ZeRO"
entry and "The 16 Bytes per Parameter Audit"]: each rank owns a partition and
the ranks gather what they need.  The pages do not fix a layout; the reading
taken here is the plainest one:

  * tensors are laid end to end in list order, with no gaps between them;
  * the flat buffer is padded at the end only, to the smallest multiple of
    N_d * align that holds every parameter;
  * the padded buffer is cut into N_d equal consecutive partitions of
    S = align * ceil(T / (N_d * align)) elements; rank r owns [r*S, (r+1)*S).

All arithmetic is on Python integers (no overflow).
"""
from typing import List, Sequence, Tuple


def _numel(shape: Sequence[int]) -> int:
    n = 1
    for d in shape:
        if int(d) < 0:
            raise ValueError("negative dimension")
        n *= int(d)
    return n


def partition_plan(shapes: Sequence[Sequence[int]], n_d: int, align: int) -> Tuple[List[int], int, int]:
    """Return (tensor_offsets, S, padded_total).

    tensor_offsets[i] is where tensor i starts in the flat buffer; S is the
    per-rank partition size; padded_total = N_d * S.
    """
    if n_d < 1 or align < 1:
        raise ValueError("n_d and align must be >= 1")
    offsets, off = [], 0
    for shape in shapes:
        offsets.append(off)
        off += _numel(shape)
    total = off
    unit = n_d * align
    units = -(-total // unit)          # ceil(T / (N_d * align))
    S = units * align
    return offsets, S, n_d * S


def rank_range(shapes: Sequence[Sequence[int]], n_d: int, align: int, rank: int) -> Tuple[int, int]:
    """[begin, end) of rank's partition in the flat buffer."""
    if not 0 <= rank < n_d:
        raise ValueError("rank out of range")
    _, S, _ = partition_plan(shapes, n_d, align)
    return rank * S, (rank + 1) * S


def rank_fragments(shapes: Sequence[Sequence[int]], n_d: int, align: int,
                   rank: int) -> List[Tuple[int, int, int, int]]:
    """Nonempty intersections of each tensor with rank's partition.

    Each fragment is (tensor index, first element within the tensor, first
    element within the shard, element count), in list order.
    """
    offsets, S, _ = partition_plan(shapes, n_d, align)
    lo, hi = rank * S, (rank + 1) * S
    if not 0 <= rank < n_d:
        raise ValueError("rank out of range")
    frags = []
    for i, shape in enumerate(shapes):
        t_lo, t_hi = offsets[i], offsets[i] + _numel(shape)
        a, b = max(lo, t_lo), min(hi, t_hi)
        if a < b:
            frags.append((i, a - t_lo, a - lo, b - a))
    return frags
