"""Whole-shard comparison with the oracle at full workload sizes: every
element of the updated state is compared, none is sampled.

The host side works through the shard one generator chunk (2^24 elements) at
a time, in a pool of threads: numpy's generators and array loops, and torch's
CPU kernels, release the interpreter lock, so the chunks run in parallel.
Each task draws a chunk's inputs from the seeded generator and runs the
oracle on it; the calling thread moves the inputs and the oracle's results
into device memory as the tasks finish, in order.  After the GPU step, torch
compares the device results with the oracle's results where both already
lie, chunk by chunk, with the bar of `parity` (the same float64 arithmetic
as parity.check_f32, check_param and strict_v), and counts every element
outside it.
"""
from collections import deque
import os
from concurrent.futures import ThreadPoolExecutor


import workloads as W
from parity import ABS, REL

THREADS = max(1, min(16, len(os.sched_getaffinity(0))))
SUB = 1 << 22           # the oracle's step runs on quarter chunks (bounded temporaries)

_pool = None


def pool() -> ThreadPoolExecutor:
    global _pool
    if _pool is None:
        _pool = ThreadPoolExecutor(THREADS, thread_name_prefix="oracle")
    return _pool


def chunk_blocks(begin: int, S: int):
    """Shard-relative ranges [lo, hi) covering [0, S), each inside one
    generator chunk of the global flat index (so no chunk is drawn twice)."""
    out, lo = [], 0
    while lo < S:
        hi = min(S, ((begin + lo) // W.CHUNK + 1) * W.CHUNK - begin)
        out.append((lo, hi))
        lo = hi
    return out


def pmap(fn, items, ahead: int = 0):
    """Yield (item, fn(item)) in order, fn running in the pool with at most
    `ahead` tasks in flight (bounds the host memory held by results)."""
    ahead = ahead or THREADS + 2
    it = iter(items)
    q = deque()
    for x in it:
        q.append((x, pool().submit(fn, x)))
        if len(q) >= ahead:
            break
    while q:
        x, f = q.popleft()
        r = f.result()
        nxt = next(it, None)
        if nxt is not None:
            q.append((nxt, pool().submit(fn, nxt)))
        yield x, r


def by_sub(n: int):
    """[a, b) pieces of at most SUB elements covering [0, n)."""
    return [(a, min(n, a + SUB)) for a in range(0, n, SUB)]


class Tally:
    """Counts elements outside the bar, keeps the worst error and a few
    offending positions (shard-relative)."""

    def __init__(self, name: str):
        self.name, self.n, self.bad, self.worst, self.examples = name, 0, 0, 0.0, []

    def add(self, n: int, bad: int, worst: float, examples):
        self.n += n
        self.bad += bad
        self.worst = max(self.worst, worst)
        if len(self.examples) < 5:
            self.examples += examples[:5 - len(self.examples)]

    def ok(self) -> bool:
        return self.bad == 0

    def __repr__(self):
        extra = f", {self.beyond_ulp} beyond 1 ulp within the value floor" if getattr(self, "beyond_ulp", 0) else ""
        return (f"{self.name}: {self.bad} of {self.n} outside the bar, worst {self.worst:.3g}{extra}"
                + (f", e.g. {self.examples}" if self.examples else ""))


def _examples(bad, got, ref, lo: int):
    import torch
    idx = torch.nonzero(bad).flatten()[:5]
    return [(lo + int(i), float(got[i]), float(ref[i])) for i in idx.tolist()]


def tally_f32(t: Tally, got, ref, lo: int, rel: float = REL, abs_: float = ABS):
    """|got - ref| <= max(rel * |ref|, abs_) for float32 tensors (either
    device); worst = the largest |got - ref| as a fraction of what the bar
    allows there (at most 1 when all pass).  NaN on either side is outside."""
    import torch
    g, r = got.double(), ref.double()
    err = (g - r).abs()
    tol = torch.clamp(r.abs() * rel, min=abs_)
    bad = ~(err <= tol)
    nbad = int(bad.sum())
    worst = float((err / tol).nan_to_num(float("inf")).max()) if err.numel() else 0.0
    t.add(err.numel(), nbad, worst, _examples(bad, got, ref, lo) if nbad else [])


def tally_strict_v(t: Tally, got, ref, lo: int):
    """Second moment: |got - ref| <= 1e-6 * |ref| + 1e-40 (parity.strict_v);
    worst as in tally_f32."""
    g, r = got.double(), ref.double()
    err = (g - r).abs()
    tol = r.abs() * 1e-6 + 1e-40
    bad = ~(err <= tol)
    nbad = int(bad.sum())
    worst = float((err / tol).nan_to_num(float("inf")).max()) if err.numel() else 0.0
    t.add(err.numel(), nbad, worst, _examples(bad, got, ref, lo) if nbad else [])


def _ordered16(b):
    """16-bit float patterns (int16 tensor) -> integers ordered like the values,
    +0 and -0 both 0 (parity.ordered16)."""
    import torch
    x = b.to(torch.int32) & 0xFFFF
    mag = x & 0x7FFF
    return torch.where((x & 0x8000) != 0, -mag, mag)


_TDT16 = {"f16": "float16", "bf16": "bfloat16"}


def _value16(b, fmt):
    import torch
    return b.view(getattr(torch, _TDT16[fmt])).double()


def tally_param(t: Tally, got16, ref16, lo: int, fmt: str, max_ulp: int = 1, abs_: float = ABS):
    """16-bit parameter copies (int16 views of format fmt): at most max_ulp
    apart on the ordered-integer line, or, where they are further apart in
    ulps, at most abs_ apart in value (parity.check_param with fmt).  worst
    is the largest ulp distance; t.beyond_ulp counts the pairs that passed
    by the value floor."""
    d = (_ordered16(got16) - _ordered16(ref16)).abs()
    far = d > max_ulp
    bad = far & ~((_value16(got16, fmt) - _value16(ref16, fmt)).abs() <= abs_)
    nbad = int(bad.sum())
    t.add(d.numel(), nbad, float(d.max()) if d.numel() else 0.0,
          _examples(bad, got16, ref16, lo) if nbad else [])
    t.beyond_ulp = getattr(t, "beyond_ulp", 0) + int(far.sum()) - nbad


def tally_writeback(t: Tally, master, got16, lo: int, fmt: str):
    """The writeback as a property of the device's own results: every 16-bit
    parameter equals the round-to-nearest-even of the float32 master beside
    it, by torch's conversion (bit for bit)."""
    import torch
    want = master.to(getattr(torch, _TDT16[fmt])).view(torch.int16)
    bad = want != got16
    nbad = int(bad.sum())
    t.add(bad.numel(), nbad, float(nbad), _examples(bad, got16, want, lo) if nbad else [])


def tally_ulp_f32(t: Tally, got, ref, lo: int):
    """float32 tensors at most one unit in the last place of ref apart."""
    import torch
    r = ref.abs()
    ulp = (torch.nextafter(r, torch.full_like(r, float("inf"))) - r).double()
    err = (got.double() - ref.double()).abs()
    bad = ~(err <= ulp)
    nbad = int(bad.sum())
    worst = float((err / ulp).max()) if err.numel() else 0.0
    t.add(err.numel(), nbad, worst, _examples(bad, got, ref, lo) if nbad else [])


def assert_all(tallies):
    """Every tally clean and non-empty; tallies whose name says "report only" are
    left out of the check."""
    tallies = [t for t in tallies if "report only" not in t.name]
    bad = [t for t in tallies if not t.ok()]
    assert not bad, "; ".join(repr(t) for t in bad)
    for t in tallies:
        assert t.n > 0, f"{t.name}: nothing compared"
