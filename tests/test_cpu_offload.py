"""The host-memory (CPU offload) shard step through the C ABI against the
oracle.  These run on the CPU: the entry points take host pointers."""
import math

import numpy as np
import pytest

import f32model
import oracle
import workloads as W
import zero_sharded_mixed_partition_amd as Z
from zero_sharded_mixed_partition_amd import _lib as L

from parity import check_norm, check_param, compare_step

CODE = {"f16": L.ZERO_F16, "bf16": L.ZERO_BF16, "f32": L.ZERO_F32}
SIZES = [1, 3, 7, 8, 2047, 2048, 2049, 65536, 65537, 200_003]


def _inputs(fmt_g, n, begin):
    w = W.GPT2_SMALL if fmt_g != "bf16" else W.LLAMA_7B
    p, m, v, g = W.shard_inputs(w, begin, n)
    if fmt_g == "f32":
        g = (W.fill(w, "master", begin + 7, n) * np.float32(1e-2)).astype(np.float32)
    return w, p, m, v, g


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("gfmt,pfmt", [("f16", "f16"), ("bf16", "bf16"), ("f32", "bf16"), ("f16", "bf16"),
                                       ("bf16", None)])
def test_cpu_step_matches_oracle(n, gfmt, pfmt):
    w, p, m, v, g = _inputs(gfmt, n, 12345 + n)
    inv = 1.0 if gfmt == "f32" else 1.0 / w.loss_scale
    sq, ovf = Z.zero_cpu_shard_unscale_norm_overflow(g, inv, grad_dtype=CODE[gfmt])
    ref_sq, ref_ovf = oracle.shard_sqnorm_overflow(g, gfmt, inv)
    assert ovf == ref_ovf is False
    check_norm(sq, ref_sq)
    P, M, V = p.copy(), m.copy(), v.copy()
    par = np.zeros(n, np.uint16) if pfmt else None
    hp = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=0.05, max_grad_norm=0.01,
              step=13, inv_loss_scale=inv)
    Z.zero_cpu_shard_adam_step(P, M, V, g, par, Z.AdamHyper(**hp), sq, ovf, grad_dtype=CODE[gfmt],
                               param_dtype=CODE[pfmt] if pfmt else None)
    ref = oracle.shard_step(p, m, v, g, gfmt, pfmt, global_sq=ref_sq, global_overflow=False, **hp)
    compare_step((P, M, V, par), ref)


@pytest.mark.parametrize("n", [1, 15, 16, 17, 2049, 65537 + 33])
@pytest.mark.parametrize("shift", [1, 5, 16])
def test_param_copy_at_any_alignment(n, shift):
    """The 16-bit copy is written with streaming stores from its first
    32-byte boundary on and ordinary stores around it: a copy that starts
    `shift` elements past an aligned address gets the same bits as an aligned
    one, and the elements on either side of it stay untouched."""
    w, p, m, v, g = _inputs("bf16", n, 77 + n)
    hp = Z.AdamHyper(lr=w.lr, weight_decay=0.05, max_grad_norm=0.01, step=5)
    sq, _ = Z.zero_cpu_shard_unscale_norm_overflow(g, 1.0, grad_dtype=L.ZERO_BF16)
    outs = []
    for off in (0, shift):
        buf = np.full(n + 64, 0xABCD, np.uint16)
        base = (-buf.ctypes.data // 2) % 16                 # first 32-byte aligned element of buf
        par = buf[base + off:base + off + n]
        Z.zero_cpu_shard_adam_step(p.copy(), m.copy(), v.copy(), g, par, hp, sq, False, grad_dtype=L.ZERO_BF16,
                                   param_dtype=L.ZERO_BF16)
        assert (buf[:base + off] == 0xABCD).all() and (buf[base + off + n:] == 0xABCD).all()
        outs.append(par.copy())
    assert (outs[0] == outs[1]).all()
    ref = oracle.shard_step(p, m, v, g, "bf16", "bf16", global_sq=sq, global_overflow=False, lr=w.lr, beta1=0.9,
                            beta2=0.999, eps=1e-8, weight_decay=0.05, max_grad_norm=0.01, step=5, inv_loss_scale=1.0)
    check_param("param", outs[1], ref[3], fmt="bf16")


def test_thread_count_does_not_change_results():
    w, p, m, v, g = _inputs("bf16", 1_000_003, 5)
    outs = []
    for t in (1, 3, 8):
        sq, ovf = Z.zero_cpu_shard_unscale_norm_overflow(g, 1.0, grad_dtype=L.ZERO_BF16, nthreads=t)
        P, M, V = p.copy(), m.copy(), v.copy()
        par = np.zeros(g.size, np.uint16)
        Z.zero_cpu_shard_adam_step(P, M, V, g, par, Z.AdamHyper(max_grad_norm=1.0, step=3), sq, ovf,
                                   grad_dtype=L.ZERO_BF16, param_dtype=L.ZERO_BF16, nthreads=t)
        outs.append((sq, P.view(np.uint32), M.view(np.uint32), V.view(np.uint32), par))
    for o in outs[1:]:
        assert o[0] == outs[0][0]
        for a, b in zip(o[1:], outs[0][1:]):
            assert (a == b).all()


@pytest.mark.parametrize("fmt", ["f16", "bf16", "f32"])
def test_overflow_and_skip(fmt):
    w, p, m, v, g = _inputs(fmt, 70_001, 99)
    for pos in (0, 35_000, 70_000):
        h = g.copy()
        if fmt == "f32":
            h[pos] = np.inf
        else:
            h[pos] = W.POS_INF_BITS[fmt]
        sq, ovf = Z.zero_cpu_shard_unscale_norm_overflow(h, 1.0, grad_dtype=CODE[fmt])
        assert ovf and math.isinf(sq)
        P = p.copy()
        par = np.full(h.size, 0x1234, np.uint16)
        Z.zero_cpu_shard_adam_step(P, m.copy(), v.copy(), h, par, Z.AdamHyper(max_grad_norm=1.0), sq, ovf,
                                   grad_dtype=CODE[fmt], param_dtype=L.ZERO_F16)
        assert (P.view(np.uint32) == p.view(np.uint32)).all() and (par == 0x1234).all()


def test_every_fp16_pattern_decodes_and_rounds():
    """All 65536 fp16 patterns through the host norm (decode) and every
    finite fp16 value of a master through the fp16 writeback (encode)."""
    allp = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    fin = allp[~oracle.is_nonfinite16(allp, "f16")]
    sq, ovf = Z.zero_cpu_shard_unscale_norm_overflow(fin, 1.0, grad_dtype=L.ZERO_F16)
    ref, _ = oracle.shard_sqnorm_overflow(fin, "f16", 1.0)
    assert not ovf and abs(sq - ref) <= 1e-15 * ref
    # writeback: with lr = 0 the update leaves the master unchanged, so the
    # parameter copy is the rounding of the given fp32 values
    rng = np.random.default_rng(0)
    x = np.concatenate([oracle.decode16(fin, "f16").astype(np.float32),
                        (rng.standard_normal(100_000) * np.exp(rng.uniform(-20, 12, 100_000))).astype(np.float32)])
    for pfmt in ("f16", "bf16"):
        par = np.zeros(x.size, np.uint16)
        z = np.zeros(x.size, np.float32)
        Z.zero_cpu_shard_adam_step(x.copy(), z.copy(), z.copy(), z.copy(), par, Z.AdamHyper(lr=0.0), 0.0, False,
                                   grad_dtype=L.ZERO_F32, param_dtype=CODE[pfmt])
        assert (par == oracle.encode16_rne(x, pfmt)).all()


def test_cpu_entry_points_reject_bad_arguments():
    a = np.zeros(16, np.float32)
    with pytest.raises(Z.ZeroShardError):
        Z.zero_cpu_shard_unscale_norm_overflow(a, 0.0)
    with pytest.raises(Z.ZeroShardError):
        Z.zero_cpu_shard_unscale_norm_overflow(a, 1.0, grad_dtype=9)
    with pytest.raises(Z.ZeroShardError):
        Z.zero_cpu_shard_adam_step(a, a, a.copy(), np.zeros(16, np.float32), None, Z.AdamHyper(), 0.0, False)
    with pytest.raises(Z.ZeroShardError):
        Z.zero_cpu_shard_adam_step(a, a.copy(), a.copy(), a.copy(), None, Z.AdamHyper(step=0), 0.0, False)
    assert Z.zero_cpu_shard_unscale_norm_overflow(np.zeros(0, np.float32), 1.0) == (0.0, False)


def test_worker_pool_survives_fork():
    """A forked child (which inherits the pool object but none of its
    threads) still completes host calls, on its own thread."""
    import os
    import signal
    g = np.ones(1 << 20, np.float32)
    assert Z.zero_cpu_shard_unscale_norm_overflow(g, 1.0) == (float(1 << 20), False)   # pool started
    pid = os.fork()
    if pid == 0:
        signal.alarm(60)
        ok = Z.zero_cpu_shard_unscale_norm_overflow(g, 1.0) == (float(1 << 20), False)
        os._exit(0 if ok else 1)
    _, status = os.waitpid(pid, 0)
    assert os.WIFEXITED(status) and os.WEXITSTATUS(status) == 0
    assert Z.zero_cpu_shard_unscale_norm_overflow(g, 2.0) == (4.0 * (1 << 20), False)


@pytest.mark.parametrize("gfmt", ["bf16", "f32"])
def test_cpu_step_huge_unclipped_gradients(gfmt):
    """Gradients whose square passes float32's range (|g| up to 4e20, no
    clipping) while (1 - beta2) g^2 does not: the second moment stays finite
    and the step matches the oracle."""
    n = 20_011
    w = W.LLAMA_7B
    p, m, v, _ = W.shard_inputs(w, 777, n)
    rng = np.random.default_rng(99)
    x = rng.normal(0.0, 1e-3, n)
    k = np.arange(0, n, 7)
    x[k] = np.sign(rng.normal(size=k.size)) * 10.0 ** rng.uniform(19.0, np.log10(4e20), k.size)
    g = x.astype(np.float32) if gfmt == "f32" else oracle.encode16_rne(x.astype(np.float32), "bf16")
    sq, ovf = Z.zero_cpu_shard_unscale_norm_overflow(g, 1.0, grad_dtype=CODE[gfmt])
    ref_sq, _ = oracle.shard_sqnorm_overflow(g, gfmt, 1.0)
    check_norm(sq, ref_sq)
    P, M, V = p.copy(), m.copy(), v.copy()
    par = np.zeros(n, np.uint16)
    hp = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=0.01, max_grad_norm=0.0,
              step=5, inv_loss_scale=1.0)
    Z.zero_cpu_shard_adam_step(P, M, V, g, par, Z.AdamHyper(**hp), sq, ovf, grad_dtype=CODE[gfmt],
                               param_dtype=L.ZERO_BF16)
    ref = oracle.shard_step(p, m, v, g, gfmt, "bf16", global_sq=ref_sq, global_overflow=False, **hp)
    assert np.isfinite(V).all()
    compare_step((P, M, V, par), ref)


@pytest.mark.parametrize("nbytes", [0, 4, 12, (1 << 18) - 4, (1 << 18) + 4, 3 * (1 << 20) + 8])
@pytest.mark.parametrize("threads", [1, 3, 0])
def test_host_copy_reference(nbytes, threads):
    """The host copy moves every byte and nothing beyond its range, for any
    thread count (chunks of 2^16 floats)."""
    rng = np.random.default_rng(nbytes + threads)
    src = rng.integers(0, 2**32, size=nbytes // 4 + 8, dtype=np.uint64).astype(np.uint32)
    dst = np.zeros_like(src)
    Z.zero_cpu_copy_reference(dst, src, nbytes, nthreads=threads)
    n = nbytes // 4
    assert (dst[:n] == src[:n]).all() and not dst[n:].any()


def test_host_copy_reference_rejects_bad_arguments():
    lib = Z._L.lib()
    a = np.zeros(64, np.uint32)
    p = a.ctypes.data
    assert lib.zero_cpu_copy_reference(p, p + 128, 6, 0) == Z._L.ZERO_EINVAL          # not a multiple of 4
    assert lib.zero_cpu_copy_reference(p, p + 128, -4, 0) == Z._L.ZERO_EINVAL
    assert lib.zero_cpu_copy_reference(None, p, 4, 0) == Z._L.ZERO_EINVAL
    assert lib.zero_cpu_copy_reference(p, p + 16, 32, 0) == Z._L.ZERO_EINVAL          # overlapping
    assert lib.zero_cpu_copy_reference(p, p + 128, 0, 0) == Z._L.ZERO_OK


@pytest.mark.parametrize("n,chunk", [(1, 1 << 25), (5000, 1024), (1_000_003, 1 << 18), (976_077_312, 1 << 25),
                                     (3 * (1 << 25) + 17, 1 << 25), (1 << 25, 1 << 25), (720_897, 1 << 18)])
def test_offload_chunks_tile_the_shard(n, chunk):
    """The offload pipeline's chunks cover [0, n) in order with no gap or
    overlap; none exceeds `chunk`; on long shards the first and last three
    ramp by doubling (chunk/8, chunk/4, chunk/2, when those are whole
    multiples of 1024 elements)."""
    class Bounds(Z.OffloadShardAdam):
        def __init__(self, n, chunk):                 # the chunking only: no buffers
            self.n, self.chunk = n, max(1024, chunk // 1024 * 1024)

    b = Bounds(n, chunk).chunk_bounds()
    assert b[0][0] == 0 and b[-1][1] == n
    assert all(lo < hi and hi - lo <= chunk for lo, hi in b)
    assert all(x[1] == y[0] for x, y in zip(b, b[1:]))
    sizes = [hi - lo for lo, hi in b]
    if chunk % 8192 == 0 and n > 2 * (chunk // 8 + chunk // 4 + chunk // 2) + chunk:
        ramp = [chunk // 8, chunk // 4, chunk // 2]
        assert sizes[:3] == ramp and sizes[-3:] == ramp[::-1]


@pytest.mark.parametrize("n", [1, 7, 2049, 65537, 200_003])
@pytest.mark.parametrize("gfmt", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("clip", [0.0, 0.01])
def test_cpu_step_equals_the_float32_model(n, gfmt, clip):
    """The host step follows the float32 operation order the header
    documents for the device update, fused multiply-adds included: master,
    m and v equal the model bit for bit (so a host step and a device step
    from the same state agree)."""
    w, p, m, v, g = _inputs(gfmt, n, 999 + n)
    inv = 1.0 if gfmt == "f32" else 1.0 / w.loss_scale
    sq, _ = Z.zero_cpu_shard_unscale_norm_overflow(g, inv, grad_dtype=CODE[gfmt])
    hp = dict(lr=3e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.05, max_grad_norm=clip, step=77,
              inv_loss_scale=inv)
    P, M, V = p.copy(), m.copy(), v.copy()
    Z.zero_cpu_shard_adam_step(P, M, V, g, None, Z.AdamHyper(**hp), sq, False, grad_dtype=CODE[gfmt])
    if gfmt == "f32":
        gv = np.asarray(g, np.float32)
    elif gfmt == "f16":
        gv = g.view(np.float16).astype(np.float32)
    else:
        gv = (g.astype(np.uint32) << 16).view(np.float32)
    for got, want in zip((P, M, V), f32model.adam_update(p, m, v, gv, sq, **hp)):
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
