"""Host-side tests of the C-ABI library (no GPU): it loads, exports every
function include/*.h declares, and its host logic (partition plan, rank
fragments, loss scaler, argument validation) agrees bit-exactly with the
oracle.  No device compute entry point is executed with valid arguments here;
the device entry points are only called with arguments the host validation
rejects before anything is enqueued."""
import ctypes
import glob
import os
import random
import re
import subprocess

import pytest

import oracle
import workloads as W
import zero_sharded_mixed_partition_amd as Z
from zero_sharded_mixed_partition_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"^[A-Za-z_][\w \*]*?\b(zero_\w+)\s*\(", text, flags=re.M))
    return names


def test_library_exports_every_declared_symbol():
    declared = _declared_functions()
    assert len(declared) >= 9
    lib = L.lib()
    for name in declared:
        assert hasattr(lib, name), name
    assert declared == set(L.SIGNATURES), "binding signatures out of sync with the header"
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (zero_\w+)", out))
    assert declared <= exported


def test_abi_version():
    assert Z.zero_abi_version() == 1


@pytest.mark.parametrize("seed", range(30))
def test_plan_matches_oracle_random(seed):
    rng = random.Random(seed)
    shapes = [tuple(rng.randint(0, 50) for _ in range(rng.randint(0, 3))) for _ in range(rng.randint(0, 12))]
    for n_d in (1, 2, 3, 8, 13):
        for align in (1, 4, 128):
            assert Z.zero_partition_plan(shapes, n_d, align) == oracle.partition_plan(shapes, n_d, align)
            for r in range(n_d):
                assert Z.zero_rank_fragments(shapes, n_d, align, r) == oracle.rank_fragments(shapes, n_d, align, r)


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_plan_matches_oracle_workloads(name):
    w = W.get(name)
    assert Z.zero_partition_plan(w.shapes, w.n_d, w.align) == oracle.partition_plan(w.shapes, w.n_d, w.align)
    for r in sorted({0, w.rank, w.n_d - 1}):
        assert Z.zero_rank_fragments(w.shapes, w.n_d, w.align, r) == oracle.rank_fragments(w.shapes, w.n_d, w.align, r)


def test_plan_errors():
    with pytest.raises(Z.ZeroShardError) as e:
        Z.zero_partition_plan([(4,)], 0, 1)
    assert e.value.status == L.ZERO_EINVAL
    with pytest.raises(Z.ZeroShardError) as e:
        Z.zero_partition_plan([(4,)], 1, 0)
    assert e.value.status == L.ZERO_EINVAL
    with pytest.raises(Z.ZeroShardError) as e:
        Z.zero_partition_plan([(-1, 3)], 2, 1)
    assert e.value.status == L.ZERO_EINVAL
    with pytest.raises(Z.ZeroShardError) as e:
        Z.zero_partition_plan([(1 << 40, 1 << 40)], 2, 1)
    assert e.value.status == L.ZERO_ERANGE
    with pytest.raises(Z.ZeroShardError) as e:
        Z.zero_partition_plan([(1 << 62,), (1 << 62,)], 1, 1)
    assert e.value.status == L.ZERO_ERANGE
    with pytest.raises(Z.ZeroShardError) as e:
        Z.zero_partition_plan([(8,)], 1 << 30, 1 << 40)
    assert e.value.status == L.ZERO_ERANGE
    with pytest.raises(Z.ZeroShardError) as e:
        Z.zero_rank_fragments([(8,)], 2, 1, 2)
    assert e.value.status == L.ZERO_EINVAL


def test_fragments_enospc_reports_count():
    dims = (ctypes.c_int64 * 3)(10, 10, 10)
    ndims = (ctypes.c_int32 * 3)(1, 1, 1)
    count = ctypes.c_int32()
    buf = (L.zero_fragment * 1)()
    st = L.lib().zero_rank_fragments(dims, ndims, 3, 1, 1, 0, buf, 1, ctypes.byref(count))
    assert st == L.ZERO_ENOSPC and count.value == 3 and buf[0].numel == 10


def test_edge_plans():
    assert Z.zero_partition_plan([], 4, 128) == ([], 0, 0)
    assert Z.zero_rank_fragments([], 4, 128, 3) == []
    assert Z.zero_partition_plan([()], 3, 1) == ([0], 1, 3)
    assert Z.zero_rank_fragments([()], 3, 1, 2) == []


def test_loss_scaler_matches_oracle():
    rng = random.Random(5)
    ours = Z.LossScaler(scale=65536.0, growth_interval=7)
    ref = oracle.LossScalerState(scale=65536.0, growth_interval=7)
    for _ in range(500):
        ovf = rng.random() < 0.1
        skip = Z.zero_loss_scaler_update(ours, ovf)
        ref, rskip = oracle.loss_scaler_update(ref, ovf)
        assert skip == rskip and ours.scale == ref.scale and ours.good_steps == ref.good_steps


def test_loss_scaler_invalid():
    with pytest.raises(Z.ZeroShardError):
        Z.zero_loss_scaler_update(Z.LossScaler(scale=0.0), False)
    with pytest.raises(Z.ZeroShardError):
        Z.zero_loss_scaler_update(Z.LossScaler(growth_interval=0), False)


def test_device_entry_points_reject_bad_arguments_on_host():
    """Arguments the host-side validation rejects: nothing reaches the GPU."""
    lib = L.lib()
    hp = L.zero_adam_params(1e-3, 0.9, 0.999, 1e-8, 0.0, 1, 1.0, 0.0)
    buf = ctypes.create_string_buffer(64)
    aligned = (ctypes.addressof(buf) + 15) & ~15
    # bad dtype / negative n / null pointers / bad hyperparameters / misalignment
    # every call below must be rejected by host validation (never a launch on
    # these host pointers): 7 is not a format code
    assert lib.zero_shard_unscale_norm_overflow(aligned, 7, 8, 1.0, aligned, aligned, aligned, 1 << 20, None) == L.ZERO_EINVAL
    assert lib.zero_shard_unscale_norm_overflow(aligned, 1, -1, 1.0, aligned, aligned, aligned, 1 << 20, None) == L.ZERO_EINVAL
    assert lib.zero_shard_unscale_norm_overflow(aligned, 1, 8, 0.0, aligned, aligned, aligned, 1 << 20, None) == L.ZERO_EINVAL
    assert lib.zero_shard_unscale_norm_overflow(aligned + 2, 1, 8, 1.0, aligned, aligned, aligned, 1 << 20, None) == L.ZERO_EALIGN
    assert lib.zero_shard_unscale_norm_overflow(aligned, 1, 8, 1.0, aligned, aligned, aligned, 0, None) == L.ZERO_ENOSPC
    A = ctypes.byref(hp)
    assert lib.zero_shard_adam_step(None, None, None, None, 1, None, 0, 8, A, None, None, None) == L.ZERO_EINVAL
    assert lib.zero_shard_adam_step(aligned, aligned, aligned, aligned, 7, None, 0, 8, A, None, None, None) == L.ZERO_EINVAL
    bad = [L.zero_adam_params(1e-3, 1.0, 0.999, 1e-8, 0.0, 1, 1.0, 0.0),
           L.zero_adam_params(1e-3, 0.9, 0.999, 1e-8, 0.0, 0, 1.0, 0.0),
           L.zero_adam_params(-1.0, 0.9, 0.999, 1e-8, 0.0, 1, 1.0, 0.0),
           L.zero_adam_params(1e-3, 0.9, 0.999, 1e-8, 0.0, 1, 0.0, 0.0),
           L.zero_adam_params(1e-3, 0.9, 0.999, 1e-8, 0.0, 1, 1.0, 1.0)]   # clip without d_global_sqnorm
    for b in bad:
        assert lib.zero_shard_adam_step(aligned, aligned + 16, aligned + 32, aligned + 48, 1, None, 0, 4,
                                        ctypes.byref(b), None, None, None) == L.ZERO_EINVAL
    assert lib.zero_shard_adam_step(aligned + 4, aligned + 16, aligned + 32, aligned + 48, 1, None, 0, 4, A,
                                    None, None, None) == L.ZERO_EALIGN
    # grad aliasing master
    assert lib.zero_shard_adam_step(aligned, aligned + 16, aligned + 32, aligned, 1, None, 0, 4, A,
                                    None, None, None) == L.ZERO_EINVAL
    # n == 0 is a no-op that needs no pointers
    assert lib.zero_shard_adam_step(None, None, None, None, 1, None, 0, 0, A, None, None, None) == L.ZERO_OK
    # gradient accumulation: fp32 input, bad sizes/scales, misalignment, aliasing
    acc = lib.zero_shard_grad_accumulate
    assert acc(aligned, aligned + 16, L.ZERO_F32, 4, 1.0, 1, None, None) == L.ZERO_EINVAL
    assert acc(aligned, aligned + 16, 7, 4, 1.0, 1, None, None) == L.ZERO_EINVAL
    assert acc(aligned, aligned + 16, L.ZERO_F16, -1, 1.0, 1, None, None) == L.ZERO_EINVAL
    assert acc(aligned, aligned + 16, L.ZERO_F16, 4, float("inf"), 1, None, None) == L.ZERO_EINVAL
    assert acc(aligned + 4, aligned + 16, L.ZERO_F16, 4, 1.0, 1, None, None) == L.ZERO_EALIGN
    assert acc(aligned, aligned + 16, L.ZERO_F16, 4, 1.0, 1, aligned + 2, None) == L.ZERO_EALIGN
    assert acc(aligned, aligned + 8 - 8, L.ZERO_BF16, 4, 1.0, 0, None, None) == L.ZERO_EINVAL   # alias
    assert acc(None, None, L.ZERO_F16, 0, 1.0, 1, None, None) == L.ZERO_OK                       # n == 0
    assert L.lib().zero_last_error() == b""


def test_workspace_size():
    assert Z.zero_norm_workspace_bytes(0) >= 12
    assert Z.zero_norm_workspace_bytes(-1) == 0
    assert Z.zero_norm_workspace_bytes(1 << 40) <= 2048 * 12 + 256
    assert Z.zero_norm_workspace_bytes(10**6) % 256 == 0


def test_coefficient_block_is_the_fp64_formulas_rounded_once():
    """zero_adam_prepare: each per-step coefficient is its float64 formula
    rounded once to float32 (lr/(1-b1^t), 1/sqrt(1-b2^t), 1-b, 1-lr*wd)."""
    import struct

    import numpy as np
    assert Z.zero_adam_coef_bytes() == struct.calcsize("<9fi2d")
    for (lr, b1, b2, eps, wd, t, inv, mx) in [(1e-3, 0.9, 0.999, 1e-8, 0.1, 1, 2.0**-16, 1.0),
                                             (3e-4, 0.95, 0.98, 1e-6, 0.0, 10000, 1.0, 0.0),
                                             (1e-2, 0.0, 0.0, 0.0, 0.5, 7, 0.25, 2.5)]:
        buf = np.zeros(Z.zero_adam_coef_bytes(), np.uint8)
        Z.zero_adam_prepare(Z.AdamHyper(lr=lr, beta1=b1, beta2=b2, eps=eps, weight_decay=wd, step=t,
                                        inv_loss_scale=inv, max_grad_norm=mx), buf)
        got = struct.unpack("<9fi2d", buf.tobytes())
        f32 = lambda x: float(np.float32(x))  # noqa: E731
        want = (f32(b1), f32(1 - b1), f32(b2), f32(1 - b2), f32(lr / (1 - b1 ** t)), f32(1 / (1 - b2 ** t) ** 0.5),
                f32(eps), f32(1 - lr * wd), f32(inv), int(mx > 0), inv, mx if mx > 0 else 0.0)
        assert got == want


def test_graph_and_coef_entry_points_reject_bad_arguments_on_host():
    """Rejected before anything is allocated, recorded or launched."""
    lib = L.lib()
    bad = L.zero_adam_params(1e-3, 1.5, 0.999, 1e-8, 0.0, 1, 1.0, 0.0)
    good = L.zero_adam_params(1e-3, 0.9, 0.999, 1e-8, 0.0, 1, 1.0, 0.0)
    out = ctypes.create_string_buffer(64)
    assert lib.zero_adam_prepare(ctypes.byref(bad), out) == L.ZERO_EINVAL
    assert lib.zero_adam_prepare(ctypes.byref(good), None) == L.ZERO_EINVAL
    buf = ctypes.create_string_buffer(256)
    al = (ctypes.addressof(buf) + 15) & ~15
    step_coef = lib.zero_shard_adam_step_coef
    assert step_coef(al, al + 16, al + 32, al + 48, 1, None, 0, 4, None, al + 64, None, None) == L.ZERO_EINVAL
    assert step_coef(al, al + 16, al + 32, al + 48, 1, None, 0, 4, al + 96, None, None, None) == L.ZERO_EINVAL
    assert step_coef(al, al + 16, al + 32, al + 48, 7, None, 0, 4, al + 96, al + 64, None, None) == L.ZERO_EINVAL
    h = ctypes.c_void_p()
    create = lib.zero_step_graph_create
    assert create(None, al, al + 16, al + 32, al + 48, 1, None, 0, 4, 1.0, al + 64, al + 72, al + 128, 1024) == L.ZERO_EINVAL
    assert create(ctypes.byref(h), al, al + 16, al + 32, al + 48, 1, None, 0, 4, 0.0, al + 64, al + 72, al + 128,
                  1024) == L.ZERO_EINVAL
    assert create(ctypes.byref(h), al, al + 16, al + 32, al + 48, 1, None, 0, 4, 1.0, al + 64, al + 72, al + 128,
                  0) == L.ZERO_ENOSPC
    assert create(ctypes.byref(h), al, al, al + 32, al + 48, 1, None, 0, 4, 1.0, al + 64, al + 72, al + 128,
                  1024) == L.ZERO_EINVAL                                   # master aliases exp_avg
    assert h.value is None
    assert lib.zero_step_graph_launch(None, ctypes.byref(good), None) == L.ZERO_EINVAL
    assert lib.zero_step_graph_overflow(None, None) == L.ZERO_EINVAL
    assert lib.zero_step_graph_destroy(None) == L.ZERO_OK


def test_copy_reference_rejects_bad_arguments_on_host():
    lib = L.lib()
    buf = ctypes.create_string_buffer(256)
    al = (ctypes.addressof(buf) + 15) & ~15
    cp = lib.zero_copy_reference
    assert cp(al, al + 64, 0, None) == L.ZERO_OK                    # empty: nothing launched
    assert cp(al, al + 64, 24, None) == L.ZERO_EINVAL               # not a multiple of 16
    assert cp(al, al + 64, -16, None) == L.ZERO_EINVAL
    assert cp(None, al, 16, None) == L.ZERO_EINVAL
    assert cp(al + 8, al + 64, 16, None) == L.ZERO_EALIGN
    assert cp(al, al + 16, 32, None) == L.ZERO_EINVAL               # overlapping
    assert cp(al, al + 64, 1 << 60, None) == L.ZERO_EINVAL           # overlapping (any size is accepted)
    wc = lib.zero_copy_widen_reference
    assert wc(al, al + 128, 0, None) == L.ZERO_OK                   # empty: nothing launched
    assert wc(al, al + 128, 12, None) == L.ZERO_EINVAL              # not a multiple of 8
    assert wc(al, al + 128, -8, None) == L.ZERO_EINVAL
    assert wc(None, al, 8, None) == L.ZERO_EINVAL
    assert wc(al + 8, al + 128, 8, None) == L.ZERO_EALIGN
    assert wc(al, al + 16, 16, None) == L.ZERO_EINVAL               # dst [al, al+32) overlaps src [al+16, al+32)
    assert wc(al, al + 64, 1 << 62, None) == L.ZERO_ERANGE          # 2 * src_bytes overflows


def test_reduce_rejects_bad_arguments_on_host():
    lib = L.lib()
    buf = ctypes.create_string_buffer(1024)
    al = (ctypes.addressof(buf) + 15) & ~15
    red = lib.zero_shard_grad_reduce

    def ptrs(*a):
        return (ctypes.c_void_p * len(a))(*a)

    two = ptrs(al + 256, al + 512)
    assert red(al, two, 2, L.ZERO_F16, 0, 1.0, None, None) == L.ZERO_OK             # n = 0: nothing launched
    assert red(al, two, 0, L.ZERO_F16, 8, 1.0, None, None) == L.ZERO_EINVAL
    assert red(al, ptrs(*([al + 256] * 17)), 17, L.ZERO_F16, 8, 1.0, None, None) == L.ZERO_EINVAL
    assert red(al, two, 2, L.ZERO_F32, 8, 1.0, None, None) == L.ZERO_EINVAL         # 16-bit slices only
    assert red(al, two, 2, L.ZERO_F16, -1, 1.0, None, None) == L.ZERO_EINVAL
    assert red(al, two, 2, L.ZERO_F16, 8, 0.0, None, None) == L.ZERO_EINVAL
    assert red(al, None, 2, L.ZERO_F16, 8, 1.0, None, None) == L.ZERO_EINVAL
    assert red(al, ptrs(al + 256, None), 2, L.ZERO_F16, 8, 1.0, None, None) == L.ZERO_EINVAL
    assert red(al, ptrs(al + 256, al + 520), 2, L.ZERO_F16, 8, 1.0, None, None) == L.ZERO_EALIGN
    assert red(al + 4, two, 2, L.ZERO_F16, 8, 1.0, None, None) == L.ZERO_EALIGN
    assert red(al, ptrs(al + 256, al + 16), 2, L.ZERO_F16, 8, 1.0, None, None) == L.ZERO_EINVAL   # acc aliases


def test_device_state_calls_reject_bad_arguments_on_host():
    lib = L.lib()
    buf = ctypes.create_string_buffer(1024)
    al = (ctypes.addressof(buf) + 15) & ~15
    hp = L.zero_adam_hyper(1e-3, 0.9, 0.999, 1e-8, 0.0, 1.0)
    bad = L.zero_adam_hyper(1e-3, 1.0, 0.999, 1e-8, 0.0, 1.0)
    step = lib.zero_shard_adam_step_dev
    args = (al, al + 64, al + 128, al + 192, L.ZERO_F16, None, 0, 4)
    assert step(*args, ctypes.byref(hp), None, al + 256, al + 264, al + 320, None) == L.ZERO_EINVAL        # state
    assert step(*args, ctypes.byref(hp), al + 4, al + 256, al + 264, al + 320, None) == L.ZERO_EALIGN      # state
    assert step(*args, ctypes.byref(hp), al + 512, al + 256, None, al + 320, None) == L.ZERO_EINVAL        # flag
    assert step(*args, ctypes.byref(hp), al + 512, None, al + 264, al + 320, None) == L.ZERO_EINVAL        # clip
    assert step(*args, ctypes.byref(hp), al + 512, al + 256, al + 264, None, None) == L.ZERO_EINVAL        # coef
    assert step(*args, ctypes.byref(bad), al + 512, al + 256, al + 264, al + 320, None) == L.ZERO_EINVAL   # beta
    assert step(*args, None, al + 512, al + 256, al + 264, al + 320, None) == L.ZERO_EINVAL
    norm = lib.zero_shard_unscale_norm_overflow_dev
    assert norm(al, L.ZERO_F16, 8, None, al + 256, al + 264, al + 320, 1024, None) == L.ZERO_EINVAL
    assert norm(al, L.ZERO_F16, 8, al + 2, al + 256, al + 264, al + 320, 1024, None) == L.ZERO_EALIGN
    acc = lib.zero_shard_grad_accumulate_dev
    assert acc(al, al + 256, L.ZERO_F16, 8, None, 1, None, None) == L.ZERO_EINVAL
    red = lib.zero_shard_grad_reduce_dev
    two = (ctypes.c_void_p * 2)(al + 256, al + 512)
    assert red(al, two, 2, L.ZERO_F16, 8, None, None, None) == L.ZERO_EINVAL


def test_coefficients_use_binary_exponentiation():
    """beta^t is taken by binary exponentiation in float64 (the same IEEE
    multiplications on host and device); over a sweep the block equals that
    formula bit for bit, and differs from a library pow by at most one float32
    rounding boundary (never observed in the sweep)."""
    import struct

    import numpy as np

    def pow_int(b, e):
        r = 1.0
        while e > 0:
            if e & 1:
                r = r * b
            b = b * b
            e >>= 1
        return r

    f32 = lambda x: float(np.float32(x))  # noqa: E731
    rng = np.random.default_rng(5)
    for _ in range(300):
        b1, b2 = float(rng.uniform(0, 0.9999)), float(rng.uniform(0, 0.99999))
        t = int(rng.integers(1, 10**6))
        lr = float(rng.uniform(1e-5, 1e-2))
        buf = np.zeros(Z.zero_adam_coef_bytes(), np.uint8)
        Z.zero_adam_prepare(Z.AdamHyper(lr=lr, beta1=b1, beta2=b2, eps=1e-8, weight_decay=0.0, step=t,
                                        inv_loss_scale=1.0, max_grad_norm=0.0), buf)
        got = struct.unpack("<9fi2d", buf.tobytes())
        assert got[4] == f32(lr / (1 - pow_int(b1, t)))
        assert got[5] == f32(1 / (1 - pow_int(b2, t)) ** 0.5)
        assert got[4] == f32(lr / (1 - b1 ** t)) and got[5] == f32(1 / (1 - b2 ** t) ** 0.5)


def test_decide_rejects_bad_arguments_on_host():
    lib = L.lib()
    buf = ctypes.create_string_buffer(1024)
    al = (ctypes.addressof(buf) + 15) & ~15
    hp = L.zero_adam_hyper(1e-3, 0.9, 0.999, 1e-8, 0.0, 1.0)
    dec = lib.zero_step_decide_dev
    assert dec(None, L.ZERO_F16, al, al + 256, al + 320, None) == L.ZERO_EINVAL
    assert dec(ctypes.byref(hp), 7, al, al + 256, al + 320, None) == L.ZERO_EINVAL
    assert dec(ctypes.byref(hp), L.ZERO_F16, None, al + 256, al + 320, None) == L.ZERO_EINVAL
    assert dec(ctypes.byref(hp), L.ZERO_F16, al, None, al + 320, None) == L.ZERO_EINVAL
    assert dec(ctypes.byref(hp), L.ZERO_F16, al, al + 257, al + 320, None) == L.ZERO_EINVAL
    assert dec(ctypes.byref(hp), L.ZERO_F16, al, al + 256, al + 324, None) == L.ZERO_EINVAL


def test_norm_decide_rejects_bad_arguments_on_host():
    lib = L.lib()
    buf = ctypes.create_string_buffer(1024)
    al = (ctypes.addressof(buf) + 15) & ~15
    hp = L.zero_adam_hyper(1e-3, 0.9, 0.999, 1e-8, 0.0, 1.0)
    nd = lib.zero_shard_norm_decide_dev
    assert nd(al, L.ZERO_F16, 8, None, al + 512, al + 256, al + 264, al + 320, al + 384, 1024, None) == L.ZERO_EINVAL
    assert nd(al, L.ZERO_F16, 8, ctypes.byref(hp), None, al + 256, al + 264, al + 320, al + 384, 1024, None) == L.ZERO_EINVAL
    assert nd(al, L.ZERO_F16, 8, ctypes.byref(hp), al + 512, al + 256, al + 264, None, al + 384, 1024, None) == L.ZERO_EINVAL
    assert nd(al, 7, 8, ctypes.byref(hp), al + 512, al + 256, al + 264, al + 320, al + 384, 1024, None) == L.ZERO_EINVAL
    assert nd(al, L.ZERO_F16, 8, ctypes.byref(hp), al + 512, al + 256, al + 264, al + 320, al + 384, 0, None) == L.ZERO_ENOSPC


def test_sum_norm_rejects_bad_arguments_on_host():
    lib = L.lib()
    buf = ctypes.create_string_buffer(2048)
    al = (ctypes.addressof(buf) + 15) & ~15
    f = lib.zero_shard_grad_sum_norm
    one = (ctypes.c_void_p * 1)(al + 256)
    ws = Z.zero_sum_norm_workspace_bytes(8)
    assert f(al, one, 0, L.ZERO_F16, 8, 0, 1.0, al + 512, al + 520, al + 768, ws, None) == L.ZERO_EINVAL
    assert f(al, one, 1, L.ZERO_F32, 8, 0, 1.0, al + 512, al + 520, al + 768, ws, None) == L.ZERO_EINVAL
    assert f(al, one, 1, L.ZERO_F16, 8, 0, 0.0, al + 512, al + 520, al + 768, ws, None) == L.ZERO_EINVAL
    assert f(al, one, 1, L.ZERO_F16, 8, 0, 1.0, None, al + 520, al + 768, ws, None) == L.ZERO_EINVAL
    assert f(al, one, 1, L.ZERO_F16, 8, 0, 1.0, al + 512, al + 520, al + 768, 0, None) == L.ZERO_ENOSPC
    assert f(al, one, 1, L.ZERO_F16, 8, 0, 1.0, al + 512, al + 520, al + 776, ws, None) == L.ZERO_EALIGN
    assert f(al, (ctypes.c_void_p * 1)(al + 8), 1, L.ZERO_F16, 8, 0, 1.0, al + 512, al + 520, al + 768, ws,
             None) == L.ZERO_EALIGN
    assert f(al, (ctypes.c_void_p * 1)(al + 16), 1, L.ZERO_F16, 8, 0, 1.0, al + 512, al + 520, al + 768, ws,
             None) == L.ZERO_EINVAL                                      # acc aliases the slice
    g = lib.zero_shard_grad_sum_norm_dev
    hp = L.zero_adam_hyper(1e-3, 0.9, 0.999, 1e-8, 0.0, 1.0)
    assert g(al, one, 1, L.ZERO_F16, 8, 0, None, None, al + 512, al + 520, None, al + 768, ws, None) == L.ZERO_EINVAL
    assert g(al, one, 1, L.ZERO_F16, 8, 0, ctypes.byref(hp), al + 1024, al + 512, al + 520, None, al + 768, ws,
             None) == L.ZERO_EINVAL                                      # decision without d_coef
    assert Z.zero_sum_norm_workspace_bytes(-1) == 0
    assert Z.zero_sum_norm_workspace_bytes(976077312) < 976077312 // 16


def test_scalar_and_workspace_aliasing_rejected_on_host():
    """A norm, flag or workspace that lies inside a buffer the same call
    writes (or reads while another block writes) is rejected before any
    launch: every layout below overlaps somewhere."""
    lib = L.lib()
    buf = ctypes.create_string_buffer(4096)
    al = (ctypes.addressof(buf) + 255) & ~255
    nrm = lib.zero_shard_unscale_norm_overflow
    need = Z.zero_norm_workspace_bytes(8)
    assert nrm(al + 1024, L.ZERO_F16, 8, 1.0, al + 512, al + 520, al + 1024, need, None) == L.ZERO_EINVAL   # grad in ws
    assert nrm(al, L.ZERO_F16, 8, 1.0, al + 1032, al + 520, al + 1024, need, None) == L.ZERO_EINVAL         # sq in ws
    assert nrm(al, L.ZERO_F16, 8, 1.0, al + 512, al + 1028, al + 1024, need, None) == L.ZERO_EINVAL         # flag in ws
    assert nrm(al, L.ZERO_F16, 8, 1.0, al + 512, al + 516, al + 1024, need, None) == L.ZERO_EINVAL          # sq over flag
    assert nrm(al, L.ZERO_F16, 0, 1.0, al + 1024, al + 520, al + 1024, need, None) == L.ZERO_EINVAL         # also at n = 0
    hp = ctypes.byref(L.zero_adam_params(1e-3, 0.9, 0.999, 1e-8, 0.0, 1, 1.0, 0.0))
    step = lib.zero_shard_adam_step
    assert step(al, al + 16, al + 32, al + 48, L.ZERO_F16, None, 0, 4, hp, None, al + 4, None) == L.ZERO_EINVAL
    assert step(al, al + 16, al + 32, al + 48, L.ZERO_F16, None, 0, 4, hp, al + 16, al + 512, None) == L.ZERO_EINVAL
    assert step(al, al + 16, al + 32, al + 48, L.ZERO_F16, al + 64, L.ZERO_F16, 4, hp, None, al + 68,
                None) == L.ZERO_EINVAL                                                          # flag in param_out
    acc = lib.zero_shard_grad_accumulate
    assert acc(al, al + 16, L.ZERO_F16, 4, 1.0, 1, al + 8, None) == L.ZERO_EINVAL
    red = lib.zero_shard_grad_reduce
    one = (ctypes.c_void_p * 1)(al + 256)
    assert red(al, one, 1, L.ZERO_F16, 4, 1.0, al + 12, None) == L.ZERO_EINVAL
    sn = lib.zero_shard_grad_sum_norm
    ws = Z.zero_sum_norm_workspace_bytes(8)
    assert sn(al, (ctypes.c_void_p * 1)(al + 1024), 1, L.ZERO_F16, 8, 0, 1.0, al + 512, al + 520, al + 1024, ws,
              None) == L.ZERO_EINVAL                                                            # slice in ws
    assert sn(al, one, 1, L.ZERO_F16, 8, 0, 1.0, al + 1024, al + 520, al + 1024, ws, None) == L.ZERO_EINVAL
    assert sn(al, one, 1, L.ZERO_F16, 8, 0, 1.0, al + 8, al + 520, al + 1024, ws, None) == L.ZERO_EINVAL  # sq in acc
    assert sn(al, one, 1, L.ZERO_F16, 8, 0, 1.0, al + 512, al + 20, al + 1024, ws, None) == L.ZERO_EINVAL  # flag in acc
    assert "lies in" in lib.zero_last_error().decode()


def test_norm_combine_rejects_bad_arguments_on_host():
    lib = L.lib()
    buf = ctypes.create_string_buffer(4096)
    al = (ctypes.addressof(buf) + 255) & ~255
    f = lib.zero_norm_combine_ranks
    # slots: 8 doubles at al, 8 flags at al + 64; outputs at al + 512 / al + 520
    assert f(al, al + 64, 0, al + 512, al + 520, None) == L.ZERO_EINVAL                   # no ranks
    assert f(al, al + 64, 65537, al + 512, al + 520, None) == L.ZERO_EINVAL               # above the maximum
    assert f(None, al + 64, 8, al + 512, al + 520, None) == L.ZERO_EINVAL
    assert f(al, al + 64, 8, None, al + 520, None) == L.ZERO_EINVAL
    assert f(al + 4, al + 64, 8, al + 512, al + 520, None) == L.ZERO_EALIGN
    assert f(al, al + 66, 8, al + 512, al + 520, None) == L.ZERO_EALIGN
    assert f(al, al + 32, 8, al + 512, al + 520, None) == L.ZERO_EINVAL                   # flags inside the sums
    assert f(al, al + 64, 8, al + 8, al + 520, None) == L.ZERO_EINVAL                     # output inside a slot array
    assert f(al, al + 64, 8, al + 512, al + 68, None) == L.ZERO_EINVAL
    assert f(al, al + 64, 8, al + 512, al + 516, None) == L.ZERO_EINVAL                   # outputs overlap


def test_noalloc_norm_rejects_bad_arguments_on_host():
    """Every argument is checked before the device is touched (no GPU here)."""
    lib = L.lib()
    buf = ctypes.create_string_buffer(256)
    al = (ctypes.addressof(buf) + 15) & ~15
    f = lib.zero_shard_unscale_norm_overflow_noalloc
    assert f(al, L.ZERO_F16, 8, 0.0, al + 64, al + 80, None) == L.ZERO_EINVAL          # inv_loss_scale
    assert f(al, L.ZERO_F16, 8, float("inf"), al + 64, al + 80, None) == L.ZERO_EINVAL
    assert f(al, L.ZERO_F16, -1, 1.0, al + 64, al + 80, None) == L.ZERO_EINVAL
    assert f(al, 7, 8, 1.0, al + 64, al + 80, None) == L.ZERO_EINVAL                   # dtype
    assert f(al, L.ZERO_F16, 8, 1.0, None, al + 80, None) == L.ZERO_EINVAL
    assert f(al, L.ZERO_F16, 8, 1.0, al + 64, None, None) == L.ZERO_EINVAL
    assert f(None, L.ZERO_F16, 8, 1.0, al + 64, al + 80, None) == L.ZERO_EINVAL
    assert f(al + 2, L.ZERO_F16, 8, 1.0, al + 64, al + 80, None) == L.ZERO_EALIGN
    assert f(al, L.ZERO_F16, 8, 1.0, al + 68, al + 80, None) == L.ZERO_EALIGN
    assert f(al, L.ZERO_F16, 8, 1.0, al + 64, al + 82, None) == L.ZERO_EALIGN
    assert f(al, L.ZERO_F16, 1 << 62, 1.0, al + 64, al + 80, None) == L.ZERO_ERANGE
