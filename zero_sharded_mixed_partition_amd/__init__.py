"""One ZeRO data-parallel rank's partitioned mixed-precision Adam step on
AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI in include/zero_shard.h (libzero_shard.so,
hand-written HIP kernels).  The functions keep the C names and only marshal
arguments: torch tensors supply device memory (their data pointers) and
torch's current HIP stream supplies the stream; every step of the update runs
in the library's kernels.

    zero_partition_plan(shapes, n_d, align) -> (offsets, S, padded_total)
    zero_rank_fragments(shapes, n_d, align, rank) -> [(tensor, tensor_begin, shard_begin, numel)]
    zero_norm_workspace_bytes(n) -> int
    zero_shard_unscale_norm_overflow(grad, inv_loss_scale, sqnorm, overflow, workspace)
    zero_shard_adam_step(master, exp_avg, exp_avg_sq, grad, param_out, hp, global_sqnorm, global_overflow)
    zero_shard_grad_accumulate(acc, grad, inv_loss_scale, first, overflow=None)
    zero_cpu_shard_unscale_norm_overflow(grad, inv_loss_scale) -> (sq, overflow)      host memory
    zero_cpu_shard_adam_step(master, exp_avg, exp_avg_sq, grad, param_out, hp, sq, overflow)  host memory
    zero_loss_scaler_update(scaler, overflow) -> skip
"""
import ctypes
from typing import List, Optional, Sequence, Tuple

from . import _lib as _L
from ._lib import (ZERO_BF16, ZERO_F16, ZERO_F32, ZeroShardError, zero_adam_hyper,  # noqa: F401
                   zero_adam_params, zero_fragment, zero_loss_scaler, zero_step_state)

__all__ = ["zero_partition_plan", "zero_rank_fragments", "zero_norm_workspace_bytes",
           "zero_shard_unscale_norm_overflow", "zero_shard_unscale_norm_overflow_noalloc", "zero_shard_adam_step",
           "zero_shard_grad_accumulate",
           "zero_cpu_shard_unscale_norm_overflow", "zero_cpu_shard_adam_step",
           "zero_loss_scaler_update", "zero_abi_version", "ZERO_F16", "ZERO_BF16", "ZERO_F32",
           "ZeroShardError", "AdamHyper",
           "LossScaler", "dtype_code", "ShardAdam", "OffloadShardAdam", "StepGraph", "zero_adam_coef_bytes",
           "zero_adam_prepare", "zero_shard_adam_step_coef", "zero_shard_grad_reduce", "zero_copy_reference",
           "zero_copy_widen_reference", "zero_cpu_copy_reference",
           "MAX_SLICES", "StepState", "zero_shard_unscale_norm_overflow_dev", "zero_shard_adam_step_dev",
           "zero_shard_grad_accumulate_dev", "zero_shard_grad_reduce_dev", "zero_step_decide_dev",
           "zero_shard_norm_decide_dev", "StepGraphDev", "zero_sum_norm_workspace_bytes", "zero_shard_grad_sum_norm",
           "zero_shard_grad_sum_norm_dev", "zero_device_alloc_contiguous", "zero_device_free",
           "zero_pool_counts", "contiguous_pool"]


def zero_abi_version() -> int:
    return int(_L.lib().zero_abi_version())


def _shape_arrays(shapes: Sequence[Sequence[int]]):
    n = len(shapes)
    flat = [int(d) for s in shapes for d in s]
    dims = (ctypes.c_int64 * max(1, len(flat)))(*flat)
    ndims = (ctypes.c_int32 * max(1, n))(*[len(s) for s in shapes])
    return dims, ndims, n


def zero_partition_plan(shapes: Sequence[Sequence[int]], n_d: int, align: int) -> Tuple[List[int], int, int]:
    dims, ndims, n = _shape_arrays(shapes)
    offs = (ctypes.c_int64 * max(1, n))()
    S, padded = ctypes.c_int64(), ctypes.c_int64()
    _L.check(_L.lib().zero_partition_plan(dims, ndims, n, n_d, align, offs, ctypes.byref(S),
                                          ctypes.byref(padded)), "zero_partition_plan")
    return list(offs[:n]), S.value, padded.value


def zero_rank_fragments(shapes: Sequence[Sequence[int]], n_d: int, align: int,
                        rank: int) -> List[Tuple[int, int, int, int]]:
    dims, ndims, n = _shape_arrays(shapes)
    count = ctypes.c_int32()
    st = _L.lib().zero_rank_fragments(dims, ndims, n, n_d, align, rank, None, 0, ctypes.byref(count))
    if st not in (_L.ZERO_OK, _L.ZERO_ENOSPC):
        _L.check(st, "zero_rank_fragments")
    buf = (zero_fragment * max(1, count.value))()
    _L.check(_L.lib().zero_rank_fragments(dims, ndims, n, n_d, align, rank, buf, count.value,
                                          ctypes.byref(count)), "zero_rank_fragments")
    return [(f.tensor, f.tensor_begin, f.shard_begin, f.numel) for f in buf[:count.value]]


def zero_norm_workspace_bytes(n: int) -> int:
    return int(_L.lib().zero_norm_workspace_bytes(n))


def dtype_code(t) -> int:
    """ZERO_F16 / ZERO_BF16 / ZERO_F32 from a torch dtype (or pass the code through)."""
    if isinstance(t, int):
        return t
    import torch
    dt = t.dtype if hasattr(t, "dtype") else t
    if dt == torch.float16:
        return ZERO_F16
    if dt == torch.bfloat16:
        return ZERO_BF16
    if dt == torch.float32:
        return ZERO_F32
    raise ValueError(f"unsupported gradient/parameter dtype {dt}")


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("device tensor expected")
    if not t.is_contiguous():
        raise ValueError("contiguous tensor expected")
    return t.data_ptr()


_ELEM_BYTES = {ZERO_F16: 2, ZERO_BF16: 2, ZERO_F32: 4}


def _dev(t, nbytes: int, what: str) -> Optional[int]:
    """_ptr(t), after checking that the tensor holds the nbytes the call reads
    or writes from its start, so that a short buffer raises here instead of
    being overrun on the device.  A raw address is taken as it is."""
    p = _ptr(t)
    if t is not None and not isinstance(t, int):
        have = t.numel() * t.element_size()
        if have < nbytes:
            raise ValueError(f"{what}: {have} bytes, the call accesses {nbytes}")
    return p


def _typed(t, dtype_name: str, count: int, what: str) -> Optional[int]:
    """Device pointer of a float64 / int32 scalar (or per-rank) buffer of at
    least count elements."""
    if t is None or isinstance(t, int):
        return t
    if str(t.dtype) != "torch." + dtype_name:
        raise ValueError(f"{what}: torch.{dtype_name} tensor expected, got {t.dtype}")
    return _dev(t, count * t.element_size(), what)


def _grad_ptr(t, gd: int, n: int, what: str = "grad") -> Optional[int]:
    return _dev(t, n * _ELEM_BYTES.get(gd, 0), what)


def _step_ptrs(master, exp_avg, exp_avg_sq, grad, gd: int, param_out, n: int):
    """Checked pointers of the five shard streams of an update over n elements."""
    return (_dev(master, 4 * n, "master"), _dev(exp_avg, 4 * n, "exp_avg"), _dev(exp_avg_sq, 4 * n, "exp_avg_sq"),
            _grad_ptr(grad, gd, n), _dev(param_out, 2 * n, "param_out"))


def _coef_ptr(d_coef) -> Optional[int]:
    return _dev(d_coef, zero_adam_coef_bytes(), "d_coef")


def zero_shard_unscale_norm_overflow(grad, inv_loss_scale: float, sqnorm, overflow, workspace,
                                     grad_dtype: Optional[int] = None, n: Optional[int] = None,
                                     stream=None) -> None:
    """Enqueue steps 1-2 on the current stream.  grad: float16/bfloat16 device
    tensor (or raw pointer with grad_dtype and n); sqnorm: float64 [1];
    overflow: int32 [1]; workspace: device tensor of at least
    zero_norm_workspace_bytes(n) bytes."""
    gd = dtype_code(grad if grad_dtype is None else grad_dtype)
    n = grad.numel() if n is None else n
    wbytes = workspace.numel() * workspace.element_size()
    _L.check(_L.lib().zero_shard_unscale_norm_overflow(_grad_ptr(grad, gd, n), gd, n, float(inv_loss_scale),
                                                       _typed(sqnorm, "float64", 1, "sqnorm"),
                                                       _typed(overflow, "int32", 1, "overflow"), _ptr(workspace),
                                                       wbytes, _stream(stream)),
             "zero_shard_unscale_norm_overflow")


def zero_shard_unscale_norm_overflow_noalloc(grad, inv_loss_scale: float, sqnorm, overflow,
                                             grad_dtype: Optional[int] = None, n: Optional[int] = None,
                                             stream=None) -> None:
    """zero_shard_unscale_norm_overflow with its partials in the library's
    fixed per-GPU array instead of a workspace: allocates nothing.  Calls
    that overlap in time on one GPU race (see include/zero_shard.h)."""
    gd = dtype_code(grad if grad_dtype is None else grad_dtype)
    n = grad.numel() if n is None else n
    _L.check(_L.lib().zero_shard_unscale_norm_overflow_noalloc(_grad_ptr(grad, gd, n), gd, n, float(inv_loss_scale),
                                                               _typed(sqnorm, "float64", 1, "sqnorm"),
                                                               _typed(overflow, "int32", 1, "overflow"),
                                                               _stream(stream)),
             "zero_shard_unscale_norm_overflow_noalloc")


class AdamHyper:
    """Adam/AdamW hyperparameters of one step (all double at the ABI)."""

    def __init__(self, lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, step=1,
                 inv_loss_scale=1.0, max_grad_norm=0.0):
        self.lr, self.beta1, self.beta2, self.eps = lr, beta1, beta2, eps
        self.weight_decay, self.step = weight_decay, step
        self.inv_loss_scale, self.max_grad_norm = inv_loss_scale, max_grad_norm

    def c(self) -> zero_adam_params:
        return zero_adam_params(float(self.lr), float(self.beta1), float(self.beta2), float(self.eps),
                                float(self.weight_decay), int(self.step), float(self.inv_loss_scale),
                                float(self.max_grad_norm))


def zero_shard_adam_step(master, exp_avg, exp_avg_sq, grad, param_out, hp: AdamHyper, global_sqnorm=None,
                         global_overflow=None, grad_dtype: Optional[int] = None,
                         param_dtype: Optional[int] = None, n: Optional[int] = None, stream=None) -> None:
    """Enqueue steps 3-4 on the current stream (see include/zero_shard.h)."""
    gd = dtype_code(grad if grad_dtype is None else grad_dtype)
    pd = 0 if param_out is None else dtype_code(param_out if param_dtype is None else param_dtype)
    n = master.numel() if n is None else n
    if not isinstance(master, int):
        for t in (exp_avg, exp_avg_sq, grad) + (() if param_out is None else (param_out,)):
            if t.numel() != n:
                raise ValueError("shard tensors differ in length")
    params = hp.c()
    pm, pe, pv, pg, pp = _step_ptrs(master, exp_avg, exp_avg_sq, grad, gd, param_out, n)
    _L.check(_L.lib().zero_shard_adam_step(pm, pe, pv, pg, gd, pp, pd, n, ctypes.byref(params),
                                           _typed(global_sqnorm, "float64", 1, "global_sqnorm"),
                                           _typed(global_overflow, "int32", 1, "global_overflow"), _stream(stream)),
             "zero_shard_adam_step")


def zero_shard_grad_accumulate(acc, grad, inv_loss_scale: float, first: bool, overflow=None,
                               grad_dtype: Optional[int] = None, n: Optional[int] = None, stream=None) -> None:
    """Enqueue acc = (first ? 0 : acc) + grad * inv_loss_scale (fp32 acc, 16-bit
    grad); overflow (int32 [1] or None) is set to 1 if grad holds an inf/NaN."""
    gd = dtype_code(grad if grad_dtype is None else grad_dtype)
    n = acc.numel() if n is None else n
    if not isinstance(acc, int) and grad.numel() != n:
        raise ValueError("acc and grad differ in length")
    _L.check(_L.lib().zero_shard_grad_accumulate(_dev(acc, 4 * n, "acc"), _grad_ptr(grad, gd, n), gd, n,
                                                 float(inv_loss_scale), 1 if first else 0,
                                                 _typed(overflow, "int32", 1, "overflow"), _stream(stream)),
             "zero_shard_grad_accumulate")


MAX_SLICES = 16


def zero_shard_grad_reduce(acc, slices, inv_loss_scale: float, overflow=None, grad_dtype: Optional[int] = None,
                           n: Optional[int] = None, stream=None) -> None:
    """acc = sum over slices (in order) of slice * inv_loss_scale, in fp32, one
    rounding per addition; overflow (device int32) is set if any slice holds
    an inf/NaN."""
    if not 1 <= len(slices) <= MAX_SLICES:
        raise ValueError(f"1 to {MAX_SLICES} slices expected, got {len(slices)}")
    gd = dtype_code(slices[0] if grad_dtype is None else grad_dtype)
    n = acc.numel() if n is None else n
    arr = (ctypes.c_void_p * len(slices))(*[_grad_ptr(t, gd, n, f"slices[{i}]") for i, t in enumerate(slices)])
    _L.check(_L.lib().zero_shard_grad_reduce(_dev(acc, 4 * n, "acc"), arr, len(slices), gd, n,
                                             float(inv_loss_scale), _typed(overflow, "int32", 1, "overflow"),
                                             _stream(stream)), "zero_shard_grad_reduce")


# ---------------------------------------------------------------- host-memory (offload) entry points

def _host_ptr(a) -> Optional[int]:
    """Address of a C-contiguous numpy array or CPU torch tensor."""
    if a is None:
        return None
    if isinstance(a, int):
        return a
    if hasattr(a, "ctypes"):
        if not a.flags["C_CONTIGUOUS"]:
            raise ValueError("C-contiguous host array expected")
        return a.ctypes.data
    if a.is_cuda or not a.is_contiguous():
        raise ValueError("contiguous host tensor expected")
    return a.data_ptr()


def _host_code(a, code: Optional[int]) -> int:
    if code is not None:
        return code
    if hasattr(a, "ctypes"):
        import numpy as np
        if a.dtype == np.float16:
            return ZERO_F16
        if a.dtype == np.float32:
            return ZERO_F32
        raise ValueError("pass grad_dtype / param_dtype for raw 16-bit patterns")
    return dtype_code(a)


def zero_cpu_shard_unscale_norm_overflow(grad, inv_loss_scale: float, grad_dtype: Optional[int] = None,
                                         n: Optional[int] = None, nthreads: int = 0):
    """Host-memory norm pass; returns (sum of squares, overflow)."""
    gd = _host_code(grad, grad_dtype)
    n = (grad.size if hasattr(grad, "ctypes") else grad.numel()) if n is None else n
    sq, ovf = ctypes.c_double(), ctypes.c_int32()
    _L.check(_L.lib().zero_cpu_shard_unscale_norm_overflow(_host_ptr(grad), gd, n, float(inv_loss_scale),
                                                           ctypes.byref(sq), ctypes.byref(ovf), int(nthreads)),
             "zero_cpu_shard_unscale_norm_overflow")
    return sq.value, bool(ovf.value)


def zero_cpu_copy_reference(dst, src, nbytes: Optional[int] = None, nthreads: int = 0) -> None:
    """Host-memory copy in the host step's chunks, threads and store style
    (synchronous): the host cores' one-read-one-write streaming rate."""
    size = lambda a: a.nbytes if hasattr(a, "ctypes") else a.numel() * a.element_size()  # noqa: E731
    nbytes = size(src) if nbytes is None else int(nbytes)
    if size(dst) < nbytes or size(src) < nbytes:
        raise ValueError(f"buffers hold {size(dst)} / {size(src)} bytes, the copy moves {nbytes}")
    _L.check(_L.lib().zero_cpu_copy_reference(_host_ptr(dst), _host_ptr(src), nbytes, int(nthreads)),
             "zero_cpu_copy_reference")


def zero_cpu_shard_adam_step(master, exp_avg, exp_avg_sq, grad, param_out, hp: AdamHyper, global_sqnorm: float,
                             global_overflow: bool, grad_dtype: Optional[int] = None,
                             param_dtype: Optional[int] = None, n: Optional[int] = None, nthreads: int = 0) -> None:
    """Host-memory fused AdamW step (synchronous)."""
    gd = _host_code(grad, grad_dtype)
    pd = 0 if param_out is None else _host_code(param_out, param_dtype)
    size = lambda a: a.size if hasattr(a, "ctypes") else a.numel()  # noqa: E731
    n = size(master) if n is None else n
    for a in (exp_avg, exp_avg_sq, grad) + (() if param_out is None else (param_out,)):
        if not isinstance(a, int) and size(a) != n:
            raise ValueError("shard arrays differ in length")
    params = hp.c()
    _L.check(_L.lib().zero_cpu_shard_adam_step(_host_ptr(master), _host_ptr(exp_avg), _host_ptr(exp_avg_sq),
                                               _host_ptr(grad), gd, _host_ptr(param_out), pd, n, ctypes.byref(params),
                                               float(global_sqnorm), 1 if global_overflow else 0, int(nthreads)),
             "zero_cpu_shard_adam_step")


def zero_adam_coef_bytes() -> int:
    return int(_L.lib().zero_adam_coef_bytes())


def zero_adam_prepare(hp: AdamHyper, coef_out) -> None:
    """Per-step coefficient block of hp into host memory coef_out (a CPU uint8
    tensor or numpy array of zero_adam_coef_bytes() bytes, or an address)."""
    params = hp.c()
    addr = coef_out if isinstance(coef_out, int) else _host_ptr(coef_out)
    _L.check(_L.lib().zero_adam_prepare(ctypes.byref(params), addr), "zero_adam_prepare")


def zero_shard_adam_step_coef(master, exp_avg, exp_avg_sq, grad, param_out, d_coef, global_sqnorm,
                              global_overflow=None, grad_dtype: Optional[int] = None,
                              param_dtype: Optional[int] = None, n: Optional[int] = None, stream=None) -> None:
    """zero_shard_adam_step with the coefficient block read from device memory d_coef."""
    gd = dtype_code(grad if grad_dtype is None else grad_dtype)
    pd = 0 if param_out is None else dtype_code(param_out if param_dtype is None else param_dtype)
    n = master.numel() if n is None else n
    pm, pe, pv, pg, pp = _step_ptrs(master, exp_avg, exp_avg_sq, grad, gd, param_out, n)
    _L.check(_L.lib().zero_shard_adam_step_coef(pm, pe, pv, pg, gd, pp, pd, n, _coef_ptr(d_coef),
                                                _typed(global_sqnorm, "float64", 1, "global_sqnorm"),
                                                _typed(global_overflow, "int32", 1, "global_overflow"),
                                                _stream(stream)),
             "zero_shard_adam_step_coef")


class StepGraph:
    """A recorded step (coefficients in, norm pass, fused update, flag out)
    over fixed buffers and a fixed loss scale; see zero_step_graph_* in the
    header.  The library allocates its pinned and device blocks; close()
    (or garbage collection) frees them."""

    def __init__(self, master, exp_avg, exp_avg_sq, grad, param_out, inv_loss_scale: float, sqnorm, overflow,
                 workspace, grad_dtype: Optional[int] = None, param_dtype: Optional[int] = None):
        gd = dtype_code(grad if grad_dtype is None else grad_dtype)
        pd = 0 if param_out is None else dtype_code(param_out if param_dtype is None else param_dtype)
        handle = ctypes.c_void_p()
        wbytes = workspace.numel() * workspace.element_size()
        n = master.numel()
        pm, pe, pv, pg, pp = _step_ptrs(master, exp_avg, exp_avg_sq, grad, gd, param_out, n)
        _L.check(_L.lib().zero_step_graph_create(ctypes.byref(handle), pm, pe, pv, pg, gd, pp, pd, n,
                                                 float(inv_loss_scale), _typed(sqnorm, "float64", 1, "sqnorm"),
                                                 _typed(overflow, "int32", 1, "overflow"), _ptr(workspace), wbytes),
                 "zero_step_graph_create")
        self._h = handle.value
        self.inv_loss_scale = float(inv_loss_scale)
        self._keep = (master, exp_avg, exp_avg_sq, grad, param_out, sqnorm, overflow, workspace)

    def launch(self, hp: AdamHyper, stream=None) -> None:
        params = hp.c()
        _L.check(_L.lib().zero_step_graph_launch(self._h, ctypes.byref(params), _stream(stream)),
                 "zero_step_graph_launch")

    def overflow(self) -> bool:
        flag = ctypes.c_int32()
        _L.check(_L.lib().zero_step_graph_overflow(self._h, ctypes.byref(flag)), "zero_step_graph_overflow")
        return bool(flag.value)

    def close(self) -> None:
        if self._h:
            _L.lib().zero_step_graph_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


MAX_RANKS = 65536


def zero_norm_combine_ranks(slot_sqnorm, slot_overflow, global_sqnorm, global_overflow, stream=None) -> None:
    """The local half of the scalars' all-reduce: global_sqnorm = the rank-order
    fp64 sum of slot_sqnorm (float64 [n_ranks]), global_overflow = the OR of
    slot_overflow (int32 [n_ranks]); all device tensors."""
    n = slot_sqnorm.numel()
    if slot_overflow.numel() != n:
        raise ValueError("slot_sqnorm and slot_overflow must have one entry per rank")
    _L.check(_L.lib().zero_norm_combine_ranks(_typed(slot_sqnorm, "float64", n, "slot_sqnorm"),
                                              _typed(slot_overflow, "int32", n, "slot_overflow"), n,
                                              _typed(global_sqnorm, "float64", 1, "global_sqnorm"),
                                              _typed(global_overflow, "int32", 1, "global_overflow"),
                                              _stream(stream)), "zero_norm_combine_ranks")


def zero_copy_reference(dst, src, nbytes: Optional[int] = None, stream=None) -> None:
    """Reference 16-byte-per-lane device copy of nbytes (default: all of src)."""
    nbytes = src.numel() * src.element_size() if nbytes is None else nbytes
    _L.check(_L.lib().zero_copy_reference(_dev(dst, int(nbytes), "dst"), _dev(src, int(nbytes), "src"), int(nbytes),
                                          _stream(stream)), "zero_copy_reference")


def zero_copy_widen_reference(dst, src, src_bytes: Optional[int] = None, stream=None) -> None:
    """Widening device copy: reads src_bytes (default: all of src), writes
    twice that to dst (8 bytes read, 16 written per lane)."""
    src_bytes = src.numel() * src.element_size() if src_bytes is None else src_bytes
    _L.check(_L.lib().zero_copy_widen_reference(_dev(dst, 2 * int(src_bytes), "dst"), _dev(src, int(src_bytes), "src"),
                                                int(src_bytes), _stream(stream)), "zero_copy_widen_reference")


class StepState:
    """The loss scaler and step counts in device memory (C struct
    zero_step_state), for the calls that keep a whole step on the device."""

    def __init__(self, scaler: "LossScaler", applied_steps: int = 0, device=None):
        import torch
        host = zero_step_state(scaler.s, int(applied_steps), 0, 0, 0)
        raw = bytes(host)
        self.tensor = torch.frombuffer(bytearray(raw), dtype=torch.uint8).to(device or "cuda")

    def ptr(self) -> int:
        return self.tensor.data_ptr()

    def read(self) -> zero_step_state:
        """Copy the state to the host (synchronises with its stream)."""
        raw = bytes(self.tensor.cpu().numpy().tobytes())
        return zero_step_state.from_buffer_copy(raw)


def _hyper(hp: "AdamHyper") -> zero_adam_hyper:
    p = hp.c()
    return zero_adam_hyper(p.lr, p.beta1, p.beta2, p.eps, p.weight_decay, p.max_grad_norm)


def zero_shard_unscale_norm_overflow_dev(grad, state: StepState, sqnorm, overflow, workspace,
                                         grad_dtype: Optional[int] = None, n: Optional[int] = None,
                                         stream=None) -> None:
    gd = dtype_code(grad if grad_dtype is None else grad_dtype)
    n = grad.numel() if n is None else n
    _L.check(_L.lib().zero_shard_unscale_norm_overflow_dev(_grad_ptr(grad, gd, n), gd, n, state.ptr(),
                                                           _typed(sqnorm, "float64", 1, "sqnorm"),
                                                           _typed(overflow, "int32", 1, "overflow"), _ptr(workspace),
                                                           workspace.numel() * workspace.element_size(),
                                                           _stream(stream)), "zero_shard_unscale_norm_overflow_dev")


def zero_shard_adam_step_dev(master, exp_avg, exp_avg_sq, grad, param_out, hp: "AdamHyper", state: StepState,
                             global_sqnorm, global_overflow, d_coef, grad_dtype: Optional[int] = None,
                             param_dtype: Optional[int] = None, n: Optional[int] = None, stream=None) -> None:
    """hp.step and hp.inv_loss_scale are ignored: t and the scale come from the device state."""
    gd = dtype_code(grad if grad_dtype is None else grad_dtype)
    pd = 0 if param_out is None else dtype_code(param_out if param_dtype is None else param_dtype)
    n = master.numel() if n is None else n
    h = _hyper(hp)
    pm, pe, pv, pg, pp = _step_ptrs(master, exp_avg, exp_avg_sq, grad, gd, param_out, n)
    _L.check(_L.lib().zero_shard_adam_step_dev(pm, pe, pv, pg, gd, pp, pd, n, ctypes.byref(h), state.ptr(),
                                               _typed(global_sqnorm, "float64", 1, "global_sqnorm"),
                                               _typed(global_overflow, "int32", 1, "global_overflow"),
                                               _coef_ptr(d_coef), _stream(stream)), "zero_shard_adam_step_dev")


def zero_shard_norm_decide_dev(grad, hp: "AdamHyper", state: StepState, sqnorm, overflow, d_coef, workspace,
                               grad_dtype: Optional[int] = None, n: Optional[int] = None, stream=None) -> None:
    """Single-rank norm pass whose final kernel also makes the step's decision."""
    gd = dtype_code(grad if grad_dtype is None else grad_dtype)
    n = grad.numel() if n is None else n
    h = _hyper(hp)
    _L.check(_L.lib().zero_shard_norm_decide_dev(_grad_ptr(grad, gd, n), gd, n, ctypes.byref(h), state.ptr(),
                                                 _typed(sqnorm, "float64", 1, "sqnorm"),
                                                 _typed(overflow, "int32", 1, "overflow"), _coef_ptr(d_coef),
                                                 _ptr(workspace),
                                                 workspace.numel() * workspace.element_size(), _stream(stream)),
             "zero_shard_norm_decide_dev")


def zero_step_decide_dev(hp: "AdamHyper", grad_dtype, state: StepState, global_overflow, d_coef,
                         stream=None) -> None:
    """The decision kernel: d_coef <- coefficients of step applied+1, state advanced by the flag."""
    h = _hyper(hp)
    _L.check(_L.lib().zero_step_decide_dev(ctypes.byref(h), dtype_code(grad_dtype), state.ptr(),
                                           _typed(global_overflow, "int32", 1, "global_overflow"),
                                           _coef_ptr(d_coef), _stream(stream)),
             "zero_step_decide_dev")


def zero_shard_grad_accumulate_dev(acc, grad, state: StepState, first: bool, overflow=None,
                                   grad_dtype: Optional[int] = None, n: Optional[int] = None, stream=None) -> None:
    gd = dtype_code(grad if grad_dtype is None else grad_dtype)
    n = acc.numel() if n is None else n
    _L.check(_L.lib().zero_shard_grad_accumulate_dev(_dev(acc, 4 * n, "acc"), _grad_ptr(grad, gd, n), gd, n,
                                                     state.ptr(), 1 if first else 0,
                                                     _typed(overflow, "int32", 1, "overflow"), _stream(stream)),
             "zero_shard_grad_accumulate_dev")


def zero_shard_grad_reduce_dev(acc, slices, state: StepState, overflow=None, grad_dtype: Optional[int] = None,
                               n: Optional[int] = None, stream=None) -> None:
    if not 1 <= len(slices) <= MAX_SLICES:
        raise ValueError(f"1 to {MAX_SLICES} slices expected, got {len(slices)}")
    gd = dtype_code(slices[0] if grad_dtype is None else grad_dtype)
    n = acc.numel() if n is None else n
    arr = (ctypes.c_void_p * len(slices))(*[_grad_ptr(t, gd, n, f"slices[{i}]") for i, t in enumerate(slices)])
    _L.check(_L.lib().zero_shard_grad_reduce_dev(_dev(acc, 4 * n, "acc"), arr, len(slices), gd, n, state.ptr(),
                                                 _typed(overflow, "int32", 1, "overflow"), _stream(stream)),
             "zero_shard_grad_reduce_dev")


def zero_sum_norm_workspace_bytes(n: int) -> int:
    return int(_L.lib().zero_sum_norm_workspace_bytes(int(n)))


def zero_shard_grad_sum_norm(acc, slices, add_to_acc: bool, inv_loss_scale: float, sqnorm, overflow, workspace,
                             grad_dtype: Optional[int] = None, n: Optional[int] = None, stream=None) -> None:
    """acc = (add_to_acc ? acc : 0) + sum_k slices[k] * inv, with the norm and
    flag of the result in the same pass (sqnorm, overflow: device scalars)."""
    if not 1 <= len(slices) <= MAX_SLICES:
        raise ValueError(f"1 to {MAX_SLICES} slices expected, got {len(slices)}")
    gd = dtype_code(slices[0] if grad_dtype is None else grad_dtype)
    n = acc.numel() if n is None else n
    arr = (ctypes.c_void_p * len(slices))(*[_grad_ptr(t, gd, n, f"slices[{i}]") for i, t in enumerate(slices)])
    _L.check(_L.lib().zero_shard_grad_sum_norm(_dev(acc, 4 * n, "acc"), arr, len(slices), gd, n,
                                               1 if add_to_acc else 0, float(inv_loss_scale),
                                               _typed(sqnorm, "float64", 1, "sqnorm"),
                                               _typed(overflow, "int32", 1, "overflow"), _ptr(workspace),
                                               workspace.numel() * workspace.element_size(), _stream(stream)),
             "zero_shard_grad_sum_norm")


def zero_shard_grad_sum_norm_dev(acc, slices, add_to_acc: bool, state: StepState, sqnorm, overflow, workspace,
                                 hp: Optional["AdamHyper"] = None, d_coef=None, grad_dtype: Optional[int] = None,
                                 n: Optional[int] = None, stream=None) -> None:
    """zero_shard_grad_sum_norm with the loss scale from the device state; with
    hp (one rank) the final kernel also makes the step's decision into d_coef."""
    if not 1 <= len(slices) <= MAX_SLICES:
        raise ValueError(f"1 to {MAX_SLICES} slices expected, got {len(slices)}")
    gd = dtype_code(slices[0] if grad_dtype is None else grad_dtype)
    n = acc.numel() if n is None else n
    arr = (ctypes.c_void_p * len(slices))(*[_grad_ptr(t, gd, n, f"slices[{i}]") for i, t in enumerate(slices)])
    h = None if hp is None else ctypes.byref(_hyper(hp))
    _L.check(_L.lib().zero_shard_grad_sum_norm_dev(_dev(acc, 4 * n, "acc"), arr, len(slices), gd, n,
                                                   1 if add_to_acc else 0, h, state.ptr(),
                                                   _typed(sqnorm, "float64", 1, "sqnorm"),
                                                   _typed(overflow, "int32", 1, "overflow"),
                                                   None if d_coef is None else _coef_ptr(d_coef),
                                                   _ptr(workspace), workspace.numel() * workspace.element_size(),
                                                   _stream(stream)), "zero_shard_grad_sum_norm_dev")


class StepGraphDev:
    """A recorded step with device state (zero_step_graph_create_dev): the
    norm pass with the decision, then the update, replayed by launch() with
    no host work besides the launch.  The library allocates the graph;
    close() (or garbage collection) frees it."""

    def __init__(self, master, exp_avg, exp_avg_sq, grad, param_out, hp: "AdamHyper", state: StepState, sqnorm,
                 overflow, d_coef, workspace, grad_dtype: Optional[int] = None, param_dtype: Optional[int] = None):
        gd = dtype_code(grad if grad_dtype is None else grad_dtype)
        pd = 0 if param_out is None else dtype_code(param_out if param_dtype is None else param_dtype)
        handle = ctypes.c_void_p()
        h = _hyper(hp)
        n = master.numel()
        pm, pe, pv, pg, pp = _step_ptrs(master, exp_avg, exp_avg_sq, grad, gd, param_out, n)
        _L.check(_L.lib().zero_step_graph_create_dev(ctypes.byref(handle), pm, pe, pv, pg, gd, pp, pd, n,
                                                     ctypes.byref(h), state.ptr(),
                                                     _typed(sqnorm, "float64", 1, "sqnorm"),
                                                     _typed(overflow, "int32", 1, "overflow"), _coef_ptr(d_coef),
                                                     _ptr(workspace),
                                                     workspace.numel() * workspace.element_size()),
                 "zero_step_graph_create_dev")
        self._h = handle.value
        self._keep = (master, exp_avg, exp_avg_sq, grad, param_out, state, sqnorm, overflow, d_coef, workspace)

    def launch(self, stream=None) -> None:
        _L.check(_L.lib().zero_step_graph_launch_dev(self._h, _stream(stream)), "zero_step_graph_launch_dev")

    def close(self) -> None:
        if self._h:
            _L.lib().zero_step_graph_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class LossScaler:
    """Host-side dynamic loss scale (C struct zero_loss_scaler)."""

    def __init__(self, scale=65536.0, min_scale=1.0, backoff=0.5, growth=2.0, growth_interval=1000,
                 good_steps=0):
        self.s = zero_loss_scaler(float(scale), float(min_scale), float(backoff), float(growth),
                                  int(growth_interval), int(good_steps))

    @property
    def scale(self) -> float:
        return self.s.scale

    @property
    def good_steps(self) -> int:
        return self.s.good_steps

    @classmethod
    def static(cls, scale=1.0):
        return cls(scale=scale, min_scale=scale, backoff=1.0, growth=1.0)


def zero_loss_scaler_update(scaler: LossScaler, overflow: bool) -> bool:
    skip = ctypes.c_int32()
    _L.check(_L.lib().zero_loss_scaler_update(ctypes.byref(scaler.s), 1 if overflow else 0, ctypes.byref(skip)),
             "zero_loss_scaler_update")
    return bool(skip.value)


from .shard import ShardAdam  # noqa: E402
from .offload import OffloadShardAdam  # noqa: E402
from . import checkpoint  # noqa: E402,F401


# ---------------------------------------------------------------- physically contiguous HBM

def zero_device_alloc_contiguous(nbytes: int) -> int:
    """Address of `nbytes` of physically contiguous device memory (0 for 0
    bytes); release it with zero_device_free."""
    p = ctypes.c_void_p()
    _L.check(_L.lib().zero_device_alloc_contiguous(ctypes.byref(p), int(nbytes)), "zero_device_alloc_contiguous")
    return p.value or 0


def zero_device_free(ptr: int) -> None:
    _L.check(_L.lib().zero_device_free(ptr or None), "zero_device_free")


def zero_pool_counts():
    """(contiguous, fallback): how many segments zero_pool_alloc has handed
    out since the library was loaded, physically contiguous and fallen back
    to ordinary device memory."""
    c, f = ctypes.c_int64(), ctypes.c_int64()
    _L.check(_L.lib().zero_pool_counts(ctypes.byref(c), ctypes.byref(f)), "zero_pool_counts")
    return c.value, f.value


_POOLS = {}


def contiguous_pool(device=None):
    """A torch memory pool whose segments are physically contiguous device
    memory (zero_pool_alloc / zero_pool_free).  Allocate a shard's buffers
    inside it:

        with torch.cuda.use_mem_pool(Z.contiguous_pool()):
            master = torch.empty(S, dtype=torch.float32, device="cuda")

    Freed tensors return to the pool; the pool (one per device, kept for the
    life of the process) must outlive them."""
    import torch
    dev = torch.cuda.current_device() if device is None else torch.device(device).index
    if dev is None:
        dev = torch.cuda.current_device()
    if dev not in _POOLS:
        _L.lib()                                   # fails loudly if the library is missing
        alloc = torch.cuda.memory.CUDAPluggableAllocator(_L.LIB_PATH, "zero_pool_alloc", "zero_pool_free")
        with torch.cuda.device(dev):
            _POOLS[dev] = (alloc, torch.cuda.MemPool(alloc.allocator()))
    return _POOLS[dev][1]
