"""ctypes loader for libzero_shard.so (C ABI declared in include/zero_shard.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation of any step.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libzero_shard.so")

ZERO_OK, ZERO_EINVAL, ZERO_EALIGN, ZERO_ERANGE, ZERO_ENOSPC, ZERO_EHIP = 0, -1, -2, -3, -4, -5
ZERO_F16, ZERO_BF16, ZERO_F32 = 1, 2, 3

c_i32, c_i64, c_dbl, c_vp, c_sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p, ctypes.c_size_t
P_i64 = ctypes.POINTER(c_i64)
P_i32 = ctypes.POINTER(c_i32)


class zero_fragment(ctypes.Structure):
    _fields_ = [("tensor", c_i32), ("reserved", c_i32), ("tensor_begin", c_i64),
                ("shard_begin", c_i64), ("numel", c_i64)]


class zero_adam_params(ctypes.Structure):
    _fields_ = [("lr", c_dbl), ("beta1", c_dbl), ("beta2", c_dbl), ("eps", c_dbl),
                ("weight_decay", c_dbl), ("step", c_i64), ("inv_loss_scale", c_dbl),
                ("max_grad_norm", c_dbl)]


class zero_loss_scaler(ctypes.Structure):
    _fields_ = [("scale", c_dbl), ("min_scale", c_dbl), ("backoff", c_dbl), ("growth", c_dbl),
                ("growth_interval", c_i64), ("good_steps", c_i64)]


class zero_adam_hyper(ctypes.Structure):
    _fields_ = [("lr", c_dbl), ("beta1", c_dbl), ("beta2", c_dbl), ("eps", c_dbl), ("weight_decay", c_dbl),
                ("max_grad_norm", c_dbl)]


class zero_step_state(ctypes.Structure):
    _fields_ = [("scaler", zero_loss_scaler), ("applied", c_i64), ("skipped", c_i64), ("last_overflow", c_i32),
                ("reserved", c_i32)]


# name -> (restype, argtypes); every symbol the header declares
SIGNATURES = {
    "zero_abi_version": (c_i32, []),
    "zero_partition_plan": (c_i32, [P_i64, P_i32, c_i32, c_i32, c_i64, P_i64, P_i64, P_i64]),
    "zero_rank_fragments": (c_i32, [P_i64, P_i32, c_i32, c_i32, c_i64, c_i32,
                                    ctypes.POINTER(zero_fragment), c_i32, P_i32]),
    "zero_norm_workspace_bytes": (c_sz, [c_i64]),
    "zero_shard_unscale_norm_overflow": (c_i32, [c_vp, c_i32, c_i64, c_dbl, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "zero_shard_unscale_norm_overflow_noalloc": (c_i32, [c_vp, c_i32, c_i64, c_dbl, c_vp, c_vp, c_vp]),
    "zero_shard_adam_step": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_i32, c_vp, c_i32, c_i64,
                                     ctypes.POINTER(zero_adam_params), c_vp, c_vp, c_vp]),
    "zero_shard_grad_accumulate": (c_i32, [c_vp, c_vp, c_i32, c_i64, c_dbl, c_i32, c_vp, c_vp]),
    "zero_shard_grad_reduce": (c_i32, [c_vp, ctypes.POINTER(c_vp), c_i32, c_i32, c_i64, c_dbl, c_vp, c_vp]),
    "zero_adam_coef_bytes": (c_sz, []),
    "zero_adam_prepare": (c_i32, [ctypes.POINTER(zero_adam_params), c_vp]),
    "zero_shard_adam_step_coef": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_i32, c_vp, c_i32, c_i64, c_vp, c_vp, c_vp, c_vp]),
    "zero_step_graph_create": (c_i32, [ctypes.POINTER(c_vp), c_vp, c_vp, c_vp, c_vp, c_i32, c_vp, c_i32, c_i64,
                                       c_dbl, c_vp, c_vp, c_vp, c_sz]),
    "zero_step_graph_launch": (c_i32, [c_vp, ctypes.POINTER(zero_adam_params), c_vp]),
    "zero_step_graph_overflow": (c_i32, [c_vp, P_i32]),
    "zero_step_graph_destroy": (c_i32, [c_vp]),
    "zero_step_graph_create_dev": (c_i32, [ctypes.POINTER(c_vp), c_vp, c_vp, c_vp, c_vp, c_i32, c_vp, c_i32, c_i64,
                                           ctypes.POINTER(zero_adam_hyper), c_vp, c_vp, c_vp, c_vp, c_vp, c_sz]),
    "zero_step_graph_launch_dev": (c_i32, [c_vp, c_vp]),
    "zero_sum_norm_workspace_bytes": (c_sz, [c_i64]),
    "zero_shard_grad_sum_norm": (c_i32, [c_vp, ctypes.POINTER(c_vp), c_i32, c_i32, c_i64, c_i32, c_dbl, c_vp, c_vp,
                                         c_vp, c_sz, c_vp]),
    "zero_shard_grad_sum_norm_dev": (c_i32, [c_vp, ctypes.POINTER(c_vp), c_i32, c_i32, c_i64, c_i32,
                                             ctypes.POINTER(zero_adam_hyper), c_vp, c_vp, c_vp, c_vp, c_vp, c_sz,
                                             c_vp]),
    "zero_cpu_shard_unscale_norm_overflow": (c_i32, [c_vp, c_i32, c_i64, c_dbl, ctypes.POINTER(c_dbl), P_i32, c_i32]),
    "zero_cpu_shard_adam_step": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_i32, c_vp, c_i32, c_i64,
                                         ctypes.POINTER(zero_adam_params), c_dbl, c_i32, c_i32]),
    "zero_cpu_copy_reference": (c_i32, [c_vp, c_vp, c_i64, c_i32]),
    "zero_loss_scaler_update": (c_i32, [ctypes.POINTER(zero_loss_scaler), c_i32, P_i32]),
    "zero_copy_reference": (c_i32, [c_vp, c_vp, c_i64, c_vp]),
    "zero_copy_widen_reference": (c_i32, [c_vp, c_vp, c_i64, c_vp]),
    "zero_device_alloc_contiguous": (c_i32, [ctypes.POINTER(c_vp), c_sz]),
    "zero_device_free": (c_i32, [c_vp]),
    "zero_pool_alloc": (c_vp, [c_sz, c_i32, c_vp]),
    "zero_pool_free": (None, [c_vp, c_sz, c_i32, c_vp]),
    "zero_pool_counts": (c_i32, [ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64)]),
    "zero_norm_combine_ranks": (c_i32, [c_vp, c_vp, c_i32, c_vp, c_vp, c_vp]),
    "zero_shard_unscale_norm_overflow_dev": (c_i32, [c_vp, c_i32, c_i64, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "zero_shard_norm_decide_dev": (c_i32, [c_vp, c_i32, c_i64, ctypes.POINTER(zero_adam_hyper), c_vp, c_vp, c_vp,
                                           c_vp, c_vp, c_sz, c_vp]),
    "zero_step_decide_dev": (c_i32, [ctypes.POINTER(zero_adam_hyper), c_i32, c_vp, c_vp, c_vp, c_vp]),
    "zero_shard_adam_step_dev": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_i32, c_vp, c_i32, c_i64,
                                         ctypes.POINTER(zero_adam_hyper), c_vp, c_vp, c_vp, c_vp, c_vp]),
    "zero_shard_grad_accumulate_dev": (c_i32, [c_vp, c_vp, c_i32, c_i64, c_vp, c_i32, c_vp, c_vp]),
    "zero_shard_grad_reduce_dev": (c_i32, [c_vp, ctypes.POINTER(c_vp), c_i32, c_i32, c_i64, c_vp, c_vp, c_vp]),
    "zero_status_string": (ctypes.c_char_p, [c_i32]),
    "zero_last_error": (ctypes.c_char_p, []),
}


class ZeroShardError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({detail})")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (loaded once).  Raises ImportError if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run "
                              "`python -m zero_sharded_mixed_partition_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


def check(status: int, where: str) -> None:
    if status != ZERO_OK:
        L = lib()
        detail = L.zero_last_error().decode() or L.zero_status_string(status).decode()
        raise ZeroShardError(status, where, detail)
