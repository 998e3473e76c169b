"""OffloadShardAdam: one rank's optimizer shard with its fp32 state in pinned
host memory (the CPU-offload lineage of ZeRO).

Per step: the norm/overflow pass runs where the gradient already is, on the
device (2 B/param at HBM speed); only its two scalars come back.  Then the
shard is processed in chunks as a pipeline over two copy streams: while the
host cores run the fused AdamW step (zero_cpu_shard_adam_step) on chunk j,
the gradient of chunk j+1 streams device-to-host and the 16-bit parameters of
chunk j-1 stream host-to-device.  Only 2 + 2 bytes per parameter cross PCIe;
the 12 bytes of fp32 state per parameter never leave host memory.  A skipped
step (overflow) moves nothing.  With device_norm=False the whole gradient is
fetched first and the norm pass also runs on the host.
"""
import time
from typing import Callable, Optional

import torch

from . import (ZERO_F32, AdamHyper, LossScaler, dtype_code, zero_cpu_shard_adam_step,
               zero_cpu_shard_unscale_norm_overflow, zero_loss_scaler_update, zero_norm_workspace_bytes,
               zero_shard_unscale_norm_overflow)


class OffloadShardAdam:
    def __init__(self, master: torch.Tensor, exp_avg: torch.Tensor, exp_avg_sq: torch.Tensor, *, grad_dtype,
                 param_dtype, lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, max_grad_norm=0.0,
                 scaler: Optional[LossScaler] = None, applied_steps: int = 0, nthreads: int = 0,
                 device_norm: bool = True, chunk: int = 1 << 25):
        n = master.numel()
        for t in (master, exp_avg, exp_avg_sq):
            if t.dtype != torch.float32 or t.is_cuda or t.numel() != n or not t.is_contiguous():
                raise ValueError("master / exp_avg / exp_avg_sq must be contiguous fp32 host tensors of equal size")
        self.master, self.exp_avg, self.exp_avg_sq, self.n = master, exp_avg, exp_avg_sq, n
        self.grad_dtype, self.param_dtype = grad_dtype, param_dtype
        self.hyper = dict(lr=lr, beta1=beta1, beta2=beta2, eps=eps, weight_decay=weight_decay,
                          max_grad_norm=max_grad_norm)
        self.scaler = scaler if scaler is not None else LossScaler.static(1.0)
        self.t = applied_steps
        self.nthreads = nthreads
        self.grad_host = torch.empty(n, dtype=grad_dtype, pin_memory=True)
        self.param_host = torch.empty(n, dtype=param_dtype, pin_memory=True)
        self.sqnorm, self.overflow = 0.0, False
        self._ready = torch.cuda.Event()
        self.device_norm, self.chunk = device_norm, max(1024, int(chunk) // 1024 * 1024)
        self._d2h = torch.cuda.Stream()        # default priority, like every stream here
        self._h2d = torch.cuda.Stream()
        self._ws = self._dsq = self._dovf = None
        self._scalars = torch.empty(2, dtype=torch.float64, pin_memory=True)
        self.last_times = {}          # seconds spent in each phase of the last step

    def chunk_bounds(self):
        """[(lo, hi)] of the pipeline's chunks.  The first and last chunks are
        small and double up to (and down from) `chunk`: the host starts once
        the first small chunk has crossed PCIe, and only a small last chunk's
        parameters cross back after the host has finished.  Bounds are
        multiples of 1024 elements except where the shard's ragged end falls."""
        ramp, s = [], max(1024, self.chunk // 8 // 1024 * 1024)
        while s < self.chunk:
            ramp.append(s)
            s *= 2
        if self.n <= 2 * sum(ramp) + self.chunk:
            return [(lo, min(self.n, lo + self.chunk)) for lo in range(0, self.n, self.chunk)]
        sizes = ramp[:]
        mid = self.n - 2 * sum(ramp)
        sizes += [self.chunk] * (mid // self.chunk) + ([mid % self.chunk] if mid % self.chunk else [])
        sizes += ramp[::-1]
        bounds, lo = [], 0
        for k in sizes:
            bounds.append((lo, lo + k))
            lo += k
        return bounds

    def fetch_grad(self, grad_dev: torch.Tensor) -> None:
        """Whole device gradient shard -> pinned host buffer (waits for the copy)."""
        self.grad_host.copy_(grad_dev, non_blocking=True)
        self._ready.record()
        self._ready.synchronize()

    def _inv(self) -> float:
        return 1.0 if dtype_code(self.grad_host) == ZERO_F32 else 1.0 / self.scaler.scale

    def unscale_norm(self) -> None:
        """Host norm pass over the fetched gradient."""
        self.sqnorm, self.overflow = zero_cpu_shard_unscale_norm_overflow(self.grad_host, self._inv(),
                                                                          nthreads=self.nthreads)

    def device_unscale_norm(self, grad_dev: torch.Tensor) -> None:
        """Norm pass on the device; brings back only (sum of squares, flag)."""
        if self._ws is None:
            dev = grad_dev.device
            self._ws = torch.empty(zero_norm_workspace_bytes(self.n), dtype=torch.uint8, device=dev)
            self._dsq = torch.empty(1, dtype=torch.float64, device=dev)
            self._dovf = torch.empty(1, dtype=torch.int32, device=dev)
        zero_shard_unscale_norm_overflow(grad_dev, self._inv(), self._dsq, self._dovf, self._ws)
        pair = torch.cat([self._dsq, self._dovf.to(torch.float64)])
        self._scalars.copy_(pair, non_blocking=True)
        self._ready.record()
        self._ready.synchronize()
        self.sqnorm, self.overflow = float(self._scalars[0]), bool(self._scalars[1] != 0)

    def step(self, grad_dev: torch.Tensor, param_dev: Optional[torch.Tensor] = None,
             allreduce: Optional[Callable[[float, bool], tuple]] = None) -> bool:
        """One step; `allreduce(sq, overflow) -> (sq, overflow)` stands for the
        data-parallel reduction of the two scalars.  Returns True if skipped."""
        t0 = time.perf_counter()
        if self.device_norm:
            self.device_unscale_norm(grad_dev)
        else:
            self.fetch_grad(grad_dev)
            self.unscale_norm()
        t1 = time.perf_counter()
        sq, ovf = (self.sqnorm, self.overflow) if allreduce is None else allreduce(self.sqnorm, self.overflow)
        hp = AdamHyper(step=self.t + 1, inv_loss_scale=self._inv(), **self.hyper)
        skip = zero_loss_scaler_update(self.scaler, ovf)
        if skip:
            self.last_times = {"norm": t1 - t0, "pipeline": 0.0}
            return True
        self.t += 1
        chunks = self.chunk_bounds()
        cur = torch.cuda.current_stream()
        arrived = []
        if self.device_norm:
            # gradient chunks stream to the host in order, behind the producer of grad_dev
            self._d2h.wait_stream(cur)
            with torch.cuda.stream(self._d2h):
                for lo, hi in chunks:
                    self.grad_host[lo:hi].copy_(grad_dev[lo:hi], non_blocking=True)
                    ev = torch.cuda.Event()
                    ev.record(self._d2h)
                    arrived.append(ev)
        if param_dev is not None:
            self._h2d.wait_stream(cur)
        for j, (lo, hi) in enumerate(chunks):
            if arrived:
                arrived[j].synchronize()
            zero_cpu_shard_adam_step(self.master[lo:hi], self.exp_avg[lo:hi], self.exp_avg_sq[lo:hi],
                                     self.grad_host[lo:hi], self.param_host[lo:hi], hp, sq, ovf,
                                     nthreads=self.nthreads)
            if param_dev is not None:
                with torch.cuda.stream(self._h2d):
                    param_dev[lo:hi].copy_(self.param_host[lo:hi], non_blocking=True)
        if param_dev is not None:
            self._h2d.synchronize()
            cur.wait_stream(self._h2d)
        t2 = time.perf_counter()
        self.last_times = {"norm": t1 - t0, "pipeline": t2 - t1}
        return False
