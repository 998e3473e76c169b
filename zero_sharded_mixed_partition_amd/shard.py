"""ShardAdam: one rank's optimizer shard driven through the C ABI.

A step is: (optionally, micro-batch by micro-batch, accumulate the 16-bit
gradients into an fp32 copy), enqueue the unscale/overflow/norm pass on the
gradient shard (16-bit, or the fp32 copy),
(in a multi-rank job: all-reduce the two scalars), enqueue the fused AdamW
pass, then read the 4-byte overflow flag back to update the loss scale and the
step counter on the host.  The flag read is the step's only device-to-host
transfer; the skip itself is decided on the device from the same flag, so the
kernels never wait for the host.

With device_state=True the loss scale and the step counter live in device
memory instead (zero_step_state): the norm pass reads the scale there, and a
one-thread kernel forms the step's coefficients and advances the scaler after
the overflow flag is known.  A step then never waits for the device; step()
returns None and read_state() brings the scaler and counts back on demand.
"""
from typing import Callable, Optional

import torch

from . import (ZERO_F32, AdamHyper, LossScaler, StepGraph, StepGraphDev, StepState, dtype_code, zero_adam_coef_bytes,
               zero_loss_scaler_update, zero_norm_workspace_bytes, zero_shard_adam_step,
               zero_shard_grad_accumulate, zero_shard_grad_accumulate_dev, zero_shard_grad_reduce,
               zero_shard_adam_step_coef, zero_shard_grad_reduce_dev, zero_shard_grad_sum_norm,
               zero_shard_grad_sum_norm_dev, zero_sum_norm_workspace_bytes, zero_shard_unscale_norm_overflow,
               zero_shard_norm_decide_dev, zero_shard_unscale_norm_overflow_dev, zero_step_decide_dev)


class ShardAdam:
    def __init__(self, master: torch.Tensor, exp_avg: torch.Tensor, exp_avg_sq: torch.Tensor, *,
                 lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, max_grad_norm=0.0,
                 scaler: Optional[LossScaler] = None, applied_steps: int = 0, graph: bool = False,
                 device_state: bool = False):
        n = master.numel()
        for t in (master, exp_avg, exp_avg_sq):
            if t.dtype != torch.float32 or not t.is_cuda or t.numel() != n or not t.is_contiguous():
                raise ValueError("master / exp_avg / exp_avg_sq must be contiguous fp32 device tensors of equal size")
        self.master, self.exp_avg, self.exp_avg_sq, self.n = master, exp_avg, exp_avg_sq, n
        self.hyper = dict(lr=lr, beta1=beta1, beta2=beta2, eps=eps, weight_decay=weight_decay,
                          max_grad_norm=max_grad_norm)
        self.scaler = scaler if scaler is not None else LossScaler.static(1.0)
        self.t = applied_steps
        dev = master.device
        self.workspace = torch.empty(zero_norm_workspace_bytes(n), dtype=torch.uint8, device=dev)
        self.sqnorm = torch.empty(1, dtype=torch.float64, device=dev)
        self.overflow = torch.empty(1, dtype=torch.int32, device=dev)
        self._flag_host = torch.empty(1, dtype=torch.int32, pin_memory=True)
        self._flag_ready = torch.cuda.Event()
        # graph mode: one recorded step replayed per step (re-recorded when the
        # buffers or the loss scale change); used when no all-reduce hook is given
        self.graph = graph
        self._graph, self._graph_key = None, None
        self.recorded_this_step = False
        self.state = StepState(self.scaler, applied_steps, dev) if device_state else None
        self._sum_ws = None           # workspace of the fused copy-and-norm pass, made on first use
        self.d_coef = torch.empty(zero_adam_coef_bytes(), dtype=torch.uint8, device=dev) if device_state else None

    def _inv_scale(self, grad: torch.Tensor) -> float:
        # an fp32 gradient is the accumulation copy, already unscaled
        return 1.0 if dtype_code(grad) == ZERO_F32 else 1.0 / self.scaler.scale

    def _sum_norm(self, acc: torch.Tensor, slices, add: bool) -> None:
        if self._sum_ws is None:
            self._sum_ws = torch.empty(zero_sum_norm_workspace_bytes(self.n), dtype=torch.uint8, device=acc.device)
        if self.state is not None:
            zero_shard_grad_sum_norm_dev(acc, slices, add, self.state, self.sqnorm, self.overflow, self._sum_ws)
        else:
            zero_shard_grad_sum_norm(acc, slices, add, 1.0 / self.scaler.scale, self.sqnorm, self.overflow,
                                     self._sum_ws)

    def accumulate(self, acc: torch.Tensor, grad: torch.Tensor, first: bool,
                   overflow: Optional[torch.Tensor] = None, last: bool = False) -> None:
        """Enqueue one micro-batch into the fp32 gradient copy `acc`
        (acc = (first ? 0 : acc) + grad / loss_scale).  last=True fuses the
        norm pass of the finished copy into this pass; then call
        step(acc, ..., norm_done=True)."""
        if last:
            self._sum_norm(acc, [grad], not first)
            return
        if self.state is not None:
            zero_shard_grad_accumulate_dev(acc, grad, self.state, first, overflow)
        else:
            zero_shard_grad_accumulate(acc, grad, 1.0 / self.scaler.scale, first, overflow)

    def reduce(self, acc: torch.Tensor, slices, overflow: Optional[torch.Tensor] = None,
               with_norm: bool = False) -> None:
        """Enqueue the reduction of the data-parallel ranks' gradient slices of
        this partition into the fp32 gradient copy `acc` (slice order,
        acc = sum_k slice_k / loss_scale).  with_norm=True fuses the norm pass
        of the copy into it; then call step(acc, ..., norm_done=True)."""
        if with_norm:
            self._sum_norm(acc, slices, False)
            return
        if self.state is not None:
            zero_shard_grad_reduce_dev(acc, slices, self.state, overflow)
        else:
            zero_shard_grad_reduce(acc, slices, 1.0 / self.scaler.scale, overflow)

    def unscale_norm(self, grad: torch.Tensor) -> None:
        """Enqueue steps 1-2: self.sqnorm, self.overflow <- this shard's values."""
        if self.state is not None:
            zero_shard_unscale_norm_overflow_dev(grad, self.state, self.sqnorm, self.overflow, self.workspace)
            return
        zero_shard_unscale_norm_overflow(grad, self._inv_scale(grad), self.sqnorm, self.overflow, self.workspace)

    def apply(self, grad: torch.Tensor, param_out: Optional[torch.Tensor], global_sqnorm=None,
              global_overflow=None) -> None:
        """Enqueue steps 3-4 for step index t+1 (skipped on device on overflow)."""
        if self.state is not None:
            self.decide(grad, global_overflow)
            self.update(grad, param_out, global_sqnorm, global_overflow)
            return
        hp = AdamHyper(step=self.t + 1, inv_loss_scale=self._inv_scale(grad), **self.hyper)
        zero_shard_adam_step(self.master, self.exp_avg, self.exp_avg_sq, grad, param_out, hp,
                             self.sqnorm if global_sqnorm is None else global_sqnorm,
                             self.overflow if global_overflow is None else global_overflow,
                             grad_dtype=dtype_code(grad))

    def norm_decide(self, grad: torch.Tensor) -> None:
        """device_state, one rank: the norm pass with the decision folded
        into its final kernel."""
        zero_shard_norm_decide_dev(grad, AdamHyper(**self.hyper), self.state, self.sqnorm, self.overflow,
                                   self.d_coef, self.workspace)

    def decide(self, grad: torch.Tensor, global_overflow=None) -> None:
        """device_state: enqueue the decision kernel (coefficients of the
        next step into d_coef, scaler and counts advanced by the flag)."""
        zero_step_decide_dev(AdamHyper(**self.hyper), grad.dtype, self.state,
                             self.overflow if global_overflow is None else global_overflow, self.d_coef)

    def update(self, grad: torch.Tensor, param_out: Optional[torch.Tensor], global_sqnorm=None,
               global_overflow=None) -> None:
        """device_state: enqueue the fused update with the coefficients in d_coef."""
        zero_shard_adam_step_coef(self.master, self.exp_avg, self.exp_avg_sq, grad, param_out, self.d_coef,
                                  self.sqnorm if global_sqnorm is None else global_sqnorm,
                                  self.overflow if global_overflow is None else global_overflow)

    def finish(self, global_overflow: Optional[torch.Tensor] = None) -> Optional[bool]:
        """Read the overflow flag, update the loss scale and t; returns skip
        (None with device_state: nothing to do on the host)."""
        if self.state is not None:
            return None
        flag = self.overflow if global_overflow is None else global_overflow
        self._flag_host.copy_(flag, non_blocking=True)
        self._flag_ready.record()
        self._flag_ready.synchronize()
        skip = zero_loss_scaler_update(self.scaler, bool(self._flag_host.item()))
        if not skip:
            self.t += 1
        return skip

    def step(self, grad: torch.Tensor, param_out: Optional[torch.Tensor] = None,
             allreduce: Optional[Callable[[torch.Tensor, torch.Tensor], None]] = None,
             norm_done: bool = False) -> Optional[bool]:
        """One full step.  `allreduce(sqnorm, overflow)`, if given, must turn
        this rank's two scalars into the data-parallel sum / OR in place (on
        one GPU the shard's own values are the global ones).  Returns True if
        the step was skipped (None with device_state, which never waits).
        norm_done: the norm and flag of `grad` (the fp32 copy) were formed by
        accumulate(last=True) or reduce(with_norm=True)."""
        if norm_done:
            if allreduce is not None:
                allreduce(self.sqnorm, self.overflow)
            if self.state is not None:
                self.decide(grad)
                self.update(grad, param_out)
                return None
            self.apply(grad, param_out)
            return self.finish()
        if self.graph and allreduce is None:
            if self.state is not None:
                self._graph_step_dev(grad, param_out)
                return None
            return self._graph_step(grad, param_out)
        if self.state is not None and allreduce is None:
            self.norm_decide(grad)          # one rank: its flag is the global one
            self.update(grad, param_out)
            return None
        self.unscale_norm(grad)
        if allreduce is not None:
            allreduce(self.sqnorm, self.overflow)
        self.apply(grad, param_out)
        return self.finish()

    def read_state(self):
        """device_state: copy the state to the host (waits for the steps
        enqueued so far), refresh self.t and self.scaler from it and return it."""
        st = self.state.read()
        self.t = st.applied
        self.scaler.s = type(self.scaler.s).from_buffer_copy(bytes(st.scaler))
        return st

    def _graph_step_dev(self, grad: torch.Tensor, param_out: Optional[torch.Tensor]) -> None:
        # with device state a recording depends only on the buffers (and the hyperparameters)
        key = ("dev", grad.data_ptr(), grad.dtype, grad.numel(),
               None if param_out is None else (param_out.data_ptr(), param_out.dtype), tuple(self.hyper.items()))
        self.recorded_this_step = key != self._graph_key
        if self.recorded_this_step:
            if self._graph is not None:
                self._graph.close()
            self._graph = StepGraphDev(self.master, self.exp_avg, self.exp_avg_sq, grad, param_out,
                                       AdamHyper(**self.hyper), self.state, self.sqnorm, self.overflow, self.d_coef,
                                       self.workspace)
            self._graph_key = key
        self._graph.launch()

    def _graph_step(self, grad: torch.Tensor, param_out: Optional[torch.Tensor]) -> bool:
        inv = self._inv_scale(grad)
        key = (grad.data_ptr(), grad.dtype, grad.numel(),
               None if param_out is None else (param_out.data_ptr(), param_out.dtype), inv)
        self.recorded_this_step = key != self._graph_key
        if self.recorded_this_step:
            if self._graph is not None:
                self._graph.close()
            self._graph = StepGraph(self.master, self.exp_avg, self.exp_avg_sq, grad, param_out, inv, self.sqnorm,
                                    self.overflow, self.workspace)
            self._graph_key = key
        self._graph.launch(AdamHyper(step=self.t + 1, inv_loss_scale=inv, **self.hyper))
        skip = zero_loss_scaler_update(self.scaler, self._graph.overflow())
        if not skip:
            self.t += 1
        return skip
