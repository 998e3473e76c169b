"""CPU oracle for one ZeRO rank's partitioned mixed-precision Adam step.

TEST INFRASTRUCTURE ONLY.  This package is the slow, plain reference that the
HIP path is checked against.  Only the test suite, the package smoke check and
the benchmark's CPU-baseline leg may import or run it; the product path never
does, and this package imports nothing from the product package (the two
share no code; only the seeded input generator in `workloads` feeds both).

It computes in float64 (Python ints for sizes) and rounds to the storage
formats (fp32 state, fp16/bf16 parameter copy) only at the end of a step.

Sources.  The method is described on three web pages about ZeRO:
  * the ZeRO method entry (Sharded Data Parallel Methods catalogue),
    "description";
  * the ZeRO glossary entry ("Zero Redundancy Optimizer"), "description";
  * the interactive explainer "Data Parallelism Without the Copies" of
    "ZeRO: Memory Optimizations Toward Training Trillion Parameter Models",
    cited below as [Explainer] with its section: "The 16 Bytes per Parameter
    Audit", Chapter 01 "Trained Everywhere, Stored Everywhere", Chapter 02
    "The Three Stages" (memory-per-parameter list, what each stage shards),
    Chapter 05 "Super-Linear Scaling" (stage table).
The pages name mixed-precision Adam but never print its update rule, loss
scaling, overflow handling or clipping.  Those steps follow the published
methods named at each function (Kingma & Ba 2015 "Adam"; Loshchilov & Hutter
2019 "Decoupled Weight Decay Regularization"; Micikevicius et al. 2018 "Mixed
Precision Training" for loss scaling; Pascanu et al. 2013 for norm clipping)
and the plainest reading the rest of the pages support.

Pins: every function here is checked by the `-m "not gpu"` tests against
facts fixed independently of this code (the pages' printed figures, closed
forms, exhaustive enumeration, library routines, brute force).  The Adam update
formula itself is not printed on the pages: there it is pinned by closed forms
and by torch.optim.AdamW on the CPU, not by the pages ("parity unpinned" by the
pages for the update formula; pinned by the textbook method).
"""
from .plan import partition_plan, rank_fragments, rank_range  # noqa: F401
from .accounting import (model_state_bytes_per_param, per_rank_state_bytes, reduction_factor,  # noqa: F401
                         communication_elements)
from .formats import decode16, is_nonfinite16, encode16_rne  # noqa: F401
from .adam import (shard_sqnorm_overflow, global_sqnorm_overflow, sqnorm_terms,  # noqa: F401
                   combine_sqnorm_terms, SqnormTerms, clip_coefficient, grad_scale, adam_update,
                   grad_accumulate, grad_reduce, LossScalerState, loss_scaler_update, shard_step)
