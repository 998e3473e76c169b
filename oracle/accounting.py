"""Model-state memory accounting (oracle).

[Explainer, "The 16 Bytes per Parameter Audit"] and [Explainer, Ch.02 "The
Three Stages", memory-per-parameter list]: with mixed-precision Adam a
parameter costs a 2-byte fp16 weight, a 4-byte fp32 master copy and two 4-byte
fp32 moments; the gradient adds bytes of its own.  The pages' own totals
disagree at the edges ("16", "16-20"; the audit's list sums to 14 before the
gradient).  The reading taken is 16 = 2 (fp16 weight) + 2 (fp16 gradient) +
12 (fp32 master, momentum, variance): it is the only split that reproduces the
pages' 7B -> ~112 GB (Audit), 100B -> ~1.6 TB ([Explainer, Ch.01 "The
Replication Trap"]) and the ~4x / ~8x stage reductions ([Explainer, Ch.01 "The
ZeRO Answer"], [Explainer, Ch.05 stage table]).  The optional fp32 gradient
copy (+4) is reported separately and not part of the 16.

Per-rank bytes by stage, Psi parameters over N_d ranks:
  baseline DP      16 Psi                  (everything replicated)
  P_os             4 Psi + 12 Psi / N_d    (optimizer states sharded)
  P_os+g           2 Psi + 14 Psi / N_d    (+ gradients)
  P_os+g+p         16 Psi / N_d            (+ parameters)

Communication per training step ([Explainer, Ch.02 "The Three Stages", what
each stage shards; Ch.05 stage table, extra-communication column]): baseline
DP all-reduces the gradient; the first two stages move about the same volume;
the third moves half as much again, gathering parameters and reduce-scattering
gradients.  Reading: ring collectives, in which a reduce-scatter or an
all-gather of a Psi-element buffer has every rank send (N_d - 1) / N_d * Psi
elements and an all-reduce is the two in turn.  DP: one all-reduce of the
gradient (2 units).  P_os and P_os+g: a reduce-scatter of the gradient, so
each rank holds the reduced gradient of its partition, then an all-gather of
the updated parameters (2 units).  P_os+g+p: each rank keeps only its
partition of the parameters, so they are all-gathered before the forward pass
and again before the backward pass, and the gradient is reduce-scattered
after it (3 units, half as much again as DP).
"""
from fractions import Fraction

FP16_WEIGHT = 2
FP16_GRAD = 2
FP32_MASTER = 4
FP32_MOMENTS = 8           # momentum + variance
FP32_GRAD_COPY = 4         # optional, not in the 16

STAGES = ("dp", "os", "os+g", "os+g+p")


def model_state_bytes_per_param(fp32_grad_copy: bool = False) -> int:
    return FP16_WEIGHT + FP16_GRAD + FP32_MASTER + FP32_MOMENTS + (FP32_GRAD_COPY if fp32_grad_copy else 0)


def per_rank_state_bytes(stage: str, psi: int, n_d: int) -> Fraction:
    """Exact bytes of model state held by one rank."""
    if stage not in STAGES:
        raise ValueError(stage)
    opt = FP32_MASTER + FP32_MOMENTS            # 12
    replicated = {"dp": FP16_WEIGHT + FP16_GRAD + opt,
                  "os": FP16_WEIGHT + FP16_GRAD,
                  "os+g": FP16_WEIGHT,
                  "os+g+p": 0}[stage]
    sharded = model_state_bytes_per_param() - replicated
    return Fraction(replicated * psi) + Fraction(sharded * psi, n_d)


def reduction_factor(stage: str, psi: int, n_d: int) -> Fraction:
    """Per-rank memory of baseline DP divided by that of `stage`."""
    return per_rank_state_bytes("dp", psi, n_d) / per_rank_state_bytes(stage, psi, n_d)


COLLECTIVES_PER_STEP = {"dp": 2, "os": 2, "os+g": 2, "os+g+p": 3}   # reduce-scatter / all-gather units


def communication_elements(stage: str, psi: int, n_d: int) -> Fraction:
    """Elements one rank sends per training step (ring collectives)."""
    if stage not in STAGES:
        raise ValueError(stage)
    if n_d < 1:
        raise ValueError("n_d >= 1")
    return COLLECTIVES_PER_STEP[stage] * Fraction((n_d - 1) * psi, n_d)
