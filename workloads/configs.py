"""Synthetic workload definitions for the partitioned mixed-precision Adam shard step.

Each workload names a model's parameter-shape list (list order = flattening
order), the data-parallel degree N_d, the partition alignment, the rank whose
shard is stepped, the 16-bit gradient/parameter format, the distributions the
seeded generator draws from, and the optimizer hyperparameters.  Nothing here
computes any part of the method: sizes, offsets and partitions are derived by
the code under test and, independently, by the oracle.

No dataset or trained weights are involved anywhere: the model families below
only fix tensor shapes, which are architecture facts (GPT-2 small, Llama-7B,
GPT-style stacks at 100B and 1T parameters).
"""
from dataclasses import dataclass, field
from typing import List, Optional, Tuple


def gpt_shapes(d: int, n_layers: int, vocab: int = 50257, n_pos: int = 2048) -> List[Tuple[int, ...]]:
    """GPT-2-style list: token + position embeddings, per layer LN1 (w,b),
    fused QKV (w,b), attention projection (w,b), LN2 (w,b), MLP up (w,b),
    MLP down (w,b); final LN (w,b)."""
    shapes: List[Tuple[int, ...]] = [(vocab, d), (n_pos, d)]
    for _ in range(n_layers):
        shapes += [(d,), (d,), (d, 3 * d), (3 * d,), (d, d), (d,),
                   (d,), (d,), (d, 4 * d), (4 * d,), (4 * d, d), (d,)]
    shapes += [(d,), (d,)]
    return shapes


def llama_shapes(d: int = 4096, n_layers: int = 32, ffn: int = 11008,
                 vocab: int = 32000) -> List[Tuple[int, ...]]:
    """Llama-style list: embedding, per layer attention RMSNorm, wq/wk/wv/wo,
    FFN RMSNorm, gate/up/down projections; final norm; untied LM head."""
    shapes: List[Tuple[int, ...]] = [(vocab, d)]
    for _ in range(n_layers):
        shapes += [(d,), (d, d), (d, d), (d, d), (d, d), (d,),
                   (ffn, d), (ffn, d), (d, ffn)]
    shapes += [(d,), (vocab, d)]
    return shapes


@dataclass(frozen=True)
class Dist:
    """A value distribution: kind is 'zero', 'normal' (mean 0, std a) or
    'uniform' on [a, b)."""
    kind: str
    a: float = 0.0
    b: float = 0.0


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int                      # seed component identifying the workload
    shapes: Tuple[Tuple[int, ...], ...]
    n_d: int
    align: int
    rank: int
    grad_dtype: str               # 'f16' or 'bf16'
    param_dtype: str              # 'f16' or 'bf16'
    master: Dist
    exp_avg: Dist
    exp_avg_sq: Dist
    grad: Dist                    # distribution of the *unscaled* gradient
    loss_scale: float             # grads are stored as 16-bit(g * loss_scale)
    step: int                     # 1-based index of the (first) step applied
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.0
    max_grad_norm: float = 0.0    # <= 0: no clipping
    param_layout: str = "zero2"   # 'zero2': param buffer is the full N_d*S flat
                                  # buffer; 'zero3': shard-local param buffer
    n_steps: int = 1              # steps in the trajectory workloads
    inf_steps: Tuple[int, ...] = field(default=())   # 1-based iterations with inf injected
    inf_fraction: float = 0.0


_ADAM_STATE = dict(exp_avg=Dist("normal", 1e-3), exp_avg_sq=Dist("uniform", 1e-8, 1e-5))

TINY = Workload(
    name="tiny_4tensors_nd4_rank1", wid=1,
    shapes=((512, 512), (512,), (1024, 512), (512,)),
    n_d=4, align=128, rank=1, grad_dtype="f16", param_dtype="f16",
    master=Dist("normal", 0.02), exp_avg=Dist("zero"), exp_avg_sq=Dist("zero"),
    grad=Dist("normal", 1e-2), loss_scale=1024.0, step=1,
    weight_decay=0.0, max_grad_norm=0.0)

GPT2_SMALL = Workload(
    name="gpt2_small_124m_nd8_rank3", wid=2,
    shapes=tuple(gpt_shapes(768, 12, n_pos=1024)),
    n_d=8, align=128, rank=3, grad_dtype="f16", param_dtype="f16",
    master=Dist("normal", 0.02), grad=Dist("normal", 1e-3), loss_scale=65536.0,
    step=100, weight_decay=0.01, max_grad_norm=1.0, **_ADAM_STATE)

LLAMA_7B = Workload(
    name="llama_7b_nd1", wid=3,
    shapes=tuple(llama_shapes()),
    n_d=1, align=512, rank=0, grad_dtype="bf16", param_dtype="bf16",
    master=Dist("normal", 0.02), grad=Dist("normal", 1e-3), loss_scale=1.0,
    step=1000, weight_decay=0.1, max_grad_norm=1.0, **_ADAM_STATE)

GPT_100B_RANK = Workload(
    name="gpt_100b_nd400_rank200", wid=4,
    shapes=tuple(gpt_shapes(8192, 124)),
    n_d=400, align=512, rank=200, grad_dtype="f16", param_dtype="f16",
    master=Dist("normal", 0.02), exp_avg=Dist("zero"), exp_avg_sq=Dist("zero"),
    grad=Dist("normal", 1e-3), loss_scale=65536.0, step=1,
    weight_decay=0.01, max_grad_norm=1.0,
    n_steps=20, inf_steps=(5, 12), inf_fraction=0.001)

GPT_1T_LAST_RANK = Workload(
    name="gpt_1t_nd1024_last_rank", wid=5,
    shapes=tuple(gpt_shapes(16384, 310)),
    n_d=1024, align=512, rank=1023, grad_dtype="bf16", param_dtype="bf16",
    master=Dist("normal", 0.02), grad=Dist("normal", 1e-4), loss_scale=1.0,
    step=10000, weight_decay=0.1, max_grad_norm=1.0, param_layout="zero3",
    **_ADAM_STATE)

WORKLOADS = {w.name: w for w in (TINY, GPT2_SMALL, LLAMA_7B, GPT_100B_RANK, GPT_1T_LAST_RANK)}
# short aliases used on command lines
ALIASES = {"tiny": TINY.name, "gpt2": GPT2_SMALL.name, "llama7b": LLAMA_7B.name,
           "gpt100b": GPT_100B_RANK.name, "gpt1t": GPT_1T_LAST_RANK.name}


def get(name: str) -> Workload:
    return WORKLOADS[ALIASES.get(name, name)]


def numel(shape: Tuple[int, ...]) -> int:
    """Element count of one tensor (a scalar has one element)."""
    n = 1
    for d in shape:
        n *= int(d)
    return n


def real_total(w: Workload) -> int:
    """Number of real (unpadded) model parameters: the generator needs it to
    emit zeros for the padding tail."""
    return sum(numel(s) for s in w.shapes)


def opt_hparams(w: Optional[Workload] = None, **over) -> dict:
    base = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                weight_decay=w.weight_decay, max_grad_norm=w.max_grad_norm) if w else {}
    base.update(over)
    return base
