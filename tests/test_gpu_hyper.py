"""GPU: the fused AdamW step over a sweep of hyperparameters and gradient
magnitudes, through both ways of supplying the step's coefficients (by value
from the host, and formed on the device from the step state), against the
oracle, and the two bit-identical to each other.

The cases reach the corners of the update rule: the first step from zero
moments, both betas zero, a short second-moment horizon with a large eps,
lr = 0, a very late step (both bias corrections round to 1 in float32),
a decay factor of one half, all-zero gradients (pure weight decay), tiny
gradients (down to 1e-15, second moments still normal float32 numbers) with
a tiny eps, a loss scale that is not a power of two, clipping
far from and exactly at its threshold, and unclipped gradients so large that
their square passes float32's range while the stored second moment does not.
"""
import numpy as np
import pytest

import oracle
import workloads as W

from parity import bits_of, check_norm, compare_step, to_device

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

N = 70_001                     # several 256-element tasks and norm blocks, ragged tail
TDT = {"f16": torch.float16, "bf16": torch.bfloat16}


@pytest.fixture(scope="module")
def Z():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import zero_sharded_mixed_partition_amd as Z
    Z._L.lib()
    return Z


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _huge_grads(fmt: str, n: int) -> np.ndarray:
    """Unclipped gradients with one element in 7 between 1e19 and 4e20 in
    magnitude: their squares overflow float32 (past 2^128), while
    (1 - beta2) g^2 stays below float32's maximum."""
    rng = np.random.default_rng(2024)
    g = rng.normal(0.0, 1e-3, n)
    k = np.arange(0, n, 7)
    g[k] = np.sign(rng.normal(size=k.size)) * 10.0 ** rng.uniform(19.0, np.log10(4e20), k.size)
    if fmt == "f32":
        return g.astype(np.float32)
    return _bf16_bits(g)


# name: (gradient format, moments, gradient kind, hyperparameter overrides)
CASES = {
    "step1_from_zero_moments": ("f16", "zero", "workload", dict(step=1, weight_decay=0.0, max_grad_norm=0.0)),
    "betas_zero": ("bf16", "random", "workload", dict(beta1=0.0, beta2=0.0, step=7, weight_decay=0.01)),
    "short_horizon_large_eps": ("f16", "random", "workload", dict(beta2=0.95, eps=1e-6, weight_decay=0.1, step=3,
                                                                  max_grad_norm=1.0)),
    "lr_zero": ("bf16", "random", "workload", dict(lr=0.0, weight_decay=0.1, step=10)),
    "step_one_million": ("bf16", "random", "workload", dict(step=1_000_000, weight_decay=0.1)),
    "decay_one_half": ("f16", "random", "workload", dict(lr=0.5, weight_decay=1.0, step=2)),
    "zero_gradients": ("bf16", "zero", "zeros", dict(weight_decay=0.1, step=5, max_grad_norm=1.0)),
    "tiny_gradients_tiny_eps": ("f16", "zero", "workload", dict(eps=1e-30, step=1, inv=2.0 ** -40)),
    "scale_not_power_of_two": ("f16", "random", "workload", dict(inv=1.0 / 3000.0, max_grad_norm=1.0, step=40)),
    "clip_far_above_norm": ("bf16", "random", "workload", dict(max_grad_norm=1e6, step=12)),
    "clip_at_norm": ("f16", "random", "workload", dict(max_grad_norm="norm", step=12)),
    "huge_bf16_unclipped": ("bf16", "random", "huge", dict(step=5, weight_decay=0.01, max_grad_norm=0.0)),
    "huge_f32_unclipped": ("f32", "random", "huge", dict(step=5, weight_decay=0.01, max_grad_norm=0.0)),
}


def _case_inputs(name):
    gfmt, moments, kind, over = CASES[name]
    w = W.GPT2_SMALL if gfmt == "f16" else W.LLAMA_7B
    begin = 5_000_011 * (sorted(CASES).index(name) + 1)
    p, m, v, g = W.shard_inputs(w, begin, N)
    if moments == "zero":
        m, v = np.zeros_like(m), np.zeros_like(v)
    if kind == "zeros":
        g = np.zeros_like(g)
    elif kind == "huge":
        g = _huge_grads(gfmt, N)
    over = dict(over)
    inv = over.pop("inv", 1.0 if gfmt == "f32" or kind == "huge" else 1.0 / w.loss_scale)
    hp = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
              max_grad_norm=w.max_grad_norm, step=w.step, inv_loss_scale=inv)
    hp.update(over)
    return w, gfmt, p, m, v, g, hp


def _dev_grad(g, gfmt):
    return to_device(g) if gfmt == "f32" else to_device(g, gfmt)


@pytest.mark.parametrize("name", sorted(CASES))
def test_update_over_hyperparameters(Z, name):
    w, gfmt, p, m, v, g, hp = _case_inputs(name)
    pfmt = "bf16" if gfmt == "f32" else gfmt
    inv = hp["inv_loss_scale"]
    ref_sq, ref_ovf = oracle.shard_sqnorm_overflow(g, gfmt, inv)
    assert not ref_ovf
    if hp["max_grad_norm"] == "norm":
        hp["max_grad_norm"] = float(np.sqrt(ref_sq))   # clip threshold exactly at the norm: coef just below 1
    G = _dev_grad(g, gfmt)

    # coefficients by value from the host
    P, M, V = to_device(p), to_device(m), to_device(v)
    par = torch.empty(N, dtype=TDT[pfmt], device="cuda")
    sq = torch.empty(1, dtype=torch.float64, device="cuda")
    ovf = torch.empty(1, dtype=torch.int32, device="cuda")
    ws = torch.empty(Z.zero_norm_workspace_bytes(N), dtype=torch.uint8, device="cuda")
    Z.zero_shard_unscale_norm_overflow(G, inv, sq, ovf, ws)
    Z.zero_shard_adam_step(P, M, V, G, par, Z.AdamHyper(**hp), sq, ovf)

    # coefficients formed on the device from the step state (scale 1/inv, step t = applied + 1)
    P2, M2, V2 = to_device(p), to_device(m), to_device(v)
    par2 = torch.empty(N, dtype=TDT[pfmt], device="cuda")
    sq2 = torch.empty(1, dtype=torch.float64, device="cuda")
    ovf2 = torch.empty(1, dtype=torch.int32, device="cuda")
    coef = torch.empty(Z.zero_adam_coef_bytes(), dtype=torch.uint8, device="cuda")
    state = Z.StepState(Z.LossScaler.static(1.0 / inv), applied_steps=hp["step"] - 1)
    h = Z.AdamHyper(**{k: x for k, x in hp.items() if k not in ("step", "inv_loss_scale")})
    Z.zero_shard_norm_decide_dev(G, h, state, sq2, ovf2, coef, ws)
    Z.zero_shard_adam_step_coef(P2, M2, V2, G, par2, coef, sq2, ovf2)
    torch.cuda.synchronize()

    assert int(ovf.item()) == int(ovf2.item()) == 0
    check_norm(sq.item(), ref_sq)
    assert sq.item() == sq2.item()
    ref = oracle.shard_step(p, m, v, g, gfmt, pfmt, global_sq=ref_sq, global_overflow=False, **hp)
    got = (P.cpu().numpy(), M.cpu().numpy(), V.cpu().numpy(), bits_of(par))
    compare_step(got, ref, what=f"{name}: ")
    assert np.isfinite(got[2]).all(), "second moment left float32's range"
    for a, b in ((P, P2), (M, M2), (V, V2)):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), name
    assert torch.equal(par.view(torch.int16), par2.view(torch.int16))
    st = state.read()
    assert (st.applied, st.skipped) == (hp["step"], 0)
    if name == "lr_zero":
        assert (got[0].view(np.uint32) == p.view(np.uint32)).all()   # p unchanged bit for bit
