"""GPU: a seeded random sweep of the whole step against the oracle.

Each case draws its own shard size (1 to 400,000 elements, so most are
ragged), gradient format (fp16, bf16, or an fp32 accumulated copy),
parameter format (or no writeback), learning rate, betas (zero included),
eps, weight decay, step index (1 to 10^6), loss scale (powers of two and
not), clipping (off, or a threshold above or below the norm), value scales
of master, moments and gradient, and whether the moments start at zero.
The step runs three ways: the norm pass with a workspace and the update
with coefficients from the host; the norm pass without a workspace; and
the norm pass that forms the coefficients on the device from the step
state, followed by the update reading them.  All three agree bit for bit;
master and moments equal, bit for bit, the float32 model of the operation
order the header documents (`f32model`); and the result is within the bar
of the oracle's, the master's absolute floor raised to 4 float32 ulps of the
larger of its two terms where they cancel (float32's own rounding, which the
bit-exact model check shows is all that differs there).
"""
import numpy as np
import pytest

import f32model
import oracle

from parity import bits_of, cancellation_floor, check_norm, compare_step, to_device

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TDT = {"f16": torch.float16, "bf16": torch.bfloat16}
N_CASES = 1024


@pytest.fixture(scope="module")
def Z():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import zero_sharded_mixed_partition_amd as Z
    Z._L.lib()
    return Z


def _bits(x: np.ndarray, fmt: str) -> np.ndarray:
    x = np.asarray(x, np.float32)
    if fmt == "f16":
        return x.astype(np.float16).view(np.uint16)
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _values(g: np.ndarray, fmt: str) -> np.ndarray:
    """Gradient values as float32: 16-bit patterns decoded exactly (IEEE
    half by numpy, bfloat16 as the upper half of a float32), or the fp32 copy."""
    if fmt == "f32":
        return np.asarray(g, np.float32)
    if fmt == "f16":
        return g.view(np.float16).astype(np.float32)
    return (g.astype(np.uint32) << 16).view(np.float32)


def _case(i: int):
    rng = np.random.default_rng(900_000 + i)
    n = int(rng.choice([1, 3, 255, 256, 257, 4099, 65537]) if i % 6 == 0 else 10 ** rng.uniform(0, np.log10(4e5)))
    gfmt = ("f16", "bf16", "f32")[i % 3]
    pfmt = None if i % 7 == 3 else ("f16", "bf16")[(i // 3) % 2]
    hp = dict(lr=float(10 ** rng.uniform(-5, -1)), beta1=float(rng.choice([0.0, 0.5, 0.9, 0.95, 0.99])),
              beta2=float(rng.choice([0.0, 0.9, 0.99, 0.999, 0.9999])), eps=float(10 ** rng.uniform(-12, -4)),
              weight_decay=float(rng.choice([0.0, 1e-4, 1e-2, 0.1])), step=int(10 ** rng.uniform(0, 6)))
    sp, sm, sg = 10 ** rng.uniform(-3, 0), 10 ** rng.uniform(-6, -2), 10 ** rng.uniform(-6, -1)
    p = (rng.standard_normal(n) * sp).astype(np.float32)
    zero_moments = rng.random() < 0.2
    m = np.zeros(n, np.float32) if zero_moments else (rng.standard_normal(n) * sm).astype(np.float32)
    v = np.zeros(n, np.float32) if zero_moments else rng.uniform(0, sm * sm, n).astype(np.float32)
    g_true = rng.standard_normal(n) * sg
    if gfmt == "f32":
        scale = 1.0                       # the accumulated copy is already unscaled
        g = g_true.astype(np.float32)
    else:
        if gfmt == "f16":
            k = int(rng.integers(0, 17))
            scale = 3000.0 if i % 5 == 1 else 2.0 ** k
            scale = min(scale, 2.0 ** np.floor(np.log2(6e4 / (8 * sg))))   # keep |g * scale| finite in fp16
        else:
            scale = float(rng.choice([1.0, 2.0 ** 8, 1000.0]))
        g = _bits(g_true * scale, gfmt)
    inv = 1.0 / scale
    clip = float(rng.choice([0.0, 0.1, 1.0, 10.0]))
    hp.update(inv_loss_scale=inv, max_grad_norm=clip)
    return n, gfmt, pfmt, p, m, v, g, hp


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_step(Z, i):
    n, gfmt, pfmt, p, m, v, g, hp = _case(i)
    inv = hp["inv_loss_scale"]
    ref_sq, ref_ovf = oracle.shard_sqnorm_overflow(g, gfmt, inv)
    assert not ref_ovf
    G = to_device(g) if gfmt == "f32" else to_device(g, gfmt)
    ws = torch.empty(Z.zero_norm_workspace_bytes(n), dtype=torch.uint8, device="cuda")

    def bufs():
        P, M, V = to_device(p), to_device(m), to_device(v)
        par = torch.empty(n, dtype=TDT[pfmt], device="cuda") if pfmt else None
        sq = torch.empty(1, dtype=torch.float64, device="cuda")
        ovf = torch.empty(1, dtype=torch.int32, device="cuda")
        return P, M, V, par, sq, ovf

    # 1: workspace norm, coefficients by value
    P, M, V, par, sq, ovf = bufs()
    Z.zero_shard_unscale_norm_overflow(G, inv, sq, ovf, ws)
    Z.zero_shard_adam_step(P, M, V, G, par, Z.AdamHyper(**hp), sq, ovf)
    # 2: the norm pass without a workspace
    P1, M1, V1, par1, sq1, ovf1 = bufs()
    Z.zero_shard_unscale_norm_overflow_noalloc(G, inv, sq1, ovf1)
    Z.zero_shard_adam_step(P1, M1, V1, G, par1, Z.AdamHyper(**hp), sq1, ovf1)
    # 3: the decision on the device from the step state
    P2, M2, V2, par2, sq2, ovf2 = bufs()
    coef = torch.empty(Z.zero_adam_coef_bytes(), dtype=torch.uint8, device="cuda")
    state = Z.StepState(Z.LossScaler.static(1.0 / inv), applied_steps=hp["step"] - 1)
    h = Z.AdamHyper(**{k: x for k, x in hp.items() if k not in ("step", "inv_loss_scale")})
    Z.zero_shard_norm_decide_dev(G, h, state, sq2, ovf2, coef, ws)
    Z.zero_shard_adam_step_coef(P2, M2, V2, G, par2, coef, sq2, ovf2)
    torch.cuda.synchronize()

    what = f"case {i} (n={n}, {gfmt}->{pfmt}, {hp}): "
    assert int(ovf.item()) == int(ovf1.item()) == int(ovf2.item()) == 0, what
    assert sq.item() == sq1.item() == sq2.item(), what
    check_norm(sq.item(), ref_sq)
    for a, b, c in ((P, P1, P2), (M, M1, M2), (V, V1, V2)) + (((par, par1, par2),) if pfmt else ()):
        iv = torch.int16 if a.element_size() == 2 else torch.int32
        assert torch.equal(a.view(iv), b.view(iv)) and torch.equal(a.view(iv), c.view(iv)), what
    # the float32 operation order the header documents, bit for bit, from the GPU's own sum of squares
    gvals = _values(g, gfmt)
    model = f32model.adam_update(p, m, v, gvals, sq.item(), **hp)
    for name, t, x in zip(("master", "exp_avg", "exp_avg_sq"), (P, M, V), model):
        assert np.array_equal(t.cpu().numpy().view(np.uint32), x.view(np.uint32)), what + name + " != float32 model"
    ref = oracle.shard_step(p, m, v, g, gfmt, pfmt, global_sq=ref_sq, global_overflow=False, **hp)
    got = (P.cpu().numpy(), M.cpu().numpy(), V.cpu().numpy(), bits_of(par) if pfmt else None)
    # the master's floor raised where its two terms cancel: float32 rounds terms near 1 to a few 1e-8
    floor = cancellation_floor(p, ref[0], 1.0 - hp["lr"] * hp["weight_decay"])
    compare_step(got, ref, what=what, pfmt=pfmt, master_floor=floor)
    assert state.read().applied == hp["step"]
