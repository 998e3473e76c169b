"""Pins for the oracle's memory accounting against the pages' printed figures
(tests/golden/zero_accounting.json, each entry citing its section)."""
import json
import os
from fractions import Fraction

import pytest

from oracle import communication_elements, model_state_bytes_per_param, per_rank_state_bytes, reduction_factor
from oracle import accounting as A


@pytest.fixture(scope="module")
def facts(golden_dir):
    with open(os.path.join(golden_dir, "zero_accounting.json")) as f:
        return {x["id"]: x for x in json.load(f)["facts"]}


def test_16_bytes(facts):
    assert model_state_bytes_per_param() == facts["bytes_per_param_mixed_precision_adam"]["value"]
    assert A.FP16_WEIGHT == facts["fp16_weight_bytes"]["value"]
    assert A.FP32_MASTER == facts["fp32_master_bytes"]["value"]
    assert A.FP32_MOMENTS == facts["adam_two_moments_bytes"]["value"]
    # the 16-20 range: without and with the optional fp32 gradient copy
    lo, hi = facts["total_bytes_per_param_range"]["value"]
    assert model_state_bytes_per_param() == lo
    assert model_state_bytes_per_param(fp32_grad_copy=True) == hi
    # "fp16 gradient + fp32 copy" = 6 bytes
    assert A.FP16_GRAD + A.FP32_GRAD_COPY == facts["fp16_grad_plus_fp32_copy_bytes"]["value"]


def test_7b_and_100b(facts):
    f7 = facts["training_state_7b"]
    assert per_rank_state_bytes("dp", int(f7["params"]), 1) == Fraction(int(f7["approx_bytes"]))
    f100 = facts["replicated_state_100b"]
    # replicated under plain DP: every rank holds all of it, whatever N_d
    for n_d in (1, 8, 400):
        assert per_rank_state_bytes("dp", int(f100["params"]), n_d) == Fraction(int(f100["approx_bytes"]))


def test_stage_reductions(facts):
    psi = 10**9
    # the printed ~4x and ~8x are the large-N_d limits (16/4, 16/2)
    r1 = reduction_factor("os", psi, 10**9)
    r2 = reduction_factor("os+g", psi, 10**9)
    assert abs(float(r1) - facts["reduction_zero1_pos"]["approx"]) < 1e-6
    assert abs(float(r2) - facts["reduction_zero2_posg"]["approx"]) < 1e-6
    # monotone in N_d and ordered across stages
    for n_d in (2, 8, 64, 1024):
        a, b, c = (reduction_factor(s, psi, n_d) for s in ("os", "os+g", "os+g+p"))
        assert 1 < a < b < c
        # ZeRO-3: exactly N_d x
        assert c == n_d
    assert reduction_factor("dp", psi, 8) == 1


def test_optimizer_states_3x(facts):
    # master + two moments = 12 B against a 4-byte (fp32) copy of the weights
    assert (A.FP32_MASTER + A.FP32_MOMENTS) / 4 == facts["optimizer_states_vs_model_size"]["approx"]


def test_exact_per_rank_formulas():
    psi, n_d = 1000, 8
    assert per_rank_state_bytes("os", psi, n_d) == 4 * psi + Fraction(12 * psi, n_d)
    assert per_rank_state_bytes("os+g", psi, n_d) == 2 * psi + Fraction(14 * psi, n_d)
    assert per_rank_state_bytes("os+g+p", psi, n_d) == Fraction(16 * psi, n_d)


def test_stage_communication(facts):
    """The stage table's extra communication: none for the first two stages,
    half as much again as plain DP for the third, at any N_d >= 2."""
    psi = 7 * 10**9
    for n_d in (2, 8, 400, 1024):
        dp = communication_elements("dp", psi, n_d)
        for stage, fid in (("os", "extra_comm_zero1_pos"), ("os+g", "extra_comm_zero2_posg"),
                           ("os+g+p", "extra_comm_zero3_posgp")):
            extra = communication_elements(stage, psi, n_d) / dp - 1
            assert extra == Fraction(facts[fid]["approx_extra_fraction"]).limit_denominator(100)
    # one rank alone sends nothing; a ring all-reduce sends 2 (N_d - 1) / N_d of the buffer
    assert communication_elements("dp", psi, 1) == 0
    assert communication_elements("dp", 1000, 4) == 1500
    assert communication_elements("os+g+p", 1000, 4) == 2250
