"""Pins of the chained-layer oracle (CPU only).

The layer composes the block oracles with residual adds and an attention
stand-in; these tests pin that composition to things other than itself:
finite differences of the whole layer, closed forms when the residual
branches are switched off, the bilinear identity of the last up projection,
and the bf16 storage rounding against an independent implementation and
hand-worked ties.
"""
import numpy as np
import pytest

import oracle
from rank_bottleneck_online_amd import synth

TINY = dict(T=3, d=8, r=2, ffn=6)


def _params(seed=1, act_scale=1.0):
    inp = synth.layer_inputs(**TINY, dtype="bf16", seed=seed)
    return inp


def _loss(inp, act, store=None):
    f = oracle.layer_forward(inp["x"], inp["qkv"], inp["o"], inp["mlp"], act, store=store)
    return float(np.sum(inp["dh3"] * f["h3"]))


def test_bf16_store_rounding_ties_and_generator():
    # ulp of bf16 at 1 is 2**-7: a half-ulp tie goes to the even neighbour
    v = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 1 + 2.0 ** -8 + 2.0 ** -20])
    want = np.array([1.0, 1 + 2.0 ** -6, -1.0, 1 + 2.0 ** -7])
    assert np.array_equal(oracle.round_to_bf16(v), want)
    # two independent implementations of round-to-nearest-even agree on
    # values already rounded to float32 (the device's intermediate)
    rng = np.random.default_rng(7)
    x = rng.standard_normal(20000).astype(np.float32).astype(np.float64) * 10.0 ** rng.integers(-3, 4, 20000)
    assert np.array_equal(oracle.round_to_bf16(x), synth.quantize(x, "bf16"))


@pytest.mark.parametrize("act", ["silu", "identity"])
def test_layer_gradients_match_finite_differences(act):
    inp = _params(seed=3)
    b = oracle.layer_backward(inp["x"], inp["qkv"], inp["o"], inp["mlp"], inp["dh3"], act)
    rng = np.random.default_rng(11)
    h = 1e-5

    def check(get, set_, grad):
        base = get()
        direc = rng.standard_normal(base.shape)
        set_(base + h * direc)
        lp = _loss(inp, act)
        set_(base - h * direc)
        lm = _loss(inp, act)
        set_(base)
        fd = (lp - lm) / (2 * h)
        an = float(np.sum(grad * direc))
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (fd, an)

    def acc(d, k):
        return (lambda: d[k]), (lambda v: d.__setitem__(k, v))

    check(*acc(inp, "x"), b["dx"])
    check(*acc(inp["qkv"], "g"), b["dg_qkv"])
    check(*acc(inp["qkv"], "A_cat"), b["dA_qkv"])
    check(*acc(inp["qkv"], "B"), b["dB_qkv"])
    check(*acc(inp["o"], "A_cat"), b["dA_o"])
    check(*acc(inp["o"], "B"), b["dB_o"])
    check(*acc(inp["mlp"], "g"), b["dg_mlp"])
    check(*acc(inp["mlp"], "A1_cat"), b["dA1_mlp"])
    check(*acc(inp["mlp"], "B1"), b["dB1_mlp"])
    check(*acc(inp["mlp"], "A2"), b["dA2_mlp"])
    check(*acc(inp["mlp"], "B2"), b["dB2_mlp"])


def test_layer_with_branches_switched_off_is_the_identity():
    inp = _params(seed=5)
    inp["o"]["B"] = np.zeros_like(inp["o"]["B"])
    inp["mlp"]["B2"] = np.zeros_like(inp["mlp"]["B2"])
    f = oracle.layer_forward(inp["x"], inp["qkv"], inp["o"], inp["mlp"], "silu")
    assert np.array_equal(f["h3"], inp["x"])
    assert np.allclose(f["sumsq_h3"], np.sum(inp["x"] ** 2, axis=1), rtol=1e-15, atol=0)
    b = oracle.layer_backward(inp["x"], inp["qkv"], inp["o"], inp["mlp"], inp["dh3"], "silu")
    assert np.array_equal(b["dx"], inp["dh3"])
    assert not np.any(b["dA_qkv"]) and not np.any(b["dB_qkv"]) and not np.any(b["dg_qkv"])


@pytest.mark.parametrize("act", ["silu", "identity"])
def test_last_up_projection_is_bilinear(act):
    # the MLP output is linear in B2, so <dB2, B2> = <dh3, h3 - h2>
    inp = _params(seed=9)
    f = oracle.layer_forward(inp["x"], inp["qkv"], inp["o"], inp["mlp"], act)
    b = oracle.layer_backward(inp["x"], inp["qkv"], inp["o"], inp["mlp"], inp["dh3"], act)
    lhs = float(np.sum(b["dB2_mlp"] * inp["mlp"]["B2"]))
    rhs = float(np.sum(inp["dh3"] * (f["h3"] - f["h2"])))
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(rhs))


def test_stored_rounding_only_perturbs_at_bf16_level():
    inp = synth.layer_inputs(T=16, d=64, r=16, ffn=48, dtype="bf16", seed=2)
    exact = oracle.layer_forward(inp["x"], inp["qkv"], inp["o"], inp["mlp"], "silu")
    stored = oracle.layer_forward(inp["x"], inp["qkv"], inp["o"], inp["mlp"], "silu", store=oracle.round_to_bf16)
    rel = np.linalg.norm(stored["h3"] - exact["h3"]) / np.linalg.norm(exact["h3"])
    assert 0 < rel < 5e-3
    assert np.array_equal(stored["h3"], oracle.round_to_bf16(stored["h3"]))
