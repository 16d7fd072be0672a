"""Parity of a chained decoder layer (QKV block, attention stand-in, O block
with the residual add and the next statistic in its up epilogue, MLP taking
that statistic and adding its own residual), forward and backward, against
the fp64 layer oracle with bf16 storage between blocks.

At the 40B layer shape the whole-layer oracle runs on sampled token rows
(every block is row-independent given the weights, so the rows of h3, its
statistic and dx are exact), and every block runs through the oracle at full
size on the inputs the GPU handed it, which checks every weight and gain
gradient of the layer.
"""
import numpy as np
import pytest
import torch

import oracle
from rank_bottleneck_online_amd import synth

from gpu_util import check, dev, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    from rank_bottleneck_online_amd import binding
    binding.lib()
    return binding


def run_layer(B, inp, dtype, act, eps=1e-5):
    x = dev(inp["x"], dtype)
    q = {k: dev(v, dtype) for k, v in inp["qkv"].items()}
    o = {k: dev(v, dtype) for k, v in inp["o"].items()}
    m = {k: dev(v, dtype) for k, v in inp["mlp"].items()}
    dh3 = dev(inp["dh3"], dtype)
    # forward
    qkv, Hq, sq, _ = B.lrblock_fwd_chained(x, q["g"], q["A_cat"], q["B"], act=act, eps=eps)
    a = B.attn_standin_fwd(qkv)
    h2, Ho, _, s2 = B.lrblock_fwd_chained(a, None, o["A_cat"], o["B"], residual=x, sumsq_next=True, act=act,
                                          norm=False)
    h2 = h2[0]
    h3, H1, H2, _, s3 = B.lrmlp_fwd_chained(h2, m["g"], m["A1_cat"], m["B1"], m["A2"], m["B2"], residual=h2,
                                            sumsq_in=s2, sumsq_next=True, act=act, eps=eps)
    # backward
    gm = B.lrmlp_bwd_chained(h2, m["g"], m["A1_cat"], m["B1"], m["A2"], m["B2"], H1, H2, s2, dh3, dx_add=dh3,
                             act=act, eps=eps)
    dh2 = gm[0]
    da, _, dAo, dBo = B.lrblock_bwd_chained(a, None, o["A_cat"], o["B"], Ho, None, dh2[None].contiguous(),
                                            act=act, norm=False)
    dqkv = B.attn_standin_bwd(da)
    dx, dgq, dAq, dBq = B.lrblock_bwd_chained(x, q["g"], q["A_cat"], q["B"], Hq, sq, dqkv, dx_add=dh2, act=act,
                                              eps=eps)
    torch.cuda.synchronize()
    return dict(h3=h3, sumsq_h3=s3, h2=h2, sumsq_h2=s2, sumsq_x=sq, qkv=qkv, a=a, dqkv=dqkv, H2=H2, dx=dx, dh2=dh2,
                da=da,
                dg_qkv=dgq, dA_qkv=dAq, dB_qkv=dBq, dA_o=dAo, dB_o=dBo,
                dg_mlp=gm[1], dA1_mlp=gm[2], dB1_mlp=gm[3], dA2_mlp=gm[4], dB2_mlp=gm[5])


def _chain_check(name, gpu, ref, frob=1e-2, maxabs=2e-2):
    """End-to-end tolerance through the whole layer: every output there sits
    behind up to three blocks, each of which may contribute the single-block
    bf16 error (<= 5e-3 relative Frobenius), so the bound is doubled."""
    from gpu_util import errors
    ma, fr = errors(gpu, ref)
    say(f"    {name:10s} (layer) max-abs/max|ref| {ma:.3e}  rel-frob {fr:.3e}")
    assert ma <= maxabs and fr <= frob, (name, ma, fr)


CASES = [(300, 512, 128, 448, "silu"), (300, 512, 128, 448, "identity"), (1, 256, 64, 192, "silu")]


def check_blocks_on_their_inputs(out, inp, act):
    """Each block of the chain against the oracle run on the inputs the GPU
    actually handed it (its residual, its statistic, its output gradient):
    the single-block tolerance applies to every output, statistic, input
    gradient and weight and gain gradient of every block."""
    q, o, m = inp["qkv"], inp["o"], inp["mlp"]
    rnd = oracle.round_to_bf16
    # QKV block
    fq = oracle.lrblock_forward(inp["x"], q["g"], q["A_cat"], q["B"], act)
    check("sumsq_x", host(out["sumsq_x"]), fq["sumsq"], "bf16")
    # stand-in: a = q + k + v, summed exactly, then rounded to fp32 and bf16
    qkv = host(out["qkv"])
    assert np.array_equal(host(out["a"]), rnd(oracle.standin_forward(qkv)))
    # O block with the residual and the next statistic
    a = host(out["a"])
    fo = oracle.lrblock_forward(a, None, o["A_cat"], o["B"], act, norm=False)
    check("h2", host(out["h2"]), inp["x"] + fo["Y"][0], "bf16")
    h2 = host(out["h2"])
    check("sumsq_h2", host(out["sumsq_h2"]), np.sum(h2 * h2, axis=1), "f32")
    # MLP with the producer's statistic, its residual and the next statistic
    fm = oracle.lrmlp_forward(h2, m["g"], m["A1_cat"], m["B1"], m["A2"], m["B2"], act)
    check("h3", host(out["h3"]), h2 + fm["Y"], "bf16")
    h3 = host(out["h3"])
    check("sumsq_h3", host(out["sumsq_h3"]), np.sum(h3 * h3, axis=1), "f32")
    # MLP backward with the residual gradient added to dx
    bm = oracle.lrmlp_backward(h2, m["g"], m["A1_cat"], m["B1"], m["A2"], m["B2"], inp["dh3"], act)
    check("dh2", host(out["dh2"]), inp["dh3"] + bm["dx"], "bf16")
    for k, rk in (("dg_mlp", "dg"), ("dA1_mlp", "dA1_cat"), ("dB1_mlp", "dB1"), ("dA2_mlp", "dA2"),
                  ("dB2_mlp", "dB2")):
        check(k, host(out[k]), bm[rk], "bf16")
    # O block backward
    dh2 = host(out["dh2"])
    bo = oracle.lrblock_backward(a, None, o["A_cat"], o["B"], dh2[None], act, norm=False)
    check("da", host(out["da"]), bo["dx"], "bf16")
    check("dA_o", host(out["dA_o"]), bo["dA_cat"], "bf16")
    check("dB_o", host(out["dB_o"]), bo["dB"], "bf16")
    # stand-in backward is three exact copies
    da = host(out["da"])
    assert np.array_equal(host(out["dqkv"]), np.stack([da, da, da]))
    # QKV block backward with the residual gradient added to dx
    bq = oracle.lrblock_backward(inp["x"], q["g"], q["A_cat"], q["B"], np.stack([da, da, da]), act)
    check("dx", host(out["dx"]), dh2 + bq["dx"], "bf16")
    for k, rk in (("dg_qkv", "dg"), ("dA_qkv", "dA_cat"), ("dB_qkv", "dB")):
        check(k, host(out[k]), bq[rk], "bf16")


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_chained_layer_blocks_on_their_inputs(B, case):
    T, d, r, ffn, act = case
    say(f"chained layer (per block) T={T} d={d} r={r} ffn={ffn} bf16 {act} seed=0")
    inp = synth.layer_inputs(T, d, r, ffn, dtype="bf16", seed=0)
    out = run_layer(B, inp, "bf16", act)
    check_blocks_on_their_inputs(out, inp, act)


@pytest.mark.parametrize("case", CASES[:2], ids=lambda c: "x".join(map(str, c)))
def test_chained_layer_end_to_end(B, case):
    T, d, r, ffn, act = case
    say(f"chained layer (end to end) T={T} d={d} r={r} ffn={ffn} bf16 {act} seed=0")
    inp = synth.layer_inputs(T, d, r, ffn, dtype="bf16", seed=0)
    out = run_layer(B, inp, "bf16", act)
    st = oracle.round_to_bf16
    ref = oracle.layer_forward(inp["x"], inp["qkv"], inp["o"], inp["mlp"], act, store=st)
    refb = oracle.layer_backward(inp["x"], inp["qkv"], inp["o"], inp["mlp"], inp["dh3"], act, store=st)
    for k in ("h2", "sumsq_h2", "h3", "sumsq_h3"):
        _chain_check(k, host(out[k]), ref[k])
    for k in ("dh2", "da", "dx", "dg_qkv", "dA_qkv", "dB_qkv", "dA_o", "dB_o", "dg_mlp", "dA1_mlp", "dB1_mlp",
              "dA2_mlp", "dB2_mlp"):
        _chain_check(k, host(out[k]), refb[k])


def test_chained_layer_40b_sampled_rows(B):
    w = synth.WORKLOADS["llama2_40b_layer_chained"]
    T, d, r, ffn = w["T"], w["d"], w["r"], w["ffn"]
    say(f"full-size chained layer T={T} d={d} r={r} ffn={ffn} bf16 silu")
    inp = synth.layer_inputs(T, d, r, ffn, dtype="bf16", seed=0)
    out = run_layer(B, inp, "bf16", "silu")
    rows = np.sort(np.random.default_rng(1).choice(T, size=24, replace=False))
    sub = dict(inp)
    sub["x"], sub["dh3"] = inp["x"][rows], inp["dh3"][rows]
    st = oracle.round_to_bf16
    ref = oracle.layer_forward(sub["x"], inp["qkv"], inp["o"], inp["mlp"], "silu", store=st)
    refb = oracle.layer_backward(sub["x"], inp["qkv"], inp["o"], inp["mlp"], sub["dh3"], "silu", store=st)
    for k in ("h3", "sumsq_h3", "h2", "sumsq_h2"):
        _chain_check(k + "[rows]", host(out[k])[rows], ref[k])
    for k in ("dx", "dh2"):
        _chain_check(k + "[rows]", host(out[k])[rows], refb[k])
    # Every block at full size against the oracle on the inputs the GPU
    # handed it: all outputs, statistics, input gradients and every weight
    # and gain gradient of the QKV, O and MLP blocks (about 5 TFLOP of fp64).
    say("  per-block oracle at full size")
    check_blocks_on_their_inputs(out, inp, "silu")
