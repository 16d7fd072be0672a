"""Parity at the full LLaMA-2-shaped workload sizes, in the launch
configuration the benchmark times (same entry points, same tile plans).

The oracle runs in full at these sizes (fp64 NumPy on the host's cores);
each test also checks homogeneity identities that need no oracle:
Y is linear in the last up weight, so <dB, B> = <dY, Y> for any activation.
"""
import numpy as np
import pytest
import torch

import oracle
from rank_bottleneck_online_amd import synth

from gpu_util import check, dev, dev_f32, host, say
from test_gpu_parity import compare_lrblock, compare_lrmlp, run_btp, run_lrblock, run_lrmlp

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    from rank_bottleneck_online_amd import binding
    binding.lib()
    return binding


def _rel(a, b):
    return abs(a - b) / max(abs(b), 1e-300)


def test_llama2_1b_qkv_forward(B):
    w = synth.WORKLOADS["llama2_1b_qkv_fwd"]
    T, d, r, G, n = w["T"], w["d"], w["r"], w["G"], w["d_out"]
    say(f"full-size 1B QKV forward T={T} d={d} r={r} G={G}")
    inp = synth.lrblock_inputs(T, d, r, G, n, dtype="bf16", seed=0)
    x, g, A, Bw = (dev(inp[k], "bf16") for k in ("x", "g", "A_cat", "B"))
    Y, H, sumsq = B.lrblock_fwd(x, g, A, Bw, act="silu", norm=True, eps=1e-5)
    torch.cuda.synchronize()
    ref = oracle.lrblock_forward(inp["x"], inp["g"], inp["A_cat"], inp["B"], act="silu", eps=1e-5)
    for k, t in (("Y", Y), ("H", H), ("sumsq", sumsq)):
        check(k, host(t), ref[k], "bf16")


def test_llama2_7b_mlp_fwd_bwd(B):
    w = synth.WORKLOADS["llama2_7b_mlp"]
    T, d, r, ffn = w["T"], w["d"], w["r"], w["ffn"]
    say(f"full-size 7B MLP fwd+bwd T={T} d={d} r={r} ffn={ffn}")
    inp = synth.lrmlp_inputs(T, d, r, ffn, dtype="bf16", seed=0)
    out = run_lrmlp(B, inp, "bf16", "silu")
    L = float(np.sum(inp["dY"] * host(out["Y"])))
    assert _rel(float(np.sum(host(out["dB2"]) * inp["B2"])), L) < 5e-3
    compare_lrmlp(out, inp, "bf16", "silu")


def test_llama2_13b_btp_share_tp4(B):
    """Share 0 of four at the 13B shape. Its backward inputs come from the
    fp64 simulation of all four shares and the consumer that sums them:
    dp = rho * dz_next and ds from the chain rule through rho (what a rank
    forms locally), rounded to their storage types (bf16, fp32)."""
    w = synth.WORKLOADS["llama2_13b_btp_share_tp4"]
    T, r, D, P = w["T"], w["r"], w["d_global"], w["P"]
    say(f"full-size 13B BTP share T={T} r={r} d_global={D} P={P}")
    inp = synth.btp_inputs(T, r, D, P, dtype="bf16", seed=0)
    shards = [synth.btp_shard(inp, p, P) for p in range(P)]
    names = ("z", "B_s", "g_s", "A_s")
    fw = [oracle.btp_share_forward(*(s[k] for k in names)) for s in shards]
    _, rho, Psum = oracle.btp_consumer([f["p"] for f in fw], [f["s"] for f in fw], 1e-5, D)
    dp, ds = oracle.btp_consumer_backward(inp["dz_next"], rho, Psum, D)
    sh = dict(shards[0], dp=oracle.round_to_bf16(dp), ds=synth.round_to_f32(ds))
    say(f"  simulated dp: rms {np.sqrt(np.mean(sh['dp'] ** 2)):.3e}; ds: rms {np.sqrt(np.mean(sh['ds'] ** 2)):.3e}")
    out = run_btp(B, sh, "bf16")
    args = [sh[k] for k in ("z", "B_s", "g_s", "A_s")]
    ref = oracle.btp_share_forward(*args)
    refb = oracle.btp_share_backward(*args, sh["dp"], sh["ds"])
    for k in ("p", "s"):
        check(k, host(out[k]), ref[k], "bf16")
    for k in ("dz", "dB_s", "dg_s", "dA_s"):
        check(k, host(out[k]), refb[k], "bf16")


@pytest.mark.parametrize("act", ["silu", "identity"])
def test_llama2_40b_layerset(B, act):
    w = synth.WORKLOADS["llama2_40b_layerset"]
    T, d, r, ffn = w["T"], w["d"], w["r"], w["ffn"]
    say(f"full-size 40B layer set ({act}) T={T} d={d} r={r} ffn={ffn}")
    inp = synth.layerset_inputs(T, d, r, ffn, dtype="bf16", seed=0)
    q = run_lrblock(B, inp["qkv"], "bf16", act, True)
    compare_lrblock(q, inp["qkv"], "bf16", act, True)
    del q
    o = run_lrblock(B, inp["o"], "bf16", act, False)
    compare_lrblock(o, inp["o"], "bf16", act, False)
    del o
    m = run_lrmlp(B, inp["mlp"], "bf16", act)
    compare_lrmlp(m, inp["mlp"], "bf16", act)
