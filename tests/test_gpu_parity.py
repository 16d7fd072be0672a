"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Every case draws seeded inputs, runs the GPU entry points, and compares each
output tensor with the oracle on the same quantized inputs (tolerances in
tests/gpu_util.py). Small cases span several tiles with ragged tails in
every dimension that can be ragged (T, and K = T for the weight gradients;
N tails where r or d_out is not a multiple of the tile width).
"""
import numpy as np
import pytest
import torch

import oracle
from rank_bottleneck_online_amd import synth

from gpu_util import check, dev, dev_f32, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    from rank_bottleneck_online_amd import binding
    binding.lib()
    return binding


def run_lrblock(B, inp, dtype, act, norm, eps=1e-5, d_norm=None):
    x, A, Bw, dY = (dev(inp[k], dtype) for k in ("x", "A_cat", "B", "dY"))
    g = dev(inp["g"], dtype) if norm else None
    Y, H, sumsq = B.lrblock_fwd(x, g, A, Bw, act=act, norm=norm, eps=eps, d_norm=d_norm)
    dx, dg, dA, dB = B.lrblock_bwd(x, g, A, Bw, H, sumsq, dY, act=act, norm=norm, eps=eps, d_norm=d_norm)
    torch.cuda.synchronize()
    return dict(Y=Y, H=H, sumsq=sumsq, dx=dx, dg=dg, dA_cat=dA, dB=dB)


def compare_lrblock(out, inp, dtype, act, norm, eps=1e-5, d_norm=None):
    ref = oracle.lrblock_forward(inp["x"], inp.get("g"), inp["A_cat"], inp["B"], act=act, norm=norm, eps=eps,
                                 d_norm=d_norm)
    refb = oracle.lrblock_backward(inp["x"], inp.get("g"), inp["A_cat"], inp["B"], inp["dY"], act=act, norm=norm,
                                   eps=eps, d_norm=d_norm)
    names = ["Y", "H"] + (["sumsq"] if norm else [])
    for k in names:
        check(k, host(out[k]), ref[k], dtype)
    for k in ["dx", "dA_cat", "dB"] + (["dg"] if norm else []):
        check(k, host(out[k]), refb[k], dtype)


LRBLOCK_CASES = [
    # (T, d, r, G, d_out, dtype, act, norm)
    (64, 256, 64, 3, 256, "f32", "silu", True),        # the tiny fp32 QKV block
    (100, 256, 64, 3, 192, "f32", "identity", True),
    (100, 128, 64, 1, 128, "f32", "silu", False),
    (300, 512, 192, 3, 320, "bf16", "silu", True),      # ragged T, r and d_out vs the tiles
    (300, 512, 192, 3, 320, "bf16", "identity", True),
    (257, 384, 128, 1, 384, "bf16", "silu", False),     # O-projection form
    (1, 256, 64, 3, 128, "bf16", "silu", True),         # a single token
    (640, 1024, 256, 2, 1024, "bf16", "silu", True),
    (130, 256, 64, 16, 128, "bf16", "silu", True),     # the most groups a descriptor takes
    (70, 128, 64, 16, 64, "f32", "identity", True),
]


@pytest.mark.parametrize("case", LRBLOCK_CASES, ids=lambda c: "x".join(map(str, c)))
def test_lrblock_parity(B, case):
    T, d, r, G, d_out, dtype, act, norm = case
    say(f"lrblock T={T} d={d} r={r} G={G} d_out={d_out} {dtype} {act} norm={norm} seed=0")
    inp = synth.lrblock_inputs(T, d, r, G, d_out, dtype=dtype, seed=0, norm=norm)
    out = run_lrblock(B, inp, dtype, act, norm)
    compare_lrblock(out, inp, dtype, act, norm)


def test_lrblock_global_width_divisor(B):
    # d_norm larger than d: the block normalises a share of a wider row.
    T, d, r, G, n = 200, 256, 64, 2, 128
    say(f"lrblock d_norm=1024 T={T} d={d}")
    inp = synth.lrblock_inputs(T, d, r, G, n, dtype="bf16", seed=3)
    out = run_lrblock(B, inp, "bf16", "silu", True, d_norm=1024)
    compare_lrblock(out, inp, "bf16", "silu", True, d_norm=1024)


@pytest.mark.parametrize("d", [256, 64, 192])
def test_lrblock_parity_256x192_tiles(B, d):
    # T = 4090, G r = 3072: 256 x 192 down tiles fill one round (16 x 16),
    # where 192 x 256 needs two (22 x 12) and 256 x 256 leaves a quarter of
    # the round idle, so the planner takes the 96-wide wave tiles whose
    # epilogue reads back 12 lanes per row; ragged T. d = 64 and 192 give
    # the down product one and three K steps, fewer than its B ring holds.
    T, r, G, n = 4090, 1024, 3, 256
    say(f"lrblock 256x192 down tiles T={T} d={d} r={r} G={G} n={n} bf16 silu seed=4")
    inp = synth.lrblock_inputs(T, d, r, G, n, dtype="bf16", seed=4)
    out = run_lrblock(B, inp, "bf16", "silu", True)
    compare_lrblock(out, inp, "bf16", "silu", True)


@pytest.mark.parametrize("r", [64, 128, 192])
def test_lrblock_short_k_on_ring_tiles(B, r):
    # T = 8190, n = d = 2048: the up product (K = r) and the input gradient
    # (K = G r) run on 256 x 256 tiles, one full round, whose operand panels
    # stream through the A and B rings; K = r of one, two and three K steps
    # covers a loop shorter than the rings (panels past K are issued out of
    # range and still counted). Ragged T.
    T, d, G, n = 8190, 2048, 1, 2048
    say(f"lrblock short-K ring tiles T={T} d={d} r={r} G={G} n={n} bf16 silu seed=5")
    inp = synth.lrblock_inputs(T, d, r, G, n, dtype="bf16", seed=5)
    out = run_lrblock(B, inp, "bf16", "silu", True)
    compare_lrblock(out, inp, "bf16", "silu", True)


def run_lrmlp(B, inp, dtype, act, eps=1e-5):
    t = {k: dev(inp[k], dtype) for k in ("x", "g", "A1_cat", "B1", "A2", "B2", "dY")}
    Y, H1, H2, sumsq = B.lrmlp_fwd(t["x"], t["g"], t["A1_cat"], t["B1"], t["A2"], t["B2"], act=act, eps=eps)
    grads = B.lrmlp_bwd(t["x"], t["g"], t["A1_cat"], t["B1"], t["A2"], t["B2"], H1, H2, sumsq, t["dY"], act=act,
                        eps=eps)
    torch.cuda.synchronize()
    out = dict(Y=Y, H1=H1, H2=H2, sumsq=sumsq)
    out.update(zip(("dx", "dg", "dA1_cat", "dB1", "dA2", "dB2"), grads))
    return out


def compare_lrmlp(out, inp, dtype, act, eps=1e-5, report=None):
    args = [inp[k] for k in ("x", "g", "A1_cat", "B1", "A2", "B2")]
    ref = oracle.lrmlp_forward(*args, act=act, eps=eps)
    refb = oracle.lrmlp_backward(*args, inp["dY"], act=act, eps=eps)
    for k in ("Y", "H1", "H2", "sumsq"):
        check(k, host(out[k]), ref[k], dtype, report)
    for k in ("dx", "dg", "dA1_cat", "dB1", "dA2", "dB2"):
        check(k, host(out[k]), refb[k], dtype, report)


@pytest.mark.parametrize("case", [(300, 256, 128, 448, "bf16", "silu"), (300, 256, 128, 448, "bf16", "identity"),
                                  (96, 128, 64, 192, "f32", "silu"), (513, 512, 128, 1408, "bf16", "silu"),
                                  (1, 128, 64, 192, "bf16", "silu"),       # a single token
                                  (70, 64, 64, 64, "f32", "identity")],    # the smallest widths, ragged T
                         ids=lambda c: "x".join(map(str, c)))
def test_lrmlp_parity(B, case):
    T, d, r, ffn, dtype, act = case
    say(f"lrmlp T={T} d={d} r={r} ffn={ffn} {dtype} {act} seed=0")
    inp = synth.lrmlp_inputs(T, d, r, ffn, dtype=dtype, seed=0)
    out = run_lrmlp(B, inp, dtype, act)
    compare_lrmlp(out, inp, dtype, act)


# Long K = T against few output tiles: the weight gradients are split along K
# (a ragged last split), written as fp32 partials and summed in split order by
# the reduction kernel, which also applies the gain to dA.
SPLITK_CASES = [
    ("lrblock", (3000, 256, 64, 2, 128, "bf16", "silu", True)),
    ("lrblock", (8000, 128, 64, 1, 64, "f32", "identity", True)),
    ("lrmlp", (2500, 128, 64, 192, "bf16", "silu")),
]


@pytest.mark.parametrize("case", SPLITK_CASES, ids=lambda c: c[0] + "x" + "x".join(map(str, c[1])))
def test_split_k_weight_gradients(B, case):
    kind, c = case
    say(f"split-K {kind} {c} seed=0")
    B.profiler_enable(None, 4096)
    try:
        if kind == "lrblock":
            T, d, r, G, d_out, dtype, act, norm = c
            inp = synth.lrblock_inputs(T, d, r, G, d_out, dtype=dtype, seed=0, norm=norm)
            out = run_lrblock(B, inp, dtype, act, norm)
        else:
            T, d, r, ffn, dtype, act = c
            inp = synth.lrmlp_inputs(T, d, r, ffn, dtype=dtype, seed=0)
            out = run_lrmlp(B, inp, dtype, act)
        rep = B.profiler_report()
    finally:
        B.profiler_disable()
    assert "splitk_reduce" in rep, sorted(rep)
    if kind == "lrblock":
        compare_lrblock(out, inp, dtype, act, norm)
    else:
        compare_lrmlp(out, inp, dtype, act)


def run_btp(B, sh, dtype):
    z, Bs, gs, As, dp = (dev(sh[k], dtype) for k in ("z", "B_s", "g_s", "A_s", "dp"))
    ds = dev_f32(sh["ds"])
    p, s = B.btp_share_fwd(z, Bs, gs, As)
    dz, dB, dg, dA = B.btp_share_bwd(z, Bs, gs, As, dp, ds)
    torch.cuda.synchronize()
    return dict(p=p, s=s, dz=dz, dB_s=dB, dg_s=dg, dA_s=dA)


def compare_btp(out, sh, dtype):
    args = [sh[k] for k in ("z", "B_s", "g_s", "A_s")]
    ref = oracle.btp_share_forward(*args)
    refb = oracle.btp_share_backward(*args, sh["dp"], sh["ds"])
    for k in ("p", "s"):
        check(k, host(out[k]), ref[k], dtype)
    for k in ("dz", "dB_s", "dg_s", "dA_s"):
        check(k, host(out[k]), refb[k], dtype)


@pytest.mark.parametrize("case", [(300, 192, 1280, 4, "bf16"), (64, 64, 512, 4, "f32"), (1, 128, 512, 4, "bf16")],
                         ids=lambda c: "x".join(map(str, c)))
def test_btp_share_parity(B, case):
    T, r, D, P, dtype = case
    say(f"btp share T={T} r={r} d_global={D} P={P} {dtype} seed=0")
    inp = synth.btp_inputs(T, r, D, P, dtype=dtype, seed=0)
    sh = synth.btp_shard(inp, 0, P)
    out = run_btp(B, sh, dtype)
    compare_btp(out, sh, dtype)


def test_bit_identical_reruns(B):
    T, d, r, ffn = 640, 512, 128, 1408
    say(f"determinism lrmlp T={T} d={d} r={r} ffn={ffn}")
    inp = synth.lrmlp_inputs(T, d, r, ffn, dtype="bf16", seed=5)
    a = run_lrmlp(B, inp, "bf16", "silu")
    b = run_lrmlp(B, inp, "bf16", "silu")
    for k in a:
        assert torch.equal(a[k], b[k]), k


def test_serialized_weight_gradients_bit_identical(B):
    # The measurement switch moves the weight gradients of every backward to
    # the caller's stream: same kernels, same sums, so every output matches
    # the overlapped run bit for bit (MLP with split-K partials, block, share).
    say("serialized weight gradients: lrmlp T=2500 (split-K), lrblock T=300, btp share T=300")
    mlp = synth.lrmlp_inputs(2500, 128, 64, 192, dtype="bf16", seed=6)
    blk = synth.lrblock_inputs(300, 256, 128, 3, 256, dtype="bf16", seed=6)
    sh = synth.btp_shard(synth.btp_inputs(300, 192, 1280, 4, dtype="bf16", seed=6), 0, 4)
    runs = []
    for serial in (False, True):
        B.profiler_serialize(serial)
        try:
            runs.append((run_lrmlp(B, mlp, "bf16", "silu"), run_lrblock(B, blk, "bf16", "silu", True),
                         run_btp(B, sh, "bf16")))
        finally:
            B.profiler_serialize(False)
    for a, b in zip(*runs):
        for k in a:
            assert torch.equal(a[k], b[k]), k


def test_scale_invariance_with_zero_eps(B):
    # Online-RMSNorm with eps = 0: scaling x by 2^k (exact in bf16) leaves the
    # block's output unchanged and stays finite far from unit scale.
    T, d, r, G, n = 256, 512, 128, 3, 256
    say("scale invariance eps=0")
    inp = synth.lrblock_inputs(T, d, r, G, n, dtype="bf16", seed=7)
    outs = []
    for k in (-20, 0, 13):
        i2 = dict(inp)
        i2["x"] = inp["x"] * 2.0 ** k
        o = run_lrblock(B, i2, "bf16", "silu", True, eps=0.0)
        assert torch.isfinite(o["Y"]).all()
        outs.append(host(o["Y"]))
    ref = oracle.lrblock_forward(inp["x"], inp["g"], inp["A_cat"], inp["B"], act="silu", eps=0.0)["Y"]
    for y in outs:
        check("Y", y, ref, "bf16")


def test_binding_rejects_mismatched_operands(B):
    """Operands that disagree with the descriptor are refused before any
    launch: a wrong down-weight shape, a gain of another dtype, a saved
    bottleneck of the wrong width, an output buffer of the wrong shape."""
    T, d, r, G, n = 64, 128, 64, 3, 128
    say("binding operand checks (no launch)")
    inp = synth.lrblock_inputs(T, d, r, G, n, dtype="bf16", seed=0)
    x, g, A, Bw, dY = (dev(inp[k], "bf16") for k in ("x", "g", "A_cat", "B", "dY"))
    with pytest.raises(ValueError, match="A_cat"):
        B.lrblock_fwd(x, g, A[:, :-64].contiguous(), Bw)
    with pytest.raises(TypeError, match="g has dtype"):
        B.lrblock_fwd(x, g.float(), A, Bw)
    Y, H, sumsq = B.lrblock_fwd(x, g, A, Bw)
    with pytest.raises(ValueError, match="H has shape"):
        B.lrblock_bwd(x, g, A, Bw, H[:, :-64].contiguous(), sumsq, dY)
    with pytest.raises(ValueError, match="dx"):
        B.lrblock_bwd(x, g, A, Bw, H, sumsq, dY, out=(torch.empty(T + 1, d, dtype=x.dtype, device=x.device),
                                                      None, None, None))
    torch.cuda.synchronize()
