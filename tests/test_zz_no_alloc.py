"""The forward that allocates nothing (boost_lrblock_fwd_noalloc) against the
workspace forward (boost_lrblock_fwd), through the C ABI.

Two calls in a row on one device share the library's fixed scratch: the
second, with a smaller input, must not see anything the first left behind.
Each result must equal the workspace forward's bit for bit (same kernels,
same plan), and both match the fp64 oracle within the bf16 tolerance. The
1B-shaped QKV forward (the largest configuration whose forward scratch fits
the fixed 64 MiB) is compared at full size; a larger descriptor is refused
before anything is launched.
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


def both(B, inp, dtype, act, norm):
    x, A, Bw = (dev(inp[k], dtype) for k in ("x", "A_cat", "B"))
    g = dev(inp["g"], dtype) if norm else None
    Y, H, s = B.lrblock_fwd(x, g, A, Bw, act=act, norm=norm)
    out = (torch.full_like(Y, float("nan")), torch.full_like(H, float("nan")),
           torch.full_like(s, float("nan")) if norm else None)
    Yn, Hn, sn = B.lrblock_fwd_noalloc(x, g, A, Bw, act=act, norm=norm, out=out)
    torch.cuda.synchronize()
    return (Y, H, s), (Yn, Hn, sn)


def same(name, a, b):
    if a is None:
        assert b is None
        return
    assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32)), name


@pytest.mark.parametrize("order", ["large_then_small"])
def test_two_calls_in_a_row_match_the_workspace_forward(B, order):
    cases = [(640, 1024, 256, 3, 768, "bf16", "silu", True),     # first call
             (300, 512, 192, 2, 320, "bf16", "identity", True)]  # smaller, ragged
    for (T, d, r, G, n, dtype, act, norm) in cases:
        say(f"  noalloc fwd T={T} d={d} r={r} G={G} d_out={n} {dtype} {act} norm={norm}")
        inp = synth.lrblock_inputs(T, d, r, G, n, dtype=dtype, seed=T, norm=norm)
        ref_ws, got = both(B, inp, dtype, act, norm)
        for k, a, b in zip(("Y", "H", "sumsq"), ref_ws, got):
            same(k, a, b)
        ref = oracle.lrblock_forward(inp["x"], inp.get("g"), inp["A_cat"], inp["B"], act=act, norm=norm)
        check("Y", host(got[0]), ref["Y"], dtype)
        check("H", host(got[1]), ref["H"], dtype)
        if norm:
            check("sumsq", host(got[2]), ref["sumsq"], dtype)


def test_full_size_1b_qkv_forward_and_the_limit(B):
    w = synth.WORKLOADS["llama2_1b_qkv_fwd"]
    T, d, r, G, n = w["T"], w["d"], w["r"], w["G"], w["d_out"]
    desc = B.lrblock_desc(T, d, r, G, n, B.DT_BF16)
    need = B.lrblock_workspace_size(desc, False)
    say(f"  1B QKV forward scratch: {need / 2**20:.1f} MiB of 64")
    assert need <= 64 << 20
    inp = synth.lrblock_inputs(T, d, r, G, n, dtype="bf16", seed=0)
    ref_ws, got = both(B, inp, "bf16", "silu", True)
    for k, a, b in zip(("Y", "H", "sumsq"), ref_ws, got):
        same(k, a, b)
    # sampled rows against the oracle
    rows = np.random.default_rng(1).choice(T, 64, replace=False)
    ref = oracle.lrblock_forward(inp["x"][rows], inp["g"], inp["A_cat"], inp["B"], act="silu", norm=True)
    check("Y rows", host(got[0])[:, rows], ref["Y"], "bf16")
    check("H rows", host(got[1])[rows], ref["H"], "bf16")
    # a forward whose scratch exceeds the fixed array is refused, nothing launched
    x = torch.zeros((T, 8192), dtype=torch.bfloat16, device="cuda")
    g = torch.ones(8192, dtype=torch.bfloat16, device="cuda")
    A = torch.zeros((8192, G * r), dtype=torch.bfloat16, device="cuda")
    Bw = torch.zeros((G, r, n), dtype=torch.bfloat16, device="cuda")
    out = (torch.zeros((G, T, n), dtype=torch.bfloat16, device="cuda"),
           torch.zeros((T, G * r), dtype=torch.float32, device="cuda"),
           torch.zeros(T, dtype=torch.float32, device="cuda"))
    big = B.lrblock_desc(T, 8192, r, G, n, B.DT_BF16)
    assert B.lrblock_workspace_size(big, False) > 64 << 20
    with pytest.raises(B.BoostError, match="UNSUPPORTED"):
        B.lrblock_fwd_noalloc(x, g, A, Bw, out=out)
    torch.cuda.synchronize()
    assert not out[0].view(torch.int16).any()
