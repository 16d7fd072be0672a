"""The C-ABI library loads, exports every symbol its header declares, and
rejects bad arguments before anything is launched (CPU only: no call here
reaches a device API)."""
import ctypes
import os
import re

import pytest

from rank_bottleneck_online_amd import build as rbo_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "boost_lrblock.h")


@pytest.fixture(scope="module")
def B():
    if not os.path.exists(rbo_build.LIB_PATH):
        rbo_build.build()
    from rank_bottleneck_online_amd import binding
    return binding


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(boost_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("boost_lrblock_fwd", "boost_lrblock_bwd", "boost_lrmlp_fwd", "boost_lrmlp_bwd",
              "boost_btp_share_fwd", "boost_btp_share_bwd", "boost_status_string",
              "boost_last_error_detail", "boost_abi_version"):
        assert n in names


def test_library_exports_every_declared_symbol(B):
    L = B.lib()
    missing = [n for n in declared_functions() if not hasattr(L, n)]
    assert not missing, missing
    # and the binding declares a signature for every one of them
    assert set(declared_functions()) <= set(B._SIGS)


def test_abi_version_and_status_strings(B):
    L = B.lib()
    assert L.boost_abi_version() == 1
    for code, name in [(0, "BOOST_OK"), (1, "BOOST_ERR_INVALID_VALUE"), (2, "BOOST_ERR_UNSUPPORTED"),
                       (3, "BOOST_ERR_MISALIGNED"), (4, "BOOST_ERR_ALIASING"), (5, "BOOST_ERR_WORKSPACE"),
                       (6, "BOOST_ERR_VERSION"), (7, "BOOST_ERR_LAUNCH")]:
        assert L.boost_status_string(code).decode() == name
    assert L.boost_status_string(99).decode() == "BOOST_ERR_UNKNOWN"


def test_serialize_switch_validates_and_toggles(B):
    L = B.lib()
    assert L.boost_profiler_serialize(2) == 1
    assert "must be 0 or 1" in L.boost_last_error_detail().decode()
    assert L.boost_profiler_serialize(1) == 0
    assert L.boost_profiler_serialize(0) == 0


# Fake, 256-byte aligned, non-overlapping "device" addresses: validation only
# compares them, it never dereferences them.
class Fake:
    def __init__(self):
        self.next = 1 << 40

    def __call__(self, nbytes):
        p = self.next
        self.next += (nbytes + 4095) // 4096 * 4096 + 4096
        return p


def lrblock_call(B, desc, fwd=True, mutate=None, ws_bytes=None):
    L = B.lib()
    T, d, r, G, n = desc.T, desc.d, desc.r, desc.G, desc.d_out
    es = 4 if desc.dtype == B.DT_F32 else 2
    f = Fake()
    try:
        need = B.lrblock_workspace_size(desc, not fwd)
    except B.BoostError:
        need = 1024  # the descriptor itself is invalid; the call must fail before the workspace check
    ws_bytes = need if ws_bytes is None else ws_bytes
    if fwd:
        args = dict(x=f(T * d * es), g=f(d * es), A=f(d * G * r * es), B=f(G * r * n * es), Y=f(G * T * n * es),
                    H=f(T * G * r * 4), s=f(T * 4), ws=f(max(ws_bytes, 1)))
        if mutate:
            mutate(args)
        return L.boost_lrblock_fwd(ctypes.byref(desc), args["x"], args["g"], args["A"], args["B"], args["Y"],
                                   args["H"], args["s"], args["ws"], ws_bytes, None)
    args = dict(x=f(T * d * es), g=f(d * es), A=f(d * G * r * es), B=f(G * r * n * es), H=f(T * G * r * 4),
                s=f(T * 4), dY=f(G * T * n * es), dx=f(T * d * es), dg=f(d * 4), dA=f(d * G * r * 4),
                dB=f(G * r * n * 4), ws=f(max(ws_bytes, 1)))
    if mutate:
        mutate(args)
    return L.boost_lrblock_bwd(ctypes.byref(desc), args["x"], args["g"], args["A"], args["B"], args["H"],
                               args["s"], args["dY"], args["dx"], args["dg"], args["dA"], args["dB"], args["ws"],
                               ws_bytes, None)


def desc_(B, **kw):
    base = dict(T=300, d=256, r=64, G=3, d_out=192, dtype=B.DT_BF16, act="silu", norm=True, eps=1e-5)
    base.update(kw)
    return B.lrblock_desc(**base)


@pytest.mark.parametrize("fwd", [True, False])
def test_lrblock_validation_errors(B, fwd):
    E_INV, E_UNS, E_MIS, E_ALI, E_WS, E_VER = 1, 2, 3, 4, 5, 6
    L = B.lib()
    dsc = desc_(B)
    dsc.abi_version = 2
    assert lrblock_call(B, dsc, fwd) == E_VER
    assert b"abi_version" in L.boost_last_error_detail()
    assert lrblock_call(B, desc_(B, d=100), fwd) == E_UNS           # not a multiple of 64
    assert lrblock_call(B, desc_(B, r=0), fwd) == E_INV
    assert lrblock_call(B, desc_(B, G=17), fwd) == E_INV
    assert lrblock_call(B, desc_(B, T=0), fwd) == E_INV
    assert lrblock_call(B, desc_(B, eps=-1.0), fwd) == E_INV
    assert lrblock_call(B, desc_(B, eps=float("nan")), fwd) == E_INV
    assert lrblock_call(B, desc_(B, d_norm=128), fwd) == E_INV      # d_norm < d
    dsc = desc_(B)
    dsc.dtype = 7
    assert lrblock_call(B, dsc, fwd) == E_INV
    dsc = desc_(B)
    dsc.act = 5
    assert lrblock_call(B, dsc, fwd) == E_INV
    dsc = desc_(B)
    dsc.norm = 2
    assert lrblock_call(B, dsc, fwd) == E_INV
    # pointers
    assert lrblock_call(B, desc_(B), fwd, mutate=lambda a: a.update(x=None)) == E_INV
    assert b"x is NULL" in L.boost_last_error_detail()
    assert lrblock_call(B, desc_(B), fwd, mutate=lambda a: a.update(g=None)) == E_INV
    assert lrblock_call(B, desc_(B), fwd, mutate=lambda a: a.update(A=a["A"] + 2)) == E_MIS
    # aliasing: an output on top of an input
    if fwd:
        assert lrblock_call(B, desc_(B), fwd, mutate=lambda a: a.update(Y=a["x"])) == E_ALI
    else:
        assert lrblock_call(B, desc_(B), fwd, mutate=lambda a: a.update(dx=a["x"])) == E_ALI
        assert lrblock_call(B, desc_(B), fwd, mutate=lambda a: a.update(ws=a["dB"])) == E_ALI
    # workspace
    need = B.lrblock_workspace_size(desc_(B), not fwd)
    assert need > 0
    assert lrblock_call(B, desc_(B), fwd, ws_bytes=need - 256) == E_WS
    assert lrblock_call(B, desc_(B), fwd, mutate=lambda a: a.update(ws=None)) == E_WS
    # a too-large tensor is refused (buffer addressing is 32-bit)
    assert lrblock_call(B, desc_(B, T=1 << 20, d=2048), fwd) == E_UNS


def test_norm0_accepts_null_gain_and_stats(B):
    # norm = 0 (an O-projection): g, sumsq and dg may be NULL. With every
    # other argument valid, only the workspace check is left to fail.
    need = B.lrblock_workspace_size(desc_(B, norm=False), True)
    r = lrblock_call(B, desc_(B, norm=False), False, ws_bytes=need - 256,
                     mutate=lambda a: a.update(g=None, s=None, dg=None))
    assert r == 5
    r = lrblock_call(B, desc_(B, norm=False), True, ws_bytes=1,
                     mutate=lambda a: a.update(g=None, s=None))
    assert r == 5


def test_mlp_and_btp_validation(B):
    L = B.lib()
    d = B.lrmlp_desc(128, 256, 64, 100, B.DT_BF16)
    n = ctypes.c_size_t(0)
    assert L.boost_lrmlp_workspace_size(ctypes.byref(d), 0, ctypes.byref(n)) == 2   # ffn % 64
    d = B.lrmlp_desc(128, 256, 64, 192, B.DT_BF16)
    d.reserved = 1
    assert L.boost_lrmlp_workspace_size(ctypes.byref(d), 0, ctypes.byref(n)) == 1
    d = B.lrmlp_desc(128, 256, 64, 192, B.DT_BF16)
    assert L.boost_lrmlp_workspace_size(ctypes.byref(d), 1, None) == 1
    f = Fake()
    args = [f(1 << 20) for _ in range(10)]
    assert L.boost_lrmlp_fwd(ctypes.byref(d), *args, None, 0, None) == 5
    args[0] = None
    assert L.boost_lrmlp_fwd(ctypes.byref(d), *args, None, 0, None) == 1
    b = B.btp_desc(128, 64, 96, B.DT_BF16)
    assert L.boost_btp_share_workspace_size(ctypes.byref(b), 0, ctypes.byref(n)) == 2
    b = B.btp_desc(128, 64, 128, B.DT_F32)
    assert L.boost_btp_share_workspace_size(ctypes.byref(b), 1, ctypes.byref(n)) == 0
    assert n.value > 0


def test_workspace_sizes_scale_with_tokens(B):
    # The token-dependent part of the workspace grows linearly with T (the
    # transposed weights are a fixed part).
    w = {T: B.lrmlp_workspace_size(B.lrmlp_desc(T, 4096, 1024, 11008, B.DT_BF16), True)
         for T in (2048, 4096, 8192)}
    assert w[8192] - w[4096] == pytest.approx(2 * (w[4096] - w[2048]), rel=0.02)
    assert w[2048] > 0


def test_chained_entry_points_validate_their_extra_arguments(B):
    E_INV, E_UNS, E_ALI, E_WS = 1, 2, 4, 5
    L = B.lib()
    f = Fake()
    T, d, r = 300, 256, 64

    def fwd(desc, residual=True, sumsq_in=False, sumsq=True, snext=True, ws_bytes=1):
        G, n = desc.G, desc.d_out
        x, g, A, Bw = f(T * d * 2), f(d * 2), f(d * G * r * 2), f(G * r * n * 2)
        return L.boost_lrblock_fwd_chained(ctypes.byref(desc), x, g, A, Bw, f(T * n * 2) if residual else None,
                                           f(T * 4) if sumsq_in else None, f(G * T * n * 2), f(T * G * r * 4),
                                           f(T * 4) if sumsq else None, f(T * 4) if snext else None, f(1 << 20),
                                           ws_bytes, None)

    # residual and the next statistic need G = 1
    assert fwd(desc_(B, G=3, d_out=256)) == E_UNS
    assert fwd(desc_(B, G=3, d_out=256), residual=False) == E_UNS
    # with G = 1 every extra argument is accepted; only the tiny workspace fails
    assert fwd(desc_(B, G=1, d_out=256)) == E_WS
    assert fwd(desc_(B, G=1, d_out=256), sumsq_in=True, sumsq=False) == E_WS
    # a producer statistic makes no sense without the norm
    assert fwd(desc_(B, G=1, d_out=256, norm=False), sumsq_in=True, sumsq=False) == E_INV
    # the residual path of the backward is only fused into the normalised dx
    dsc = desc_(B, G=1, d_out=256, norm=False)
    args = [f(1 << 20) for _ in range(12)]
    assert L.boost_lrblock_bwd_chained(ctypes.byref(dsc), *args, f(1 << 20), 1, None) == E_UNS
    # stand-in: dims and overlap
    qkv, a = f(3 * T * d * 2), f(T * d * 2)
    assert L.boost_attn_standin_fwd(B.DT_BF16, T, 100, qkv, a, None) == E_UNS
    assert L.boost_attn_standin_fwd(B.DT_BF16, T, d, qkv, qkv, None) == E_ALI
    assert L.boost_attn_standin_bwd(B.DT_BF16, T, d, None, qkv, None) == E_INV
    # MLP chained forward: extra arguments accepted, then the workspace check
    m = B.lrmlp_desc(128, 256, 64, 192, B.DT_BF16)
    margs = [f(1 << 20) for _ in range(6)] + [f(1 << 20), f(1 << 20)] + [f(1 << 20) for _ in range(4)] + [f(1 << 20)]
    assert L.boost_lrmlp_fwd_chained(ctypes.byref(m), *margs, f(1 << 20), 1, None) == E_WS


def test_binding_checks_operands_against_the_descriptor():
    """The binding rejects operands whose shape, dtype or layout differ from
    what the descriptor implies (the C ABI takes plain pointers and cannot)."""
    import torch

    from rank_bottleneck_online_amd import binding
    x = torch.zeros(4, 8, dtype=torch.bfloat16)
    assert binding._arg(torch.zeros(8, dtype=torch.bfloat16), (8,), torch.bfloat16, x, "g") is not None
    with pytest.raises(ValueError, match="shape"):
        binding._arg(torch.zeros(9, dtype=torch.bfloat16), (8,), torch.bfloat16, x, "g")
    with pytest.raises(TypeError, match="dtype"):
        binding._arg(torch.zeros(8, dtype=torch.float32), (8,), torch.bfloat16, x, "g")
    with pytest.raises(ValueError, match="contiguous"):
        binding._arg(torch.zeros(8, 4, dtype=torch.bfloat16).t(), (4, 8), torch.bfloat16, x, "A")
    with pytest.raises(TypeError, match="torch.Tensor"):
        binding._arg([0.0] * 8, (8,), torch.bfloat16, x, "g")
    assert binding._opt(None, (8,), torch.bfloat16, x, "g") is None
    with pytest.raises(ValueError, match="GPU"):
        binding._anchor(x, "x")
    assert binding._nbytes(torch.zeros(10, dtype=torch.float32)) == 40


def test_workspace_limit_applies_per_buffer_not_to_the_whole_workspace(B):
    """Each buffer carved from a workspace is addressed on its own, so only
    those buffers (and every tensor) must stay below 2 GiB: the 40B-shaped
    MLP backward at T = 16384 needs a workspace above 2 GiB and is accepted
    (the call goes on to the workspace-size check), while a descriptor whose
    largest workspace buffer reaches 2 GiB, or a tensor of 2 GiB, is refused."""
    E_UNS, E_WS = 2, 5
    L = B.lib()
    d, r, ffn = 8192, 2048, 22016
    desc = B.lrmlp_desc(16384, d, r, ffn, B.DT_BF16)
    need = B.lrmlp_workspace_size(desc, True)
    assert need > (1 << 31)
    f = Fake()
    T = desc.T
    es = 2
    ins = [f(T * d * es), f(d * es), f(d * 2 * r * es), f(2 * r * ffn * es), f(ffn * r * es), f(r * d * es),
           f(T * 2 * r * 4), f(T * r * 4), f(T * 4), f(T * d * es)]
    outs = [f(T * d * es), f(d * 4), f(d * 2 * r * 4), f(2 * r * ffn * 4), f(ffn * r * 4), f(r * d * 4)]
    ws = f(need)
    assert L.boost_lrmlp_bwd(ctypes.byref(desc), *ins, *outs, ws, need - 256, None) == E_WS
    assert b"workspace of" in L.boost_last_error_detail()
    # T = 32768: every tensor is below 2 GiB, but the [2, T, ffn] gradient
    # buffer of the workspace is 2.9 GB
    big = B.lrmlp_desc(32768, d, r, ffn, B.DT_BF16)
    n = ctypes.c_size_t(0)
    assert L.boost_lrmlp_workspace_size(ctypes.byref(big), 1, ctypes.byref(n)) == E_UNS
    assert b"smaller than 2 GiB" in L.boost_last_error_detail()
    # a 2 GiB input tensor is refused
    huge = B.lrmlp_desc(131072, d, r, ffn, B.DT_BF16)
    T = huge.T
    ins = [f(T * d * es)] + ins[1:6] + [f(T * 2 * r * 4), f(T * r * 4), f(T * 4), f(T * d * es)]
    outs = [f(T * d * es)] + outs[1:]
    assert L.boost_lrmlp_bwd(ctypes.byref(huge), *ins, *outs, f(1 << 20), 1 << 20, None) == E_UNS
    assert b"x is" in L.boost_last_error_detail()
