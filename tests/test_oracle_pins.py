"""Pins of the fp64 oracle to things other than itself (CPU only).

Each oracle function is checked against at least one of: hand-worked values
(tests/golden), brute-force scalar loops on tiny non-square inputs, central
finite differences, a library SVD special case, exact homogeneity /
scale-invariance identities, and the sharded-equals-unsharded simulation of
the tensor-parallel share. The plausible mistakes these catch: a dropped
eps or wrong divisor (golden, unit-RMS), transposed or swapped operands
(brute force on non-square shapes, SVD), wrong signs or missing terms in a
gradient (finite differences, identities).
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import method_form
from rank_bottleneck_online_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def rng(seed=1):
    return np.random.default_rng(seed)


def block_inputs(T, d, r, G, d_out, seed=3):
    R = rng(seed)
    return dict(x=R.standard_normal((T, d)),
                g=1.0 + 0.3 * R.standard_normal(d),
                A_cat=R.standard_normal((d, G * r)) / math.sqrt(d),
                B=R.standard_normal((G, r, d_out)) / math.sqrt(r),
                dY=R.standard_normal((G, T, d_out)))


def mlp_inputs(T, d, r, ffn, seed=4):
    R = rng(seed)
    return dict(x=R.standard_normal((T, d)),
                g=1.0 + 0.3 * R.standard_normal(d),
                A1_cat=R.standard_normal((d, 2 * r)) / math.sqrt(d),
                B1=R.standard_normal((2, r, ffn)) / math.sqrt(r),
                A2=R.standard_normal((ffn, r)) / math.sqrt(ffn),
                B2=R.standard_normal((r, d)) / math.sqrt(r),
                dY=R.standard_normal((T, d)))


def btp_inputs(T, r, ds_, seed=5):
    R = rng(seed)
    return dict(z=R.standard_normal((T, r)),
                B_s=R.standard_normal((r, ds_)) / math.sqrt(r),
                g_s=1.0 + 0.3 * R.standard_normal(ds_),
                A_s=R.standard_normal((ds_, r)) / math.sqrt(4 * ds_),
                dp=R.standard_normal((T, r)),
                ds=0.01 * R.standard_normal(T))


# ---------------------------------------------------------------------------
# Hand-worked RMSNorm values and RMSNorm properties
# ---------------------------------------------------------------------------

def test_golden_rmsnorm_worked_examples():
    cases = json.load(open(os.path.join(GOLDEN, "rmsnorm_worked.json")))["cases"]
    for c in cases:
        x = np.array([c["x"]], np.float64)
        d = x.shape[1]
        # Through the whole block with identity factors: Y = RMSNorm(x) * g.
        out = oracle.lrblock_forward(x, np.array(c["g"], np.float64), np.eye(d),
                                     np.eye(d)[None], act="identity", norm=True,
                                     eps=c["eps"], d_norm=c["d_norm"])
        np.testing.assert_allclose(out["Y"][0, 0], c["y"], rtol=0, atol=1e-15)
        assert out["sumsq"][0] == pytest.approx(sum(v * v for v in c["x"]), abs=0)


def test_rmsnorm_rows_have_unit_rms_and_scale_invariance():
    R = rng(7)
    x = R.standard_normal((9, 24)) * R.uniform(0.01, 100, size=(9, 1))
    y, rho, sumsq = oracle.rmsnorm(x, np.ones(24), 0.0, 24)
    np.testing.assert_allclose(np.mean(y * y, axis=1), 1.0, rtol=1e-14)
    y2, _, _ = oracle.rmsnorm(x * 2.0 ** 7, np.ones(24), 0.0, 24)
    np.testing.assert_allclose(y2, y, rtol=1e-14)
    np.testing.assert_allclose(sumsq, [math.fsum(v * v for v in row) for row in x], rtol=1e-14)


# ---------------------------------------------------------------------------
# Brute force: scalar Python loops on tiny, non-square inputs
# ---------------------------------------------------------------------------

def _silu_s(z):
    return z / (1.0 + math.exp(-z))


def _bf_rms(x, g, eps, d_norm):
    out = []
    for row in x:
        rho = 1.0 / math.sqrt(math.fsum(v * v for v in row) / d_norm + eps)
        out.append([rho * v * gi for v, gi in zip(row, g)])
    return out


def _bf_mm(a, b):
    n_in, n_out = len(b), len(b[0])
    return [[math.fsum(a[t][k] * b[k][n] for k in range(n_in)) for n in range(n_out)]
            for t in range(len(a))]


@pytest.mark.parametrize("act", ["silu", "identity"])
@pytest.mark.parametrize("norm", [True, False])
def test_bruteforce_lrblock_forward(act, norm):
    T, d, r, G, d_out = 3, 8, 2, 3, 5
    inp = block_inputs(T, d, r, G, d_out, seed=11)
    out = oracle.lrblock_forward(inp["x"], inp["g"], inp["A_cat"], inp["B"], act=act,
                                 norm=norm, eps=1e-3)
    x = inp["x"].tolist()
    xh = _bf_rms(x, inp["g"].tolist(), 1e-3, d) if norm else x
    f = _silu_s if act == "silu" else (lambda z: z)
    for j in range(G):
        Aj = [[inp["A_cat"][i][j * r + k] for k in range(r)] for i in range(d)]
        Hj = _bf_mm(xh, Aj)
        Sj = [[f(v) for v in row] for row in Hj]
        Yj = _bf_mm(Sj, inp["B"][j].tolist())
        np.testing.assert_allclose(out["H"][:, j * r:(j + 1) * r], Hj, rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(out["Y"][j], Yj, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("act", ["silu", "identity"])
def test_bruteforce_lrmlp_forward(act):
    T, d, r, ffn = 3, 8, 2, 6
    inp = mlp_inputs(T, d, r, ffn, seed=12)
    out = oracle.lrmlp_forward(inp["x"], inp["g"], inp["A1_cat"], inp["B1"], inp["A2"],
                               inp["B2"], act=act, eps=1e-3)
    f = _silu_s if act == "silu" else (lambda z: z)
    xh = _bf_rms(inp["x"].tolist(), inp["g"].tolist(), 1e-3, d)
    H1 = _bf_mm(xh, inp["A1_cat"].tolist())
    S1 = [[f(v) for v in row] for row in H1]
    Yg = _bf_mm([row[:r] for row in S1], inp["B1"][0].tolist())
    Yu = _bf_mm([row[r:] for row in S1], inp["B1"][1].tolist())
    M = [[_silu_s(a) * b for a, b in zip(ra, rb)] for ra, rb in zip(Yg, Yu)]
    H2 = _bf_mm(M, inp["A2"].tolist())
    Y = _bf_mm([[f(v) for v in row] for row in H2], inp["B2"].tolist())
    np.testing.assert_allclose(out["H1"], H1, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(out["H2"], H2, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(out["Y"], Y, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(out["sumsq"], [math.fsum(v * v for v in row) for row in inp["x"]],
                               rtol=1e-14)


def test_bruteforce_btp_share_forward():
    T, r, dsh = 3, 5, 4
    inp = btp_inputs(T, r, dsh, seed=13)
    out = oracle.btp_share_forward(inp["z"], inp["B_s"], inp["g_s"], inp["A_s"])
    u = _bf_mm(inp["z"].tolist(), inp["B_s"].tolist())
    a = [[_silu_s(v) for v in row] for row in u]
    s = [math.fsum(v * v for v in row) for row in a]
    ag = [[v * gi for v, gi in zip(row, inp["g_s"])] for row in a]
    p = _bf_mm(ag, inp["A_s"].tolist())
    np.testing.assert_allclose(out["p"], p, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(out["s"], s, rtol=1e-14)


# ---------------------------------------------------------------------------
# Library special case: SVD-style factors of a dense weight
# ---------------------------------------------------------------------------

def test_svd_variant_reconstructs_truncated_dense_layer():
    R = rng(21)
    T, d = 7, 16
    x = R.standard_normal((T, d))
    g = 1.0 + 0.2 * R.standard_normal(d)
    W = R.standard_normal((d, d)) / 4.0
    U, sv, Vt = np.linalg.svd(W)
    xh = x / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + 1e-5) * g
    for r in (5, d):
        A = U[:, :r] * np.sqrt(sv[:r])
        B = (np.sqrt(sv[:r])[:, None] * Vt[:r])[None]
        Y = oracle.lrblock_forward(x, g, A, B, act="identity", norm=True, eps=1e-5)["Y"][0]
        W_r = (U[:, :r] * sv[:r]) @ Vt[:r]
        assert rel(Y, xh @ W_r) < 1e-12
    assert rel(Y, xh @ W) < 1e-12   # full rank: the dense layer itself


# ---------------------------------------------------------------------------
# Method form (deferred scale, grouped products, checkpointed backward)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("act", ["silu", "identity"])
def test_deferred_grouped_forward_equals_plain(act):
    inp = block_inputs(64, 256, 64, 3, 256, seed=31)
    a = oracle.lrblock_forward(inp["x"], inp["g"], inp["A_cat"], inp["B"], act=act, eps=1e-5)
    b = method_form.lrblock_forward_deferred(inp["x"], inp["g"], inp["A_cat"], inp["B"], act=act,
                                             eps=1e-5)
    for k in ("Y", "H", "sumsq"):
        assert rel(b[k], a[k]) < 1e-13, k


@pytest.mark.parametrize("act", ["silu", "identity"])
def test_checkpointed_backward_equals_full_store(act):
    inp = block_inputs(64, 256, 64, 3, 256, seed=32)
    f = oracle.lrblock_forward(inp["x"], inp["g"], inp["A_cat"], inp["B"], act=act, eps=1e-5)
    a = oracle.lrblock_backward(inp["x"], inp["g"], inp["A_cat"], inp["B"], inp["dY"], act=act,
                                eps=1e-5)
    b = method_form.lrblock_backward_checkpointed(inp["x"], inp["g"], inp["A_cat"], inp["B"],
                                                  f["H"], f["sumsq"], inp["dY"], act=act, eps=1e-5)
    for k in ("dx", "dg", "dA_cat", "dB"):
        assert rel(b[k], a[k]) < 1e-12, k


# ---------------------------------------------------------------------------
# Finite differences on L = <dY, Y> (and <dp,p> + <ds,s> for the share)
# ---------------------------------------------------------------------------

def _fd_check(loss, params, grads, seed, h=1e-5, tol=1e-7):
    R = rng(seed)
    for name in params:
        v = R.standard_normal(params[name].shape)
        p0 = params[name]
        params[name] = p0 + h * v
        lp = loss(params)
        params[name] = p0 - h * v
        lm = loss(params)
        params[name] = p0
        fd = (lp - lm) / (2 * h)
        an = float(np.sum(grads[name] * v))
        assert abs(fd - an) <= tol * max(abs(an), 1e-3), (name, fd, an)


@pytest.mark.parametrize("act", ["silu", "identity"])
@pytest.mark.parametrize("norm", [True, False])
@pytest.mark.parametrize("shape", [(3, 8, 2, 3, 5), (64, 256, 64, 3, 256)])
def test_fd_lrblock(act, norm, shape):
    inp = block_inputs(*shape, seed=41)
    params = {k: inp[k] for k in ("x", "g", "A_cat", "B")}
    if not norm:
        params.pop("g")

    def loss(p):
        Y = oracle.lrblock_forward(p["x"], p.get("g"), p["A_cat"], p["B"], act=act, norm=norm,
                                   eps=1e-5)["Y"]
        return float(np.sum(inp["dY"] * Y))

    gr = oracle.lrblock_backward(inp["x"], inp.get("g"), inp["A_cat"], inp["B"], inp["dY"],
                                 act=act, norm=norm, eps=1e-5)
    grads = {"x": gr["dx"], "g": gr["dg"], "A_cat": gr["dA_cat"], "B": gr["dB"]}
    _fd_check(loss, params, grads, seed=42)


@pytest.mark.parametrize("act", ["silu", "identity"])
@pytest.mark.parametrize("shape", [(3, 8, 2, 6), (32, 128, 64, 192)])
def test_fd_lrmlp(act, shape):
    inp = mlp_inputs(*shape, seed=43)
    names = ("x", "g", "A1_cat", "B1", "A2", "B2")
    params = {k: inp[k] for k in names}

    def loss(p):
        Y = oracle.lrmlp_forward(*(p[k] for k in names), act=act, eps=1e-5)["Y"]
        return float(np.sum(inp["dY"] * Y))

    gr = oracle.lrmlp_backward(*(inp[k] for k in names), inp["dY"], act=act, eps=1e-5)
    grads = {"x": gr["dx"], "g": gr["dg"], "A1_cat": gr["dA1_cat"], "B1": gr["dB1"],
             "A2": gr["dA2"], "B2": gr["dB2"]}
    _fd_check(loss, params, grads, seed=44)


@pytest.mark.parametrize("shape", [(3, 5, 4), (32, 64, 128)])
def test_fd_btp_share(shape):
    inp = btp_inputs(*shape, seed=45)
    names = ("z", "B_s", "g_s", "A_s")
    params = {k: inp[k] for k in names}

    def loss(p):
        o = oracle.btp_share_forward(*(p[k] for k in names))
        return float(np.sum(inp["dp"] * o["p"]) + np.sum(inp["ds"] * o["s"]))

    gr = oracle.btp_share_backward(*(inp[k] for k in names), inp["dp"], inp["ds"])
    grads = {"z": gr["dz"], "B_s": gr["dB_s"], "g_s": gr["dg_s"], "A_s": gr["dA_s"]}
    _fd_check(loss, params, grads, seed=46)


# ---------------------------------------------------------------------------
# Exact identities (also usable on full-size GPU outputs)
# ---------------------------------------------------------------------------

def _dot(a, b):
    return float(np.sum(np.asarray(a) * np.asarray(b)))


@pytest.mark.parametrize("act", ["silu", "identity"])
def test_lrblock_homogeneity_identities(act):
    inp = block_inputs(16, 64, 16, 3, 48, seed=51)
    f = oracle.lrblock_forward(inp["x"], inp["g"], inp["A_cat"], inp["B"], act=act, eps=0.0)
    gr = oracle.lrblock_backward(inp["x"], inp["g"], inp["A_cat"], inp["B"], inp["dY"], act=act,
                                 eps=0.0)
    L = _dot(inp["dY"], f["Y"])
    assert _dot(gr["dB"], inp["B"]) == pytest.approx(L, rel=1e-12)       # Y linear in B
    if act == "identity":                                                # ... and in A, g
        assert _dot(gr["dA_cat"], inp["A_cat"]) == pytest.approx(L, rel=1e-12)
        assert _dot(gr["dg"], inp["g"]) == pytest.approx(L, rel=1e-12)
    # eps = 0: Y is invariant to scaling a row of x, so <dx_t, x_t> = 0.
    per_row = np.sum(gr["dx"] * inp["x"], axis=1)
    assert np.max(np.abs(per_row)) < 1e-12 * np.max(np.abs(gr["dx"])) * inp["x"].shape[1]


@pytest.mark.parametrize("act", ["silu", "identity"])
def test_lrmlp_homogeneity_identities(act):
    inp = mlp_inputs(16, 64, 16, 96, seed=52)
    names = ("x", "g", "A1_cat", "B1", "A2", "B2")
    f = oracle.lrmlp_forward(*(inp[k] for k in names), act=act, eps=0.0)
    gr = oracle.lrmlp_backward(*(inp[k] for k in names), inp["dY"], act=act, eps=0.0)
    L = _dot(inp["dY"], f["Y"])
    assert _dot(gr["dB2"], inp["B2"]) == pytest.approx(L, rel=1e-12)
    if act == "identity":
        assert _dot(gr["dA2"], inp["A2"]) == pytest.approx(L, rel=1e-12)
        assert _dot(gr["dB1"][1], inp["B1"][1]) == pytest.approx(L, rel=1e-12)
    per_row = np.sum(gr["dx"] * inp["x"], axis=1)
    assert np.max(np.abs(per_row)) < 1e-12 * np.max(np.abs(gr["dx"])) * inp["x"].shape[1]


def test_btp_share_linearity_identities():
    inp = btp_inputs(16, 32, 64, seed=53)
    names = ("z", "B_s", "g_s", "A_s")
    f = oracle.btp_share_forward(*(inp[k] for k in names))
    gr = oracle.btp_share_backward(*(inp[k] for k in names), inp["dp"], inp["ds"])
    Lp = _dot(inp["dp"], f["p"])
    assert _dot(gr["dA_s"], inp["A_s"]) == pytest.approx(Lp, rel=1e-12)
    assert _dot(gr["dg_s"], inp["g_s"]) == pytest.approx(Lp, rel=1e-12)


# ---------------------------------------------------------------------------
# Tensor-parallel share: P shares reproduce the unsharded pair
# ---------------------------------------------------------------------------

def test_btp_shards_reproduce_unsharded_pair():
    T, r, D, P, eps = 24, 32, 128, 4, 1e-5
    R = rng(61)
    z = R.standard_normal((T, r))
    B_full = R.standard_normal((r, D)) / math.sqrt(r)
    A_full = R.standard_normal((D, r)) / math.sqrt(D)
    g_full = 1.0 + 0.3 * R.standard_normal(D)
    dz_next = R.standard_normal((T, r))
    w = D // P
    shards = [dict(z=z, B_s=B_full[:, p * w:(p + 1) * w], g_s=g_full[p * w:(p + 1) * w],
                   A_s=A_full[p * w:(p + 1) * w]) for p in range(P)]
    fw = [oracle.btp_share_forward(**s) for s in shards]
    z_next, rho, Psum = oracle.btp_consumer([f["p"] for f in fw], [f["s"] for f in fw], eps, D)

    # Unsharded: a = SiLU(z B_full); z_next = RMSNorm(a; g_full, global width) A_full.
    u = z @ B_full
    a = oracle.silu(u)
    ref = oracle.lrblock_forward(a, g_full, A_full, np.eye(r)[None], act="identity", norm=True,
                                 eps=eps, d_norm=D)
    assert rel(z_next, ref["Y"][0]) < 1e-12
    assert rel(sum(f["s"] for f in fw), ref["sumsq"]) < 1e-13

    # Backward: the gradients of one share's outputs are local (no exchange).
    dp, ds = oracle.btp_consumer_backward(dz_next, rho, Psum, D)
    bw = [oracle.btp_share_backward(**s, dp=dp, ds=ds) for s in shards]
    ub = oracle.lrblock_backward(a, g_full, A_full, np.eye(r)[None], dz_next[None],
                                 act="identity", norm=True, eps=eps, d_norm=D)
    du = ub["dx"] * oracle.silu_grad(u)
    assert rel(np.concatenate([b["dA_s"] for b in bw], axis=0), ub["dA_cat"]) < 1e-12
    assert rel(np.concatenate([b["dg_s"] for b in bw]), ub["dg"]) < 1e-12
    assert rel(np.concatenate([b["dB_s"] for b in bw], axis=1), z.T @ du) < 1e-12
    assert rel(sum(b["dz"] for b in bw), du @ B_full.T) < 1e-12


# ---------------------------------------------------------------------------
# The seeded generator (shared by both sides) is deterministic and exact
# ---------------------------------------------------------------------------

def test_generator_deterministic_and_bf16_exact():
    a = synth.lrblock_inputs(8, 64, 16, 3, 64, dtype="bf16", seed=0)
    b = synth.lrblock_inputs(8, 64, 16, 3, 64, dtype="bf16", seed=0)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])
        bits = synth.storage_bits(a[k], "bf16")
        np.testing.assert_array_equal(synth.from_bits(bits, "bf16"), a[k])


def test_bf16_rounding_ties_to_even():
    # 1 + 2^-8 lies halfway between bf16 neighbours 1 and 1 + 2^-7: ties go to
    # the even significand (1); 1 + 3*2^-8 ties up to 1 + 2^-6.
    v = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 1 + 2.0 ** -8 + 2.0 ** -30])
    np.testing.assert_array_equal(synth.round_to_bf16(v), [1.0, 1 + 2.0 ** -6, -1.0, 1 + 2.0 ** -7])


def test_stored_results_round_through_fp32():
    # A stored result is the fp32 value rounded to bf16, as a device stores
    # its fp32 results. The stand-in sum -1.0703125 - (2^-26 + 2^-28) -
    # 0.35546875 lies 1.86e-8 beyond the bf16 midpoint -1.42578125; that is
    # under half an fp32 ulp (5.96e-8), so fp32 holds the midpoint itself and
    # the tie goes to the even neighbour -1.421875 (a single rounding of the
    # exact sum would give -1.4296875).
    qkv = np.array([[[-1.0703125]], [[-(2.0 ** -26 + 2.0 ** -28)]], [[-0.35546875]]])
    s = oracle.standin_forward(qkv)
    assert s[0, 0] == -1.0703125 - (2.0 ** -26 + 2.0 ** -28) - 0.35546875
    assert oracle.round_to_bf16(s)[0, 0] == -1.421875
