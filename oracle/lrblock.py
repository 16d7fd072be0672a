"""Plain fp64 CPU oracle of the low-rank bottleneck block.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. It shares no
code with the GPU path and never imports it.

What it computes follows the BOOST summary pages ("BOOST: BOttleneck-
Optimized Scalable Training Framework for Low-Rank Large Language Models",
gist.science, paper 2512.12131; technical summary):

* §1 and §2.1: a low-rank bottleneck layer replaces a dense d x d_out weight
  by a down factor (d x r) and an up factor (r x d_out);
* §4: the bottleneck variants CoLA (a nonlinearity between the factors,
  taken here as SiLU) and SVD (identity between the factors);
* §2.2 "Online-RMSNorm": the block's input is RMS-normalised; the method
  computes local statistics and defers the global normalisation, which the
  page states is mathematically equal to plain RMSNorm. The oracle is the
  plain RMSNorm;
* §2.2 "linear-layer grouping": the down projections that share an input
  are grouped into one product with concatenated weights, and the up
  projections are run as one batched product. The oracle computes every
  group's product separately (the plain definition);
* §2.2 "communication-free low-rank activation checkpointing": the method
  keeps only the bottleneck activations and recomputes the rest in the
  backward. The oracle's backward instead keeps every intermediate of its
  own forward (the plain definition; the checkpointed form must give the
  same numbers);
* §2.1 "BTP": one tensor-parallel share runs a column slice of the up
  projection, the intermediate ops on the sharded activation, and a row
  slice of the following down projection; RMSNorm statistics are local
  per-row partial sums.

Readings where the pages are silent (all written down in the design notes):
eps sits inside the square root and is added to the mean square; the
mean-square divisor ``d_norm`` is the global width; the local statistic is
the per-row sum of squares; the gain multiplies the normalised input
elementwise; SwiGLU is SiLU(gate) * up with gate = group 0 and up = group 1.

All arithmetic is fp64 on fp64 arrays. Parity unpinned: nothing. Every
function here is pinned by the CPU tests (brute-force scalar loops on tiny
inputs, finite differences, a library-SVD special case, a hand-worked
RMSNorm example, homogeneity and scale-invariance identities, and the
sharded-equals-unsharded simulation).
"""
from __future__ import annotations

import numpy as np

ACTS = ("silu", "identity")


# ---------------------------------------------------------------------------
# Elementwise functions
# ---------------------------------------------------------------------------

def sigmoid(z):
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def silu(z):
    """SiLU(z) = z * sigmoid(z) (CoLA's bottleneck nonlinearity)."""
    return z * sigmoid(z)


def silu_grad(z):
    """d/dz SiLU(z) = s + z * s * (1 - s), s = sigmoid(z)."""
    s = sigmoid(z)
    return s * (1.0 + z * (1.0 - s))


def act_fn(z, act):
    if act == "silu":
        return silu(z)
    if act == "identity":
        return np.array(z, dtype=np.float64, copy=True)
    raise ValueError(f"unknown bottleneck activation {act!r}")


def act_grad(z, act):
    if act == "silu":
        return silu_grad(z)
    if act == "identity":
        return np.ones_like(z, dtype=np.float64)
    raise ValueError(f"unknown bottleneck activation {act!r}")


# ---------------------------------------------------------------------------
# RMSNorm (plain, global statistics)
# ---------------------------------------------------------------------------

def rmsnorm(x, g, eps, d_norm):
    """Plain RMSNorm of each row of x[T,d]: rho_t * x_t * g with
    rho_t = 1/sqrt(sum_i x_ti^2 / d_norm + eps).

    Returns (x_hat, rho[T], sumsq[T]).
    """
    x = np.asarray(x, dtype=np.float64)
    sumsq = np.sum(x * x, axis=1)
    rho = 1.0 / np.sqrt(sumsq / d_norm + eps)
    return rho[:, None] * x * np.asarray(g, dtype=np.float64)[None, :], rho, sumsq


# ---------------------------------------------------------------------------
# Grouped low-rank block (QKV-style; O-projection when norm is False)
# ---------------------------------------------------------------------------

def _group_cols(r, j):
    return slice(j * r, (j + 1) * r)


def lrblock_forward(x, g, A_cat, B, act="silu", norm=True, eps=1e-5, d_norm=None,
                    keep=False):
    """Forward of the grouped low-rank block.

    x[T,d], g[d] (ignored when norm is False), A_cat[d,G*r] (group j owns
    columns j*r..(j+1)*r-1), B[G,r,d_out].

    H_j = RMSNorm(x) @ A_j (one product per group), S_j = act(H_j),
    Y_j = S_j @ B_j. Returns Y[G,T,d_out], H[T,G*r], sumsq[T] (None when
    norm is False); with keep=True also every intermediate.
    """
    x = np.asarray(x, np.float64)
    A_cat = np.asarray(A_cat, np.float64)
    B = np.asarray(B, np.float64)
    G, r, _ = B.shape
    d = x.shape[1]
    if d_norm is None:
        d_norm = d
    if norm:
        xhat, rho, sumsq = rmsnorm(x, g, eps, d_norm)
    else:
        xhat, rho, sumsq = x, None, None
    H_parts = [xhat @ A_cat[:, _group_cols(r, j)] for j in range(G)]
    S_parts = [act_fn(h, act) for h in H_parts]
    Y = np.stack([S_parts[j] @ B[j] for j in range(G)])
    H = np.concatenate(H_parts, axis=1)
    out = {"Y": Y, "H": H, "sumsq": sumsq}
    if keep:
        out.update(xhat=xhat, rho=rho, S=np.concatenate(S_parts, axis=1))
    return out


def lrblock_backward(x, g, A_cat, B, dY, act="silu", norm=True, eps=1e-5, d_norm=None):
    """Backward of :func:`lrblock_forward` from a forward whose every
    intermediate is kept (x_hat, rho, H, S).

    Returns dx[T,d], dg[d] (None when norm is False), dA_cat[d,G*r],
    dB[G,r,d_out].
    """
    x = np.asarray(x, np.float64)
    A_cat = np.asarray(A_cat, np.float64)
    B = np.asarray(B, np.float64)
    dY = np.asarray(dY, np.float64)
    G, r, _ = B.shape
    d = x.shape[1]
    if d_norm is None:
        d_norm = d
    f = lrblock_forward(x, g, A_cat, B, act, norm, eps, d_norm, keep=True)
    xhat, rho, H, S = f["xhat"], f["rho"], f["H"], f["S"]
    dB = np.stack([S[:, _group_cols(r, j)].T @ dY[j] for j in range(G)])
    dA_cat = np.zeros_like(A_cat)
    dxhat = np.zeros_like(x)
    for j in range(G):
        cols = _group_cols(r, j)
        dS_j = dY[j] @ B[j].T
        dH_j = dS_j * act_grad(H[:, cols], act)
        dA_cat[:, cols] = xhat.T @ dH_j
        dxhat += dH_j @ A_cat[:, cols].T
    if not norm:
        return {"dx": dxhat, "dg": None, "dA_cat": dA_cat, "dB": dB}
    g = np.asarray(g, np.float64)
    # x_hat = rho * x * g, rho = (sum x^2 / d_norm + eps)^(-1/2)
    dg = np.sum(rho[:, None] * x * dxhat, axis=0)
    w = np.sum(x * g[None, :] * dxhat, axis=1)  # sum_i x_ti g_i dxhat_ti
    dx = rho[:, None] * (g[None, :] * dxhat) - (rho ** 3 / d_norm)[:, None] * x * w[:, None]
    return {"dx": dx, "dg": dg, "dA_cat": dA_cat, "dB": dB}


# ---------------------------------------------------------------------------
# Low-rank SwiGLU MLP
# ---------------------------------------------------------------------------

def lrmlp_forward(x, g, A1_cat, B1, A2, B2, act="silu", eps=1e-5, d_norm=None, keep=False):
    """Forward of the low-rank SwiGLU MLP.

    H1 = RMSNorm(x) @ A1_cat [T,2r]; S1 = act(H1);
    Yg = S1[:, :r] @ B1[0]; Yu = S1[:, r:] @ B1[1]  (each [T,ffn]);
    M = SiLU(Yg) * Yu; H2 = M @ A2 [T,r]; S2 = act(H2); Y = S2 @ B2 [T,d].
    SwiGLU uses SiLU whatever the bottleneck activation is.
    """
    x = np.asarray(x, np.float64)
    A1_cat = np.asarray(A1_cat, np.float64)
    B1 = np.asarray(B1, np.float64)
    A2 = np.asarray(A2, np.float64)
    B2 = np.asarray(B2, np.float64)
    r = B1.shape[1]
    if d_norm is None:
        d_norm = x.shape[1]
    xhat, rho, sumsq = rmsnorm(x, g, eps, d_norm)
    H1g = xhat @ A1_cat[:, :r]
    H1u = xhat @ A1_cat[:, r:]
    Yg = act_fn(H1g, act) @ B1[0]
    Yu = act_fn(H1u, act) @ B1[1]
    M = silu(Yg) * Yu
    H2 = M @ A2
    S2 = act_fn(H2, act)
    Y = S2 @ B2
    out = {"Y": Y, "H1": np.concatenate([H1g, H1u], axis=1), "H2": H2, "sumsq": sumsq}
    if keep:
        out.update(xhat=xhat, rho=rho, Yg=Yg, Yu=Yu, M=M, S2=S2,
                   S1=np.concatenate([act_fn(H1g, act), act_fn(H1u, act)], axis=1))
    return out


def lrmlp_backward(x, g, A1_cat, B1, A2, B2, dY, act="silu", eps=1e-5, d_norm=None):
    """Backward of :func:`lrmlp_forward` from fully kept intermediates.

    Returns dx, dg, dA1_cat, dB1, dA2, dB2.
    """
    x = np.asarray(x, np.float64)
    A2 = np.asarray(A2, np.float64)
    B2 = np.asarray(B2, np.float64)
    dY = np.asarray(dY, np.float64)
    if d_norm is None:
        d_norm = x.shape[1]
    f = lrmlp_forward(x, g, A1_cat, B1, A2, B2, act, eps, d_norm, keep=True)
    dB2 = f["S2"].T @ dY
    dH2 = (dY @ B2.T) * act_grad(f["H2"], act)
    dA2 = f["M"].T @ dH2
    dM = dH2 @ A2.T
    Yg, Yu = f["Yg"], f["Yu"]
    dYg = dM * Yu * silu_grad(Yg)
    dYu = dM * silu(Yg)
    b1 = lrblock_backward(x, g, A1_cat, B1, np.stack([dYg, dYu]), act, True, eps, d_norm)
    return {"dx": b1["dx"], "dg": b1["dg"], "dA1_cat": b1["dA_cat"], "dB1": b1["dB"],
            "dA2": dA2, "dB2": dB2}


# ---------------------------------------------------------------------------
# One tensor-parallel share of a bottleneck pair (BTP)
# ---------------------------------------------------------------------------

def btp_share_forward(z, B_s, g_s, A_s, keep=False):
    """One share: u = z @ B_s (column slice of the up projection);
    a = SiLU(u) (op on the sharded activation); s = rowsum(a^2) (local
    RMSNorm statistic, a partial sum over this share's columns);
    p = (a * g_s) @ A_s (row slice of the next down projection, a partial
    sum over shares). No cross-share sum and no 1/rms scale here.
    """
    z = np.asarray(z, np.float64)
    u = z @ np.asarray(B_s, np.float64)
    a = silu(u)
    s = np.sum(a * a, axis=1)
    p = (a * np.asarray(g_s, np.float64)[None, :]) @ np.asarray(A_s, np.float64)
    out = {"p": p, "s": s}
    if keep:
        out.update(u=u, a=a)
    return out


def btp_share_backward(z, B_s, g_s, A_s, dp, ds):
    """Backward of one share given the gradients of its own outputs,
    dp[T,r] and ds[T]. Returns dz (this share's partial), dB_s, dg_s, dA_s.
    """
    B_s = np.asarray(B_s, np.float64)
    A_s = np.asarray(A_s, np.float64)
    g_s = np.asarray(g_s, np.float64)
    dp = np.asarray(dp, np.float64)
    ds = np.asarray(ds, np.float64)
    f = btp_share_forward(z, B_s, g_s, A_s, keep=True)
    u, a = f["u"], f["a"]
    e = dp @ A_s.T                       # gradient w.r.t. (a * g_s)
    dA_s = (a * g_s[None, :]).T @ dp
    dg_s = np.sum(a * e, axis=0)
    da = g_s[None, :] * e + 2.0 * ds[:, None] * a
    du = da * silu_grad(u)
    dB_s = np.asarray(z, np.float64).T @ du
    dz = du @ B_s.T
    return {"dz": dz, "dB_s": dB_s, "dg_s": dg_s, "dA_s": dA_s}


def btp_consumer(p_parts, s_parts, eps, d_norm):
    """What follows the shares once the one exchange has summed them:
    z_next = rho * sum_p p_p with rho = (sum_p s_p / d_norm + eps)^(-1/2)."""
    P = np.sum(np.stack(p_parts), axis=0)
    S = np.sum(np.stack(s_parts), axis=0)
    rho = 1.0 / np.sqrt(S / d_norm + eps)
    return rho[:, None] * P, rho, P


def btp_consumer_backward(dz_next, rho, Psum, d_norm):
    """Gradients of every share's own outputs from the consumer's output
    gradient dz_next (BOOST summary, technical summary 2.1 and 2.2: each rank
    forms them locally, with no exchange). From z_next = rho * Psum and
    rho = (S / d_norm + eps)^(-1/2) with S = sum_p s_p:
      dp = rho * dz_next                            (the same for every share)
      ds = d rho / d S * <dz_next, Psum>_row = -(rho^3 / (2 d_norm)) <dz_next, Psum>_row
    """
    dz_next = np.asarray(dz_next, np.float64)
    dp = rho[:, None] * dz_next
    ds = -(rho ** 3) / (2.0 * d_norm) * np.sum(dz_next * Psum, axis=1)
    return dp, ds
