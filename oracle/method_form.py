"""The method's own (deferred, grouped, checkpointed) form, in fp64.

TEST INFRASTRUCTURE, like the rest of this package: only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may use
it. It is not used for parity; the CPU tests check it against the plain
definitions in :mod:`oracle.lrblock`, which pins the algebra the GPU path
relies on.

Follows the BOOST summary pages, technical summary §2.2:

* Online-RMSNorm: keep the per-row sum of squares as the local statistic and
  apply 1/rms later, as a row scale of the down product,
  H = rho * ((x * g) @ A_cat), which equals the plain form because a
  diagonal row scale commutes with right multiplication;
* linear-layer grouping: one product with the concatenated down weights;
* low-rank activation checkpointing: the backward sees only the inputs, the
  bottleneck H and the statistic sumsq, and recomputes act(H), act'(H) and
  rho from them.
"""
from __future__ import annotations

import numpy as np

from .lrblock import act_fn, act_grad


def lrblock_forward_deferred(x, g, A_cat, B, act="silu", eps=1e-5, d_norm=None):
    x = np.asarray(x, np.float64)
    g = np.asarray(g, np.float64)
    B = np.asarray(B, np.float64)
    G, r, _ = B.shape
    if d_norm is None:
        d_norm = x.shape[1]
    sumsq = np.sum(x * x, axis=1)
    U = (x * g[None, :]) @ np.asarray(A_cat, np.float64)      # one grouped product
    rho = 1.0 / np.sqrt(sumsq / d_norm + eps)
    H = rho[:, None] * U                                       # deferred row scale
    S = act_fn(H, act)
    Y = np.einsum("tgk,gkn->gtn", S.reshape(len(x), G, r), B)  # batched up product
    return {"Y": Y, "H": H, "sumsq": sumsq}


def lrblock_backward_checkpointed(x, g, A_cat, B, H, sumsq, dY, act="silu", eps=1e-5,
                                  d_norm=None):
    """Backward from (x, g, A_cat, B, H, sumsq, dY) only."""
    x = np.asarray(x, np.float64)
    g = np.asarray(g, np.float64)
    A_cat = np.asarray(A_cat, np.float64)
    B = np.asarray(B, np.float64)
    H = np.asarray(H, np.float64)
    dY = np.asarray(dY, np.float64)
    G, r, _ = B.shape
    T, d = x.shape
    if d_norm is None:
        d_norm = d
    rho = 1.0 / np.sqrt(np.asarray(sumsq, np.float64) / d_norm + eps)
    S = act_fn(H, act).reshape(T, G, r)
    dB = np.einsum("tgk,gtn->gkn", S, dY)
    dS = np.einsum("gtn,gkn->tgk", dY, B).reshape(T, G * r)
    dH = dS * act_grad(H, act)
    dU = rho[:, None] * dH
    drho = np.sum(dH * H, axis=1) / rho
    dA_cat = (x * g[None, :]).T @ dU
    dxt = dU @ A_cat.T
    dx = g[None, :] * dxt - ((rho ** 3) * drho / d_norm)[:, None] * x
    dg = np.sum(x * dxt, axis=0)
    return {"dx": dx, "dg": dg, "dA_cat": dA_cat, "dB": dB}
