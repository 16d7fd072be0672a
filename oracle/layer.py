"""Plain fp64 CPU oracle of a chained decoder layer built from low-rank
bottleneck blocks.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. It shares no
code with the GPU path and never imports it.

The BOOST summary pages (gist.science, paper 2512.12131, technical summary
§2.2 "Online-RMSNorm") describe the normalisation of a block's input as
local statistics that the producer of that input can emit; §4 names
LLaMA-2-shaped models, i.e. pre-norm decoder layers whose attention and MLP
sub-layers add into a residual stream. The pages define no layer code, so
this module takes the plainest reading (all of it written down in the design
notes):

* a layer is  h2 = x + O(attn(QKV(x))),  h3 = h2 + MLP(h2)  with QKV the
  grouped block (G = 3, RMSNorm on x), O the ungrouped block without a norm,
  MLP the low-rank SwiGLU MLP (RMSNorm on h2);
* the attention core is outside the method; a parameter-free stand-in takes
  its place: attn(q, k, v) = q + k + v (elementwise), so every projection
  receives a gradient;
* the statistic the next block's Online-RMSNorm needs is the row sum of
  squares of its input, computed here from the stored residual stream;
* every tensor the layer stores between blocks (q, k, v, the stand-in
  output, h2, h3 and, in the backward, the gradients handed from block to
  block) is held in the activation dtype. ``store`` is the rounding applied
  at those points (None = exact fp64, used by the pins); this is the same
  convention as a single block, whose input x is always given in the dtype.

Every function is pinned by the CPU tests (finite differences of the whole
layer, zeroed-branch closed forms, and the bilinear identity of the last up
projection).
"""
from __future__ import annotations

import numpy as np

from .lrblock import lrblock_backward, lrblock_forward, lrmlp_backward, lrmlp_forward


def round_to_bf16(a):
    """Store fp64 values as bfloat16 the way a device stores an fp32 result:
    round to float32, then to the nearest bfloat16 with ties to even (on the
    float32 bit pattern: add 0x7FFF plus the lowest kept bit, truncate the
    low 16 bits). Returned as fp64. Finite inputs only."""
    f = np.asarray(a, dtype=np.float64).astype(np.float32)
    bits = f.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + lsb) >> 16) << 16
    return rounded.astype(np.uint32).view(np.float32).astype(np.float64)


def standin_forward(qkv):
    """Attention stand-in: a = q + k + v for qkv[3,T,d]."""
    qkv = np.asarray(qkv, np.float64)
    return qkv[0] + qkv[1] + qkv[2]


def standin_backward(da):
    """Gradient of the stand-in: each of q, k, v receives da."""
    da = np.asarray(da, np.float64)
    return np.stack([da, da, da])


def _identity(t):
    return t


def layer_forward(x, qkv, o, mlp, act="silu", eps=1e-5, store=None, keep=False):
    """Forward of one chained layer.

    x[T,d]; qkv = dict(g, A_cat[d,3r], B[3,r,d]); o = dict(A_cat[d,r],
    B[1,r,d]); mlp = dict(g, A1_cat[d,2r], B1[2,r,ffn], A2[ffn,r], B2[r,d]).
    Returns h3[T,d], the next layer's statistic sumsq_h3[T] = sum_i h3_ti^2,
    the MLP's input statistic sumsq_h2[T], and the blocks' saved bottlenecks.
    """
    rnd = store or _identity
    x = np.asarray(x, np.float64)
    fq = lrblock_forward(x, qkv["g"], qkv["A_cat"], qkv["B"], act, True, eps)
    qkv_out = rnd(fq["Y"])
    a = rnd(standin_forward(qkv_out))
    fo = lrblock_forward(a, None, o["A_cat"], o["B"], act, False)
    h2 = rnd(x + fo["Y"][0])
    fm = lrmlp_forward(h2, mlp["g"], mlp["A1_cat"], mlp["B1"], mlp["A2"], mlp["B2"], act, eps)
    h3 = rnd(h2 + fm["Y"])
    out = {"h3": h3, "sumsq_h3": np.sum(h3 * h3, axis=1), "h2": h2, "sumsq_h2": np.sum(h2 * h2, axis=1),
           "sumsq_x": fq["sumsq"], "H_qkv": fq["H"], "H_o": fo["H"], "H1": fm["H1"], "H2": fm["H2"]}
    if keep:
        out.update(qkv=qkv_out, a=a)
    return out


def layer_backward(x, qkv, o, mlp, dh3, act="silu", eps=1e-5, store=None):
    """Backward of :func:`layer_forward` for the output gradient dh3[T,d].

    Returns dx (= dh1) and every weight/gain gradient, from block backwards
    that keep all their intermediates (the plain definition).
    """
    rnd = store or _identity
    f = layer_forward(x, qkv, o, mlp, act, eps, store, keep=True)
    dh3 = np.asarray(dh3, np.float64)
    bm = lrmlp_backward(f["h2"], mlp["g"], mlp["A1_cat"], mlp["B1"], mlp["A2"], mlp["B2"], dh3, act, eps)
    dh2 = rnd(dh3 + bm["dx"])
    bo = lrblock_backward(f["a"], None, o["A_cat"], o["B"], dh2[None], act, False)
    da = rnd(bo["dx"])
    dqkv = rnd(standin_backward(da))
    bq = lrblock_backward(x, qkv["g"], qkv["A_cat"], qkv["B"], dqkv, act, True, eps)
    dx = dh2 + bq["dx"]
    return {"dx": dx, "dg_qkv": bq["dg"], "dA_qkv": bq["dA_cat"], "dB_qkv": bq["dB"],
            "dA_o": bo["dA_cat"], "dB_o": bo["dB"],
            "dg_mlp": bm["dg"], "dA1_mlp": bm["dA1_cat"], "dB1_mlp": bm["dB1"],
            "dA2_mlp": bm["dA2"], "dB2_mlp": bm["dB2"], "dh2": dh2, "da": da}
