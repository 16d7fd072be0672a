"""Seeded synthetic inputs for the low-rank bottleneck block.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark. It holds no arithmetic of the method itself: it only draws
Gaussian tensors in a fixed order from a seeded PCG64 generator and rounds
them to the storage dtype, so that both sides of a parity check receive
bit-identical values.

Workload recipe (the pages measure LLaMA-2-family low-rank models trained on
a corpus that is not available here; seeded Gaussian tensors of the same
shapes stand in for it):

* activations and upstream gradients ~ N(0, 1);
* every weight ~ N(0, 1/fan_in) (the second argument is a variance), where
  fan_in is the layer's input width;
* RMSNorm gains g = 1 + N(0, 0.1);
* draws are fp64, in the order the tensors are listed by each function, from
  ``numpy.random.default_rng(seed)``; every value is then rounded to the
  storage dtype with round-to-nearest-even.

The rounded values are returned as fp64 arrays (exactly representable in the
storage dtype) together with the raw storage bits for upload.
"""
from __future__ import annotations

import numpy as np

DTYPES = ("bf16", "f32")


def round_to_bf16(v: np.ndarray) -> np.ndarray:
    """Round fp64 values to the nearest bfloat16 value (ties to even).

    bfloat16 keeps 8 significant bits. ``frexp`` writes v = m * 2**e with
    0.5 <= |m| < 1; scaling m by 2**8 and rounding half-to-even with ``rint``
    keeps 8 significant bits exactly in fp64 arithmetic (no double rounding).
    Finite, normal-range inputs only (Gaussian draws never leave that range).
    """
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)


def round_to_f32(v: np.ndarray) -> np.ndarray:
    """Round fp64 values to fp32 (ties to even), returned as fp64."""
    return np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)


def quantize(v: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_to_bf16(v)
    if dtype == "f32":
        return round_to_f32(v)
    raise ValueError(f"unknown dtype {dtype!r}")


def storage_bits(v: np.ndarray, dtype: str) -> np.ndarray:
    """Raw storage representation of already-quantized values.

    bf16 -> uint16 bit patterns (the upper half of the fp32 pattern, exact
    because the value is bf16-representable); f32 -> float32.
    """
    v = np.ascontiguousarray(v, dtype=np.float64)
    f = v.astype(np.float32)
    if dtype == "f32":
        return f
    if dtype == "bf16":
        bits = f.view(np.uint32)
        if np.any(bits & 0xFFFF):
            raise ValueError("value is not bf16-representable; quantize first")
        return (bits >> 16).astype(np.uint16)
    raise ValueError(f"unknown dtype {dtype!r}")


def from_bits(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Inverse of :func:`storage_bits` (device results back to fp64)."""
    if dtype == "f32":
        return np.asarray(bits, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
        return b.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


class _Draw:
    def __init__(self, seed: int, dtype: str):
        self.rng = np.random.default_rng(seed)
        self.dtype = dtype

    def normal(self, shape, var: float = 1.0, mean: float = 0.0) -> np.ndarray:
        z = self.rng.standard_normal(size=shape)
        return quantize(mean + np.sqrt(var) * z, self.dtype)


def lrblock_inputs(T, d, r, G, d_out, dtype="bf16", seed=0, norm=True, draw=None):
    """Inputs of one grouped low-rank block (QKV-style, or O-proj when
    ``norm`` is False: no gain is drawn then).

    Draw order: x[T,d], A_cat[d,G*r], B[G,r,d_out], g[d] (norm only),
    dY[G,T,d_out].
    """
    dr = draw or _Draw(seed, dtype)
    out = {}
    out["x"] = dr.normal((T, d))
    out["A_cat"] = dr.normal((d, G * r), 1.0 / d)
    out["B"] = dr.normal((G, r, d_out), 1.0 / r)
    if norm:
        out["g"] = dr.normal((d,), 0.1, mean=1.0)
    out["dY"] = dr.normal((G, T, d_out))
    return out


def lrmlp_inputs(T, d, r, ffn, dtype="bf16", seed=0, draw=None):
    """Inputs of the low-rank SwiGLU MLP.

    Draw order: x[T,d], A1_cat[d,2r], B1[2,r,ffn], A2[ffn,r], B2[r,d], g[d],
    dY[T,d].
    """
    dr = draw or _Draw(seed, dtype)
    out = {}
    out["x"] = dr.normal((T, d))
    out["A1_cat"] = dr.normal((d, 2 * r), 1.0 / d)
    out["B1"] = dr.normal((2, r, ffn), 1.0 / r)
    out["A2"] = dr.normal((ffn, r), 1.0 / ffn)
    out["B2"] = dr.normal((r, d), 1.0 / r)
    out["g"] = dr.normal((d,), 0.1, mean=1.0)
    out["dY"] = dr.normal((T, d))
    return out


def btp_inputs(T, r, d_global, P, dtype="bf16", seed=0, draw=None):
    """Inputs of one tensor-parallel share of a bottleneck pair.

    Full (unsharded) weights are drawn so that every shard is a slice of one
    consistent layer. Draw order: z[T,r], B_full[r,d_global],
    A_full[d_global,r], g_full[d_global], dz_next[T,r], then the upstream
    gradients of one share's own outputs, dp[T,r] ~ N(0,1) and
    ds[T] ~ N(0,1e-4).
    """
    if d_global % P:
        raise ValueError("d_global must divide by P")
    dr = draw or _Draw(seed, dtype)
    out = {}
    out["z"] = dr.normal((T, r))
    out["B_full"] = dr.normal((r, d_global), 1.0 / r)
    out["A_full"] = dr.normal((d_global, r), 1.0 / d_global)
    out["g_full"] = dr.normal((d_global,), 0.1, mean=1.0)
    out["dz_next"] = dr.normal((T, r))
    out["dp"] = dr.normal((T, r))
    # ds is a per-row fp32 statistic gradient: drawn in fp32 whatever dtype is.
    out["ds"] = round_to_f32(np.sqrt(1e-4) * dr.rng.standard_normal(size=(T,)))
    return out


def btp_shard(inp, p, P):
    """Slice shard ``p`` of ``P`` out of :func:`btp_inputs` (pure indexing)."""
    dg = inp["B_full"].shape[1] // P
    sl = slice(p * dg, (p + 1) * dg)
    return {
        "z": inp["z"],
        "B_s": np.ascontiguousarray(inp["B_full"][:, sl]),
        "g_s": np.ascontiguousarray(inp["g_full"][sl]),
        "A_s": np.ascontiguousarray(inp["A_full"][sl, :]),
        "dp": inp["dp"],
        "ds": inp["ds"],
    }


def layerset_inputs(T, d, r, ffn, dtype="bf16", seed=0):
    """Inputs of the decoder-layer bottleneck set: a QKV block (G=3, with
    Online-RMSNorm), an O-projection block (G=1, no norm) and the SwiGLU MLP,
    drawn from one generator in that order."""
    dr = _Draw(seed, dtype)
    return {
        "qkv": lrblock_inputs(T, d, r, 3, d, norm=True, draw=dr),
        "o": lrblock_inputs(T, d, r, 1, d, norm=False, draw=dr),
        "mlp": lrmlp_inputs(T, d, r, ffn, draw=dr),
    }


def layer_inputs(T, d, r, ffn, dtype="bf16", seed=0):
    """Inputs of one chained decoder layer: the layer-set draws (same order),
    of which the layer uses the QKV block's x as its input x, the MLP's dY as
    the output gradient dh3, and every block's weights and gains."""
    s = layerset_inputs(T, d, r, ffn, dtype, seed)
    q, o, m = s["qkv"], s["o"], s["mlp"]
    return {
        "x": q["x"],
        "qkv": {"g": q["g"], "A_cat": q["A_cat"], "B": q["B"]},
        "o": {"A_cat": o["A_cat"], "B": o["B"]},
        "mlp": {k: m[k] for k in ("g", "A1_cat", "B1", "A2", "B2")},
        "dh3": m["dY"],
    }


# Named workloads (LLaMA-2-family shapes). T = batch * sequence length.
WORKLOADS = {
    "tiny_qkv_f32": dict(kind="lrblock", T=64, d=256, r=64, G=3, d_out=256, dtype="f32"),
    "llama2_1b_qkv_fwd": dict(kind="lrblock", T=16384, d=2048, r=512, G=3, d_out=2048, dtype="bf16"),
    "llama2_7b_mlp": dict(kind="lrmlp", T=8192, d=4096, r=1024, ffn=11008, dtype="bf16"),
    "llama2_13b_btp_share_tp4": dict(kind="btp", T=8192, r=1280, d_global=5120, P=4, dtype="bf16"),
    "llama2_40b_layerset": dict(kind="layerset", T=4096, d=8192, r=2048, ffn=22016, dtype="bf16"),
    "llama2_40b_layer_chained": dict(kind="layer", T=4096, d=8192, r=2048, ffn=22016, dtype="bf16"),
}
