"""Parity over seeded random shapes, through the C ABI, against the oracle.

The shapes are drawn once from a fixed seed: ragged token counts (1 to
8192), widths and ranks that are multiples of 64, one to three groups, both
bottleneck activations, with and without the statistic; a class of large
T x d_out up products at small K = r that run on the panel-ring tiles for
one to five K steps; the SwiGLU MLP; and one share of a two- or four-way
tensor-parallel pair. Every output and gradient is checked at the standard
tolerance.
"""
import random

import pytest

from rank_bottleneck_online_amd import synth

from gpu_util import say
from test_gpu_parity import B, compare_btp, compare_lrblock, compare_lrmlp, run_btp, run_lrblock, run_lrmlp  # noqa: F401

pytestmark = pytest.mark.gpu


def _cases():
    rng = random.Random(2026)

    def m64(lo, hi):
        return 64 * rng.randint(lo // 64, hi // 64)

    out = []
    for _ in range(8):
        T = rng.choice([1, 7, 63, 65, 300, 511, 1000, 2049, 4097])
        out.append(("lrblock", (T, m64(64, 1024), m64(64, 512), rng.randint(1, 3), m64(64, 1024),
                                rng.choice(["silu", "identity"]), rng.random() < 0.8)))
    for _ in range(6):
        T = rng.choice([4090, 4096, 8190, 8192])
        out.append(("lrblock", (T, m64(64, 256), m64(64, 320), rng.randint(1, 3), rng.choice([1024, 2048, 2112]),
                                "silu", True)))
    for _ in range(5):
        T = rng.choice([1, 100, 513, 1500, 3000])
        out.append(("lrmlp", (T, m64(64, 768), m64(64, 256), m64(64, 2048), rng.choice(["silu", "identity"]))))
    for _ in range(4):
        P = rng.choice([2, 4])
        out.append(("btp", (rng.choice([1, 300, 2000, 8192]), m64(64, 1280), 64 * P * rng.randint(1, 8), P)))
    return out


CASES = _cases()


@pytest.mark.parametrize("i", range(len(CASES)), ids=lambda i: f"{CASES[i][0]}-{'x'.join(map(str, CASES[i][1]))}")
def test_random_shape(B, i):  # noqa: F811
    kind, c = CASES[i]
    seed = 200 + i
    say(f"sweep {kind} {c} bf16 seed={seed}")
    if kind == "lrblock":
        T, d, r, G, n, act, norm = c
        inp = synth.lrblock_inputs(T, d, r, G, n, dtype="bf16", seed=seed, norm=norm)
        compare_lrblock(run_lrblock(B, inp, "bf16", act, norm), inp, "bf16", act, norm)
    elif kind == "lrmlp":
        T, d, r, ffn, act = c
        inp = synth.lrmlp_inputs(T, d, r, ffn, dtype="bf16", seed=seed)
        compare_lrmlp(run_lrmlp(B, inp, "bf16", act), inp, "bf16", act)
    else:
        T, r, D, P = c
        inp = synth.btp_inputs(T, r, D, P, dtype="bf16", seed=seed)
        sh = synth.btp_shard(inp, 0, P)
        compare_btp(run_btp(B, sh, "bf16"), sh, "bf16")
