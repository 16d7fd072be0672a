"""The entry points under HIP graph capture.

The library allocates no device memory and issues no memsets; its side
stream is forked from and joined back into the caller's stream with events,
so a whole forward + backward can be captured into one graph and replayed.
Each replay here follows eager work of the program's own (the outputs are
overwritten with NaN, then synchronised) and must reproduce the eager
result bit for bit (the kernels are deterministic).
"""
import pytest
import torch

from rank_bottleneck_online_amd import synth

from gpu_util import dev, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    from rank_bottleneck_online_amd import binding
    binding.lib()
    return binding


def _replay_and_check(step, outs, replays=3):
    """step() enqueues the work writing into `outs` (a list of tensors)."""
    step()  # eager reference (also creates the library's side stream)
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(replays):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, r) in enumerate(zip(outs, ref)):
            bits = torch.int16 if o.dtype == torch.bfloat16 else torch.int32
            same = torch.equal(o.view(bits), r.view(bits))
            assert same, f"replay {rep}: output {i} differs from the eager run"
        say(f"    replay {rep}: {len(outs)} outputs bit-identical to the eager run")


def test_lrmlp_step_graph_replay(B):
    T, d, r, ffn = 513, 512, 128, 1408
    say(f"graph capture: lrmlp fwd+bwd T={T} d={d} r={r} ffn={ffn} bf16 silu seed=0")
    inp = synth.lrmlp_inputs(T, d, r, ffn, dtype="bf16", seed=0)
    t = {k: dev(inp[k], "bf16") for k in ("x", "g", "A1_cat", "B1", "A2", "B2", "dY")}
    fdesc = B.lrmlp_desc(T, d, r, ffn, B._dtype_code(t["x"]))
    wf = torch.empty(max(B.lrmlp_workspace_size(fdesc, False), 1), dtype=torch.uint8, device="cuda")
    wb = torch.empty(max(B.lrmlp_workspace_size(fdesc, True), 1), dtype=torch.uint8, device="cuda")
    f32 = dict(dtype=torch.float32, device="cuda")
    fo = (torch.empty(T, d, dtype=torch.bfloat16, device="cuda"), torch.empty(T, 2 * r, **f32),
          torch.empty(T, r, **f32), torch.empty(T, **f32))
    bo = (torch.empty(T, d, dtype=torch.bfloat16, device="cuda"), torch.empty(d, **f32),
          torch.empty(d, 2 * r, **f32), torch.empty(2, r, ffn, **f32), torch.empty(ffn, r, **f32),
          torch.empty(r, d, **f32))

    def step():
        Y, H1, H2, sumsq = B.lrmlp_fwd(t["x"], t["g"], t["A1_cat"], t["B1"], t["A2"], t["B2"], out=fo, ws=wf)
        B.lrmlp_bwd(t["x"], t["g"], t["A1_cat"], t["B1"], t["A2"], t["B2"], H1, H2, sumsq, t["dY"], out=bo,
                    ws=wb)

    _replay_and_check(step, list(fo) + list(bo))


def test_lrblock_step_graph_replay(B):
    T, d, r, G, n = 640, 1024, 256, 2, 1024
    say(f"graph capture: lrblock fwd+bwd T={T} d={d} r={r} G={G} d_out={n} bf16 silu seed=0")
    inp = synth.lrblock_inputs(T, d, r, G, n, dtype="bf16", seed=0)
    x, g, A, Bw, dY = (dev(inp[k], "bf16") for k in ("x", "g", "A_cat", "B", "dY"))
    desc = B.lrblock_desc(T, d, r, G, n, B._dtype_code(x))
    wf = torch.empty(max(B.lrblock_workspace_size(desc, False), 1), dtype=torch.uint8, device="cuda")
    wb = torch.empty(max(B.lrblock_workspace_size(desc, True), 1), dtype=torch.uint8, device="cuda")
    f32 = dict(dtype=torch.float32, device="cuda")
    fo = (torch.empty(G, T, n, dtype=torch.bfloat16, device="cuda"), torch.empty(T, G * r, **f32),
          torch.empty(T, **f32))
    bo = (torch.empty(T, d, dtype=torch.bfloat16, device="cuda"), torch.empty(d, **f32),
          torch.empty(d, G * r, **f32), torch.empty(G, r, n, **f32))

    def step():
        Y, H, sumsq = B.lrblock_fwd(x, g, A, Bw, out=fo, ws=wf)
        B.lrblock_bwd(x, g, A, Bw, H, sumsq, dY, out=bo, ws=wb)

    _replay_and_check(step, list(fo) + list(bo))
