#!/usr/bin/env python3
"""Throughput of the low-rank bottleneck block on one MI355X.

A step is one forward + backward pass of the whole block (every product,
the fused Online-RMSNorm statistics and scale, SiLU/SwiGLU and their
recompute) over one batch of seeded synthetic input resident in HBM. The
default workload is the LLaMA-2-7B-shaped low-rank SwiGLU MLP (T = 8192
tokens, d = 4096, r = 1024, ffn = 11008, bf16 with fp32 accumulation).

Prints one JSON line on stdout. Besides the contract fields it carries:
  roofline      the dominant kernel's algorithmic TFLOP/s (per-launch flops /
                average launch time from HIP events recorded around that
                kernel on its launch stream during the timed steps), against
                the bf16 dense MFMA peak, and its HBM traffic from committed
                rocprofv3 counters when they match the current sources;
  cpu_baseline  the fp64 CPU oracle timed on a bounded sample of the same
                workload on this host (a baseline, not a target).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from rank_bottleneck_online_amd import synth  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3        # MI355X dense fp32 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
METRIC = "low-rank block fwd+bwd TFLOP/s (% bf16 MFMA peak) + tokens/s, 7B shape"
def traffic_json_path(workload: str) -> str:
    """Counter-measured traffic of a workload's launches (written by --traffic)."""
    return os.path.join(ROOT, "profiles", f"{workload}_traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def code_text(src: str) -> str:
    """C/C++ source without its comments and with whitespace runs collapsed:
    what the compiler sees, so that edits to comments leave the digest of
    the kernels unchanged."""
    import re
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def source_digest() -> str:
    """Digest of the code of the library's sources and header (comments and
    layout excluded), recorded with counter measurements so that they are
    reported only while the kernels are unchanged."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "rank_bottleneck_online_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        h.update(f.encode())
        h.update(code_text(open(os.path.join(csrc, f)).read()).encode())
    h.update(code_text(open(os.path.join(ROOT, "include", "boost_lrblock.h")).read()).encode())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------------------
# Algorithmic flops (the method's own products, with its prescribed recompute)
# ---------------------------------------------------------------------------

def mlp_kernel_flops(T, d, r, ffn):
    return {
        "mlp_down1": 2 * T * d * 2 * r,
        "mlp_up1_swiglu": 2 * 2 * T * r * ffn,
        "mlp_down2": 2 * T * ffn * r,
        "mlp_up2": 2 * T * r * d,
        "mlp_ds2": 2 * T * d * r,
        "mlp_dB2": 2 * r * d * T,
        "mlp_recompute_swiglu_bwd": 3 * 2 * T * r * ffn,  # gate and up recompute + dM, one launch
        "mlp_dA2": 2 * ffn * r * T,
        "mlp1_ds": 2 * 2 * T * ffn * r,
        "mlp1_dB": 2 * 2 * r * ffn * T,
        "mlp1_dA": 2 * d * 2 * r * T,
        "mlp1_dx": 2 * T * 2 * r * d,
    }


def mlp_kernel_rw(T, d, r, ffn):
    """Algorithmic HBM bytes per launch of the MLP step's kernels as (read,
    written): each input read once, each output written once (bf16 2 B,
    fp32 4 B)."""
    b, f = 2, 4
    return {
        "mlp_down1": (T * d * b + d * 2 * r * b, T * 2 * r * (f + b) + T * f),
        "mlp_up1_swiglu": (T * 2 * r * b + 2 * r * ffn * b, T * ffn * b),
        "mlp_down2": (T * ffn * b + ffn * r * b, T * r * (f + b)),
        "mlp_up2": (T * r * b + r * d * b, T * d * b),
        "mlp_ds2": (T * d * b + r * d * b + T * r * f, 2 * T * r * b),
        "mlp_dB2": (T * r * b + T * d * b, r * d * f),
        "mlp_recompute_swiglu_bwd": (T * 2 * r * b + 2 * r * ffn * b + T * r * b + ffn * r * b, 3 * T * ffn * b),
        "mlp_dA2": (T * ffn * b + T * r * b, ffn * r * f),
        "mlp1_ds": (2 * T * ffn * b + 2 * r * ffn * b + T * 2 * r * f, T * 2 * r * b),
        "mlp1_dB": (T * 2 * r * b + 2 * T * ffn * b, 2 * r * ffn * f),
        "mlp1_dA": (T * d * b + T * 2 * r * b, d * 2 * r * f),
        "mlp1_dx": (T * 2 * r * b + d * 2 * r * b + T * d * b, T * d * b),
    }


def mlp_kernel_bytes(T, d, r, ffn):
    """Algorithmic HBM bytes per launch (read + written)."""
    return {k: rd + wr for k, (rd, wr) in mlp_kernel_rw(T, d, r, ffn).items()}


def lrblock_kernel_flops(T, d, r, G, n, bwd=True):
    f = {"lrblock_down": 2 * T * d * G * r, "lrblock_up": 2 * G * T * r * n}
    if bwd:
        f.update({"lrblock_ds": 2 * G * T * n * r, "lrblock_dB": 2 * G * r * n * T,
                  "lrblock_dA": 2 * d * G * r * T, "lrblock_dx": 2 * T * G * r * d})
    return f


def recompute_flops(kind, w) -> float:
    """Flops of the prescribed recompute in one step (the gate/up re-forward
    of each MLP, u of the BTP share)."""
    mlp = 2 * 2 * w["T"] * w["r"] * w.get("ffn", 0)
    if kind in ("lrmlp", "layerset", "layer"):
        return float(mlp)
    if kind == "btp":
        return float(2 * w["T"] * w["r"] * (w["d_global"] // w["P"]))
    return 0.0
# Weight-gradient launches of the block and MLP backward: the library runs
# them on its side stream concurrently with the input-gradient chain, so
# their event durations include sharing the GPU and they are not roofline
# candidates. (The tensor-parallel share runs all of its launches on the
# caller's stream.)
SIDE_STREAM_LABELS = ("mlp_dB2", "mlp_dA2", "mlp1_dB", "mlp1_dA", "lrblock_dB", "lrblock_dA", "splitk_reduce")


def btp_kernel_flops(T, r, ds):
    # btp_u_re: the recompute u = z @ B_s; btp_u_bwd: e = dp @ A_s^T with the
    # bottleneck backward in its epilogue.
    return {"btp_u": 2 * T * r * ds, "btp_p": 2 * T * ds * r, "btp_u_re": 2 * T * r * ds,
            "btp_u_bwd": 2 * T * r * ds, "btp_dA": 2 * ds * r * T, "btp_dB": 2 * r * ds * T,
            "btp_dz": 2 * T * ds * r}


# ---------------------------------------------------------------------------
# Workloads: inputs on the GPU, a step closure, flops, and an oracle sample
# ---------------------------------------------------------------------------

class Workload:
    def __init__(self, name):
        import torch
        from rank_bottleneck_online_amd import binding as B
        self.name = name
        self.w = w = synth.WORKLOADS[name]
        self.kind = w["kind"]
        self.dtype = w["dtype"]
        self.B = B
        self.torch = torch
        self.bwd = name != "llama2_1b_qkv_fwd"
        self.acts = ["silu"]
        if self.kind == "layerset":
            self.acts = ["silu", "identity"]
        self._setup()

    def dev(self, a):
        return self.B.upload(a, self.dtype)

    def _setup(self):
        B, torch, w = self.B, self.torch, self.w
        dt = B.DT_BF16 if self.dtype == "bf16" else B.DT_F32
        if self.kind == "lrmlp":
            T, d, r, ffn = w["T"], w["d"], w["r"], w["ffn"]
            inp = synth.lrmlp_inputs(T, d, r, ffn, dtype=self.dtype, seed=0)
            t = {k: self.dev(v) for k, v in inp.items()}
            desc = B.lrmlp_desc(T, d, r, ffn, dt)
            ws_f = torch.empty(B.lrmlp_workspace_size(desc, False), dtype=torch.uint8, device="cuda")
            ws_b = torch.empty(B.lrmlp_workspace_size(desc, True), dtype=torch.uint8, device="cuda")
            fo = B.lrmlp_fwd(t["x"], t["g"], t["A1_cat"], t["B1"], t["A2"], t["B2"], ws=ws_f)
            bo = B.lrmlp_bwd(t["x"], t["g"], t["A1_cat"], t["B1"], t["A2"], t["B2"], *fo[1:], t["dY"], ws=ws_b)
            args = [t[k] for k in ("x", "g", "A1_cat", "B1", "A2", "B2")]

            def fwd():
                B.lrmlp_fwd(*args, out=fo, ws=ws_f)

            def bwd():
                B.lrmlp_bwd(*args, *fo[1:], t["dY"], out=bo, ws=ws_b)

            self.fwd, self.bwd_fn = fwd, bwd
            self.tokens = T
            self.kflops = mlp_kernel_flops(T, d, r, ffn)
            self.kbytes = mlp_kernel_bytes(T, d, r, ffn)
            self.shape = dict(T=T, d=d, r=r, ffn=ffn)
        elif self.kind == "lrblock":
            T, d, r, G, n = w["T"], w["d"], w["r"], w["G"], w["d_out"]
            inp = synth.lrblock_inputs(T, d, r, G, n, dtype=self.dtype, seed=0)
            t = {k: self.dev(v) for k, v in inp.items()}
            desc = B.lrblock_desc(T, d, r, G, n, dt)
            ws_f = torch.empty(B.lrblock_workspace_size(desc, False), dtype=torch.uint8, device="cuda")
            ws_b = torch.empty(B.lrblock_workspace_size(desc, True), dtype=torch.uint8, device="cuda")
            fo = B.lrblock_fwd(t["x"], t["g"], t["A_cat"], t["B"], ws=ws_f)
            bo = B.lrblock_bwd(t["x"], t["g"], t["A_cat"], t["B"], fo[1], fo[2], t["dY"], ws=ws_b) \
                if self.bwd else None

            def fwd():
                B.lrblock_fwd(t["x"], t["g"], t["A_cat"], t["B"], out=fo, ws=ws_f)

            def bwd():
                B.lrblock_bwd(t["x"], t["g"], t["A_cat"], t["B"], fo[1], fo[2], t["dY"], out=bo, ws=ws_b)

            self.fwd, self.bwd_fn = fwd, (bwd if self.bwd else None)
            self.tokens = T
            self.kflops = lrblock_kernel_flops(T, d, r, G, n, self.bwd)
            if not self.bwd:
                self.kbytes = {k: rd + wr for k, (rd, wr) in lrblock_fwd_kernel_rw(T, d, r, G, n).items()}
            self.shape = dict(T=T, d=d, r=r, G=G, d_out=n)
        elif self.kind == "btp":
            T, r, D, P = w["T"], w["r"], w["d_global"], w["P"]
            inp = synth.btp_inputs(T, r, D, P, dtype=self.dtype, seed=0)
            sh = synth.btp_shard(inp, 0, P)
            t = {k: self.dev(sh[k]) for k in ("z", "B_s", "g_s", "A_s", "dp")}
            ds = self.B.upload(sh["ds"], "f32")
            desc = B.btp_desc(T, r, D // P, dt)
            ws_f = torch.empty(B.btp_workspace_size(desc, False), dtype=torch.uint8, device="cuda")
            ws_b = torch.empty(B.btp_workspace_size(desc, True), dtype=torch.uint8, device="cuda")
            args = [t[k] for k in ("z", "B_s", "g_s", "A_s")]
            fo = B.btp_share_fwd(*args, ws=ws_f)
            bo = B.btp_share_bwd(*args, t["dp"], ds, ws=ws_b)

            def fwd():
                B.btp_share_fwd(*args, out=fo, ws=ws_f)

            def bwd():
                B.btp_share_bwd(*args, t["dp"], ds, out=bo, ws=ws_b)

            self.fwd, self.bwd_fn = fwd, bwd
            self.tokens = T
            self.kflops = btp_kernel_flops(T, r, D // P)
            self.shape = dict(T=T, r=r, d_shard=D // P, d_global=D, tp=P)
        elif self.kind == "layerset":
            T, d, r, ffn = w["T"], w["d"], w["r"], w["ffn"]
            inp = synth.layerset_inputs(T, d, r, ffn, dtype=self.dtype, seed=0)
            q = {k: self.dev(v) for k, v in inp["qkv"].items()}
            o = {k: self.dev(v) for k, v in inp["o"].items()}
            m = {k: self.dev(v) for k, v in inp["mlp"].items()}
            dq = B.lrblock_desc(T, d, r, 3, d, dt)
            do = B.lrblock_desc(T, d, r, 1, d, dt, norm=False)
            dm = B.lrmlp_desc(T, d, r, ffn, dt)
            sizes = [B.lrblock_workspace_size(dq, 0), B.lrblock_workspace_size(dq, 1),
                     B.lrblock_workspace_size(do, 0), B.lrblock_workspace_size(do, 1),
                     B.lrmlp_workspace_size(dm, 0), B.lrmlp_workspace_size(dm, 1)]
            ws = torch.empty(max(sizes), dtype=torch.uint8, device="cuda")
            state = {}
            for act in self.acts:
                qf = B.lrblock_fwd(q["x"], q["g"], q["A_cat"], q["B"], act=act, ws=ws)
                qb = B.lrblock_bwd(q["x"], q["g"], q["A_cat"], q["B"], qf[1], qf[2], q["dY"], act=act, ws=ws)
                of = B.lrblock_fwd(o["x"], None, o["A_cat"], o["B"], act=act, norm=False, ws=ws)
                ob = B.lrblock_bwd(o["x"], None, o["A_cat"], o["B"], of[1], None, o["dY"], act=act, norm=False,
                                   ws=ws)
                ma = [m[k] for k in ("x", "g", "A1_cat", "B1", "A2", "B2")]
                mf = B.lrmlp_fwd(*ma, act=act, ws=ws)
                mb = B.lrmlp_bwd(*ma, *mf[1:], m["dY"], act=act, ws=ws)
                state[act] = (qf, qb, of, ob, mf, mb)
            self.act = self.acts[0]

            ma = [m[k] for k in ("x", "g", "A1_cat", "B1", "A2", "B2")]

            def fwd():
                act = self.act
                qf, qb, of, ob, mf, mb = state[act]
                B.lrblock_fwd(q["x"], q["g"], q["A_cat"], q["B"], act=act, out=qf, ws=ws)
                B.lrblock_fwd(o["x"], None, o["A_cat"], o["B"], act=act, norm=False, out=of, ws=ws)
                B.lrmlp_fwd(*ma, act=act, out=mf, ws=ws)

            def bwd():
                act = self.act
                qf, qb, of, ob, mf, mb = state[act]
                B.lrblock_bwd(q["x"], q["g"], q["A_cat"], q["B"], qf[1], qf[2], q["dY"], act=act, out=qb, ws=ws)
                B.lrblock_bwd(o["x"], None, o["A_cat"], o["B"], of[1], None, o["dY"], act=act, norm=False,
                              out=ob, ws=ws)
                B.lrmlp_bwd(*ma, *mf[1:], m["dY"], act=act, out=mb, ws=ws)

            self.fwd, self.bwd_fn = fwd, bwd
            self.tokens = T
            # QKV and O launches share the lrblock_* labels with different
            # per-launch flops, so only the MLP kernels get a roofline here.
            self.kflops = mlp_kernel_flops(T, d, r, ffn)
            self.shape = dict(T=T, d=d, r=r, ffn=ffn)
        elif self.kind == "layer":
            T, d, r, ffn = w["T"], w["d"], w["r"], w["ffn"]
            inp = synth.layer_inputs(T, d, r, ffn, dtype=self.dtype, seed=0)
            x, dh3 = self.dev(inp["x"]), self.dev(inp["dh3"])
            q = {k: self.dev(v) for k, v in inp["qkv"].items()}
            o = {k: self.dev(v) for k, v in inp["o"].items()}
            m = {k: self.dev(v) for k, v in inp["mlp"].items()}
            dq = B.lrblock_desc(T, d, r, 3, d, dt)
            do = B.lrblock_desc(T, d, r, 1, d, dt, norm=False)
            dm = B.lrmlp_desc(T, d, r, ffn, dt)
            sizes = [B.lrblock_workspace_size(dq, 0), B.lrblock_workspace_size(dq, 1),
                     B.lrblock_workspace_size(do, 0), B.lrblock_workspace_size(do, 1),
                     B.lrmlp_workspace_size(dm, 0), B.lrmlp_workspace_size(dm, 1)]
            ws = torch.empty(max(sizes), dtype=torch.uint8, device="cuda")
            act = "silu"
            ma = [m[k] for k in ("g", "A1_cat", "B1", "A2", "B2")]
            # outputs and saved tensors, allocated once
            qf = B.lrblock_fwd_chained(x, q["g"], q["A_cat"], q["B"], act=act, ws=ws)
            a = B.attn_standin_fwd(qf[0])
            of = B.lrblock_fwd_chained(a, None, o["A_cat"], o["B"], residual=x, sumsq_next=True, act=act,
                                       norm=False, ws=ws)
            h2 = of[0][0]
            mf = B.lrmlp_fwd_chained(h2, *ma, residual=h2, sumsq_in=of[3], sumsq_next=True, act=act, ws=ws)
            mb = B.lrmlp_bwd_chained(h2, *ma, mf[1], mf[2], of[3], dh3, dx_add=dh3, act=act, ws=ws)
            ob = B.lrblock_bwd_chained(a, None, o["A_cat"], o["B"], of[1], None, mb[0][None], act=act, norm=False,
                                       ws=ws)
            dqkv = B.attn_standin_bwd(ob[0])
            qb = B.lrblock_bwd_chained(x, q["g"], q["A_cat"], q["B"], qf[1], qf[2], dqkv, dx_add=mb[0], act=act,
                                       ws=ws)

            def fwd():
                B.lrblock_fwd_chained(x, q["g"], q["A_cat"], q["B"], act=act, out=qf, ws=ws)
                B.attn_standin_fwd(qf[0], out=a)
                B.lrblock_fwd_chained(a, None, o["A_cat"], o["B"], residual=x, sumsq_next=True, act=act,
                                      norm=False, out=of, ws=ws)
                B.lrmlp_fwd_chained(h2, *ma, residual=h2, sumsq_in=of[3], sumsq_next=True, act=act, out=mf,
                                    ws=ws)

            def bwd():
                B.lrmlp_bwd_chained(h2, *ma, mf[1], mf[2], of[3], dh3, dx_add=dh3, act=act, out=mb, ws=ws)
                B.lrblock_bwd_chained(a, None, o["A_cat"], o["B"], of[1], None, mb[0][None], act=act, norm=False,
                                      out=ob, ws=ws)
                B.attn_standin_bwd(ob[0], out=dqkv)
                B.lrblock_bwd_chained(x, q["g"], q["A_cat"], q["B"], qf[1], qf[2], dqkv, dx_add=mb[0], act=act,
                                      out=qb, ws=ws)

            self.fwd, self.bwd_fn = fwd, bwd
            self.act = act
            self.tokens = T
            # the QKV and O launches share the lrblock_* labels, so only the
            # MLP kernels get a per-kernel roofline here
            self.kflops = mlp_kernel_flops(T, d, r, ffn)
            self.kbytes = mlp_kernel_bytes(T, d, r, ffn)
            self.shape = dict(T=T, d=d, r=r, ffn=ffn)
        if not hasattr(self, "kbytes"):
            self.kbytes = {}
        self.flops = self.step_flops()
        self.model_flops = self.step_flops(model_only=True)

    def step(self):
        self.fwd()
        if self.bwd_fn is not None:
            self.bwd_fn()

    def step_flops(self, model_only: bool = False) -> float:
        """Algorithmic flops of one step; model_only drops the prescribed
        recompute (the gate/up re-forward of the MLP, u of the BTP share)."""
        w = self.w
        sub = recompute_flops(self.kind, w) if model_only else 0.0

        def tot(f):
            return float(sum(f.values()))

        if self.kind == "lrmlp":
            return tot(mlp_kernel_flops(w["T"], w["d"], w["r"], w["ffn"])) - sub
        if self.kind == "lrblock":
            return tot(lrblock_kernel_flops(w["T"], w["d"], w["r"], w["G"], w["d_out"], self.bwd)) - sub
        if self.kind == "btp":
            return tot(btp_kernel_flops(w["T"], w["r"], w["d_global"] // w["P"])) - sub
        T, d, r, ffn = w["T"], w["d"], w["r"], w["ffn"]
        # layer set and chained layer: the same products (QKV, O, MLP)
        return (tot(lrblock_kernel_flops(T, d, r, 3, d)) + tot(lrblock_kernel_flops(T, d, r, 1, d)) +
                tot(mlp_kernel_flops(T, d, r, ffn))) - sub


# ---------------------------------------------------------------------------
# CPU baseline: the fp64 oracle on a bounded sample of the same workload
# ---------------------------------------------------------------------------

def cpu_baseline(name, target_s):
    import oracle  # test infrastructure; used here only for the CPU baseline leg
    w = synth.WORKLOADS[name]
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))

    def run(Ts):
        if w["kind"] == "lrmlp":
            inp = synth.lrmlp_inputs(Ts, w["d"], w["r"], w["ffn"], dtype=w["dtype"], seed=0)
            a = [inp[k] for k in ("x", "g", "A1_cat", "B1", "A2", "B2")]
            t0 = time.perf_counter()
            oracle.lrmlp_forward(*a)
            oracle.lrmlp_backward(*a, inp["dY"])
            dt = time.perf_counter() - t0
            return dt, float(sum(mlp_kernel_flops(Ts, w["d"], w["r"], w["ffn"]).values()))
        if w["kind"] == "lrblock":
            inp = synth.lrblock_inputs(Ts, w["d"], w["r"], w["G"], w["d_out"], dtype=w["dtype"], seed=0)
            a = [inp[k] for k in ("x", "g", "A_cat", "B")]
            bwd = name != "llama2_1b_qkv_fwd"
            t0 = time.perf_counter()
            oracle.lrblock_forward(*a)
            if bwd:
                oracle.lrblock_backward(*a, inp["dY"])
            dt = time.perf_counter() - t0
            return dt, float(sum(lrblock_kernel_flops(Ts, w["d"], w["r"], w["G"], w["d_out"], bwd).values()))
        if w["kind"] == "btp":
            inp = synth.btp_inputs(Ts, w["r"], w["d_global"], w["P"], dtype=w["dtype"], seed=0)
            sh = synth.btp_shard(inp, 0, w["P"])
            a = [sh[k] for k in ("z", "B_s", "g_s", "A_s")]
            t0 = time.perf_counter()
            oracle.btp_share_forward(*a)
            oracle.btp_share_backward(*a, sh["dp"], sh["ds"])
            dt = time.perf_counter() - t0
            return dt, float(sum(btp_kernel_flops(Ts, w["r"], w["d_global"] // w["P"]).values()))
        if w["kind"] == "layer":
            inp = synth.layer_inputs(Ts, w["d"], w["r"], w["ffn"], dtype=w["dtype"], seed=0)
            t0 = time.perf_counter()
            oracle.layer_backward(inp["x"], inp["qkv"], inp["o"], inp["mlp"], inp["dh3"], "silu",
                                  store=oracle.round_to_bf16)
            dt = time.perf_counter() - t0
            T, d, r, ffn = Ts, w["d"], w["r"], w["ffn"]
            fl = (sum(lrblock_kernel_flops(T, d, r, 3, d).values()) +
                  sum(lrblock_kernel_flops(T, d, r, 1, d).values()) + sum(mlp_kernel_flops(T, d, r, ffn).values()))
            return dt, float(fl)
        inp = synth.layerset_inputs(Ts, w["d"], w["r"], w["ffn"], dtype=w["dtype"], seed=0)
        t0 = time.perf_counter()
        q, o, m = inp["qkv"], inp["o"], inp["mlp"]
        oracle.lrblock_backward(q["x"], q["g"], q["A_cat"], q["B"], q["dY"])
        oracle.lrblock_backward(o["x"], None, o["A_cat"], o["B"], o["dY"], norm=False)
        ma = [m[k] for k in ("x", "g", "A1_cat", "B1", "A2", "B2")]
        oracle.lrmlp_backward(*ma, m["dY"])
        dt = time.perf_counter() - t0
        T, d, r, ffn = Ts, w["d"], w["r"], w["ffn"]
        fl = (sum(lrblock_kernel_flops(T, d, r, 3, d).values()) + sum(lrblock_kernel_flops(T, d, r, 1, d).values())
              + sum(mlp_kernel_flops(T, d, r, ffn).values()))
        return dt, float(fl)

    T = w["T"]
    probe = min(128, T)
    dt, _ = run(probe)
    Ts = int(min(T, max(probe, probe * target_s / max(dt, 1e-3))))
    Ts = max(64, Ts // 64 * 64) if T >= 64 else T
    # Where the whole workload takes less than the target, it is timed over
    # several passes (each timed on its own; inputs drawn outside the timing).
    dt, fl = run(Ts)
    passes = 1
    while dt < 0.8 * target_s and passes < 8:
        d2, f2 = run(Ts)
        dt, fl, passes = dt + d2, fl + f2, passes + 1
    cpu_model, blas = "unknown", "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        blas = np.show_config(mode="dicts")["Build Dependencies"]["blas"]["name"]
    except Exception:
        pass
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": cpu_model, "blas": blas,
            "sample": f"fp64 NumPy oracle, fwd+bwd of the first {Ts} of {T} tokens of the same workload "
                      f"(algorithmic flops scaled to the sample), {passes} pass(es), {dt:.1f} s",
            "tokens_per_s": Ts * passes / dt}



# ---------------------------------------------------------------------------
# rocprofv3 post-processing (CSV output of --kernel-trace --stats and --pmc)
# ---------------------------------------------------------------------------

# Kernels of the MLP step whose instantiation (epilogue type) is unique, so a
# rocprofv3 kernel name identifies the launch label.
MLP_LABEL_PATTERNS = {
    "mlp_recompute_swiglu_bwd": "NS_12EpiSwigluBwd",
    "mlp_up1_swiglu": "NS_9EpiSwigluE",
    "mlp_down1": "NS_7EpiDownILb1",
    "mlp_down2": "NS_7EpiDownILb0",
    "mlp1_dx": "NS_5EpiDXE",
    "mlp1_ds": "NS_5EpiDSILb1",
    "mlp_ds2": "NS_5EpiDSILb0",
    # weight-gradient products: one kernel instantiation per launch tag
    "mlp1_dB": "NS_8EpiStoreILb1EEELi1EE",
    "mlp1_dA": "NS_8EpiStoreILb1EEELi2EE",
    "mlp_dB2": "NS_8EpiStoreILb1EEELi3EE",
    "mlp_dA2": "NS_8EpiStoreILb1EEELi4EE",
}


# The forward of a grouped block (the QKV workload): down product with the
# statistic and activation, batched up product with a plain store.
LRBLOCK_FWD_LABEL_PATTERNS = {
    "lrblock_down": "NS_7EpiDownILb1",
    "lrblock_up": "NS_8EpiStoreILb0",
}


def lrblock_fwd_kernel_rw(T, d, r, G, d_out):
    """(read, written) algorithmic bytes of the grouped block's forward
    launches (bf16 operands, fp32 H and statistic)."""
    b, f = 2, 4
    return {"lrblock_down": (T * d * b + d * G * r * b, T * G * r * (f + b) + T * f),
            "lrblock_up": (T * G * r * b + G * r * d_out * b, G * T * d_out * b)}


# The tensor-parallel share: every launch has an instantiation of its own.
BTP_LABEL_PATTERNS = {
    "btp_u": "NS_7EpiBtpUE",
    "btp_p": "NS_7EpiBtpPE",
    "btp_u_re": "NS_8EpiStoreILb1EEELi0EE",
    "btp_u_bwd": "NS_10EpiBtpEBwdE",
    "btp_dz": "NS_8EpiStoreILb0EEELi0EE",
    "btp_dA": "NS_8EpiStoreILb1EEELi5EE",
    "btp_dB": "NS_8EpiStoreILb1EEELi6EE",
}


def btp_kernel_rw(T, r, S):
    """(read, written) algorithmic bytes of the share's launches (bf16
    operands; fp32 statistic, u handed over in fp32, fp32 weight gradients)."""
    b, f = 2, 4
    return {"btp_u": (T * r * b + r * S * b + S * b, T * S * b + T * f),
            "btp_p": (T * S * b + S * r * b, T * r * b + T * f),
            "btp_u_re": (T * r * b + r * S * b, T * S * f),
            "btp_u_bwd": (T * r * b + S * r * b + T * S * f + S * b + T * f, 2 * T * S * b),
            "btp_dz": (T * S * b + r * S * b, T * r * b),
            "btp_dA": (T * S * b + T * r * b, S * r * f),
            "btp_dB": (T * r * b + T * S * b, r * S * f)}


def counter_workload(workload: str):
    """(label patterns, {label: flops}, {label: (read, written)}) of a
    workload whose launches the counter summaries attribute to labels, or
    (None, {}, {}) for one whose kernel instantiations serve several
    launches (the chained layer and the layer set): those are summarised
    per instantiation."""
    w = synth.WORKLOADS[workload]
    if w["kind"] == "lrmlp":
        a = {k: w[k] for k in ("T", "d", "r", "ffn")}
        return MLP_LABEL_PATTERNS, mlp_kernel_flops(**a), mlp_kernel_rw(**a)
    if w["kind"] == "lrblock" and workload.endswith("_fwd"):
        return (LRBLOCK_FWD_LABEL_PATTERNS, lrblock_kernel_flops(w["T"], w["d"], w["r"], w["G"], w["d_out"], False),
                lrblock_fwd_kernel_rw(w["T"], w["d"], w["r"], w["G"], w["d_out"]))
    if w["kind"] == "btp":
        S = w["d_global"] // w["P"]
        return BTP_LABEL_PATTERNS, btp_kernel_flops(w["T"], w["r"], S), btp_kernel_rw(w["T"], w["r"], S)
    if w["kind"] in ("layer", "layerset"):
        return None, {}, {}
    raise SystemExit(f"no counter summary for workload {workload}")


def instantiation_patterns(*per_kernel_maps):
    """{short name: full name} of every GEMM instantiation in counter maps."""
    names = sorted({k for m in per_kernel_maps for k in m if "gemm_kernel" in k})
    return {short_kernel_name(k): k for k in names}


def short_kernel_name(n: str) -> str:
    import re
    m = re.search(r"CfgI(DF16b|f)Li(\d+)ELi(\d+)ELi(\d)ELi(\d)ELb(\d)ELb(\d)ELi(\d)EEENS_(\d+)", n)
    if m:
        t = "bf16" if m.group(1) == "DF16b" else "f32"
        lay = ("KC" if m.group(6) == "1" else "MC") + "/" + ("KC" if m.group(7) == "1" else "NC")
        rest = n[m.end():]
        epi = rest[:int(m.group(9))]  # mangled <length><name>
        flags = re.match(r"I((?:Lb\d+E)+)E", rest[len(epi):])
        if flags:
            epi += "<" + ",".join(re.findall(r"Lb(\d+)E", flags.group(1))) + ">"
        tag = re.search(r"EELi(\d+)EEEv", n)
        tag = f" tag {tag.group(1)}" if tag and tag.group(1) != "0" else ""
        return f"gemm {t} {m.group(2)}x{m.group(3)} waves {m.group(4)}x{m.group(5)} {lay} nacc={m.group(8)} {epi}{tag}"
    return n.split("(")[0].replace("void ", "")


def summarize_stats(csv_path: str, title: str, command: str) -> str:
    """Markdown table from a rocprofv3 kernel_stats.csv."""
    import csv
    rows = list(csv.DictReader(open(csv_path)))
    out = [f"# {title}", "", "Command:", "", "```", command, "```", "",
           "| kernel | calls | avg (us) | min (us) | max (us) | total (us) | % |", "|---|---|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| {short_kernel_name(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                   f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                   f"{float(r['TotalDurationNs']) / 1e3:.1f} | {float(r['Percentage']):.1f} |")
    return "\n".join(out) + "\n"


def counter_per_kernel(csv_path: str, counter: str):
    """{kernel name: [per-dispatch values]} of one counter from counter_collection.csv."""
    import csv
    per = {}
    for r in csv.DictReader(open(csv_path)):
        if r["Counter_Name"] != counter:
            continue
        per.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return per


def dispatch_ns(csv_path: str, pattern: str):
    """Durations (ns) of the dispatches whose kernel name contains pattern,
    one per dispatch, from a counter_collection.csv."""
    import csv
    seen, out = set(), []
    for r in csv.DictReader(open(csv_path)):
        if pattern not in r["Kernel_Name"] or not r.get("Start_Timestamp") or r.get("Dispatch_Id") in seen:
            continue
        seen.add(r.get("Dispatch_Id"))
        out.append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    return out


def mfma_summary(csv_path: str, title: str, command: str, workload: str = "llama2_7b_mlp") -> str:
    """Markdown table of MFMA utilisation (rocprofv3 derived counter MfmaUtil)
    and hardware-counted bf16 MFMA flops (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512)
    per labelled kernel of the workload's step, against its algorithmic flops."""
    util = counter_per_kernel(csv_path, "MfmaUtil")
    mops = counter_per_kernel(csv_path, "SQ_INSTS_VALU_MFMA_MOPS_BF16")
    patterns, kf, _ = counter_workload(workload)
    out = [f"# {title}", "", "Command:", "", "```", command, "```", ""]
    if patterns is None:
        # Instantiations shared by several launches: per-dispatch means over
        # every launch an instantiation served (several shapes).
        out += ["One row per kernel instantiation; an instantiation that serves several launches of the step "
                "(e.g. the weight gradients of the QKV, O and MLP blocks) averages over all of them.", "",
                "| kernel | dispatches | MFMA busy (% of SIMD cycles, mean) | counted MFMA GF per dispatch (mean) |",
                "|---|---|---|---|"]
        for short, full in instantiation_patterns(util, mops).items():
            u, m = util.get(full), mops.get(full)
            if not u or not m:
                continue
            out.append(f"| {short} | {len(u)} | {sum(u) / len(u):.1f} | {sum(m) / len(m) * 512 / 1e9:.1f} |")
        return "\n".join(out) + "\n"
    out += ["| launch | kernel | MFMA busy (% of SIMD cycles) | counted MFMA GF | algorithmic GF | counted / algorithmic |",
            "|---|---|---|---|---|---|"]
    for label, pat in patterns.items():
        un = [k for k in util if pat in k]
        mn = [k for k in mops if pat in k]
        if len(un) != 1 or len(mn) != 1:
            continue
        u = sum(util[un[0]]) / len(util[un[0]])
        gf = sum(mops[mn[0]]) / len(mops[mn[0]]) * 512 / 1e9
        out.append(f"| {label} | {short_kernel_name(un[0])} | {u:.1f} | {gf:.1f} | {kf[label] / 1e9:.1f} | "
                   f"{gf * 1e9 / kf[label]:.3f} |")
    return "\n".join(out) + "\n"


def traffic_json(fetch_csv: str, write_csv: str, workload: str, copy_mib: int) -> dict:
    """Per-launch HBM bytes of the labelled kernels, each counter scaled by the
    factor that makes the calibration copy (copy_mib MiB read and written by
    one blit kernel) read exactly its size."""
    fetch = counter_per_kernel(fetch_csv, "FETCH_SIZE")
    write = counter_per_kernel(write_csv, "WRITE_SIZE")
    known = float(copy_mib << 20)

    def copy_kib(per):
        vals = [max(v) for k, v in per.items() if "copyBuffer" in k or "copy" in k.lower()]
        return max(vals) if vals else None

    fk, wk = copy_kib(fetch), copy_kib(write)
    if not fk or not wk:
        raise SystemExit("no calibration copy kernel in the counter files")
    f_scale, w_scale = known / (fk * 1024.0), known / (wk * 1024.0)
    kernels = {}
    patterns = counter_workload(workload)[0]
    if patterns is None:
        patterns = instantiation_patterns(fetch, write)
    for label, pat in patterns.items():
        fn = [k for k in fetch if pat in k]
        wn = [k for k in write if pat in k]
        if len(fn) != 1 or len(wn) != 1:
            continue
        fv, wv = fetch[fn[0]], write[wn[0]]
        kernels[label] = {"kernel": short_kernel_name(fn[0]), "dispatches": len(fv),
                          "fetch_bytes": round(sum(fv) / len(fv) * 1024.0 * f_scale),
                          "write_bytes": round(sum(wv) / len(wv) * 1024.0 * w_scale)}
        durs = dispatch_ns(fetch_csv, pat) + dispatch_ns(write_csv, pat)
        if durs:
            kernels[label]["avg_ms_profiled"] = round(sum(durs) / len(durs) / 1e6, 5)
    return {"source_digest": source_digest(), "workload": workload,
            "calibration": {"copy_bytes": int(known), "fetch_kib_read": fk, "write_kib_read": wk,
                            "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4)},
            "kernels": kernels}

def traffic_table(json_path: str, title: str, command: str) -> str:
    """Markdown table of the per-launch traffic in a traffic JSON against the
    algorithmic bytes of each launch."""
    tj = json.load(open(json_path))
    rw = counter_workload(tj["workload"])[2]
    cal = tj["calibration"]
    out = [f"# {title}", "", "Commands (R = repository root):", "", "```", command, "```", "",
           f"Calibration: each run first copies {cal['copy_bytes'] >> 20} MiB with one blit kernel. FETCH_SIZE read "
           f"{cal['fetch_kib_read']:.0f} KiB for it (scale x{cal['fetch_scale']}), WRITE_SIZE "
           f"{cal['write_kib_read']:.0f} KiB (scale x{cal['write_scale']}); both scales are applied below. "
           "FETCH_SIZE counts every L2 miss that goes to the memory fabric, so reads served by the 256 MB "
           "last-level (MALL) cache count too: fetched bytes are upper bounds on DRAM bytes.", "",
           f"Source digest of the kernels measured: `{tj['source_digest']}`.", "",
           "Algorithmic bytes: each input read once, each output written once (the operands of every launch are "
           "listed in `mlp_kernel_rw`, `lrblock_fwd_kernel_rw` and `btp_kernel_rw` in bench.py; a workload whose "
           "kernel instantiations serve several launches is listed per instantiation, as means over its "
           "dispatches, without algorithmic bytes). Fetched bytes above the algorithmic "
           "reads are operand panels "
           "that many tiles share and that leave an XCD's 4 MB L2 between the waves of tiles using them (the "
           "up projections and the recompute, with K = r, re-read their S1/B1 panels once per wave of tiles); "
           "they are served from the fabric (MALL or DRAM).", "",
           "Rates: the counted bytes (fetched + written) and the algorithmic bytes over each launch's average "
           "duration in the two counter runs (kernels run one at a time under counter collection), against the "
           f"{PEAK_HBM_GBS / 1e3:.0f} TB/s HBM peak.", "",
           "| launch | kernel | fetched MB | written MB | algorithmic read MB | algorithmic write MB | "
           "fetched / algorithmic read | us (profiled) | counted GB/s | % of HBM peak | algorithmic GB/s |",
           "|---|---|---|---|---|---|---|---|---|---|---|"]
    for label, k in tj["kernels"].items():
        # Per-instantiation rows (shared by launches of several shapes) have
        # no algorithmic bytes of their own.
        rd, wr = rw.get(label, (None, None))
        ms = k.get("avg_ms_profiled")
        alg = "- | - | -" if rd is None else f"{rd / 1e6:.0f} | {wr / 1e6:.0f} | {k['fetch_bytes'] / rd:.2f}"
        if ms:
            cg = (k["fetch_bytes"] + k["write_bytes"]) / (ms * 1e-3) / 1e9
            ag = "-" if rd is None else f"{(rd + wr) / (ms * 1e-3) / 1e9:.0f}"
            rates = f"{ms * 1e3:.1f} | {cg:.0f} | {100 * cg / PEAK_HBM_GBS:.1f} | {ag}"
        else:
            rates = "- | - | - | -"
        kern = k["kernel"] if k["kernel"] != label else f"mean of {k['dispatches']} dispatches"
        out.append(f"| {label} | {kern} | {k['fetch_bytes'] / 1e6:.0f} | {k['write_bytes'] / 1e6:.0f} | "
                   f"{alg} | {rates} |")
    return "\n".join(out) + "\n"

def r_sweep(B, torch, ranks, steps, warmup):
    """Per-launch kernel times of the 7B-shaped MLP block at several ranks."""
    w = synth.WORKLOADS["llama2_7b_mlp"]
    T, d, ffn = w["T"], w["d"], w["ffn"]
    gen = torch.Generator(device="cuda").manual_seed(0)
    for r in ranks:
        def rn(*shape, std=1.0):
            return (torch.randn(*shape, device="cuda", generator=gen) * std).bfloat16()
        x, dY = rn(T, d), rn(T, d)
        g = (1 + 0.1 * torch.randn(d, device="cuda", generator=gen)).bfloat16()
        args = [x, g, rn(d, 2 * r, std=d ** -0.5), rn(2, r, ffn, std=r ** -0.5), rn(ffn, r, std=ffn ** -0.5),
                rn(r, d, std=r ** -0.5)]
        for _ in range(max(1, warmup)):
            fo = B.lrmlp_fwd(*args)
            B.lrmlp_bwd(*args, *fo[1:], dY)
        torch.cuda.synchronize()
        B.profiler_enable(None, 4096)
        for _ in range(max(1, steps)):
            fo = B.lrmlp_fwd(*args)
            B.lrmlp_bwd(*args, *fo[1:], dY)
        torch.cuda.synchronize()
        rep = B.profiler_report()
        B.profiler_disable()
        print(json.dumps({"T": T, "d": d, "r": r, "ffn": ffn,
                          "kernel_ms": {k: round(v[1] / v[0], 4) for k, v in sorted(rep.items())}}), flush=True)


# ---------------------------------------------------------------------------

def peak_of(wl) -> float:
    return PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_F32_TFLOPS


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--split-steps", type=int, default=10,
                    help="steps of the untimed pass that splits forward and backward with events (default 10)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warm-up steps (default: as many as fill --warmup-s seconds, at least 3)")
    ap.add_argument("--warmup-s", type=float, default=0.5, help="seconds of warm-up when --warmup is not given")
    ap.add_argument("--workload", default="llama2_7b_mlp", choices=sorted(synth.WORKLOADS))
    ap.add_argument("--act", default=None, help="bottleneck activation for the layer set (silu|identity)")
    ap.add_argument("--cpu-baseline", default="on", choices=["on", "off"])
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--graph-steps", type=int, default=0,
                    help="after the timed steps, capture one forward+backward step into a HIP graph and time this "
                         "many replays (reported under timing.graph; `value` stays the eager rate)")
    ap.add_argument("--flush-steps", type=int, default=5,
                    help="steps of a second, untimed-for-value pass with the last-level cache flushed before each")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="before timing, copy this many MiB once with a plain device copy, so that a "
                         "counter profile of this run holds a copy kernel of known traffic")
    ap.add_argument("--summarize-stats", metavar="CSV", help="print a markdown summary of a rocprofv3 "
                    "kernel_stats.csv (with --title, --command) and exit")
    ap.add_argument("--traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="print the per-launch HBM traffic JSON from two rocprofv3 --pmc counter_collection.csv "
                         "files (FETCH_SIZE, WRITE_SIZE; runs made with --calibrate-copy-mib) and exit")
    ap.add_argument("--mfma-summary", metavar="CSV", help="print MFMA utilisation per kernel from a rocprofv3 "
                    "--pmc MfmaUtil SQ_INSTS_VALU_MFMA_MOPS_BF16 counter_collection.csv (with --title, --command) "
                    "and exit")
    ap.add_argument("--traffic-table", metavar="JSON", help="print a markdown table of a traffic JSON (written "
                    "by --traffic) against the algorithmic bytes (with --title, --command) and exit")
    ap.add_argument("--r-sweep", metavar="R,R,...", help="time the 7B-shaped MLP block (T, d, ffn of the default "
                    "workload) at each listed rank r with seeded Gaussian inputs generated on the GPU, print one JSON "
                    "line of per-launch kernel times (ms, library events, mean of --steps steps) per rank, and exit. "
                    "The K = r products have a fixed tile count, so their time against r separates the fixed "
                    "per-tile cost from the main loop")
    ap.add_argument("--isolate-steps", type=int, default=3,
                    help="after the timed steps, run this many more (not part of `value`) with every product "
                         "on the caller's stream, one launch at a time, and report each product's own time "
                         "as `kernels_isolated` (0: skip)")
    ap.add_argument("--title", default="")
    ap.add_argument("--command", default="")
    args = ap.parse_args()
    if args.summarize_stats:
        sys.stdout.write(summarize_stats(args.summarize_stats, args.title, args.command))
        return
    if args.mfma_summary:
        sys.stdout.write(mfma_summary(args.mfma_summary, args.title, args.command, args.workload))
        return
    if args.traffic_table:
        sys.stdout.write(traffic_table(args.traffic_table, args.title, args.command))
        return
    if args.traffic:
        print(json.dumps(traffic_json(args.traffic[0], args.traffic[1], args.workload,
                                      args.calibrate_copy_mib or 1024), indent=1))
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(collectives, sharding and rank code are not part of it). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(1)
    from rank_bottleneck_online_amd import binding as B
    B.lib()

    if args.r_sweep:
        r_sweep(B, torch, [int(v) for v in args.r_sweep.split(",")], args.steps,
                3 if args.warmup is None else args.warmup)
        return

    wl = Workload(args.workload)
    if args.act and wl.kind == "layerset":
        wl.act = args.act
    log(f"workload {args.workload} {wl.shape}; step flops {wl.flops / 1e9:.1f} GF")

    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy: {n} bytes read, {n} bytes written")
        del src, dst

    # Warm-up: W steps, or by default as many as fill --warmup-s seconds (at
    # least 3). From idle the GPU needs tens of milliseconds under load to
    # reach its working clock, longer than a few steps of the smaller
    # workloads (a 0.25 ms step timed after 3 warm-up steps reads 15% slow).
    if args.warmup is None:
        warmup, t_end = 0, time.perf_counter() + args.warmup_s
        while warmup < 3 or time.perf_counter() < t_end:
            wl.step()
            warmup += 1
            if warmup % 8 == 0:
                torch.cuda.synchronize()  # the host stays within 8 steps of the GPU
    else:
        warmup = args.warmup
        for _ in range(warmup):
            wl.step()
    torch.cuda.synchronize()

    # Which kernel dominates the step (untimed discovery pass over three
    # steps: the first launch after the timer is switched on reads a few
    # microseconds long, enough to tip a choice between equal products).
    n_disc = 3
    B.profiler_enable(None, 4096)
    for _ in range(n_disc):
        wl.step()
    rep = B.profiler_report()
    B.profiler_disable()
    per_kernel = {k: v[1] / n_disc for k, v in rep.items()}
    # The roofline kernel: the longest launch on the caller's stream among
    # those with algorithmic flops (not the transposes or reductions).
    main_kernels = {k: v for k, v in per_kernel.items() if k not in SIDE_STREAM_LABELS and k in wl.kflops}
    cands = main_kernels or {k: v for k, v in per_kernel.items() if k in wl.kflops} or per_kernel
    dom = max(cands, key=cands.get)
    log("kernel times in one step (ms):", json.dumps({k: round(v, 4) for k, v in
                                                       sorted(per_kernel.items(), key=lambda kv: -kv[1])}))

    # Timed region: K steps between two events, plus the library's events
    # around the dominant kernel's launches (created without the system-scope
    # fence, so they cost the stream almost nothing).
    B.profiler_enable(dom, 64 * max(1, args.steps))
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e_start, e_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e_start.record(stream)
    for i in range(args.steps):
        wl.step()
    e_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e_start.elapsed_time(e_end) / args.steps
    rep = B.profiler_report()
    B.profiler_disable()

    # Forward / backward split, not part of `value`: a separate pass with an
    # event at every boundary. An event recorded on the stream costs it a few
    # microseconds (its cache write-back), which is why these stay out of the
    # timed region; the split's step times include them.
    n_split = max(1, min(args.steps, args.split_steps))
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n_split + 1)]
    ev[0].record(stream)
    for i in range(n_split):
        wl.fwd()
        ev[2 * i + 1].record(stream)
        if wl.bwd_fn is not None:
            wl.bwd_fn()
        ev[2 * i + 2].record(stream)
    torch.cuda.synchronize()
    fwd_ms = [ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(n_split)]
    bwd_ms = [ev[2 * i + 1].elapsed_time(ev[2 * i + 2]) for i in range(n_split)]
    step_ms = [a + b for a, b in zip(fwd_ms, bwd_ms)]

    # Second pass, not part of `value`: the 256 MB last-level cache is flushed
    # (a 512 MB buffer is written) before every step, so inputs come from HBM.
    flushed = None
    if args.flush_steps > 0:
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        fl = []
        for i in range(args.flush_steps):
            scratch.fill_(i & 0xFF)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            wl.step()
            b.record(stream)
            fl.append((a, b))
        torch.cuda.synchronize()
        fms = sorted(a.elapsed_time(b) for a, b in fl)
        flushed = {"steps": args.flush_steps, "ms_median": round(fms[len(fms) // 2], 4), "ms_min": round(fms[0], 4),
                   "tflops_median": round(wl.flops / (fms[len(fms) // 2] * 1e-3) / 1e12, 2)}
        del scratch

    # Third pass, not part of `value`: every product alone. The weight
    # gradients leave the side stream for the caller's (the library's
    # measurement switch), so no launch shares the GPU with another and each
    # product's time is its own (the cache state is still that of a step).
    isolated = None
    if args.isolate_steps > 0:
        B.profiler_serialize(True)
        B.profiler_enable(None, 4096)
        for _ in range(args.isolate_steps):
            wl.step()
        torch.cuda.synchronize()
        rep_iso = B.profiler_report()
        B.profiler_disable()
        B.profiler_serialize(False)
        isolated = {}
        for k, (c, t) in sorted(rep_iso.items(), key=lambda kv: -kv[1][1]):
            kms = t / args.isolate_steps
            isolated[k] = {"ms": round(kms, 4), "launches_per_step": c / args.isolate_steps}
            kf = wl.kflops.get(k)
            if kf and kms > 0:
                isolated[k]["tflops"] = round(kf / (kms * 1e-3) / 1e12, 1)
                isolated[k]["frac"] = round(kf / (kms * 1e-3) / 1e12 / peak_of(wl), 4)
        log("kernel times in one step, each product alone (ms):",
            json.dumps({k: v["ms"] for k, v in isolated.items()}))

    # Optional: the same step captured into a HIP graph and replayed (the
    # library allocates nothing and forks its side stream with events, which
    # capture records as graph dependencies); launch-bound workloads show the
    # launch overhead this removes.
    graph = None
    if args.graph_steps > 0:
        cg = torch.cuda.CUDAGraph()
        with torch.cuda.graph(cg):
            wl.step()
        torch.cuda.synchronize()
        gl = []
        for _ in range(args.graph_steps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            cg.replay()
            b.record(stream)
            gl.append((a, b))
        torch.cuda.synchronize()
        gms = sorted(a.elapsed_time(b) for a, b in gl)
        graph = {"steps": args.graph_steps, "ms_median": round(gms[len(gms) // 2], 4), "ms_min": round(gms[0], 4),
                 "tflops_median": round(wl.flops / (gms[len(gms) // 2] * 1e-3) / 1e12, 3)}
        del cg

    cnt, tot = rep.get(dom, (0, 0.0))
    avg_ms = tot / max(cnt, 1)
    launches_per_step = cnt / args.steps
    dom_flops = wl.kflops.get(dom)
    value = wl.flops / (ms * 1e-3) / 1e12
    peak = peak_of(wl)
    roofline = None
    if dom_flops:
        achieved = dom_flops / (avg_ms * 1e-3) / 1e12
        traffic = None
        if os.path.exists(traffic_json_path(args.workload)):
            tj = json.load(open(traffic_json_path(args.workload)))
            if tj.get("source_digest") == source_digest() and tj.get("workload") == args.workload:
                k = tj.get("kernels", {}).get(dom)
                if k:
                    traffic = k["fetch_bytes"] + k["write_bytes"]
        roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                    "frac": round(achieved / peak, 4), "traffic": traffic, "kernel": dom,
                    "kernel_avg_ms": round(avg_ms, 5), "launches_per_step": launches_per_step,
                    "algorithmic_gflop_per_launch": round(dom_flops / 1e9, 3)}

    def med(v):
        return sorted(v)[len(v) // 2]

    kernels = {}
    for k, kms in sorted(per_kernel.items(), key=lambda kv: -kv[1]):
        kf = wl.kflops.get(k)
        kernels[k] = {"ms": round(kms, 4), "stream": "side" if k in SIDE_STREAM_LABELS else "caller"}
        if kf and kms > 0:
            kernels[k]["tflops"] = round(kf / (kms * 1e-3) / 1e12, 1)
            kernels[k]["frac"] = round(kf / (kms * 1e-3) / 1e12 / peak, 4)
            kb = wl.kbytes.get(k)
            if kb:
                # roofline time max(F/peak, B/HBM) over the measured time
                t_mfma, t_hbm = kf / (peak * 1e12), kb / (PEAK_HBM_GBS * 1e9)
                kernels[k]["alg_gb"] = round(kb / 1e9, 3)
                kernels[k]["alg_gbs"] = round(kb / (kms * 1e-3) / 1e9, 1)
                kernels[k]["roofline_bound"] = "mfma" if t_mfma >= t_hbm else "hbm"
                kernels[k]["roofline_frac"] = round(max(t_mfma, t_hbm) / (kms * 1e-3), 4)

    cpu = None
    if args.cpu_baseline == "on":
        log("timing the CPU oracle on a bounded sample ...")
        cpu = cpu_baseline(args.workload, args.cpu_seconds)

    if cpu:
        cpu["gpu_over_cpu"] = round(value / cpu["value"], 1)
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded Gaussian, LLaMA-2 shapes)",
        "config": {"workload": args.workload, **wl.shape, **({"act": wl.act} if wl.kind == "layerset" else {})},
        "tokens_per_s": round(wl.tokens / (ms * 1e-3), 1),
        "pct_of_peak": round(100.0 * value / peak, 2),
        "algorithmic_gflop_per_step": round(wl.flops / 1e9, 2),
        "wall_s_timed": round(wall, 4),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "timing": {"split_steps": n_split,
                   "step_ms_median": round(med(step_ms), 4), "step_ms_min": round(min(step_ms), 4),
                   "fwd_ms_median": round(med(fwd_ms), 4), "fwd_ms_min": round(min(fwd_ms), 4),
                   "bwd_ms_median": round(med(bwd_ms), 4) if wl.bwd_fn else None,
                   "bwd_ms_min": round(min(bwd_ms), 4) if wl.bwd_fn else None,
                   "model_only_tflops": round(wl.model_flops / (ms * 1e-3) / 1e12, 2),
                   "model_only_gflop_per_step": round(wl.model_flops / 1e9, 2),
                   "mall_flushed": flushed, "graph": graph},
        "kernels": kernels,
        "kernels_isolated": isolated,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
