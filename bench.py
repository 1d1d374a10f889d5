"""Benchmark of the NVFP4 W4A16 MTP draft-head hot path on one MI355X.

A step is one draft step of a Qwen-shaped MTP head at M decode rows: the
fc / q|k|v (grouped) / o W4A16 GEMVs, the routed MoE FFN (256 NVFP4
experts, top-8) and the full-vocabulary (151936 x 2048) NVFP4 LM head fused
with argmax, whose draft ids stay on the device: the same call runs the next
step's fc over the embedding row of each id (lmhead_gemv_argmax_fc: one
launch at M = 1, the LM head's workgroups finishing the fc once the last of
them has published the id), so each step runs its fc with the previous
step's head (device-resident chaining).  The step is captured
in a HIP graph and replayed in rotation over NCOPIES independent copies of
every weight (5.5 GB, 21x the 256 MB Infinity Cache), each step with its own
router logits, so the weights stream from HBM as in serving.  The headline
is M = 1; M = 4 and 8 are timed in the same run.  All inputs are seeded
synthetic data resident in HBM before the timed region.

Printed: one JSON line.  `value` = algorithmic HBM bytes of the step (NVFP4
codes + scales + globals actually read, activations in, results out) per
second at M = 1.  Extra fields: drafts/s of the LM head, a roofline object
for the dominant kernel (the LM-head GEMV+argmax, timed with HIP events on
the stream it runs on), per-row measurements (each decode kernel over at
least 1 GiB of distinct weights, the quantizer, the prefill GEMM,
DeepSeek-shaped rows) with the committed counter passes attached where the
kernel sources still match, and the CPU oracle timed on bounded samples at
one thread and at every host core.

Other modes: --gemm-only (every prefill GEMM shape), --counters (the decode
rows once each, separated by marker kernels, for rocprofv3 counter passes),
--summarize-counters (turns those passes into the committed summary),
--calibrate-copy (a plain 1 GiB copy for the byte-counter calibration),
--moe-timeline (the one-token MoE's phase timestamps, moe_w4a16_gemv_trace).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
H, I, E, TOPK, VOCAB = 2048, 1024, 256, 8, 151936
PROJ = [("fc", 2048, 4096), ("q", 8192, 2048), ("k", 512, 2048), ("v", 512, 2048), ("o", 2048, 4096)]
NCOPIES = 5                 # weight copies of the whole step (1.1 GB each)
ROT_BYTES = 1 << 30         # distinct weight bytes a timed row rotates through (4x the Infinity Cache)
MIN_LAUNCHES = 30           # launches per timed graph at least
COUNTER_PROFILE = os.path.join(ROOT, "profiles", "decode_kernels_counters.md")
SOURCES = ("gemv.hip", "gemv_core.hpp", "common.hpp", "moe.hip", "quantize.hip")


def nvfp4_bytes(n, k):
    return n * k // 2 + n * k // 16 + 16


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-rows", action="store_true", help="skip the per-row measurements")
    p.add_argument("--gemm-only", action="store_true",
                   help="only time the prefill GEMM at every prompt-chunk shape (one JSON line)")
    p.add_argument("--counters", action="store_true",
                   help="run each decode row once (no graphs), rows separated by a marker kernel")
    p.add_argument("--summarize-counters", nargs="+", metavar="DIR",
                   help="rocprofv3 output dirs of the --counters passes -> markdown summary on stdout")
    p.add_argument("--copy-dirs", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="with --summarize-counters: the FETCH_SIZE and WRITE_SIZE passes of --calibrate-copy")
    p.add_argument("--moe-timeline", action="store_true",
                   help="phase timestamps of the one-token MoE launch (medians over launches) and exit")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run a plain 1 GiB device copy (PMC byte-counter calibration)")
    return p.parse_args()


# ------------------------------------------------------------------ set-up
class Env:
    def __init__(self, nv, torch):
        self.nv, self.torch = nv, torch
        self.dev = torch.device("cuda:0")
        self.gen = torch.Generator(device=self.dev)
        self.gen.manual_seed(0)
        self.s = torch.cuda.Stream()

    def randn(self, shape, std=1.0, dtype=None):
        t = self.torch.randn(shape, generator=self.gen, device=self.dev, dtype=self.torch.float32)
        if std != 1.0:
            t.mul_(std)
        return t.to(dtype or self.torch.bfloat16)


def quantized_pool(env, n, k, copies):
    """`copies` distinct NVFP4 matrices [n, k]: seeded N(0, 0.02) bf16
    weights quantized on the GPU, several copies per quantizer call (row
    views of one quantized pool, one global scale per call)."""
    nv = env.nv
    per_call = max(1, min(copies, (1 << 28) // (n * k)))
    out = []
    while len(out) < copies:
        cc = min(per_call, copies - len(out))
        q = nv.nvfp4_quantize(env.randn((cc * n, k), 0.02))
        for j in range(cc):
            out.append(nv.NVFP4Weight(q.codes[j * n:(j + 1) * n], q.scales[j * n:(j + 1) * n], q.glob, n, k))
    return out


def expert_stack(env, num_experts=E, hidden=H, inter=I):
    """One stack of routed experts (gate/up [E][I][H], down [E][H][I]), each
    projection quantized from seeded N(0, 0.02) bf16 weights in one call
    (its global scale repeated per expert)."""
    nv = env.nv
    parts = []
    for rows, cols in ((inter, hidden), (inter, hidden), (hidden, inter)):
        q = nv.nvfp4_quantize(env.randn((num_experts * rows, cols), 0.02))
        parts += [q.codes.view(num_experts, rows, cols // 2), q.scales.view(num_experts, rows, cols // 16),
                  q.glob.repeat(num_experts, 1).contiguous()]
    return nv.NVFP4Experts(*parts)


def rot_copies(bytes_per_launch):
    """Distinct weight copies a timed row rotates through: ROT_BYTES of them."""
    return max(1, math.ceil(ROT_BYTES / bytes_per_launch))


def launches(copies):
    return max(MIN_LAUNCHES, copies)


def _time(torch, fn, reps, stream):
    """Average launch time of fn(i), i = 0..reps-1, back to back on `stream`
    between two HIP events recorded on that stream."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        fn(0)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(reps):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def _time_graph(torch, fn, reps, stream):
    """Per-launch device time of fn: `reps` launches (each on its own weight
    copy or routing) captured in one HIP graph, replayed 3 times between two
    events.  Host launch overhead is excluded; the kernel boundaries inside
    the graph are included, as in a captured draft step."""
    with torch.cuda.stream(stream):
        fn(0)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(reps):
                fn(i)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(3):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) / (3 * reps)


def _row(ms, nbytes, **extra):
    gbs = nbytes / (ms * 1e-3) / 1e9
    r = {"ms": round(ms, 5), "gbs": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4)}
    r.update(extra)
    return r


def moe_bytes(nd, M, hidden=H, inter=I, experts=E):
    return nd * 3 * nvfp4_bytes(inter, hidden) + M * hidden * 2 + M * experts * 4 + M * hidden * 4 + 2 * M * TOPK * 4


def distinct_experts(nv, torch, x, routers, ex, ws, M):
    ids = torch.empty((M, TOPK), dtype=torch.int32, device=x.device)
    out = []
    for r in routers:
        nv.moe_w4a16_gemv(x, r, TOPK, ex, workspace=ws, topk_ids=ids)
        out.append(len(set(ids.cpu().numpy().ravel().tolist())))
    return out


# ------------------------------------------------------- the draft step
def draft_step(env, copies, lm_pool, embed_table, M, steps, warmup):
    """Times `steps` chained draft steps at M rows (graphs of NCOPIES steps,
    one per weight copy, each with its own router logits)."""
    nv, torch, dev = env.nv, env.torch, env.dev
    xs = {name: env.randn((M, k)) for name, n, k in PROJ}
    xm = env.randn((M, H))
    routers = [env.randn((M, E), dtype=torch.float32) for _ in range(NCOPIES)]
    hl = env.randn((M, H))
    ys = {name: torch.empty((M, n), dtype=torch.float32, device=dev) for name, n, k in PROJ}
    ymoe = torch.empty((M, H), dtype=torch.float32, device=dev)
    ids = torch.empty((M, TOPK), dtype=torch.int32, device=dev)
    wts = torch.empty((M, TOPK), dtype=torch.float32, device=dev)
    moe_ws = nv.moe_workspace(M, TOPK, copies[0]["moe"], dev)
    lm_ws = nv.lmhead_workspace(M, VOCAB, dev)
    out_idx = torch.zeros(M, dtype=torch.int32, device=dev)
    out_max = torch.empty(M, dtype=torch.float32, device=dev)
    draft_log = torch.zeros(NCOPIES * M, dtype=torch.int32, device=dev)

    hfc = env.randn((M, H))   # the hidden-state half of the fc input rows

    def step(c):
        ws = copies[c]
        # (this step's fc over [embedding of the previous draft | hidden
        # state] ran with the previous step's LM head, below)
        nv.w4a16_gemv_grouped(xs["q"], [ws["q"], ws["k"], ws["v"]], outs=[ys["q"], ys["k"], ys["v"]])
        nv.w4a16_gemv(xs["o"], ws["o"], out=ys["o"])
        nv.moe_w4a16_gemv(xm, routers[c], TOPK, ws["moe"], workspace=moe_ws, out=ymoe, topk_ids=ids, topk_w=wts)
        # the draft ids stay on the device; the same call runs the next
        # step's fc over the embedding row of each id (one launch at M = 1)
        nv.lmhead_gemv_argmax_fc(hl, lm_pool[c], embed_table, hfc, copies[(c + 1) % NCOPIES]["fc"], vocab_rows=VOCAB,
                                 workspace=lm_ws, out_idx=draft_log[c * M:(c + 1) * M], out_max=out_max,
                                 out=ys["fc"])

    nd = distinct_experts(nv, torch, xm, routers, copies[0]["moe"], moe_ws, M)
    gemv_b = sum(nvfp4_bytes(n, k) + M * n * 4 for name, n, k in PROJ) + M * 2 * (4096 + 2048 + 4096)
    lm_b = nvfp4_bytes(VOCAB, H) + M * H * 2 + M * 8
    emb_b = M * 4                          # the draft id the fc reads (its embedding row is in gemv_b)
    step_b = gemv_b + float(np.mean([moe_bytes(n, M) for n in nd])) + lm_b + emb_b

    s = env.s
    with torch.cuda.stream(s):
        for c in range(NCOPIES):       # warm the kernels before capture
            step(c)
        torch.cuda.synchronize()
        g_all = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_all, stream=s):
            for c in range(NCOPIES):
                step(c)
        singles = []
        for c in range(NCOPIES):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                step(c)
            singles.append(g)
    torch.cuda.synchronize()

    def run(k):
        for _ in range(k // NCOPIES):
            g_all.replay()
        for i in range(k % NCOPIES):
            singles[i].replay()

    with torch.cuda.stream(s):
        run(warmup)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        run(steps)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    nv.moe_workspace_status(moe_ws)      # raises if a down pass gave up its wait
    ms = (t1 - t0) * 1e3 / steps
    del g_all, singles
    return {"ms_per_step": ms, "step_bytes": step_b, "distinct_experts": nd, "hl": hl, "lm_ws": lm_ws,
            "out_idx": out_idx, "out_max": out_max}


# ------------------------------------------------------------- decode rows
def decode_rows(env, M, copies_moe, lm_pool, counters=False, reps_cap=None):
    """Per-launch device time of each decode kernel at M rows, every timed
    graph rotating over at least ROT_BYTES of distinct weights (the MoE over
    the expert copies, each launch with its own router logits).  With
    counters: each row's launches run once, eagerly, after a marker kernel
    (no timing) -- the input of the rocprofv3 counter passes."""
    nv, torch, dev = env.nv, env.torch, env.dev
    out, order = {}, []

    def measure(name, fn, reps, nbytes, **extra):
        if reps_cap:
            reps = min(reps, reps_cap)
        if counters:
            torch.cuda.synchronize()
            torch.cuda._sleep(1000)            # markers: a row's launches lie between two of these kernels
            for i in range(reps):
                fn(i)
            torch.cuda._sleep(1000)
            torch.cuda.synchronize()
            order.append({"row": name, "launches": reps, "bytes": nbytes})
            return
        extra["launches"] = reps
        out[name] = _row(_time_graph(torch, fn, reps, env.s), nbytes, **extra)

    sfx = "" if M == 1 else f"_m{M}"
    pools = {}
    for name, n, k in PROJ:
        if name in ("k", "v") and M != 1:
            continue
        b = nvfp4_bytes(n, k) + M * k * 2 + M * n * 4
        L = rot_copies(nvfp4_bytes(n, k))
        pool = quantized_pool(env, n, k, L)
        x = env.randn((M, k))
        y = torch.empty((M, n), dtype=torch.float32, device=dev)
        measure(f"gemv_{name}{sfx}", lambda i: nv.w4a16_gemv(x, pool[i % L], out=y), launches(L), b, copies=L)
        if name in ("q", "k", "v"):
            pools[name] = pool
        del pool
    if M == 1:
        qkv = [pools["q"], pools["k"], pools["v"]]
    else:
        nq = len(pools["q"])
        qkv = [pools["q"], quantized_pool(env, 512, 2048, nq), quantized_pool(env, 512, 2048, nq)]
    L = len(qkv[0])
    x = env.randn((M, 2048))
    yq = [torch.empty((M, n), dtype=torch.float32, device=dev) for n in (8192, 512, 512)]
    b = sum(nvfp4_bytes(n, 2048) + M * n * 4 for n in (8192, 512, 512)) + M * 2048 * 2
    measure(f"gemv_qkv_grouped{sfx}", lambda i: nv.w4a16_gemv_grouped(x, [p[i % L] for p in qkv], outs=yq),
            launches(L), b, copies=L)
    del qkv, pools
    torch.cuda.empty_cache()
    # LM head: the full vocabulary (and its log-probability variant) over the
    # head copies; the 32768-row head over its own pool
    hl = env.randn((M, H))
    oi = torch.empty(M, dtype=torch.int32, device=dev)
    om = torch.empty(M, dtype=torch.float32, device=dev)
    olp = torch.empty(M, dtype=torch.float32, device=dev)
    ws = nv.lmhead_workspace(M, VOCAB, dev)
    nl = len(lm_pool)
    b = nvfp4_bytes(VOCAB, H) + M * H * 2 + M * 8
    measure(f"lmhead_v{VOCAB}{sfx}", lambda i: nv.lmhead_gemv_argmax(hl, lm_pool[i % nl], workspace=ws, out_idx=oi,
                                                                     out_max=om), launches(nl), b,
            copies=nl, drafts_per_s=None)
    if M == 1:
        measure(f"lmhead_logprob_v{VOCAB}", lambda i: nv.lmhead_gemv_argmax_logprob(
            hl, lm_pool[i % nl], workspace=ws, out_idx=oi, out_max=om, out_logprob=olp), launches(nl), b + 4 * M,
            copies=nl, drafts_per_s=None)
    L = rot_copies(nvfp4_bytes(32768, H))
    small = quantized_pool(env, 32768, H, L)
    b = nvfp4_bytes(32768, H) + M * H * 2 + M * 8
    measure(f"lmhead_v32768{sfx}", lambda i: nv.lmhead_gemv_argmax(hl, small[i % L], workspace=ws, out_idx=oi,
                                                                   out_max=om), launches(L), b, copies=L,
            drafts_per_s=None)
    del small
    torch.cuda.empty_cache()
    # MoE: 64 launches, each its own router logits, over the expert copies
    nr = 64
    xm = env.randn((M, H))
    routers = [env.randn((M, E), dtype=torch.float32) for _ in range(nr)]
    mws = nv.moe_workspace(M, TOPK, copies_moe[0], dev)
    ym = torch.empty((M, H), dtype=torch.float32, device=dev)
    ids = torch.empty((M, TOPK), dtype=torch.int32, device=dev)
    wts = torch.empty((M, TOPK), dtype=torch.float32, device=dev)
    nc = len(copies_moe)
    nd = distinct_experts(nv, torch, xm, routers, copies_moe[0], mws, M)
    mb = float(np.mean([moe_bytes(n, M) for n in nd]))
    measure(f"moe{sfx}", lambda i: nv.moe_w4a16_gemv(xm, routers[i % nr], TOPK, copies_moe[i % nc], workspace=mws,
                                                     out=ym, topk_ids=ids, topk_w=wts), nr, mb,
            mean_distinct_experts=float(np.mean(nd)))
    nv.moe_workspace_status(mws)
    for name, r in out.items():
        if "drafts_per_s" in r:
            r["drafts_per_s"] = round(M / (r["ms"] * 1e-3), 1)
    return order if counters else out


def moe_layer_row(env, copies_moe):
    """The complete MoE layer: NVFP4 router + routed experts + gated shared expert."""
    nv, torch, dev = env.nv, env.torch, env.dev
    nc = len(copies_moe)
    lay = [(quantized_pool(env, E, H, 1)[0], *quantized_pool(env, I, H, 2), quantized_pool(env, H, I, 1)[0])
           for _ in range(nc)]
    sgw = env.randn(H, 0.02)
    xm = env.randn((1, H))
    lws = nv.moe_layer_workspace(1, TOPK, copies_moe[0], dev)
    ym = torch.empty((1, H), dtype=torch.float32, device=dev)
    ids = torch.empty((1, TOPK), dtype=torch.int32, device=dev)
    wts = torch.empty((1, TOPK), dtype=torch.float32, device=dev)
    rl = torch.empty((1, E), dtype=torch.float32, device=dev)
    ms = _time_graph(torch, lambda i: nv.moe_layer_w4a16(xm, lay[i % nc][0], TOPK, copies_moe[i % nc], *lay[i % nc][1:],
                                                         shared_gate_w=sgw, workspace=lws, out=ym, topk_ids=ids,
                                                         topk_w=wts, router_logits=rl), 2 * nc, env.s)
    extra = nvfp4_bytes(E, H) + 3 * nvfp4_bytes(I, H)
    return _row(ms, moe_bytes(8, 1) + extra + E * 4, extra_weight_bytes=extra)


def quantizer_row(env):
    nv, torch = env.nv, env.torch
    wq = env.randn((VOCAB, H), 0.02)
    qo = nv.nvfp4_quantize(wq)
    ms = _time(torch, lambda i: nv.nvfp4_quantize(wq, out=qo), 10, env.s)
    return _row(ms, 2 * VOCAB * H * 2 + nvfp4_bytes(VOCAB, H))


# prefill GEMM shapes: (name, N, K, M) -- prompt chunks of 128, 1024 and 8192
# rows through the fc, k/v and the dense-head FFN projections
GEMM_SHAPES = tuple((name, n, k, m) for name, n, k in (("fc", 2048, 4096), ("kv", 512, 2048), ("gate_up", 17408, 5120),
                                                      ("down", 5120, 17408)) for m in (128, 1024, 8192))


def gemm_rows(env, shapes):
    """Back-to-back launch time of w4a16_gemm_m128 (bf16 output) per shape."""
    nv, torch, dev = env.nv, env.torch, env.dev
    out = {}
    for name, n, k, m in shapes:
        w = nv.nvfp4_quantize(env.randn((n, k), 0.02))
        x = env.randn((m, k))
        y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        ws = nv.gemm_workspace(m, n, k, dev)
        ms = _time(torch, lambda i: nv.w4a16_gemm_m128(x, w, out=y, workspace=ws), 10, env.s)
        tf = 2.0 * m * n * k / (ms * 1e-3) / 1e12
        out[f"gemm_{name}_m{m}"] = {"ms": round(ms, 4), "tflops": round(tf, 1),
                                    "frac_mfma": round(tf / BF16_MFMA_PEAK_TFLOPS, 4)}
        del w, x, y
    return out


DS_H, DS_V, DS_I, DS_E = 7168, 129280, 2048, 256


def deepseek_rows(env, M):
    """DeepSeek-shaped head (hidden 7168, vocabulary 129280, 256 experts of
    width 2048, top-8): LM head + argmax (two copies, 1.04 GB), the routed
    MoE (each launch its own routing over 6.3 GB of experts) and a
    18432 x 7168 GEMV (over 1 GiB of copies), graph-timed like the other rows."""
    nv, torch, dev = env.nv, env.torch, env.dev
    out = {}
    lm = quantized_pool(env, DS_V, DS_H, 2)
    hl = env.randn((M, DS_H))
    ws = nv.lmhead_workspace(M, DS_V, dev)
    oi = torch.empty(M, dtype=torch.int32, device=dev)
    om = torch.empty(M, dtype=torch.float32, device=dev)
    ms = _time_graph(torch, lambda i: nv.lmhead_gemv_argmax(hl, lm[i % 2], workspace=ws, out_idx=oi, out_max=om),
                     MIN_LAUNCHES, env.s)
    out["lmhead_v129280_k7168"] = _row(ms, nvfp4_bytes(DS_V, DS_H) + M * DS_H * 2 + M * 8,
                                       drafts_per_s=round(M / (ms * 1e-3), 1))
    del lm
    torch.cuda.empty_cache()
    experts = expert_stack(env, DS_E, DS_H, DS_I)
    xm = env.randn((M, DS_H))
    routers = [env.randn((M, DS_E), dtype=torch.float32) for _ in range(MIN_LAUNCHES)]
    mws = nv.moe_workspace(M, TOPK, experts, dev)
    ym = torch.empty((M, DS_H), dtype=torch.float32, device=dev)
    ids = torch.empty((M, TOPK), dtype=torch.int32, device=dev)
    wts = torch.empty((M, TOPK), dtype=torch.float32, device=dev)
    nd = distinct_experts(nv, torch, xm, routers, experts, mws, M)
    ms = _time_graph(torch, lambda i: nv.moe_w4a16_gemv(xm, routers[i], TOPK, experts, workspace=mws, out=ym,
                                                        topk_ids=ids, topk_w=wts), MIN_LAUNCHES, env.s)
    nv.moe_workspace_status(mws)
    b = float(np.mean([moe_bytes(n, M, DS_H, DS_I, DS_E) for n in nd]))
    out["moe_256x2048x7168_top8"] = _row(ms, b, mean_distinct_experts=float(np.mean(nd)))
    del experts
    torch.cuda.empty_cache()
    L = rot_copies(nvfp4_bytes(18432, DS_H))
    gws = quantized_pool(env, 18432, DS_H, L)
    xg = env.randn((M, DS_H))
    yg = torch.empty((M, 18432), dtype=torch.float32, device=dev)
    ms = _time_graph(torch, lambda i: nv.w4a16_gemv(xg, gws[i % L], out=yg), launches(L), env.s)
    out["gemv_18432x7168"] = _row(ms, nvfp4_bytes(18432, DS_H) + M * DS_H * 2 + M * 18432 * 4, copies=L)
    del gws
    torch.cuda.empty_cache()
    return out


# ------------------------------------------------------- committed counters
def sources_sha256():
    h = hashlib.sha256()
    for f in SOURCES:
        with open(os.path.join(ROOT, "nvfp4_w4a16_mtp_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _profile_fields(path):
    fields = {}
    if os.path.exists(path):
        for line in open(path):
            if ":" in line and not line.startswith(("|", " ", "#", "-")):
                key, val = line.split(":", 1)
                fields[key.strip()] = val.strip()
    return fields


def counter_table():
    """The committed per-row counter figures, or {} when the kernel sources
    changed since the counter passes were taken."""
    f = _profile_fields(COUNTER_PROFILE)
    if f.get("source_sha256") != sources_sha256():
        return {}
    return json.loads(f.get("rows_json", "{}"))


def lmhead_traffic(lm_bytes):
    """HBM bytes per LM-head launch (M = 1): the counter passes' FETCH_SIZE +
    WRITE_SIZE ratio to the algorithmic bytes, or None."""
    ratio = counter_table().get(f"lmhead_v{VOCAB}", {}).get("traffic_ratio")
    return round(ratio * lm_bytes) if ratio else None


def attach_counters(rows):
    """Adds each row's counter figures (traffic ratio, VALUBusy, median
    launch time, clock) from the committed summary, if the kernel sources
    still match."""
    table = counter_table()
    for name, vals in table.items():
        if name in rows:
            rows[name]["counters"] = vals
    return bool(table)


def _csv_records(d):
    rows = []
    for path in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
                       + glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)):
        with open(path) as fh:
            rows += list(csv.DictReader(fh))
    return rows


def copy_calibration(fetch_dir, write_dir):
    """Bytes moved per counted KiB: the 1 GiB copy's dispatches (the kernel
    that runs 5 times) read 1 GiB and write 1 GiB."""
    out = {}
    for key, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        by_name = {}
        for r in _csv_records(d):
            if r.get("Counter_Name") == key:
                by_name.setdefault(r["Kernel_Name"], {}).setdefault(int(r["Dispatch_Id"]), 0.0)
                by_name[r["Kernel_Name"]][int(r["Dispatch_Id"])] += float(r["Counter_Value"])
        vals = next(list(v.values()) for v in by_name.values() if len(v) == 5)
        kib = statistics.median(vals)
        out[key] = {"kib_per_copy": kib, "factor": (1 << 30) / (kib * 1024)}
    return out


def summarize_counters(dirs, copy_dirs):
    """Markdown table of the --counters passes (rocprofv3 output dirs: any of
    FETCH_SIZE, WRITE_SIZE and VALUBusy passes and a kernel trace), rows
    split at the marker kernels, row order from
    gpurun_out/counters_order.json; byte counters scaled by the plain-copy
    calibration passes."""
    cal = copy_calibration(*copy_dirs)
    records = _csv_records
    def split(rows):
        """Library dispatches of each row, in dispatch order."""
        by_id = {}
        for r in rows:
            did = int(r["Dispatch_Id"])
            rec = by_id.setdefault(did, {"name": r["Kernel_Name"], "vals": {}, "start": r.get("Start_Timestamp"),
                                         "end": r.get("End_Timestamp")})
            if r.get("Counter_Name"):
                rec["vals"][r["Counter_Name"]] = rec["vals"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        seq, marks = {}, 0
        for did in sorted(by_id):
            rec = by_id[did]
            if "spin_kernel" in rec["name"]:
                marks += 1
            elif marks % 2 == 1 and "nvfp4::" in rec["name"]:     # inside row (marks - 1) / 2
                seq.setdefault(marks // 2, []).append(rec)
        return seq

    out_dir = os.path.join(ROOT, "gpurun_out")
    order = json.load(open(os.path.join(out_dir, "counters_order.json")))
    passes = [split(records(d)) for d in dirs]
    lines = [f"Calibration (plain 1 GiB copy): FETCH_SIZE {cal['FETCH_SIZE']['kib_per_copy']:.1f} KiB a copy "
             f"(factor {cal['FETCH_SIZE']['factor']:.4f}), WRITE_SIZE {cal['WRITE_SIZE']['kib_per_copy']:.1f} KiB "
             f"(factor {cal['WRITE_SIZE']['factor']:.4f}).", "",
             "| row | kernels | launches | dispatches | median us a launch | algorithmic bytes | FETCH+WRITE bytes "
             "(scaled) | ratio | GB/s (algorithmic) | VALUBusy % |", "|---|---|---|---|---|---|---|---|---|---|"]
    table = {}
    for i, o in enumerate(order):
        recs = [r for p in passes for r in p.get(i, [])]
        L = o["launches"]

        def per_launch(key):
            v = [r["vals"][key] for r in recs if key in r["vals"]]
            return sum(v) / L if v else None

        fetch, write = per_launch("FETCH_SIZE"), per_launch("WRITE_SIZE")
        valu = [r["vals"]["VALUBusy"] for r in recs if "VALUBusy" in r["vals"]]
        traced = [r for r in recs if not r["vals"] and r["start"] and r["end"]]
        n_disp = len(traced) // L if traced else None
        # launch time: the sum of one launch's dispatches (median of each position)
        med = None
        if traced and n_disp:
            med = sum(statistics.median((int(traced[j * n_disp + q]["end"]) - int(traced[j * n_disp + q]["start"]))
                                        / 1e3 for j in range(L)) for q in range(n_disp))
        traffic = fetch * 1024 * cal["FETCH_SIZE"]["factor"] + write * 1024 * cal["WRITE_SIZE"]["factor"] \
            if fetch is not None and write is not None else None
        ent = {"traffic_ratio": round(traffic / o["bytes"], 4) if traffic else None,
               "valu_busy_pct": round(statistics.median(valu), 1) if valu else None,
               "median_us": round(med, 2) if med else None,
               "gbs": round(o["bytes"] / (med * 1e-6) / 1e9, 1) if med else None}
        table[o["row"]] = ent
        names = sorted({r["name"].split("(")[0].replace("void ", "") for r in recs})
        lines.append(f"| {o['row']} | {'<br>'.join('`' + n + '`' for n in names)} | {L} | {n_disp} | "
                     f"{ent['median_us']} | {round(o['bytes'])} | {round(traffic) if traffic else None} | "
                     f"{ent['traffic_ratio']} | {ent['gbs']} | {ent['valu_busy_pct']} |")
    lines += ["", f"source_sha256: {sources_sha256()}", f"rows_json: {json.dumps(table)}"]
    return "\n".join(lines)


# ------------------------------------------------------------ CPU baseline
def cpu_baseline(step_bytes_m1):
    """The CPU oracle (plain C, fp64 accumulation, loops over independent
    outputs on OpenMP threads) timed on bounded samples of the workload's
    rows: median of 5 runs after one warm-up, at one thread and at every
    core the process may use."""
    import oracle
    from tests import synth
    cores = len(os.sched_getaffinity(0))
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    rng = np.random.default_rng(0)
    W = {name: synth.quantized_domain_weight(rng, n, k) for name, n, k in PROJ}
    lm = synth.quantized_domain_weight(rng, VOCAB, H)
    ex = synth.moe_quantized_experts(0, 16, H, I)          # the routed subset is what the oracle reads
    x1 = {name: synth.acts_bf16(1, 1, k) for name, n, k in PROJ}
    x8 = synth.acts_bf16(2, 8, 2048)
    xm = synth.acts_bf16(3, 8, H)
    r = synth.router_logits(3, 8, 16)
    xg = synth.acts_bf16(4, 128, 4096)

    def step():
        for name, n, k in PROJ:
            oracle.gemv(x1[name], *W[name])
        oracle.moe(xm[:1], r[:1], TOPK, *ex)
        oracle.lmhead_argmax(x1["q"], *lm)

    cases = [
        ("draft_step_m1", step, step_bytes_m1),
        ("lmhead_v151936_m1", lambda: oracle.lmhead_argmax(x1["q"], *lm), nvfp4_bytes(VOCAB, H)),
        ("gemv_q_m8", lambda: oracle.gemv(x8, *W["q"]), nvfp4_bytes(8192, 2048)),
        ("moe_m8_16_experts", lambda: oracle.moe(xm, r, TOPK, *ex), 16 * 3 * nvfp4_bytes(I, H)),
        ("gemm_fc_m128", lambda: oracle.gemv(xg, *W["fc"]), None),
    ]
    n0 = oracle.get_threads()
    res = {}
    t_all0 = time.perf_counter()
    for threads in (1, cores):
        oracle.set_threads(threads)
        for name, fn, nbytes in cases:
            fn()
            ts = []
            for _ in range(5):
                t0 = time.perf_counter()
                fn()
                ts.append(time.perf_counter() - t0)
            med = statistics.median(ts)
            e = res.setdefault(name, {})
            e[f"ms_{threads}t"] = round(med * 1e3, 2)
            if nbytes:
                e[f"gbs_{threads}t"] = round(nbytes / med / 1e9, 3)
            if name == "gemm_fc_m128":
                e[f"tflops_{threads}t"] = round(2 * 128 * 2048 * 4096 / med / 1e12, 4)
    oracle.set_threads(n0)
    step_ms = res["draft_step_m1"][f"ms_{cores}t"]
    return {"value": round(step_bytes_m1 / (step_ms * 1e-3) / 1e9, 3), "unit": "GB/s", "cores": cores,
            "kind": "oracle", "cpu_model": model,
            "sample": "whole draft step at M=1 (5 GEMVs, MoE over 8 of 16 synthetic experts standing in for the "
                      "routed 8 of 256, LM head 151936x2048) on synthetic NVFP4 weights; value at every core, "
                      f"median of 5 runs after one warm-up; rows at 1 thread and {cores} threads",
            "single_thread_value": round(step_bytes_m1 / (res["draft_step_m1"]["ms_1t"] * 1e-3) / 1e9, 3),
            "rows": res, "seconds": round(time.perf_counter() - t_all0, 1)}


# ------------------------------------------------------------------- main
def moe_timeline(env, launches=40, skip=5):
    """Phase timestamps of the one-token MoE (bench shapes: 256 experts,
    top-8, 2048 x 1024): each launch starts on an idle GPU, after a spin
    kernel that covers the host's queueing; per launch, each event's
    [min, median, max] over the workgroups in microseconds from the first
    workgroup's start; then the median of each over the launches after
    `skip` warm-up ones."""
    nv, torch = env.nv, env.torch
    experts = [expert_stack(env) for _ in range(3)]
    x = env.randn((1, H))
    routers = [env.randn((1, E), dtype=torch.float32) for _ in range(launches)]
    ws = nv.moe_workspace(1, TOPK, experts[0], env.dev)
    y = torch.empty((1, H), dtype=torch.float32, device=env.dev)
    ev, groups = nv.moe_trace_events(TOPK, experts[0])
    gate_up = (I + 15) // 16 * TOPK
    trace = torch.zeros((ev, groups), dtype=torch.int64, device=env.dev)
    names = {"gate_up": ("start", "routed", "stored", "counted"),
             "down": ("start", "weights_issued", "go_seen", "staged", "sums_done", "written")}
    per = []
    for i in range(launches):
        torch.cuda._sleep(100000)
        nv.moe_w4a16_gemv(x, routers[i], TOPK, experts[i % 3], workspace=ws, out=y, trace=trace)
        torch.cuda.synchronize()
        if i < skip:
            continue
        t = trace.cpu().numpy().astype(np.int64)
        t0 = t[0].min()
        row = {}
        for role, cols in (("gate_up", t[:, :gate_up]), ("down", t[:, gate_up:])):
            for e, name in enumerate(names[role]):
                v = (cols[e] - t0) / 100.0   # 100 MHz ticks -> us
                row[f"{role}.{name}"] = [float(v.min()), float(np.median(v)), float(v.max())]
        per.append(row)
    nv.moe_workspace_status(ws)
    return {k: [round(float(np.median([r[k][j] for r in per])), 2) for j in range(3)] for k in per[0]}


def main():
    a = parse()
    if a.summarize_counters:
        print(summarize_counters(a.summarize_counters, a.copy_dirs))
        return
    if a.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {a.gpus} is not supported: the library's kernels run on a "
              "single MI355X", file=sys.stderr)
        sys.exit(2)
    import torch
    torch.cuda.set_device(0)
    if a.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": 1 << 30, "launches": 5}))
        return
    import nvfp4_w4a16_mtp_amd as nv
    nv.lib()
    env = Env(nv, torch)
    if a.gemm_only:
        print(json.dumps({"prefill_gemm": gemm_rows(env, GEMM_SHAPES)}), flush=True)
        return
    if a.moe_timeline:
        print(json.dumps({"moe_timeline_us": moe_timeline(env)}), flush=True)
        return

    # ---------------- weights: NCOPIES copies of the step, quantized on the GPU
    t0 = time.perf_counter()
    copies = []
    for c in range(NCOPIES):
        ws = {name: quantized_pool(env, n, k, 1)[0] for name, n, k in PROJ}
        ws["moe"] = expert_stack(env)
        copies.append(ws)
    lm_pool = quantized_pool(env, VOCAB, H, rot_copies(nvfp4_bytes(VOCAB, H)))   # 7 heads, 1.2 GB
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t0
    moe_copies = [c["moe"] for c in copies]

    if a.counters:
        order = []
        for M in (1, 4, 8):
            order += decode_rows(env, M, moe_copies, lm_pool, counters=True, reps_cap=96)
        os.makedirs(os.path.join(ROOT, "gpurun_out"), exist_ok=True)
        with open(os.path.join(ROOT, "gpurun_out", "counters_order.json"), "w") as fh:
            json.dump(order, fh)
        print(json.dumps({"counters_rows": order}), flush=True)
        return

    embed_table = env.randn((VOCAB, H))
    steps = {M: draft_step(env, copies, lm_pool, embed_table, M, a.steps, a.warmup) for M in (1, 4, 8)}
    r1 = steps[1]
    # the dominant kernel: LM-head GEMV + argmax at M = 1, launched back to
    # back over the head copies, timed with events on its own stream
    nl = len(lm_pool)
    lm_ms = _time(torch, lambda i: nv.lmhead_gemv_argmax(r1["hl"], lm_pool[i % nl], vocab_rows=VOCAB,
                                                         workspace=r1["lm_ws"], out_idx=r1["out_idx"],
                                                         out_max=r1["out_max"]), max(a.steps, 5 * nl), env.s)
    lm_bytes = nvfp4_bytes(VOCAB, H) + H * 2 + 8
    lm_gbs = lm_bytes / (lm_ms * 1e-3) / 1e9
    lm_traffic = lmhead_traffic(lm_bytes)
    ms_per_step = r1["ms_per_step"]
    value = r1["step_bytes"] / (ms_per_step * 1e-3) / 1e9
    rot_b = NCOPIES * (sum(nvfp4_bytes(n, k) for _, n, k in PROJ) + 3 * E * nvfp4_bytes(I, H)) \
        + nl * nvfp4_bytes(VOCAB, H)

    result = {
        "metric": "W4A16 GEMV achieved HBM GB/s (% peak) + MTP drafts/sec (LM-head GEMV+argmax)",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "nvfp4 weights x bf16 activations, fp32 accumulate",
        "data": "synthetic (seeded normal bf16 weights quantized on the GPU, normal activations and router logits)",
        "config": {"workload": "qwen_mtp_draft_step", "m_rows": 1, "hidden": H,
                   "proj": {n: [r_, c_] for n, r_, c_ in PROJ}, "moe": {"experts": E, "top_k": TOPK, "inter": I},
                   "lm_head": [VOCAB, H], "weight_copies_rotated": NCOPIES, "weight_bytes_allocated": int(rot_b),
                   "graph": f"{NCOPIES} steps per graph, each its own weight copy and router logits",
                   "chained": "the LM head call runs the next step's fc over the embedding row of its draft id"},
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "step_bytes": round(r1["step_bytes"]),
        "drafts_per_s": round(1 / (lm_ms * 1e-3), 1),
        "step_drafts_per_s": round(1 / (ms_per_step * 1e-3), 1),
        "steps_by_m": {str(M): {"ms_per_step": round(r["ms_per_step"], 5), "step_bytes": round(r["step_bytes"]),
                                "gbs": round(r["step_bytes"] / (r["ms_per_step"] * 1e-3) / 1e9, 1),
                                "frac": round(r["step_bytes"] / (r["ms_per_step"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                "step_drafts_per_s": round(M / (r["ms_per_step"] * 1e-3), 1),
                                "distinct_experts": r["distinct_experts"]} for M, r in steps.items()},
        "roofline": {"kernel": "lmhead_gemv_argmax (151936 x 2048 NVFP4, M = 1)", "bound": "hbm",
                     "achieved": round(lm_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(lm_gbs / HBM_PEAK_GBS, 4),
                     "traffic": (round(lm_traffic / (lm_ms * 1e-3) / 1e9, 1) if lm_traffic else None),
                     "bytes_per_launch": lm_bytes, "traffic_bytes_per_launch": lm_traffic,
                     "avg_launch_ms": round(lm_ms, 5)},
        "setup_s": round(setup_s, 2),
    }
    del steps
    torch.cuda.empty_cache()
    if not a.no_rows:
        rows = {}
        for M in (1, 4, 8):
            rows.update(decode_rows(env, M, moe_copies, lm_pool))
        rows["moe_layer_router_shared"] = moe_layer_row(env, moe_copies)
        del copies, moe_copies, lm_pool
        torch.cuda.empty_cache()
        rows["quantize_151936x2048"] = quantizer_row(env)
        rows.update(gemm_rows(env, (("fc", 2048, 4096, 1024), ("gate_up", 17408, 5120, 1024),
                                    ("down", 5120, 17408, 1024), ("gate_up", 17408, 5120, 8192))))
        result["counters_attached"] = attach_counters(rows)
        result["rows"] = rows
        result["rows_deepseek_shaped"] = deepseek_rows(env, 1)
    if not a.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(r1["step_bytes"])
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
