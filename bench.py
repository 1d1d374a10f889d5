"""Benchmark of the NVFP4 W4A16 MTP draft-head hot path on one MI355X.

A step is one draft step of a Qwen-shaped MTP head at M decode rows: the
fc / q|k|v (grouped) / o W4A16 GEMVs, the routed MoE FFN (256 NVFP4
experts, top-8) and the full-vocabulary (151936 x 2048) NVFP4 LM head fused
with argmax, whose last workgroup gathers the draft token's embedding into
the next step's fc input (device-resident chaining).  The step is captured once per weight copy in a HIP graph and the
graphs are replayed in rotation over three independent copies of every
weight (~1.5 GB in total, several times the 256 MB Infinity Cache), so the
weights stream from HBM as they would in serving.  All inputs are seeded
synthetic data resident in HBM before the timed region.

Printed: one JSON line.  `value` = algorithmic HBM bytes of the step (NVFP4
codes + scales + globals actually read, activations in, results out) per
second.  Extra fields: drafts/s of the LM head, a roofline object for the
dominant kernel (the LM-head GEMV+argmax, timed with HIP events on the
stream it runs on), per-row measurements (quantizer, each GEMV, MoE, LM
head, the prefill GEMM) and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
H, I, E, TOPK, VOCAB = 2048, 1024, 256, 8, 151936
PROJ = [("fc", 2048, 4096), ("q", 8192, 2048), ("k", 512, 2048), ("v", 512, 2048), ("o", 2048, 4096)]
NCOPIES = 3


def nvfp4_bytes(n, k):
    return n * k // 2 + n * k // 16 + 16


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--m", type=int, default=1, help="decode rows per step (1..8)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-rows", action="store_true", help="skip the per-row measurements")
    p.add_argument("--gemm-only", action="store_true",
                   help="only time the prefill GEMM at every prompt-chunk shape (one JSON line)")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run a plain 1 GiB device copy (PMC byte-counter calibration)")
    return p.parse_args()


def main():
    a = parse()
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
    if a.gemm_only:
        s = torch.cuda.Stream()
        print(json.dumps({"prefill_gemm": gemm_rows(nv, torch, torch.device("cuda:0"), s, GEMM_SHAPES)}), flush=True)
        return
    M = a.m
    assert 1 <= M <= 8
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)

    def randn_bf16(shape, std):
        return (torch.randn(shape, generator=gen, device=dev, dtype=torch.float32) * std).to(torch.bfloat16)

    # ---------------- weights: NCOPIES copies, quantized on the GPU ----------------
    qev0, qev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    quant_bytes = 0
    quant_ms = 0.0
    copies = []
    for c in range(NCOPIES):
        ws = {}
        for name, n, k in PROJ + [("lm", VOCAB, H)]:
            w = randn_bf16((n, k), 0.02)
            qev0.record()
            ws[name] = nv.nvfp4_quantize(w)
            qev1.record()
            torch.cuda.synchronize()
            quant_ms += qev0.elapsed_time(qev1)
            quant_bytes += 2 * (n * k * 2) + nvfp4_bytes(n, k)
            del w
        # experts: stacked [E, rows, cols]; each matrix quantized with its own global scale
        ex = {}
        for proj, rows, cols in (("gate", I, H), ("up", I, H), ("down", H, I)):
            codes = torch.empty((E, rows, cols // 2), dtype=torch.uint8, device=dev)
            scales = torch.empty((E, rows, cols // 16), dtype=torch.uint8, device=dev)
            glob = torch.empty((E, 4), dtype=torch.float32, device=dev)
            for e in range(E):
                w = randn_bf16((rows, cols), 0.02)
                nv.nvfp4_quantize(w, out=nv.NVFP4Weight(codes[e], scales[e], glob[e], rows, cols))
            ex[proj] = (codes, scales, glob)
        ws["moe"] = nv.NVFP4Experts(*ex["gate"], *ex["up"], *ex["down"])
        copies.append(ws)
    torch.cuda.synchronize()

    # ---------------- activations and outputs (resident) ----------------
    xs = {name: randn_bf16((M, k), 1.0) for name, n, k in PROJ}
    xm = randn_bf16((M, H), 1.0)
    router = torch.randn((M, E), generator=gen, device=dev, dtype=torch.float32)
    hl = randn_bf16((M, H), 1.0)
    ys = {name: torch.empty((M, n), dtype=torch.float32, device=dev) for name, n, k in PROJ}
    ymoe = torch.empty((M, H), dtype=torch.float32, device=dev)
    ids = torch.empty((M, TOPK), dtype=torch.int32, device=dev)
    wts = torch.empty((M, TOPK), dtype=torch.float32, device=dev)
    moe_ws = nv.moe_workspace(M, TOPK, copies[0]["moe"], dev)
    lm_ws = nv.lmhead_workspace(M, VOCAB, dev)
    out_idx = torch.empty(M, dtype=torch.int32, device=dev)
    out_max = torch.empty(M, dtype=torch.float32, device=dev)

    # device-resident chaining: the LM head of each step gathers the embedding
    # of its draft token into the first half of the next step's fc input and
    # logs the id on the device (no host round trip between draft steps)
    embed_table = randn_bf16((VOCAB, H), 1.0)
    draft_log = torch.zeros(NCOPIES * M, dtype=torch.int32, device=dev)
    out_idx.zero_()

    def step(ws, slot=0):
        # fc, then q|k|v in one grouped launch (they share the normed hidden
        # state), then o
        nv.w4a16_gemv(xs["fc"], ws["fc"], out=ys["fc"])
        nv.w4a16_gemv_grouped(xs["q"], [ws["q"], ws["k"], ws["v"]], outs=[ys["q"], ys["k"], ys["v"]])
        nv.w4a16_gemv(xs["o"], ws["o"], out=ys["o"])
        nv.moe_w4a16_gemv(xm, router, TOPK, ws["moe"], workspace=moe_ws, out=ymoe, topk_ids=ids, topk_w=wts)
        # LM head + argmax; its last workgroup gathers the draft token's
        # embedding into the next step's fc input and logs the id
        nv.lmhead_gemv_argmax_embed(hl, ws["lm"], embed_table, xs["fc"][:, :H], vocab_rows=VOCAB,
                                    id_log=draft_log[slot * M:(slot + 1) * M], workspace=lm_ws, out_idx=out_idx,
                                    out_max=out_max)

    # distinct experts hit by the routing (same router logits every step)
    step(copies[0])
    torch.cuda.synchronize()
    n_distinct = len(set(ids.cpu().numpy().ravel().tolist()))
    moe_bytes = n_distinct * 3 * nvfp4_bytes(I, H) + M * H * 2 + M * E * 4 + M * H * 4 + 2 * M * TOPK * 4
    # q, k and v read one activation block (grouped launch)
    gemv_bytes = sum(nvfp4_bytes(n, k) + M * n * 4 for name, n, k in PROJ) + M * 2 * (4096 + 2048 + 4096)
    lm_bytes = nvfp4_bytes(VOCAB, H) + M * H * 2 + M * 8
    embed_bytes = M * (4 + 2 * H * 2)          # draft id in, embedding row read and written
    step_bytes = gemv_bytes + moe_bytes + lm_bytes + embed_bytes

    # ---------------- capture one graph per copy; LM head bracketed by events ----------------
    s = torch.cuda.Stream()
    # One graph holds NCOPIES consecutive draft steps (one per weight copy),
    # as a multi-draft propose loop would; single-step graphs cover a
    # remainder so that exactly `steps` steps are timed.
    graphs = []
    with torch.cuda.stream(s):
        for c in range(NCOPIES):      # warm the kernels before capture
            step(copies[c], c)
        torch.cuda.synchronize()
        g_all = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_all, stream=s):
            for c in range(NCOPIES):
                step(copies[c], c)
        for c in range(NCOPIES):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                step(copies[c], c)
            graphs.append(g)
    torch.cuda.synchronize()

    def run_steps(k):
        for _ in range(k // NCOPIES):
            g_all.replay()
        for i in range(k % NCOPIES):
            graphs[i].replay()

    # The LM-head launch duration is timed with HIP events on stream s over
    # back-to-back launches that rotate over the weight copies, after the
    # timed region (an event pair around every single launch would add its
    # own gaps to the figure).
    with torch.cuda.stream(s):
        run_steps(a.warmup)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        run_steps(a.steps)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    lm_ms = _time(torch, lambda i: nv.lmhead_gemv_argmax(hl, copies[i % NCOPIES]["lm"], vocab_rows=VOCAB, workspace=lm_ws,
                                                         out_idx=out_idx, out_max=out_max), max(a.steps, 30), s)
    ms_per_step = (t1 - t0) * 1e3 / a.steps
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    lm_gbs = lm_bytes / (lm_ms * 1e-3) / 1e9
    lm_traffic = lmhead_traffic(M)

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
        "data": "synthetic (seeded normal bf16 weights quantized on the GPU, normal activations)",
        "config": {"workload": "qwen_mtp_draft_step", "m_rows": M, "hidden": H, "proj": {n: [r, c] for n, r, c in PROJ},
                   "moe": {"experts": E, "top_k": TOPK, "inter": I, "distinct_experts": n_distinct},
                   "lm_head": [VOCAB, H], "weight_copies_rotated": NCOPIES, "graph": f"{NCOPIES} steps per graph",
                   "chained": "the LM head gathers the draft token's embedding into the next step's fc input"},
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "step_bytes": step_bytes,
        "drafts_per_s": round(M / (lm_ms * 1e-3), 1),
        "step_drafts_per_s": round(M / (ms_per_step * 1e-3), 1),
        "roofline": {"kernel": "lmhead_gemv_argmax (151936 x 2048 NVFP4)", "bound": "hbm", "achieved": round(lm_gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(lm_gbs / HBM_PEAK_GBS, 4),
                     "traffic": (round(lm_traffic / (lm_ms * 1e-3) / 1e9, 1) if lm_traffic else None),
                     "bytes_per_launch": lm_bytes, "traffic_bytes_per_launch": lm_traffic, "avg_launch_ms": round(lm_ms, 5)},
        "load_time_quantizer": {"bytes": quant_bytes, "ms": round(quant_ms, 3),
                                "gbs": round(quant_bytes / (quant_ms * 1e-3) / 1e9, 1)},
    }
    if not a.no_rows:
        result["rows"] = rows_measure(nv, torch, copies, xs, ys, xm, router, hl, M, s)
        del copies
        torch.cuda.empty_cache()
        result["rows_deepseek_shaped"] = deepseek_rows(nv, torch, M, s)
    if not a.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(M, step_bytes, n_distinct)
    print(json.dumps(result), flush=True)


def lmhead_traffic(M):
    """HBM bytes per LM-head launch from the committed FETCH_SIZE / WRITE_SIZE
    counter passes (scaled by the plain-copy calibration), or None when the
    kernel sources have changed since those counters were taken or M differs."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "lmhead_v151936_m1_traffic.md")
    if M != 1 or not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith(("|", " ", "#")):
            key, val = line.split(":", 1)
            fields[key.strip()] = val.strip()
    h = hashlib.sha256()
    for f in ("gemv.hip", "gemv_core.hpp", "common.hpp"):
        with open(os.path.join(ROOT, "nvfp4_w4a16_mtp_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if fields.get("source_sha256") != h.hexdigest() or "traffic_bytes_per_launch" not in fields:
        return None
    return int(fields["traffic_bytes_per_launch"])


def _time(torch, fn, reps, stream):
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        fn(0)
        torch.cuda.synchronize()
        e0.record()
        for i in range(reps):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def _time_graph(torch, fn, reps, stream):
    """Per-launch device time of fn: `reps` launches (rotating weight copies)
    captured in one HIP graph, replayed 3 times between two events.  Host
    launch overhead is excluded; the kernel boundaries inside the graph are
    included, as in a captured draft step."""
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
        e0.record()
        for _ in range(3):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (3 * reps)


def randn_like_rows(torch, m, k, dev):
    """Seeded N(0, 1) activations [m, k] in bf16."""
    g = torch.Generator(device=dev)
    g.manual_seed(1000 + m * 7 + k)
    return torch.randn((m, k), generator=g, device=dev).to(torch.bfloat16)


def rows_measure(nv, torch, copies, xs, ys, xm, router, hl, M, s):
    """Per-row device timings (graph-captured launches over rotating weight
    copies), each with its roofline fraction."""
    out = {}
    reps = 30
    for name, n, k in PROJ:
        ms = _time_graph(torch, lambda i: nv.w4a16_gemv(xs[name], copies[i % NCOPIES][name], out=ys[name]), reps, s)
        b = nvfp4_bytes(n, k) + M * k * 2 + M * n * 4
        out[f"gemv_{name}"] = {"ms": round(ms, 5), "gbs": round(b / ms / 1e6, 1), "frac": round(b / ms / 1e6 / HBM_PEAK_GBS, 4)}
    ms = _time_graph(torch, lambda i: nv.w4a16_gemv_grouped(xs["q"], [copies[i % NCOPIES][nm] for nm in "qkv"],
                                                            outs=[ys[nm] for nm in "qkv"]), reps, s)
    b = sum(nvfp4_bytes(n, k) + M * n * 4 for name, n, k in PROJ if name in "qkv") + M * 2048 * 2
    out["gemv_qkv_grouped"] = {"ms": round(ms, 5), "gbs": round(b / ms / 1e6, 1), "frac": round(b / ms / 1e6 / HBM_PEAK_GBS, 4)}
    # LM head at both vocabulary sizes of the workload
    for v in (32768, VOCAB):
        ws = nv.lmhead_workspace(M, v, hl.device)
        oi = torch.empty(M, dtype=torch.int32, device=hl.device)
        om = torch.empty(M, dtype=torch.float32, device=hl.device)
        ms = _time_graph(torch, lambda i: nv.lmhead_gemv_argmax(hl, copies[i % NCOPIES]["lm"], vocab_rows=v, workspace=ws,
                                                                out_idx=oi, out_max=om), reps, s)
        b = nvfp4_bytes(v, H) + M * H * 2 + M * 8
        out[f"lmhead_v{v}"] = {"ms": round(ms, 5), "gbs": round(b / ms / 1e6, 1), "frac": round(b / ms / 1e6 / HBM_PEAK_GBS, 4),
                               "drafts_per_s": round(M / (ms * 1e-3), 1)}
    # the same head with the top-1 log-probability (online log-sum-exp in the same pass)
    ws = nv.lmhead_workspace(M, VOCAB, hl.device)
    oi = torch.empty(M, dtype=torch.int32, device=hl.device)
    om = torch.empty(M, dtype=torch.float32, device=hl.device)
    olp = torch.empty(M, dtype=torch.float32, device=hl.device)
    ms = _time_graph(torch, lambda i: nv.lmhead_gemv_argmax_logprob(hl, copies[i % NCOPIES]["lm"], vocab_rows=VOCAB,
                                                                    workspace=ws, out_idx=oi, out_max=om,
                                                                    out_logprob=olp), reps, s)
    b = nvfp4_bytes(VOCAB, H) + M * H * 2 + M * 12
    out[f"lmhead_logprob_v{VOCAB}"] = {"ms": round(ms, 5), "gbs": round(b / ms / 1e6, 1),
                                       "frac": round(b / ms / 1e6 / HBM_PEAK_GBS, 4), "drafts_per_s": round(M / (ms * 1e-3), 1)}
    ws = nv.moe_workspace(M, TOPK, copies[0]["moe"], hl.device)
    ymo = torch.empty((M, H), dtype=torch.float32, device=hl.device)
    ids = torch.empty((M, TOPK), dtype=torch.int32, device=hl.device)
    wts = torch.empty((M, TOPK), dtype=torch.float32, device=hl.device)
    ms = _time_graph(torch, lambda i: nv.moe_w4a16_gemv(xm, router, TOPK, copies[i % NCOPIES]["moe"], workspace=ws, out=ymo,
                                                        topk_ids=ids, topk_w=wts), reps, s)
    nd = len(set(ids.cpu().numpy().ravel().tolist()))   # distinct routed experts
    mb = nd * 3 * nvfp4_bytes(I, H) + M * H * 2 + M * E * 4 + M * H * 4 + 2 * M * TOPK * 4
    out["moe"] = {"ms": round(ms, 5), "gbs": round(mb / ms / 1e6, 1), "frac": round(mb / ms / 1e6 / HBM_PEAK_GBS, 4),
                  "distinct_experts": nd}
    # the complete MoE layer: NVFP4 router + routed experts + gated shared expert
    gen2 = torch.Generator(device=hl.device)
    gen2.manual_seed(2)

    def qw(n, k):
        return nv.nvfp4_quantize((torch.randn((n, k), generator=gen2, device=hl.device) * 0.02).to(torch.bfloat16))
    lay = [(qw(E, H), qw(I, H), qw(I, H), qw(H, I)) for _ in range(NCOPIES)]
    sgw = (torch.randn(H, generator=gen2, device=hl.device) * 0.02).to(torch.bfloat16)
    lws = nv.moe_layer_workspace(M, TOPK, copies[0]["moe"], hl.device)
    rl = torch.empty((M, E), dtype=torch.float32, device=hl.device)
    ms = _time_graph(torch, lambda i: nv.moe_layer_w4a16(xm, lay[i % NCOPIES][0], TOPK, copies[i % NCOPIES]["moe"],
                                                         *lay[i % NCOPIES][1:], shared_gate_w=sgw, workspace=lws,
                                                         out=ymo, topk_ids=ids, topk_w=wts, router_logits=rl), reps, s)
    nvfp4_lay = nvfp4_bytes(E, H) + 3 * nvfp4_bytes(I, H)
    lb = mb + nvfp4_lay + M * E * 4
    out["moe_layer_router_shared"] = {"ms": round(ms, 5), "extra_weight_bytes": nvfp4_lay,
                                      "gbs": round(lb / ms / 1e6, 1), "frac": round(lb / ms / 1e6 / HBM_PEAK_GBS, 4)}
    del lay
    # the decode rows of the workload at several tokens (M = 4, 8): the q
    # projection, the LM head and the MoE (rotating weight copies, graph-timed)
    if M == 1:
        rows_m = {}
        for mm in (4, 8):
            xq = randn_like_rows(torch, mm, 2048, hl.device)
            yq = torch.empty((mm, 8192), dtype=torch.float32, device=hl.device)
            ms = _time_graph(torch, lambda i: nv.w4a16_gemv(xq, copies[i % NCOPIES]["q"], out=yq), reps, s)
            b = nvfp4_bytes(8192, 2048) + mm * 2048 * 2 + mm * 8192 * 4
            rows_m[f"gemv_q_m{mm}"] = {"ms": round(ms, 5), "gbs": round(b / ms / 1e6, 1),
                                       "frac": round(b / ms / 1e6 / HBM_PEAK_GBS, 4)}
            wsm = nv.lmhead_workspace(mm, VOCAB, hl.device)
            oim = torch.empty(mm, dtype=torch.int32, device=hl.device)
            omm = torch.empty(mm, dtype=torch.float32, device=hl.device)
            hm = randn_like_rows(torch, mm, H, hl.device)
            ms = _time_graph(torch, lambda i: nv.lmhead_gemv_argmax(hm, copies[i % NCOPIES]["lm"], vocab_rows=VOCAB,
                                                                    workspace=wsm, out_idx=oim, out_max=omm), reps, s)
            b = nvfp4_bytes(VOCAB, H) + mm * H * 2 + mm * 8
            rows_m[f"lmhead_v{VOCAB}_m{mm}"] = {"ms": round(ms, 5), "gbs": round(b / ms / 1e6, 1),
                                                "frac": round(b / ms / 1e6 / HBM_PEAK_GBS, 4),
                                                "drafts_per_s": round(mm / (ms * 1e-3), 1)}
            xmm = randn_like_rows(torch, mm, H, hl.device)
            rm = torch.randn((mm, E), generator=torch.Generator(device=hl.device).manual_seed(10 + mm), device=hl.device)
            wsq = nv.moe_workspace(mm, TOPK, copies[0]["moe"], hl.device)
            ymm = torch.empty((mm, H), dtype=torch.float32, device=hl.device)
            idm = torch.empty((mm, TOPK), dtype=torch.int32, device=hl.device)
            wtm = torch.empty((mm, TOPK), dtype=torch.float32, device=hl.device)
            ms = _time_graph(torch, lambda i: nv.moe_w4a16_gemv(xmm, rm, TOPK, copies[i % NCOPIES]["moe"], workspace=wsq,
                                                                out=ymm, topk_ids=idm, topk_w=wtm), reps, s)
            ndm = len(set(idm.cpu().numpy().ravel().tolist()))
            b = ndm * 3 * nvfp4_bytes(I, H) + mm * H * 2 + mm * E * 4 + mm * H * 4 + 2 * mm * TOPK * 4
            rows_m[f"moe_m{mm}"] = {"ms": round(ms, 5), "gbs": round(b / ms / 1e6, 1),
                                    "frac": round(b / ms / 1e6 / HBM_PEAK_GBS, 4), "distinct_experts": ndm}
        out["rows_m4_m8"] = rows_m
    # quantizer on the largest matrix (the LM head): clear, absmax and encode
    # launches back to back; bytes = 2 reads of the bf16 tensor + the NVFP4 write
    wq = (torch.randn((VOCAB, H), generator=gen2, device=hl.device) * 0.02).to(torch.bfloat16)
    qo = nv.nvfp4_quantize(wq)
    ms = _time(torch, lambda i: nv.nvfp4_quantize(wq, out=qo), 10, s)
    qb = 2 * VOCAB * H * 2 + nvfp4_bytes(VOCAB, H)
    out["quantize_151936x2048"] = {"ms": round(ms, 4), "gbs": round(qb / ms / 1e6, 1),
                                   "frac": round(qb / ms / 1e6 / HBM_PEAK_GBS, 4)}
    del wq, qo
    # prefill GEMM: fc (2048 x 4096) and the dense-FFN gate/up (17408 x 5120)
    out.update(gemm_rows(nv, torch, hl.device, s, (("fc", 2048, 4096, 1024), ("gate_up", 17408, 5120, 1024),
                                                   ("gate_up", 17408, 5120, 8192))))
    return out


# prefill GEMM shapes: (name, N, K, M) -- prompt chunks of 128, 1024 and 8192
# rows through the fc, k/v and the dense-head FFN projections
GEMM_SHAPES = tuple((name, n, k, m) for name, n, k in (("fc", 2048, 4096), ("kv", 512, 2048), ("gate_up", 17408, 5120),
                                                      ("down", 5120, 17408)) for m in (128, 1024, 8192))


def gemm_rows(nv, torch, dev, s, shapes):
    """Back-to-back launch time of w4a16_gemm_m128 (bf16 output) per shape."""
    out = {}
    gen = torch.Generator(device=dev)
    gen.manual_seed(1)
    for name, n, k, m in shapes:
        w = nv.nvfp4_quantize((torch.randn((n, k), generator=gen, device=dev) * 0.02).to(torch.bfloat16))
        x = torch.randn((m, k), generator=gen, device=dev).to(torch.bfloat16)
        y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        ms = _time(torch, lambda i: nv.w4a16_gemm_m128(x, w, out=y), 10, s)
        tf = 2.0 * m * n * k / (ms * 1e-3) / 1e12
        out[f"gemm_{name}_m{m}"] = {"ms": round(ms, 4), "tflops": round(tf, 1), "frac_mfma": round(tf / BF16_MFMA_PEAK_TFLOPS, 4)}
        del w, x, y
    return out


DS_H, DS_V, DS_I, DS_E = 7168, 129280, 2048, 256


def deepseek_rows(nv, torch, M, s):
    """DeepSeek-shaped head (hidden 7168, vocabulary 129280, 256 experts of
    width 2048, top-8): LM head + argmax, the routed MoE (a different routing
    per launch, so experts stream from HBM) and a 18432 x 7168 GEMV (four
    rotated copies), graph-timed like the other rows."""
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    out = {}

    def q(n, k, into=None):
        w = (torch.randn((n, k), generator=gen, device=dev, dtype=torch.float32) * 0.02).to(torch.bfloat16)
        return nv.nvfp4_quantize(w, out=into)

    reps = 30
    lm = q(DS_V, DS_H)
    hl = (torch.randn((M, DS_H), generator=gen, device=dev)).to(torch.bfloat16)
    ws = nv.lmhead_workspace(M, DS_V, dev)
    oi = torch.empty(M, dtype=torch.int32, device=dev)
    om = torch.empty(M, dtype=torch.float32, device=dev)
    ms = _time_graph(torch, lambda i: nv.lmhead_gemv_argmax(hl, lm, workspace=ws, out_idx=oi, out_max=om), reps, s)
    b = nvfp4_bytes(DS_V, DS_H) + M * DS_H * 2 + M * 8
    out["lmhead_v129280_k7168"] = {"ms": round(ms, 5), "gbs": round(b / ms / 1e6, 1),
                                   "frac": round(b / ms / 1e6 / HBM_PEAK_GBS, 4), "drafts_per_s": round(M / (ms * 1e-3), 1)}
    del lm
    ex = {}
    for proj, rows, cols in (("gate", DS_I, DS_H), ("up", DS_I, DS_H), ("down", DS_H, DS_I)):
        codes = torch.empty((DS_E, rows, cols // 2), dtype=torch.uint8, device=dev)
        scales = torch.empty((DS_E, rows, cols // 16), dtype=torch.uint8, device=dev)
        glob = torch.empty((DS_E, 4), dtype=torch.float32, device=dev)
        for e in range(DS_E):
            q(rows, cols, into=nv.NVFP4Weight(codes[e], scales[e], glob[e], rows, cols))
        ex[proj] = (codes, scales, glob)
    experts = nv.NVFP4Experts(*ex["gate"], *ex["up"], *ex["down"])
    xm = torch.randn((M, DS_H), generator=gen, device=dev).to(torch.bfloat16)
    routers = [torch.randn((M, DS_E), generator=gen, device=dev) for _ in range(reps)]
    mws = nv.moe_workspace(M, TOPK, experts, dev)
    ym = torch.empty((M, DS_H), dtype=torch.float32, device=dev)
    ids = torch.empty((M, TOPK), dtype=torch.int32, device=dev)
    wts = torch.empty((M, TOPK), dtype=torch.float32, device=dev)
    nd = []
    for r in routers:
        nv.moe_w4a16_gemv(xm, r, TOPK, experts, workspace=mws, out=ym, topk_ids=ids, topk_w=wts)
        nd.append(len(set(ids.cpu().numpy().ravel().tolist())))
    ms = _time_graph(torch, lambda i: nv.moe_w4a16_gemv(xm, routers[i % reps], TOPK, experts, workspace=mws, out=ym,
                                                        topk_ids=ids, topk_w=wts), reps, s)
    b = float(np.mean(nd)) * 3 * nvfp4_bytes(DS_I, DS_H) + M * DS_H * 6 + M * DS_E * 4
    out["moe_256x2048x7168_top8"] = {"ms": round(ms, 5), "gbs": round(b / ms / 1e6, 1),
                                     "frac": round(b / ms / 1e6 / HBM_PEAK_GBS, 4), "mean_distinct_experts": float(np.mean(nd))}
    del ex, experts
    gws = [q(18432, DS_H) for _ in range(4)]
    xg = torch.randn((M, DS_H), generator=gen, device=dev).to(torch.bfloat16)
    yg = torch.empty((M, 18432), dtype=torch.float32, device=dev)
    ms = _time_graph(torch, lambda i: nv.w4a16_gemv(xg, gws[i % 4], out=yg), reps, s)
    b = nvfp4_bytes(18432, DS_H) + M * DS_H * 2 + M * 18432 * 4
    out["gemv_18432x7168"] = {"ms": round(ms, 5), "gbs": round(b / ms / 1e6, 1), "frac": round(b / ms / 1e6 / HBM_PEAK_GBS, 4)}
    del gws
    torch.cuda.empty_cache()
    return out


def cpu_baseline(M, step_bytes, n_distinct):
    """The CPU oracle (single-threaded C, fp64 accumulation) timed on a bounded
    sample: whole draft steps of the same shapes on synthetic NVFP4 weights,
    repeated for about 10 s."""
    import oracle
    from tests import synth
    rng = np.random.default_rng(0)
    W = {name: synth.quantized_domain_weight(rng, n, k) for name, n, k in PROJ}
    lm = synth.quantized_domain_weight(rng, VOCAB, H)
    ex = synth.moe_quantized_experts(0, 16, H, I)          # the routed subset is what the oracle reads
    x = {name: synth.acts_bf16(1, M, k) for name, n, k in PROJ}
    xm = synth.acts_bf16(2, M, H)
    r = synth.router_logits(3, M, 16)
    topk = min(TOPK, 16)
    t0 = time.perf_counter()
    nsteps = 0
    while True:
        for name, n, k in PROJ:
            oracle.gemv(x[name], *W[name])
        oracle.moe(xm, r, topk, *ex)
        oracle.lmhead_argmax(x["q"], *lm)
        nsteps += 1
        if time.perf_counter() - t0 > 10.0:
            break
    dt = (time.perf_counter() - t0) / nsteps
    return {"value": round(step_bytes / dt / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{nsteps} whole draft step(s) at M={M} (5 GEMVs, MoE over {min(16, M * topk)} of 16 experts "
                      f"standing in for the {n_distinct} routed of 256, LM head 151936x2048) on synthetic NVFP4 "
                      f"weights (the 4 KiB embedding gather is left out); {dt:.2f} s per step",
            "ms_per_step": round(dt * 1e3, 1)}


if __name__ == "__main__":
    main()
