"""Benchmark: one forward round of chunk-causal attention over a rolling paged KV cache.

A step is the whole hot path for one new chunk, once per layer:
  evict the oldest chunk (once the 21-frame window is full) -> append the new
  chunk's K/V (page scatter) -> chunk-causal attention of its 4680 query rows
  over the 32760-key window.
Default workload: Wan2.1-1.3B shape, 30 layers, 12 heads x 128, bf16, paged
ring of 21 pages x 1560 tokens per layer (random page table per layer).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload round|call|wave|fp8round|frameround]

Prints one JSON line.  Inputs are synthetic (seeded on the device) and already
resident in HBM when the timed region starts.  The default workload also
reports, under "extras" (after the headline measurement, which they do not
change): the same round replayed from captured HIP graphs, the same round on
peaked scores (the online softmax's re-form path fires), the 14B-shaped fp8
round, and that round with the quantising append.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
FP8_PEAK_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
HBM_PEAK_GBPS = 8000.0
FRAME = 1560
CHUNK = 3 * FRAME
WINDOW = 21 * FRAME
METRIC = "chunk-attn TFLOP/s + % bf16 MFMA peak (1 GPU); KV-append GB/s; chunks/s"

WORKLOADS = {
    "round": dict(layers=30, H=12, D=128, dtype="bf16", std=0.5,
                  name="wan1.3b forward round: 30 layers x (evict + append 4680 tok + attend 4680 q x 32760 k), "
                       "H12 D128 bf16, paged ring P1560 T21"),
    "fp8round": dict(layers=40, H=40, D=128, dtype="fp8", std=1.0,
                     name="14b forward round: 40 layers x (evict + append 4680 tok + attend 4680 q x 32760 k), "
                          "H40 D128 bf16 Q / e4m3 K,V, paged ring P1560 T21"),
    "frameround": dict(layers=30, H=12, D=128, dtype="bf16", std=0.5, chunk=FRAME,
                       name="wan1.3b frame-wise round: 30 layers x (evict + append 1560 tok + attend 1560 q x "
                            "32760 k), H12 D128 bf16, paged ring P1560 T21"),
    "call": dict(layers=1, H=12, D=128, dtype="bf16", std=0.5,
                 name="wan1.3b single call: 4680 q x 18720 k, H12 D128 bf16"),
    "wave": dict(layers=1, H=12, D=128, dtype="bf16", std=0.5,
                 name="wave: 4 chunks x 4680 q, prefixes 4680..18720, H12 D128 bf16"),
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="round", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=4680, help="query rows in the oracle timing sample")
    ap.add_argument("--schedule", default="balanced", choices=["balanced", "tile"],
                    help="balanced: pass a workspace, so the library may choose its split schedule (key "
                         "parts merged by log-sum-exp) where it applies; tile: no workspace, one workgroup "
                         "per query tile.  The JSON line reports the schedule the library took")
    ap.add_argument("--quantize-append", action="store_true",
                    help="fp8round: new K/V arrive as bf16 and the append quantises them to E4M3FN "
                         "(wf_kv_append_quantize) instead of copying pre-quantised pages")
    ap.add_argument("--graph", action="store_true",
                    help="round workloads: after the eager run, replay the round from captured HIP graphs "
                         "(one per ring phase) for the same number of steps and report its rate")
    ap.add_argument("--no-extras", action="store_true",
                    help="round workload: skip the extra measurements (graph replay, peaked scores, fp8 round, "
                         "quantising append)")
    ap.add_argument("--peaked", action="store_true",
                    help="round workloads: peaked scores -- dim 0 of every key rises along the chunk "
                         "(16 log2 units of score per 256 keys against a query dim 0 of 8), so later key tiles "
                         "outscore earlier ones and the softmax re-forms P with a new maximum")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after the timed run, copy a buffer of this many MiB once (a plain copy kernel of "
                         "known size that scales the FETCH_SIZE / WRITE_SIZE counters of a profiled run)")
    return ap.parse_args()


def kernel_of(dtype):
    """Attention kernel the library launches for a workload (the dispatch rule of wf_chunk_attn_fwd:
    caches with pages of >= 64 tokens take the LDS-DMA kernels, bf16 or fp8 MFMA)."""
    return "attn_fwd_pp_kernel<128>" if dtype == "bf16" else "attn_fwd_fp8_kernel<128>"


def code_text(src):
    """C/C++ source with its comments removed and runs of white space folded to one space, so
    that an edit of comments or layout alone leaves the hash unchanged."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return re.sub(r"\s+", " ", "".join(out)).strip()


def source_sha(name):
    """sha256 over the code of a kernel source and of the local headers it includes
    (recursively), in include order, comments and layout left out: a change to the code of any
    of them invalidates counters taken before it."""
    csrc = os.path.join(ROOT, "chunk_causal_dit_wf_amd", "csrc")
    seen, order = set(), []

    def visit(path):
        path = os.path.normpath(path)
        if path in seen or not os.path.exists(path):
            return
        seen.add(path)
        order.append(path)
        for inc in re.findall(r'^#include "([^"]+)"', open(path).read(), re.M):
            visit(os.path.join(os.path.dirname(path), inc))

    visit(os.path.join(csrc, name))
    h = hashlib.sha256()
    for path in order:
        with open(path, encoding="utf-8") as f:
            h.update(code_text(f.read()).encode())
        h.update(b"\0")
    return h.hexdigest()


def hbm_traffic(kernel, workload, source):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE, each scaled by a plain copy of known size).  None when no summary
    exists or the kernel source changed after the counters were taken."""
    path = os.path.join(ROOT, "profiles", "%s_%s_hbm_traffic.md" % (kernel, workload))
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    sha = re.search(r"^source_sha256: *([0-9a-f]{64})", txt, re.M)
    val = re.search(r"^hbm_bytes_per_launch: *([0-9.eE+]+)", txt, re.M)
    if sha is None or val is None or sha.group(1) != source_sha(source):
        return None
    return float(val.group(1))


def pct(xs, q):
    ys = sorted(xs)
    return ys[min(len(ys) - 1, max(0, int(round(q * (len(ys) - 1)))))]


PEAK_Q0 = 8.0              # query dim 0 of the peaked variant
PEAK_RISE_LOG2 = 16.0      # score rise per PEAK_STEP keys, log2 units
PEAK_STEP = 256


def make_peaked(torch, q, k, D):
    """Peaked scores: q[:, :, 0] = PEAK_Q0 and k[r, :, 0] rising linearly with the row r of the chunk,
    PEAK_RISE_LOG2 log2 units of sigma q.k per PEAK_STEP rows (sigma = 1/sqrt(D))."""
    n = k.shape[0]
    per_key = PEAK_RISE_LOG2 / PEAK_STEP / (PEAK_Q0 * 1.4426950408889634 / D ** 0.5)
    q[:, :, 0] = PEAK_Q0
    k[:, :, 0] = (torch.arange(n, device=k.device, dtype=torch.float32) * per_key)[:, None].to(k.dtype)


class Layer:
    """One layer's cache plus the device inputs of its chunk."""

    def __init__(self, wf, torch, synth, cfg, layer, gen, bf16_source=False, peaked=False):
        H, D, dt = cfg["H"], cfg["D"], cfg["dtype"]
        n = cfg.get("chunk", CHUNK)
        table = synth.permuted_table(synth.W_WAN_ROUND if dt == "bf16" else synth.W_14B_FP8, layer, 21)
        self.cache = wf.KVCache(21, FRAME, H, D, dt, table.tolist(), device="cuda")
        std = cfg["std"]
        self.q = (torch.randn((n, H, D), generator=gen, device="cuda") * std).to(torch.bfloat16)
        self.o = torch.empty_like(self.q)
        if dt == "bf16" or bf16_source:
            self.k = (torch.randn((n, H, D), generator=gen, device="cuda") * std).to(torch.bfloat16)
            self.v = (torch.randn((n, H, D), generator=gen, device="cuda") * std).to(torch.bfloat16)
            self.ks = self.vs = None
            if peaked:
                make_peaked(torch, self.q, self.k, D)
        else:
            self.k, self.ks = quantize_dev(torch, torch.randn((n, H, D), generator=gen, device="cuda") * std)
            self.v, self.vs = quantize_dev(torch, torch.randn((n, H, D), generator=gen, device="cuda") * std)


def quantize_dev(torch, x):
    """Synthetic E4M3FN pages: per (page, head, 128-token block) amax/448 scales (input preparation)."""
    n, H, D = x.shape
    pages = n // FRAME
    nblk = -(-FRAME // 128)
    xs = x.view(pages, FRAME, H, D)
    pad = nblk * 128 - FRAME
    xp = torch.nn.functional.pad(xs.abs(), (0, 0, 0, 0, 0, pad)).view(pages, nblk, 128, H, D)
    amax = xp.amax(dim=(2, 4))                                  # [pages, nblk, H]
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    sc = scale.permute(0, 2, 1).contiguous()                    # [pages, H, nblk]
    per_tok = scale.repeat_interleave(128, dim=1)[:, :FRAME]    # [pages, FRAME, H]
    q = (xs / per_tok[..., None]).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    return q.view(n, H, D).contiguous(), sc


def attn_flops(H, D, rows, keys):
    return 4.0 * D * H * rows * keys


def run_round(args, cfg):
    import torch
    import chunk_causal_dit_wf_amd as wf
    import synth

    wf.lib()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(synth.SEED)
    quant = cfg["dtype"] == "fp8" and getattr(args, "quantize_append", False)
    peaked = cfg["dtype"] == "bf16" and getattr(args, "peaked", False)
    layers = [Layer(wf, torch, synth, cfg, l, gen, bf16_source=quant, peaked=peaked) for l in range(cfg["layers"])]

    def append(L, pos):
        if quant:
            wf.wf_kv_append_quantize(L.cache, pos, L.k, L.v)
        else:
            wf.wf_kv_append(L.cache, pos, L.k, L.v, L.ks, L.vs)
    H, D = cfg["H"], cfg["D"]
    n = cfg.get("chunk", CHUNK)
    # prefill 18 frames per layer with the layer's chunk data
    for L in layers:
        for c in range(18 * FRAME // n):
            append(L, c * n)
    torch.cuda.synchronize()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    ws = wf.workspace_for(layers[0].cache, "cuda") if args.schedule == "balanced" else None

    def step(record):
        marks = []
        for L in layers:
            c = L.cache
            if c.end - c.start + n > c.capacity:
                wf.wf_kv_evict(c, n)
            e0 = ev() if record else None
            if record:
                e0.record()
            append(L, c.end)
            e1 = ev() if record else None
            if record:
                e1.record()
            kb = max(c.start, c.end - WINDOW)
            wf.wf_chunk_attn_fwd(c, L.q, [0, n], [kb], [c.end], o=L.o, workspace=ws)
            if record:
                e2 = ev()
                e2.record()
                marks.append((e0, e1, e2, c.end - kb))
        return marks

    for _ in range(max(1, args.warmup)):
        step(False)
    torch.cuda.synchronize()
    c0 = layers[0].cache
    plan = wf.wf_chunk_attn_plan(c0, [0, n], [max(c0.start, c0.end - WINDOW)], [c0.end], "bf16",
                                 0 if ws is None else ws.numel())
    t_start, t_end = ev(), ev()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record()
    all_marks = []
    for _ in range(args.steps):
        all_marks += step(True)
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)
    app_ms = [a.elapsed_time(b) for a, b, _, _ in all_marks]
    att_ms = [b.elapsed_time(c) for _, b, c, _ in all_marks]
    keys = [k for _, _, _, k in all_marks]
    flops_per_launch = attn_flops(H, D, n, keys[0])
    assert all(k == WINDOW for k in keys)
    esize = 2 if cfg["dtype"] == "bf16" else 1
    app_bytes = 2 * 2 * n * H * D * esize
    if cfg["dtype"] == "fp8":
        app_bytes += 2 * 2 * (n // FRAME) * H * (-(-FRAME // 128)) * 4
    if quant:  # read bf16, write e4m3 codes and the scales
        app_bytes = 2 * n * H * D * (2 + 1) + 2 * (n // FRAME) * H * (-(-FRAME // 128)) * 4
    total_flops = flops_per_launch * len(att_ms)
    ms_step = total_ms / args.steps
    avg_att = sum(att_ms) / len(att_ms)
    avg_app = sum(app_ms) / len(app_ms)
    graph = None
    if getattr(args, "graph", False) and not quant:
        from chunk_causal_dit_wf_amd.round import Layer as RLayer, StreamingRound
        rr = StreamingRound([RLayer(L.cache, L.q, L.k, L.v, L.o, L.ks, L.vs) for L in layers], n, WINDOW,
                            workspace=ws)
        rr.capture()
        for _ in range(rr.period):
            rr.replay()
        torch.cuda.synchronize()
        g0, g1 = ev(), ev()
        g0.record()
        for _ in range(args.steps):
            rr.replay()
        g1.record()
        torch.cuda.synchronize()
        gms = g0.elapsed_time(g1) / args.steps
        graph = dict(ms_per_step=round(gms, 4), chunks_per_s=round(1000.0 / gms, 3),
                     tflops=round(flops_per_launch * cfg["layers"] / (gms * 1e-3) / 1e12, 2),
                     phases=rr.period, steps=args.steps)
    del layers
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return dict(
        plan=plan, graph=graph,
        ms_per_step=ms_step, wall_s=wall, value=total_flops / (total_ms * 1e-3) / 1e12,
        attn_kernel_ms=avg_att, attn_tflops=flops_per_launch / (avg_att * 1e-3) / 1e12, att_ms=att_ms,
        append_kernel_ms=avg_app, append_gbps=app_bytes / (avg_app * 1e-3) / 1e9, app_ms=app_ms,
        chunks_per_s=1000.0 / ms_step, flops_per_launch=flops_per_launch, append_bytes=app_bytes,
        H=H, D=D, layers=cfg["layers"])


def run_single(args, cfg, wave):
    import torch
    import chunk_causal_dit_wf_amd as wf
    import synth

    wf.lib()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(synth.SEED)
    H, D = cfg["H"], cfg["D"]
    cache = wf.KVCache(12, FRAME, H, D, "bf16", list(range(12)), device="cuda")
    for c in range(4):
        k = (torch.randn((CHUNK, H, D), generator=gen, device="cuda") * 0.5).to(torch.bfloat16)
        wf.wf_kv_append(cache, c * CHUNK, k, k.clone())
    rows = 4 * CHUNK if wave else CHUNK
    q = (torch.randn((rows, H, D), generator=gen, device="cuda") * 0.5).to(torch.bfloat16)
    o = torch.empty_like(q)
    if wave:
        q_off, kb, ke = [0, CHUNK, 2 * CHUNK, 3 * CHUNK, 4 * CHUNK], [0] * 4, [CHUNK * (j + 1) for j in range(4)]
        flops = sum(attn_flops(H, D, CHUNK, e) for e in ke)
    else:
        q_off, kb, ke = [0, CHUNK], [0], [4 * CHUNK]
        flops = attn_flops(H, D, CHUNK, 4 * CHUNK)
    ws = wf.workspace_for(cache, "cuda") if args.schedule == "balanced" else None
    plan = wf.wf_chunk_attn_plan(cache, q_off, kb, ke, "bf16", 0 if ws is None else ws.numel())
    for _ in range(args.warmup):
        wf.wf_chunk_attn_fwd(cache, q, q_off, kb, ke, o=o, workspace=ws)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for a, b in evs:
        a.record()
        wf.wf_chunk_attn_fwd(cache, q, q_off, kb, ke, o=o, workspace=ws)
        b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = [a.elapsed_time(b) for a, b in evs]
    avg = sum(ms) / len(ms)
    return dict(plan=plan, ms_per_step=avg, wall_s=wall, value=flops / (avg * 1e-3) / 1e12, attn_kernel_ms=avg,
                attn_tflops=flops / (avg * 1e-3) / 1e12, flops_per_launch=flops, H=H, D=D, layers=1, att_ms=ms,
                append_kernel_ms=None, append_gbps=None, chunks_per_s=None, append_bytes=None, app_ms=None)


def calib_copy(mib):
    """One plain device copy of `mib` MiB (read mib, write mib): the reference kernel for counter scaling."""
    import torch
    x = torch.ones(mib * 1024 * 1024 // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    y.copy_(x)
    torch.cuda.synchronize()
    del x, y


def copy_calibration(nbytes, nbuf=30, reps=3):
    """Achievable rate of a plain device copy moving the append's bytes (read nbytes, write nbytes),
    over nbuf distinct source/destination pairs (the rounds' per-layer rotation, so no copy is served
    from the previous one's lines in the 256 MB MALL): the practical HBM ceiling for a single
    kernel of the append's size, launch and ramp included.  Two copies are timed: torch's copy_ and
    the library's wf_stream_copy (persistent grid, nontemporal 16-byte loads and stores, the
    fastest copy shape measured at this size)."""
    import torch
    import chunk_causal_dit_wf_amd as wf
    nbytes -= nbytes % 16
    src = [torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(i) for i in range(nbuf)]
    dst = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(nbuf)]

    def timed(copy):
        for a, b in zip(src, dst):
            copy(a, b)
        torch.cuda.synchronize()
        ms = []
        for _ in range(reps):
            for a, b in zip(src, dst):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                copy(a, b)
                e1.record()
                ms.append((e0, e1))
        torch.cuda.synchronize()
        t = sorted(a.elapsed_time(b) for a, b in ms)
        med = t[len(t) // 2]
        return dict(GBps=round(2 * nbytes / (med * 1e-3) / 1e9, 1), ms=round(med, 5), copies=len(t))

    out = timed(lambda a, b: b.copy_(a))
    out.update(bytes_per_copy=2 * nbytes, kernel="torch copy_ (a plain device copy kernel)")
    sc = timed(lambda a, b: wf.wf_stream_copy(a, b))
    sc["kernel"] = "wf_stream_copy (persistent grid, nontemporal 16-byte loads and stores)"
    out["stream_copy"] = sc
    del src, dst
    torch.cuda.empty_cache()
    return out


def cpu_baseline(rows, H, D, keys):
    """Time the float64 oracle on the host for one layer's attention (rows x keys x H)."""
    import numpy as np
    import oracle

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    rng = np.random.default_rng(42)
    q = rng.standard_normal((rows, H, D)) * 0.5
    k = rng.standard_normal((keys, H, D)) * 0.5
    v = rng.standard_normal((keys, H, D)) * 0.5
    t0 = time.perf_counter()
    oracle.chunk_attention(q, k, v, [0, rows], [0], [keys])
    dt = time.perf_counter() - t0
    return dict(value=attn_flops(H, D, rows, keys) / dt / 1e12, unit="TFLOP/s", cores=threads, kind="oracle",
                sample="float64 oracle, one layer's attention: %d query rows x %d keys x %d heads x D%d (%.1f s)"
                       % (rows, keys, H, D, dt))


def extras(args):
    """Extra measurements of the default run (each a short run of its own after the headline)."""
    import copy
    import torch
    out = {}

    def sub_args(**kw):
        a = copy.copy(args)
        a.graph = a.peaked = a.quantize_append = False
        a.steps, a.warmup = kw.pop("steps", 5), kw.pop("warmup", 2)
        for k, v in kw.items():
            setattr(a, k, v)
        return a

    def summary(r, peak):
        d = dict(value=round(r["value"], 3), unit="TFLOP/s", ms_per_step=round(r["ms_per_step"], 4),
                 chunks_per_s=round(r["chunks_per_s"], 3), attn_kernel_tflops=round(r["attn_tflops"], 2),
                 attn_frac_of_peak=round(r["attn_tflops"] / peak, 4), kv_append_GBps=round(r["append_gbps"], 1),
                 schedule=r["plan"]["schedule"], attn_grid=r["plan"]["grid"])
        return d

    r = run_round(sub_args(steps=args.steps, warmup=args.warmup, graph=True), WORKLOADS["round"])
    out["graph_replay"] = dict(r["graph"], workload="the headline round replayed from one captured HIP graph "
                                                    "per ring phase (evict metadata on the host)")
    r = run_round(sub_args(peaked=True), WORKLOADS["round"])
    out["peaked"] = dict(summary(r, BF16_PEAK_TFLOPS), workload="the headline round on peaked scores: "
                         "query dim 0 = %g, key dim 0 rising %g log2 units of score per %d keys" %
                         (PEAK_Q0, PEAK_RISE_LOG2, PEAK_STEP), steps=5)
    r = run_round(sub_args(steps=3, warmup=1), WORKLOADS["fp8round"])
    out["fp8round"] = dict(summary(r, FP8_PEAK_TFLOPS), workload=WORKLOADS["fp8round"]["name"], steps=3,
                           append_bytes_per_launch=r["append_bytes"], attn_kernel=kernel_of("fp8"),
                           attn_hbm_traffic=hbm_traffic("attn_fwd_fp8_kernel", "fp8round", "attn_fp8.hip"))
    r = run_round(sub_args(steps=3, warmup=1, quantize_append=True), WORKLOADS["fp8round"])
    out["quantize_append"] = dict(
        kv_append_GBps=round(r["append_gbps"], 1), append_kernel_ms=round(r["append_kernel_ms"], 5),
        append_frac_of_hbm=round(r["append_gbps"] / HBM_PEAK_GBPS, 4), bytes_per_launch=r["append_bytes"],
        chunks_per_s=round(r["chunks_per_s"], 3), steps=3,
        workload="the 14B fp8 round with bf16 K/V quantised to E4M3FN by the append (quant_append_kernel)")
    torch.cuda.synchronize()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path, so there is nothing to "
              "run on more (requested --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    cfg = WORKLOADS[args.workload]
    if args.workload in ("round", "fp8round", "frameround"):
        r = run_round(args, cfg)
    else:
        r = run_single(args, cfg, wave=args.workload == "wave")
    peak = FP8_PEAK_TFLOPS if cfg["dtype"] == "fp8" else BF16_PEAK_TFLOPS
    kernel = kernel_of(cfg["dtype"])
    kname = kernel.split("<")[0]
    traffic = hbm_traffic(kname, args.workload, "attn_fwd.hip" if cfg["dtype"] == "bf16" else "attn_fp8.hip")
    att = r["att_ms"]
    out = {
        "metric": METRIC,
        "value": round(r["value"], 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg["dtype"] == "bf16" else "e4m3 (fp8 MFMA; bf16 Q and P quantised in-kernel, e4m3 K,V)",
        "append_mode": ("quantising bf16 -> e4m3" if getattr(args, "quantize_append", False) and cfg["dtype"] == "fp8"
                        else "copy"),
        "data": ("synthetic (seeded N(0, s^2) on device, random page tables%s)" %
                 (", peaked scores" if args.peaked else "")),
        "config": {"workload": cfg["name"], "layers": cfg["layers"], "heads": r["H"], "head_dim": r["D"],
                   "query_rows": cfg.get("chunk", CHUNK), "keys": WINDOW if "round" in args.workload else None,
                   "parallelism": "single GPU", "schedule": r["plan"]["schedule"],
                   "attn_grid": r["plan"]["grid"]},
        "pct_bf16_peak": round(100.0 * r["value"] / BF16_PEAK_TFLOPS, 2),
        "attn_kernel_tflops": round(r["attn_tflops"], 2),
        "attn_kernel_ms": round(r["attn_kernel_ms"], 4),
        "attn_kernel_ms_p10_p50_p90": [round(pct(att, q), 4) for q in (0.1, 0.5, 0.9)],
        "kv_append_GBps": None if r["append_gbps"] is None else round(r["append_gbps"], 1),
        "append_kernel_ms": None if r["append_kernel_ms"] is None else round(r["append_kernel_ms"], 5),
        "chunks_per_s": None if r["chunks_per_s"] is None else round(r["chunks_per_s"], 3),
        "roofline": {"bound": "mfma", "achieved": round(r["attn_tflops"], 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(r["attn_tflops"] / peak, 4), "traffic": traffic,
                     "kernel": kernel, "flops_per_launch": r["flops_per_launch"]},
    }
    if r["append_gbps"] is not None:
        app = r["app_ms"]
        out["append_kernel_ms_p10_p50_p90"] = [round(pct(app, q), 5) for q in (0.1, 0.5, 0.9)]
        out["append_roofline"] = {"bound": "hbm", "achieved": round(r["append_gbps"], 1), "peak": HBM_PEAK_GBPS,
                                  "unit": "GB/s", "frac": round(r["append_gbps"] / HBM_PEAK_GBPS, 4),
                                  "traffic": (hbm_traffic("append_kernel", args.workload, "kv_cache.hip")
                                              if out["append_mode"] == "copy" else None),
                                  "kernel": ("quant_append_kernel<128>" if out["append_mode"] != "copy" else
                                             "append_kernel<%d, 128>" % (2 if cfg["dtype"] == "bf16" else 1)),
                                  "bytes_per_launch": r["append_bytes"]}
        if not args.no_extras:
            cal = copy_calibration(r["append_bytes"] // 2)
            cal["append_frac_of_copy"] = round(r["append_gbps"] / cal["GBps"], 4)
            cal["append_frac_of_stream_copy"] = round(r["append_gbps"] / cal["stream_copy"]["GBps"], 4)
            out["append_roofline"]["copy_calibration"] = cal
    if r.get("graph"):
        out["graph_replay"] = r["graph"]
    if args.workload == "round" and not args.no_extras and not args.peaked:
        out["extras"] = extras(args)
    if args.calib_copy_mib > 0:
        calib_copy(args.calib_copy_mib)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(min(args.cpu_rows, CHUNK), r["H"], r["D"],
                                           WINDOW if "round" in args.workload else 4 * CHUNK)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
