#!/usr/bin/env python3
"""Benchmark of the compressed-KV sparse attention hot path on one MI355X.

A step is one decode step of one c4a layer at 128k context for a batch of 16
sequences: compress_append -> indexer_topk -> sparse_swa_attn through the C
ABI's single decode-step call, inputs resident in HBM (fp8 E4M3 attention
cache with fp32 row scales, bf16 indexer cache, 64 query heads x 512, top-k
512).  The timed loop replays a captured HIP graph of one step.  Alongside
it the script reports:

* roofline of the step's dominant kernel (the projection + indexer scan
  launch): its algorithmic bytes per launch / its average duration from HIP
  events its own dispatch stamps, and its HBM traffic from recorded counters;
* the whole step's algorithmic bytes against HBM peak;
* the other decode workloads (c4a at 64k for 32 sequences, c128a at up to 1M
  tokens, the 128k c128a and window-only layers) and a context sweep of the
  64k-workload shapes from 4k to 128k;
* the 4096-token chunked prefill at position 61440 (tokens/s and the share of
  bf16 MFMA peak of its algorithmic flops);
* the whole 43-layer Flash stack (2 window-only, 21 c4a, 20 c128a layers) at
  the same batch and context, one graph per step;
* the CPU oracle timed on the host cores on the same inputs (a baseline).

    python bench.py [--steps K] [--warmup W] [--gpus 1]
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

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16
ALGO_ROW_BYTES = {"f32": lambda d: 4 * d, "bf16": lambda d: 2 * d,
                  "e4m3": lambda d: (d - 64) + 128 + 4}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# --------------------------------------------------------------------------- setup

def make_layer(cfg, wts, cache, max_chunk=0):
    """A DeviceLayer holding the drawn cache.  A paged workload gets a pool of
    its own with every block's page drawn from a seeded permutation (the
    pages of a sequence scattered over the pool, as after many allocations)."""
    from compressed_kv_sparse_amd import DeviceLayer, PagePools
    from compressed_kv_sparse_amd import _lib as L
    pools = None
    if cfg.paged and cfg.ratio:
        nb = cfg.comp_cap // (256 // cfg.ratio)
        rb = L.row_bytes(L.FMT[cfg.kv_fmt], cfg.head_dim, cfg.n_rot)
        irb = L.idx_row_bytes(L.FMT[cfg.idx_fmt], cfg.idx_dim) if cfg.ratio == 4 else 0
        npg = cfg.batch * nb
        pools = PagePools(kv_row_bytes=rb, idx_row_bytes=irb, pages_c4a=npg if cfg.ratio == 4 else 0,
                          pages_c128a=npg if cfg.ratio == 128 else 0)
    dl = DeviceLayer(ratio=cfg.ratio, hidden=cfg.hidden, head_dim=cfg.head_dim, n_heads=cfg.n_heads,
                     batch=cfg.batch, idx_heads=cfg.idx_heads, idx_dim=cfg.idx_dim, top_k=cfg.top_k,
                     comp_cap=cfg.comp_cap, kv_fmt=cfg.kv_fmt, idx_fmt=cfg.idx_fmt, act_fmt=cfg.act_fmt,
                     w_fmt=cfg.w_fmt, rope_base=cfg.rope_base, norm_eps=cfg.norm_eps, max_chunk=max_chunk,
                     rope_base_comp=cfg.rope_base_comp or 0.0, flags=cfg.flags, pages=pools)
    if pools is not None:
        perm = np.random.default_rng(cfg.seed).permutation(npg)
        for b in range(cfg.batch):
            dl.map_rows(b, cfg.comp_cap, order=perm[b * nb:(b + 1) * nb])
    if wts is not None:
        dl.set_weights(wkv=wts.wkv, wgate=wts.wgate, ape=wts.ape, gamma=wts.gamma, idx_wkv=wts.idx_wkv,
                       idx_wgate=wts.idx_wgate, idx_ape=wts.idx_ape, idx_gamma=wts.idx_gamma)
    dl.load_cache(raw=cache.raw, comp=cache.comp, idx=cache.idx, st_kv=cache.st_kv, st_sc=cache.st_sc,
                  ist_kv=cache.ist_kv, ist_sc=cache.ist_sc, n_tokens=cache.first_live)
    return dl


def dev(a):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


# --------------------------------------------------------------------------- algorithmic work

def idx_row_bytes(cfg):
    """Bytes of one stored indexer row: f32 / bf16 values, or the fp4 record
    (codes at 4 bits plus one scale byte per 32 channels)."""
    DI = cfg.idx_dim
    return {"f32": 4 * DI, "bf16": 2 * DI, "fp4": DI // 2 + DI // 32}[cfg.idx_fmt]


def decode_step_bytes(cfg, n):
    """Bytes one decode step must move (reads + writes), per the method."""
    d, D, H, HI, DI, k, r = cfg.head_dim, cfg.hidden, cfg.n_heads, cfg.idx_heads, cfg.idx_dim, cfg.top_k, cfg.ratio
    rho = ALGO_ROW_BYTES[cfg.kv_fmt](d)
    rho_i = idx_row_bytes(cfg) if r == 4 else 0
    s_a = 2 if cfg.act_fmt == "bf16" else 4
    s_w = 2 if cfg.w_fmt == "bf16" else 4
    W = cfg.window
    nl = cfg.lanes   # two-lane compressors: twice the projection and state bytes
    total = 0.0
    for nb in n:
        p = nb - 1
        V = (nb // r) if r else 0
        C = min(k, V) if r == 4 else (V if r == 128 else 0)
        b = 0.0
        if r == 4:
            b += V * rho_i + HI * (DI * s_a + 4) + 8 * k
        out_b = H * (d + 4 * (d // 128)) if cfg.flags & 32 else H * d * s_a   # fp8 output records
        b += (min(nb, 128) + C) * rho + H * d * s_a + out_b + d * s_a + rho
        if r:
            b += D * s_a + 8 * nl * (d + (DI if r == 4 else 0))
            if (p + 1) % r == 0:
                b += W * 8 * nl * (d + (DI if r == 4 else 0)) + rho + rho_i
        total += b
    if r:
        total += nl * (2 * D * (d + (DI if r == 4 else 0)) * s_w + W * 4 * (d + (DI if r == 4 else 0)))
    return total


def step_scan_bytes(cfg, n):
    """Algorithmic bytes of the decode step's projection + scan launch: every
    indexer row it scores (all visible rows but the one the step's own token
    closes, which the selection block scores), the four projection weight
    matrices, x, q^I and the head weights.  The keys it writes are workspace,
    not part of the method's traffic."""
    rho_i = idx_row_bytes(cfg)
    s_a = 2 if cfg.act_fmt == "bf16" else 4
    s_w = 2 if cfg.w_fmt == "bf16" else 4
    tot = 2.0 * cfg.hidden * (cfg.head_dim + cfg.idx_dim) * s_w
    for nb in n:
        V = nb // 4
        scanned = V - 1 if nb % 4 == 0 else V
        tot += scanned * rho_i + cfg.hidden * s_a + cfg.idx_heads * (cfg.idx_dim * s_a + 4)
    return tot


STEP_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "step_scan_traffic_c5.md")


def _code(text):
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (re.sub(r"//.*$", "", ln).rstrip() for ln in text.splitlines())
    return "\n".join(ln for ln in lines if ln.strip())


def step_scan_source_hash():
    """sha256 of the step scan kernel's code (comments and blank lines left
    out): the score body and the fused-step section of k_indexer.hip, the
    projection tile and the device helpers.  A recorded HBM traffic figure is
    valid only for the code it was measured on."""
    import hashlib
    csrc = os.path.join(ROOT, "compressed_kv_sparse_amd", "csrc")
    src = open(os.path.join(csrc, "k_indexer.hip")).read()
    parts = [src[src.index("// ---------------------------------------------------------------- MFMA score"):
                 src.index("// ---------------------------------------------------------------- prefill score GEMM")],
             src[src.index("// ---------------------------------------------------------------- fused decode step"):
                 src.index("// k_step_select: one block")],
             open(os.path.join(csrc, "proj_dec.h")).read(),
             open(os.path.join(csrc, "ckv_device.h")).read()]
    h = hashlib.sha256()
    for part in parts:
        h.update(_code(part).encode())
    return h.hexdigest()


def recorded_traffic(path, source_hash):
    """HBM bytes per launch from a committed counter summary (FETCH_SIZE and
    WRITE_SIZE, each scaled by what the counter reads for a copy of known
    size), or None when the kernel's source has changed since."""
    try:
        lines = open(path).read().splitlines()
    except OSError:
        return None
    kv = {}
    for ln in lines:
        if ln.startswith("- ") and ": " in ln:
            k, v = ln[2:].split(": ", 1)
            kv[k.strip()] = v.strip().strip("`")
    if kv.get("source_sha256") != source_hash:
        return None
    return int(kv["traffic_bytes_per_launch"])


def prefill_flops(cfg, pos0, T):
    d, D, H, HI, DI, k = cfg.head_dim, cfg.hidden, cfg.n_heads, cfg.idx_heads, cfg.idx_dim, cfg.top_k
    f = 2.0 * T * D * 2 * (d + DI) * cfg.lanes   # the projections (two-lane compressors: both lanes)
    for p in range(pos0, pos0 + T):
        V = (p + 1) // 4
        f += 2.0 * HI * DI * V + 4.0 * H * d * (min(128, p + 1) + min(k, V))
    return f


# --------------------------------------------------------------------------- decode

def bench_decode(cfg, steps, warmup, with_kernel=True, api="step", copies=3):
    """Decode steps of one layer.  ``copies`` independent instances of the layer
    (each with its own caches, all drawn from the same seed) take the steps in
    turn, so that the caches one step reads were last touched ``copies`` steps
    earlier: with three copies of the 128k-context layer (about 1.2 GB) nothing
    a step reads is still in the 256 MB last-level cache from the previous one,
    and every cache byte comes from HBM, as it does in a deep layer stack."""
    import torch
    from workloads import make_decode_inputs, make_layer_weights
    from workloads.gen import context_lengths
    from compressed_kv_sparse_amd import _lib as L

    t0 = time.time()
    inp = make_decode_inputs(cfg)
    wts = make_layer_weights(cfg)
    n = context_lengths(cfg)
    log(f"[bench] {cfg.name}: inputs drawn in {time.time() - t0:.1f}s")
    layers = [make_layer(cfg, wts, inp.cache) for _ in range(max(1, copies))]
    x, u, q, pos = dev(inp.x), dev(inp.u), dev(inp.q), dev(inp.pos)
    qI = dev(inp.qI) if inp.qI is not None else None
    w = dev(inp.w) if inp.w is not None else None
    B = cfg.batch
    out = layers[0].new_out(B)
    topk = torch.empty((B, cfg.top_k), dtype=torch.int32, device="cuda") if cfg.ratio == 4 else None

    def step(dl):
        if api == "step":
            dl.decode_step(x, u, q, qI, w, pos, out=out, topk=topk)
        else:
            dl.decode(x, u, q, qI, w, pos, out=out, topk=topk)

    step(layers[0])
    torch.cuda.synchronize()
    assert int(layers[0].status.abs().sum()) == 0, "device status set"
    ref_out = out.clone()
    ref_tk = topk.clone() if topk is not None else None
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for dl in layers:
            step(dl)
    torch.cuda.current_stream().wait_stream(s)
    graphs = []
    for dl in layers:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(dl)
        graphs.append(g)
    for _ in range(3):          # replays interleaved with eager checks; every copy gives the same result
        for g in graphs:
            out.zero_()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), "graph replay differs"
            if ref_tk is not None:
                assert torch.equal(topk, ref_tk), "graph replay top-k differs"
    for i in range(warmup):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    res = {"ms_per_step": dt * 1e3, "tok_s": B / dt, "step_bytes": decode_step_bytes(cfg, n),
           "layer_copies": len(layers)}
    res["step_gbs"] = res["step_bytes"] / dt / 1e9
    res["step_hbm_frac"] = res["step_gbs"] / HBM_PEAK_GBS

    if with_kernel and cfg.ratio == 4 and api == "step":
        # the step's dominant kernel: the projection + indexer scan launch of
        # the decode-step call, timed by a pair of HIP events its own dispatch
        # stamps at the kernel's start and end (hipExtLaunchKernel), on the
        # stream it runs on; the copies take the steps in turn as above
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for a, b in evs:        # torch creates an event at its first record
            a.record()
            b.record()
        for i in range(warmup + steps):
            if i >= warmup:
                L.time_next_score(*evs[i - warmup])
            step(layers[i % len(layers)])
        torch.cuda.synchronize()
        assert int(layers[0].status.abs().sum()) == 0, "device status set"
        ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
        kb = step_scan_bytes(cfg, n)
        res["kernel"] = {"name": "k_step_scan", "avg_us": ms * 1e3, "bytes": kb,
                         "gbs": kb / (ms * 1e-3) / 1e9}
    res["_inp"] = inp
    res["_wts"] = wts
    return res


# --------------------------------------------------------------------------- context sweep

SWEEP_CONTEXTS = (4096, 8192, 16384, 32768, 65536, 131072)


def bench_sweep(steps, warmup, copies=3, contexts=SWEEP_CONTEXTS):
    """Decode throughput against context length ("throughput per context
    frontier"): the 64k workload's layer shape (c4a, 32 sequences, bf16,
    8 x 128 indexer, top-k 512) at each context, caches filled on the device
    as at a warm context, ``copies`` layer instances taking the steps in turn
    so that every cache byte comes from HBM."""
    import torch
    from compressed_kv_sparse_amd import DeviceLayer
    from workloads import get_config
    from workloads.device_gen import draw_step_inputs, draw_weights, fill_layer_cache
    from workloads.gen import context_lengths

    rows = []
    for n_ctx in contexts:
        cfg = get_config("c2").with_(n_ctx=n_ctx, comp_cap=n_ctx // 4, name=f"c2_sweep_{n_ctx}")
        layers = []
        for _ in range(copies):
            dl = DeviceLayer(ratio=4, hidden=cfg.hidden, head_dim=cfg.head_dim, n_heads=cfg.n_heads,
                             batch=cfg.batch, idx_heads=cfg.idx_heads, idx_dim=cfg.idx_dim, top_k=cfg.top_k,
                             comp_cap=cfg.comp_cap, kv_fmt=cfg.kv_fmt, idx_fmt=cfg.idx_fmt,
                             rope_base=cfg.rope_base, norm_eps=cfg.norm_eps)
            fill_layer_cache(dl, cfg)
            dl.set_weights(**draw_weights(cfg))
            layers.append(dl)
        a = draw_step_inputs(cfg)
        out = layers[0].new_out(cfg.batch)
        topk = torch.empty((cfg.batch, cfg.top_k), dtype=torch.int32, device="cuda")
        graphs = []
        for dl in layers:
            dl.decode_step(a["x"], a["u"], a["q"], a["qI"], a["w"], a["pos"], out=out, topk=topk)
        torch.cuda.synchronize()
        assert all(int(dl.status.abs().sum()) == 0 for dl in layers), "device status set"
        for dl in layers:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                dl.decode_step(a["x"], a["u"], a["q"], a["qI"], a["w"], a["pos"], out=out, topk=topk)
            graphs.append(g)
        for i in range(warmup):
            graphs[i % copies].replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            graphs[i % copies].replay()
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / steps
        nb = decode_step_bytes(cfg, context_lengths(cfg))
        rows.append({"context": n_ctx, "us_per_step": round(dt * 1e6, 2), "tok_s": round(cfg.batch / dt, 1),
                     "hbm_frac": round(nb / dt / 1e9 / HBM_PEAK_GBS, 4)})
        log(f"[bench] sweep {n_ctx}: {dt * 1e6:.1f} us/step, {cfg.batch / dt:.0f} tok/s, "
            f"{100 * nb / dt / 1e9 / HBM_PEAK_GBS:.1f}% HBM")
        del layers, graphs
        torch.cuda.empty_cache()
    return {"workload": "c2 shapes (c4a, B=32, bf16, indexer 8x128, top-k 512), caches filled on the device",
            "points": rows}


# --------------------------------------------------------------------------- layer stack

def bench_stack(steps, warmup, paged=False):
    """The 43-layer Flash stack at 128k context, batch 16: one decode step of
    every layer (window-only, c4a and c128a per the schedule), replayed as one
    captured HIP graph.  Caches, weights and inputs are seeded device-side draws.
    paged: the compressed rows in page pools all layers share."""
    import torch
    from compressed_kv_sparse_amd.stack import DeviceStack, StackShape
    from workloads.configs import stack_layer
    from workloads.device_gen import draw_step_inputs, draw_weights, fill_layer_cache
    from workloads.gen import context_lengths

    t0 = time.time()
    stk = DeviceStack(StackShape(paged=paged))
    inputs, nbytes = [], 0.0
    for il, dl in enumerate(stk.layers):
        cfg = stack_layer(il)
        assert cfg.ratio == dl.ratio
        fill_layer_cache(dl, cfg)
        wts = draw_weights(cfg)
        if wts:
            dl.set_weights(**wts)
        inputs.append(draw_step_inputs(cfg))
        nbytes += decode_step_bytes(cfg, context_lengths(cfg))
    outs, topks = stk.buffers()
    torch.cuda.synchronize()
    log(f"[bench] stack: {len(stk)} layers set up in {time.time() - t0:.1f}s")

    def step():
        stk.decode(inputs, outs, topks)

    step()
    torch.cuda.synchronize()
    assert all(int(dl.status.abs().sum()) == 0 for dl in stk.layers), "device status set"
    ref = [o.clone() for o in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    g.replay()
    torch.cuda.synchronize()
    assert all(torch.equal(o.view(torch.int16), r.view(torch.int16)) for o, r in zip(outs, ref)), \
        "stack graph replay differs"
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    B = stk.shape.batch
    return {"workload": "c5_flash_stack_43L_b16_ctx131072_fp8" + ("_paged" if paged else ""), "layers": len(stk),
            "ms_per_step": round(dt * 1e3, 4), "tok_s": round(B / dt, 1), "bytes": int(nbytes),
            "achieved_gbs": round(nbytes / dt / 1e9, 1), "frac": round(nbytes / dt / 1e9 / HBM_PEAK_GBS, 4)}


# --------------------------------------------------------------------------- prefill

def bench_prefill(cfg, steps, warmup, side=False):
    """One chunk per run: the three prefill calls, or (side) one
    ckv_prefill_chunk call with the indexer branch on a second stream."""
    import torch
    from workloads import make_layer_weights, make_prefill_inputs

    inp = make_prefill_inputs(cfg)
    wts = make_layer_weights(cfg)
    dl = make_layer(cfg.with_(batch=1), wts, inp.cache, max_chunk=inp.T)
    x, u, q, qI, w = dev(inp.x), dev(inp.u), dev(inp.q), dev(inp.qI), dev(inp.w)
    T = inp.T
    out = dl.new_out(T)
    topk = torch.empty((T, cfg.top_k), dtype=torch.int32, device="cuda")
    # the chunk rewrites the raw ring and the compressor state; restoring them
    # before each run keeps every run identical (a few hundred KiB of copies,
    # outside the timed span: HIP events on the stream bracket the three
    # prefill calls alone)
    saved = [(t, t.clone()) for t in (dl.raw, dl.st_kv, dl.st_sc, dl.ist_kv, dl.ist_sc, dl.n_tokens)
             if t is not None]
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    side_st = torch.cuda.Stream() if side else None

    def run(ev=None):
        for t, c in saved:
            t.copy_(c)
        if ev is not None:
            ev[0].record()
        if side_st is None:
            dl.prefill(0, inp.pos0, x, u, q, qI, w, out=out, topk=topk)
        else:
            dl.prefill_chunk(0, inp.pos0, x, u, q, qI, w, out=out, topk=topk, side_stream=side_st)
        if ev is not None:
            ev[1].record()

    for _ in range(max(1, warmup)):
        run()
    torch.cuda.synchronize()
    for i in range(steps):
        run(evs[i])
    torch.cuda.synchronize()
    dt = float(np.mean([a.elapsed_time(b) for a, b in evs])) * 1e-3
    fl = prefill_flops(cfg, inp.pos0, T)
    return {"ms_per_chunk": dt * 1e3, "tok_s": T / dt, "tflops": fl / dt / 1e12,
            "mfma_frac": fl / dt / 1e12 / MFMA_BF16_PEAK_TFLOPS, "flops": fl}


# --------------------------------------------------------------------------- Hyper-Connection mixer

def bench_hc(T, D=4096, steps=20, copies=3):
    """The Hyper-Connection mixer around the attention block (split + Sinkhorn +
    pre mix, then the post mix) for T tokens of hidden D, bf16 streams; copies
    of the buffers taken in turn (the T = 4096 streams, 134 MB a copy, then come
    from HBM).  Algorithmic bytes: pre reads the mixer row and four streams and
    writes the block input and the split; post reads the split, four streams and
    the block output and writes four streams."""
    import torch
    from compressed_kv_sparse_amd import HCMixer
    g = torch.Generator(device="cuda")
    g.manual_seed(T)
    m = HCMixer(D, act_fmt="bf16")
    bufs = []
    for _ in range(copies):
        mix = torch.randn((T, 24), generator=g, device="cuda")
        h = torch.randn((T, 4, D), generator=g, device="cuda").to(torch.bfloat16)
        y = torch.randn((T, D), generator=g, device="cuda").to(torch.bfloat16)
        x = torch.empty((T, D), dtype=torch.bfloat16, device="cuda")
        coef = torch.empty((T, 24), dtype=torch.float32, device="cuda")
        out = torch.empty_like(h)
        bufs.append((mix, h, y, x, coef, out))

    def run(b):
        mix, h, y, x, coef, out = b
        m.pre(mix, h, x=x, coef=coef)
        m.post(coef, h, y, out=out)

    for i in range(3):
        run(bufs[i % copies])
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i, (a, b) in enumerate(evs):
        a.record()
        run(bufs[i % copies])
        b.record()
    torch.cuda.synchronize()
    dt = float(np.median([a.elapsed_time(b) for a, b in evs])) * 1e-3
    nbytes = T * (96 + 8 * D + 2 * D + 96) + T * (96 + 8 * D + 2 * D + 8 * D)
    return {"T": T, "hidden": D, "us": round(dt * 1e6, 2), "bytes": nbytes,
            "gbs": round(nbytes / dt / 1e9, 1), "hbm_frac": round(nbytes / dt / 1e9 / HBM_PEAK_GBS, 4)}


# --------------------------------------------------------------------------- CPU oracle

def cpu_baseline(cfg, inp, wts, budget_s=12.0):
    """The oracle on the host cores, on the same inputs: whole decode steps
    (compressor, indexer scores, full-sort top-k, attention) per sequence."""
    import oracle as O
    from threadpoolctl import threadpool_info
    L = O.layer_from(cfg, wts)
    c = inp.cache
    done, t0 = 0, time.perf_counter()
    while True:
        for b in range(cfg.batch):
            seq = O.OracleSequence(L, raw_rec=c.raw[b], comp_rec=c.comp[b] if c.comp is not None else None,
                                   idx_vals=c.idx[b] if c.idx is not None else None,
                                   st_kv=c.st_kv[b] if c.st_kv is not None else None,
                                   st_sc=c.st_sc[b] if c.st_sc is not None else None,
                                   ist_kv=c.ist_kv[b] if c.ist_kv is not None else None,
                                   ist_sc=c.ist_sc[b] if c.ist_sc is not None else None,
                                   first_live=int(c.first_live[b]))
            seq.step(int(inp.pos[b]), inp.x[b], inp.u[b], inp.q[b],
                     None if inp.qI is None else inp.qI[b], None if inp.w is None else inp.w[b])
            done += 1
            if time.perf_counter() - t0 > budget_s and done >= 2:
                break
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    model = ""
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": done / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "host_cpus": os.cpu_count(), "cpu_model": model,
            "sample": f"{done} sequence decode steps of {cfg.name} (p={int(inp.pos[0])}), "
                      f"{dt:.1f}s on the host, numpy fp64 ({threads} BLAS threads of {os.cpu_count()} host CPUs)"}


def cpu_baseline_extra(budget_s=4.0):
    """Further oracle timings on the host: the 1024-token tiny workload's
    decode step and the 64k workload's decode step on one thread each (the
    history fed once, then repeated steps at the last position, each
    recomputing what a new token changes), and a sample of the 4096-token
    prefill chunk's queries on the BLAS thread pool."""
    import oracle as O
    from threadpoolctl import threadpool_limits
    from workloads import get_config, make_decode_inputs, make_layer_weights, make_prefill_inputs
    from workloads import gen as G
    out = {}

    def timed_steps(seq, p, x, u, q, qI, w):
        n, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < budget_s or n < 2:
            seq.step(p, x, u, q, qI, w)
            n += 1
        return n / (time.perf_counter() - t0), n

    with threadpool_limits(1):
        cfg = get_config("c1")
        wts = make_layer_weights(cfg)
        x, u, q, qI, w = G.make_token_stream(cfg, cfg.n_ctx)
        seq = O.OracleSequence(O.layer_from(cfg, wts))
        p = cfg.n_ctx - 1
        seq.feed(0, x[:p], u[:p])
        v, n = timed_steps(seq, p, x[p], u[p], q[p], qI[p], w[p])
        out["c1_decode_1thread"] = {"value": round(v, 2), "unit": "tokens/s", "steps": n}
        cfg = get_config("c2").with_(batch=1)
        inp = make_decode_inputs(cfg)
        wts = make_layer_weights(cfg)
        c = inp.cache
        seq = O.OracleSequence(O.layer_from(cfg, wts), raw_rec=c.raw[0], comp_rec=c.comp[0], idx_vals=c.idx[0],
                               st_kv=c.st_kv[0], st_sc=c.st_sc[0], ist_kv=c.ist_kv[0], ist_sc=c.ist_sc[0],
                               first_live=int(c.first_live[0]))
        v, n = timed_steps(seq, int(inp.pos[0]), inp.x[0], inp.u[0], inp.q[0], inp.qI[0], inp.w[0])
        out["c2_decode_1thread"] = {"value": round(v, 2), "unit": "tokens/s", "steps": n}
    cfg = get_config("c4")
    inp = make_prefill_inputs(cfg)
    seq = O.OracleSequence(O.layer_from(cfg, make_layer_weights(cfg)), raw_rec=inp.cache.raw[0],
                           comp_rec=inp.cache.comp[0], idx_vals=inp.cache.idx[0], st_kv=inp.cache.st_kv[0],
                           st_sc=inp.cache.st_sc[0], ist_kv=inp.cache.ist_kv[0], ist_sc=inp.cache.ist_sc[0],
                           first_live=inp.pos0)
    t0 = time.perf_counter()
    seq.feed(inp.pos0, inp.x, inp.u)
    n = 0
    while time.perf_counter() - t0 < budget_s or n < 2:
        seq.query(inp.pos0 + 8 * n, inp.q[8 * n], inp.qI[8 * n], inp.w[8 * n])
        n += 1
    dt = time.perf_counter() - t0
    out["c4_prefill_sample"] = {"value": round(n / dt, 2), "unit": "tokens/s",
                                "sample": f"the chunk's projection and {n} of its 4096 queries (every 8th)"}
    return out


# --------------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c5")
    ap.add_argument("--api", choices=("step", "calls"), default="step",
                    help="decode through the single decode-step entry point or the three stage calls")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--prefill-steps", type=int, default=3)
    ap.add_argument("--side-stream", action="store_true",
                    help="--part prefill: one ckv_prefill_chunk call with the indexer branch on a second stream")
    ap.add_argument("--no-stack", action="store_true")
    ap.add_argument("--part", choices=("all", "decode", "prefill", "stack", "hc"), default="all",
                    help="time one part alone and print its own JSON line (for kernel profiles)")
    ap.add_argument("--stack-steps", type=int, default=20)
    ap.add_argument("--no-extra", action="store_true", help="skip the other decode workloads")
    ap.add_argument("--no-sweep", action="store_true", help="skip the context sweep")
    ap.add_argument("--layer-copies", type=int, default=3,
                    help="independent layer instances taking the decode steps in turn (1: one layer re-read every "
                         "step, partly from the last-level cache)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first run 3 elementwise copies (neg) of MIB MiB: a known-size reference for HBM counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(decode batches would shard by sequence, each GPU running this path on its own sequences).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    from workloads import get_config

    if args.copy_calibration:
        # an elementwise kernel that reads MIB MiB and writes MIB MiB: the
        # reference for what FETCH_SIZE / WRITE_SIZE read per byte moved
        n = (args.copy_calibration << 20) // 4
        a = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
        b = torch.empty_like(a)
        for _ in range(3):
            torch.neg(a, out=b)
        torch.cuda.synchronize()
        del a, b
    if args.part == "prefill":
        pcfg = get_config(args.workload if args.workload.startswith("c4") else "c4")
        p = bench_prefill(pcfg, args.prefill_steps, 1, side=args.side_stream)
        print(json.dumps({"part": "prefill", "workload": pcfg.name, "side_stream": args.side_stream,
                          **{k: round(v, 4) for k, v in p.items()}}), flush=True)
        return
    if args.part == "hc":
        for T in (16, 4096):
            print(json.dumps({"part": "hc", **bench_hc(T)}), flush=True)
        return
    if args.part == "stack":
        print(json.dumps({"part": "stack", **bench_stack(args.stack_steps, 3)}), flush=True)
        if not args.no_extra:
            print(json.dumps({"part": "stack", **bench_stack(args.stack_steps, 3, paged=True)}), flush=True)
        return
    cfg = get_config(args.workload)
    r = bench_decode(cfg, args.steps, args.warmup, api=args.api, copies=args.layer_copies)
    log(f"[bench] decode {cfg.name}: {r['ms_per_step'] * 1e3:.1f} us/step, {r['tok_s']:.0f} tok/s, "
        f"step {r['step_gbs']:.0f} GB/s ({100 * r['step_hbm_frac']:.1f}% of HBM)")
    kern = r.get("kernel")
    roof = None
    if kern:
        log(f"[bench] {kern['name']}: {kern['avg_us']:.1f} us, {kern['gbs']:.0f} GB/s")
        roof = {"bound": "hbm", "kernel": kern["name"], "achieved": round(kern["gbs"], 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(kern["gbs"] / HBM_PEAK_GBS, 4),
                "avg_us": round(kern["avg_us"], 2), "bytes_per_launch": int(kern["bytes"]),
                "traffic": (recorded_traffic(STEP_TRAFFIC_FILE, step_scan_source_hash())
                            if cfg.name.startswith("c5_c4a") and args.layer_copies == 3 else None)}
    if args.part == "decode":
        print(json.dumps({"part": "decode", "workload": cfg.name, "us_per_step": round(r["ms_per_step"] * 1e3, 2),
                          "roofline": roof}), flush=True)
        return
    extra = {}
    if not args.no_extra:
        for name in ("c2", "c3", "c5_c128a", "c5_swa", "c5_fp4idx", "c5_out8", "c5_qnorm", "c5_paged", "c5_two_lane"):
            e = bench_decode(get_config(name), args.steps, args.warmup, with_kernel=name == "c5_fp4idx",
                             copies=args.layer_copies)
            extra[name] = {k: round(v, 4) for k, v in e.items() if not k.startswith("_") and isinstance(v, float)}
            if "kernel" in e:   # the fp4 indexer's projection + scan launch
                kk = e["kernel"]
                extra[name]["scan_us"] = round(kk["avg_us"], 2)
                extra[name]["scan_hbm_frac"] = round(kk["gbs"] / HBM_PEAK_GBS, 4)
            log(f"[bench] decode {name}: {e['ms_per_step'] * 1e3:.1f} us/step, {e['tok_s']:.0f} tok/s, "
                f"{100 * e['step_hbm_frac']:.1f}% HBM")
            del e
    if not args.no_extra:   # the Hyper-Connection mixer around the block (decode and prefill token counts)
        for T in (16, 4096):
            e = bench_hc(T)
            extra[f"hc_T{T}"] = {k: v for k, v in e.items() if k in ("us", "gbs", "hbm_frac")}
            log(f"[bench] hc mixer T={T}: {e['us']:.1f} us, {e['gbs']:.0f} GB/s ({100 * e['hbm_frac']:.1f}% of HBM)")
    sweep = None
    if not args.no_sweep:
        sweep = bench_sweep(args.steps, args.warmup, copies=args.layer_copies)
    pre = None
    if not args.no_prefill:
        p = bench_prefill(get_config("c4"), args.prefill_steps, 1)
        pre = {"workload": get_config("c4").name, "tok_s": round(p["tok_s"], 1),
               "ms_per_chunk": round(p["ms_per_chunk"], 3), "tflops": round(p["tflops"], 2),
               "mfma_frac": round(p["mfma_frac"], 4)}
        log(f"[bench] prefill: {p['ms_per_chunk']:.2f} ms/chunk, {p['tok_s']:.0f} tok/s, "
            f"{p['tflops']:.1f} TFLOP/s ({100 * p['mfma_frac']:.1f}% of bf16 MFMA)")
        if not args.no_extra:   # one call, the indexer on a second stream
            pp = bench_prefill(get_config("c4"), args.prefill_steps, 1, side=True)
            pre["side_stream"] = {"ms_per_chunk": round(pp["ms_per_chunk"], 3), "tok_s": round(pp["tok_s"], 1),
                                  "mfma_frac": round(pp["mfma_frac"], 4)}
            log(f"[bench] prefill (indexer on a second stream): {pp['ms_per_chunk']:.2f} ms/chunk, "
                f"{pp['tok_s']:.0f} tok/s")
        if not args.no_extra:   # the same chunk with the fp4 indexer cache
            c4f = get_config("c4_fp4idx")
            pf = bench_prefill(c4f, args.prefill_steps, 1)
            pre["fp4_indexer"] = {"workload": c4f.name, "tok_s": round(pf["tok_s"], 1),
                                  "ms_per_chunk": round(pf["ms_per_chunk"], 3)}
            log(f"[bench] prefill (fp4 indexer): {pf['ms_per_chunk']:.2f} ms/chunk, {pf['tok_s']:.0f} tok/s")
    stack = None
    if not args.no_stack:
        stack = bench_stack(args.stack_steps, 3)
        log(f"[bench] stack {stack['layers']} layers: {stack['ms_per_step']:.3f} ms/step, {stack['tok_s']:.0f} tok/s, "
            f"{100 * stack['frac']:.1f}% of HBM")
        if not args.no_extra:   # the same stack with every compressed row in shared page pools
            sp = bench_stack(args.stack_steps, 3, paged=True)
            stack["paged"] = {k: sp[k] for k in ("workload", "ms_per_step", "tok_s", "frac")}
            log(f"[bench] stack (paged): {sp['ms_per_step']:.3f} ms/step, {sp['tok_s']:.0f} tok/s")
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(cfg, r["_inp"], r["_wts"])
        log(f"[bench] cpu oracle: {cpu['value']:.2f} tok/s on {cpu['cores']} threads")
        cpu["others"] = cpu_baseline_extra()
        log(f"[bench] cpu oracle, other workloads: {cpu['others']}")
    line = {
        "metric": "decode tokens/s + HBM GB/s % peak, c4a sparse attn @128k ctx; prefill tok/s",
        "value": round(r["tok_s"], 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(r["ms_per_step"], 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16+fp8",
        "data": "synthetic (seeded draws of the workload's shapes)",
        "config": {"workload": cfg.name, "batch": cfg.batch, "context": cfg.n_ctx, "head_dim": cfg.head_dim,
                   "heads": cfg.n_heads, "indexer": f"{cfg.idx_heads}x{cfg.idx_dim}", "top_k": cfg.top_k,
                   "kv_cache": cfg.kv_fmt, "indexer_cache": cfg.idx_fmt, "layer_copies": r["layer_copies"],
                   "parallelism": "1 GPU"},
        "step_hbm": {"bytes": int(r["step_bytes"]), "achieved": round(r["step_gbs"], 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(r["step_hbm_frac"], 4)},
        "roofline": roof,
        "prefill": pre,
        "stack": stack,
        "cpu_baseline": cpu,
    }
    if extra:
        line["extra"] = extra
    if sweep:
        line["sweep"] = sweep
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
