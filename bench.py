"""Benchmark of the MLA latent-cache decode hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input,
with every input already resident in HBM:
    mla_absorb_q -> mla_decode_attention (split-KV kernel + LSE merge) -> mla_decompress_v
(the decode call alone where the absorbed queries are given).
Default workload: DeepSeek-V3-shaped ragged decode (128 heads, 576-wide
absorbed queries given directly, kv_rank 512 + rope 64; 64 requests with
lengths uniform in [0, 32768], requests 0 and 63 empty; 16-row blocks; bf16).
The GLM-5.2, causal t_q = 4 and NoPE workloads are timed the same way and
reported under "workloads".

Consecutive steps cycle through --copies independent copies of every input
(cache, block table, queries, weights), so the 256 MB Infinity Cache cannot
serve a step from the previous one.  After the --warmup steps, untimed steps
run for --settle-ms of wall time (the first tens of milliseconds of sustained
load run slower than the steady state).  The timed region replays one HIP graph
per input copy holding the step's kernels (--eager launches them from the
host instead); the decode call's own duration for the roofline comes from
HIP events on its stream around each call.  The CPU baseline runs the oracle
over the same workload on the host cores (and on one thread for the tiny
workload and a GLM-5.2 sample).

Prints one JSON line.  Throughput `value` is algorithmic decode-path bytes
per second (GB/s): KV rows read once, queries, weights, outputs, block table
and lengths; the split partials are not counted.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode GB/s & TFLOP/s (% HBM/MFMA roofline); tokens·heads/s vs CPU oracle"
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA

# Measured HBM traffic of one decode call (FETCH_SIZE and WRITE_SIZE counter
# runs, calibrated against a device copy of known size) lives in profile
# summaries (profiles/decode_*_hbm_traffic.md), each tagged with its workload
# and a hash of the sources it was measured on; a figure is reported only
# while those sources are unchanged.
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ["mla_latent_cache_amd/csrc/decode.hip", "mla_latent_cache_amd/csrc/decode_flat.hip",
                  "mla_latent_cache_amd/csrc/decode_common.hpp", "mla_latent_cache_amd/csrc/device_common.hpp",
                  "mla_latent_cache_amd/csrc/kernels.hpp", "mla_latent_cache_amd/csrc/mla_api.cpp"]


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """Bytes per decode call from a committed counter summary, or None when
    there is none for this workload or the kernel sources changed since."""
    import glob
    import re
    for path in sorted(glob.glob(os.path.join(PROFILES, "decode_*_hbm_traffic.md"))):
        text = open(path).read()
        m = re.search(r"<!-- traffic: (\{.*?\}) -->", text, re.S)
        if not m:
            continue
        rec = json.loads(m.group(1))
        if rec.get("workload") == workload and rec.get("source_sha256") == kernel_source_hash():
            return int(rec["bytes_per_call"])
    return None


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def work_figures(spec, seq_lens):
    """Algorithmic bytes / flops / tokens*heads of one step, per stage."""
    import numpy as np
    L = np.asarray(seq_lens, dtype=np.int64)
    B, T, H, D, R = spec.batch, spec.t_q, spec.n_head, spec.D, spec.kv_rank
    e = 4 if spec.dtype == "f32" else 2
    n_tok = B * T
    vis = 0
    for l in L:
        if l > 0:
            vis += sum(int(l) - T + i + 1 for i in range(T))
    kv_rows = int(L[L > 0].sum())
    blocks = int(((L[L > 0] + 15) // 16).sum())
    f = {}
    f["absorb_bytes"] = 0 if spec.q_given else (n_tok * H * (spec.d_nope + spec.d_rope) * e
                                                + H * spec.d_nope * R * e + n_tok * H * D * e)
    f["absorb_flops"] = 0 if spec.q_given else 2 * n_tok * H * spec.d_nope * R
    f["decode_bytes"] = (kv_rows * D * e + n_tok * H * D * e + n_tok * H * R * e + n_tok * H * 4
                         + blocks * 4 + B * 4)
    f["decode_flops"] = vis * H * 2 * (D + R)
    f["decompress_bytes"] = 0 if spec.q_given else (n_tok * H * R * e + H * spec.d_v * R * e
                                                    + n_tok * H * spec.d_v * e)
    f["decompress_flops"] = 0 if spec.q_given else 2 * n_tok * H * spec.d_v * R
    f["kv_bytes"] = kv_rows * D * e
    f["tokens_heads"] = vis * H
    f["bytes"] = f["absorb_bytes"] + f["decode_bytes"] + f["decompress_bytes"]
    f["flops"] = f["absorb_flops"] + f["decode_flops"] + f["decompress_flops"]
    return f


def cpu_baseline(spec, case, figs, max_items: int):
    """The oracle (absorbed form) timed on the host cores over the workload, or
    over a seeded sample of max_items (request, query, head) items."""
    import numpy as np
    import mla_inputs as mi
    import oracle

    n_all = spec.batch * spec.t_q * spec.n_head
    d = oracle.Dims(spec.n_head, spec.d_nope, spec.d_rope, spec.d_v, spec.kv_rank)
    paged = oracle.Paged(case.kv, case.block_table, case.seq_lens)
    sel = None if n_all <= max_items else mi.sample_items(spec.seed + 1, spec.batch, spec.t_q, spec.n_head,
                                                          max_items)
    n = n_all if sel is None else len(sel)
    t0 = time.perf_counter()
    if spec.q_given:
        oracle.decode(d, spec.t_q, case.q_abs, paged, case.scale, sel=sel)
    else:
        oracle.attend_absorbed(d, spec.t_q, case.q_nope, case.q_pe, case.w_uk, case.w_uv, paged, case.scale,
                               sel=sel)
    dt = time.perf_counter() - t0
    frac = n / n_all  # items are independent: the sample does this share of the step's work
    gbs = figs["bytes"] * frac / dt / 1e9
    return {
        "value": round(gbs, 3),
        "unit": "GB/s",
        "cores": oracle.threads(),
        "kind": "oracle",
        "sample": ("whole workload" if sel is None else f"{n} of {n_all} (request, query, head) items, seeded")
                  + (", paged decode of the given absorbed queries" if spec.q_given else ", absorbed form")
                  + f" in float64, {dt:.2f} s wall",
        "tokens_heads_per_s": round(figs["tokens_heads"] * frac / dt, 1),
        "seconds": round(dt, 3),
    }


def append_bytes(spec, n_tok: int, with_q: bool) -> int:
    """Algorithmic bytes of one cache append of n_tok tokens (all written):
    c_kv and k_pe read, the cache row written, q_pe read and written,
    position and slot read, gamma read once."""
    e = 2 if spec.dtype == "bf16" else 4
    per_tok = (spec.kv_rank + spec.d_rope) * e * 2 + 4 + 8
    if with_q and spec.d_rope:
        per_tok += 2 * spec.n_head * spec.d_rope * e
    return n_tok * per_tok + spec.kv_rank * e


def time_prolog(spec, case, dims, kv, stream, reps: int = 20, chunk: int = 4096):
    """The cache-append prolog timed on its own (HIP events on its stream):
    the decode step's new tokens written into the step's cache, and a
    prefill-sized chunk of `chunk` tokens written into a cache of its own."""
    import numpy as np
    import torch

    import mla_inputs as mi
    import mla_latent_cache_amd as mla

    def dev(a):
        if a is None or a.size == 0:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    def timed(args_):
        c, k, q, g, pos, slots, cache = args_
        es = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for _ in range(3):
            mla.mla_cache_append(dims, c, k, g, mi.RMS_EPS, pos, mi.ROPE_BASE, mla.MLA_ROPE_NEOX, q, slots, cache,
                                 None, stream)
        for a, b in es:
            a.record(stream)
            mla.mla_cache_append(dims, c, k, g, mi.RMS_EPS, pos, mi.ROPE_BASE, mla.MLA_ROPE_NEOX, q, slots, cache,
                                 None, stream)
            b.record(stream)
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in es) / reps * 1e-3  # seconds

    ap = mi.step_append(spec, case.seq_lens, case.block_table)
    n_step = ap.slots.shape[0]
    step_args = (dev(ap.c_kv), dev(ap.k_pe), dev(ap.q_pe), dev(ap.gamma),
                 torch.from_numpy(ap.positions).cuda(), torch.from_numpy(ap.slots).cuda(), kv)
    t_step = timed(step_args)
    c, k, q, g = mi.append_values(spec, chunk, tag="bench_chunk")
    cache = torch.empty(chunk // 16, 16, spec.D, dtype=kv.dtype, device="cuda")
    chunk_args = (dev(c), dev(k), dev(q), dev(g), torch.arange(chunk, dtype=torch.int32, device="cuda"),
                  torch.arange(chunk, dtype=torch.int64, device="cuda"), cache)
    t_chunk = timed(chunk_args)
    b_step = append_bytes(spec, n_step, True)
    b_chunk = append_bytes(spec, chunk, True)
    return {
        "kernel": "cache_append_kernel (RmsNorm + rope + slot-mapped write, q_pe rope in place)",
        "decode_step_tokens": n_step,
        "decode_step_us": round(t_step * 1e6, 2),
        "decode_step_bytes": b_step,
        "chunk_tokens": chunk,
        "chunk_us": round(t_chunk * 1e6, 2),
        "chunk_bytes": b_chunk,
        "chunk_gbs": round(b_chunk / t_chunk / 1e9, 1),
        "chunk_frac": round(b_chunk / t_chunk / 1e9 / HBM_PEAK_GBS, 4),
    }


def time_dcp(spec, case, dims, q_abs, stream, world: int = 8, interleave: int = 1, reps: int = 20):
    """One GPU's part of context-parallel decode at `world` ranks, timed with
    HIP events: rank 0's share of the workload (its rows only, float32 partial
    and LSE), and the combine of `world` shares into the final bf16 result.
    The all-gather between the two runs over the GPU links and is not part of
    one GPU's work."""
    import numpy as np
    import torch

    import mla_inputs as mi
    import mla_latent_cache_amd as mla

    B, T, H, D, R = spec.batch, spec.t_q, spec.n_head, spec.D, spec.kv_rank
    e = 2 if spec.dtype == "bf16" else 4
    kv, bt, n_loc = mi.dcp_local(case, world, 0, interleave)

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    kv_d, bt_d, sl_d = dev(kv), dev(bt), dev(case.seq_lens)
    o = torch.empty(B, T, H, R, dtype=torch.float32, device="cuda")
    lse = torch.empty(B, T, H, dtype=torch.float32, device="cuda")
    ws = torch.empty(mla.mla_decode_workspace_size(dims, B, T, bt.shape[1], 16, 0), dtype=torch.uint8, device="cuda")
    n = B * T * H
    o_parts = torch.empty(world, n, R, dtype=torch.float32, device="cuda")
    l_parts = torch.empty(world, n, dtype=torch.float32, device="cuda")
    out = torch.empty(n, R, dtype=torch.bfloat16, device="cuda")
    lse_out = torch.empty(n, dtype=torch.float32, device="cuda")

    def share():
        mla.mla_decode_attention_dcp(dims, case.scale, q_abs, kv_d, bt_d, sl_d, world, 0, interleave, o, lse, ws,
                                     0, stream)

    def combine():
        mla.mla_lse_combine(o_parts, l_parts, out, lse_out, stream)

    def timed(fn):
        for _ in range(3):
            fn()
        es = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in es:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in es) / reps * 1e-3

    t_share = timed(share)
    if mla.mla_decode_status(ws, stream) != 0:
        raise RuntimeError("context-parallel benchmark: the share reported a data error")
    for k in range(world):  # every part a valid share (the combine's time does not depend on values)
        o_parts[k].copy_(o.reshape(n, R))
        l_parts[k].copy_(lse.reshape(n))
    t_comb = timed(combine)
    rows = int(np.asarray(n_loc, dtype=np.int64).sum())
    b_share = rows * D * e + n * D * e + n * R * 4 + n * 4 + int(((n_loc + 15) // 16).sum()) * 4 + B * 4
    b_comb = world * n * (R + 1) * 4 + n * R * 2 + n * 4
    return {
        "layout": f"{world} ranks, rows dealt in runs of {interleave} (row j on rank (j / {interleave}) % {world})",
        "share_rows": rows,
        "share_us": round(t_share * 1e6, 2),
        "share_bytes": b_share,
        "share_gbs": round(b_share / t_share / 1e9, 1),
        "share_frac": round(b_share / t_share / 1e9 / HBM_PEAK_GBS, 4),
        "combine_parts": world,
        "combine_us": round(t_comb * 1e6, 2),
        "combine_bytes": b_comb,
        "combine_gbs": round(b_comb / t_comb / 1e9, 1),
        "combine_frac": round(b_comb / t_comb / 1e9 / HBM_PEAK_GBS, 4),
    }


def time_mlaprolog(spec, case, dims, reps: int = 20):
    """The fused prolog for the decode step's new tokens (one per request and
    query), timed with HIP events: hidden states -> absorbed queries and cache
    rows, at hidden and q_rank widths of the mla_inputs defaults."""
    import numpy as np
    import torch

    import mla_inputs as mi
    import mla_latent_cache_amd as mla

    n_tok = spec.batch * spec.t_q
    hid, qr = mi.PROLOG_HIDDEN, mi.PROLOG_Q_RANK
    p = mi.prolog_inputs(spec, n_tok, hid, qr, tag="bench_prolog")

    def dev(a):
        if a is None or a.size == 0:
            return None
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)

    ap = mi.step_append(spec, case.seq_lens, case.block_table)
    H, D, e = spec.n_head, spec.D, 2
    cache = torch.zeros(case.num_blocks, 16, D, dtype=torch.bfloat16, device="cuda")
    q_abs = torch.empty(n_tok, H, D, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(mla.mla_prolog_workspace_size(dims, hid, qr, n_tok), dtype=torch.uint8, device="cuda")
    args = [dev(p.x), dev(p.w_dq), dev(p.w_uq), dev(p.w_qr), dev(case.w_uk), dev(p.w_dkv), dev(p.w_kr),
            dev(p.gamma_q), dev(p.gamma_kv)]
    pos = torch.from_numpy(ap.positions).cuda()
    slots = torch.from_numpy(ap.slots).cuda()
    stream = torch.cuda.current_stream()

    def call():
        mla.mla_prolog(dims, *args, mi.RMS_EPS, mi.RMS_EPS, pos, mi.ROPE_BASE, mla.MLA_ROPE_NEOX, slots, cache, q_abs,
                       ws, None, stream)

    for _ in range(3):
        call()
    es = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in es:
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize()
    t = sum(a.elapsed_time(b) for a, b in es) / reps * 1e-3
    w_bytes = (qr * hid + spec.kv_rank * hid + spec.d_rope * hid + H * (spec.d_nope + spec.d_rope) * qr
               + H * spec.d_nope * spec.kv_rank + qr + spec.kv_rank) * e
    io_bytes = n_tok * hid * e + n_tok * H * D * e + n_tok * D * e + n_tok * (4 + 8)
    byts = w_bytes + io_bytes
    return {
        "kernels": "skinny_gemm x2 (split-K MFMA), prolog_finish1/2, cache_append_kernel, absorb_mfma",
        "tokens": n_tok,
        "hidden": hid,
        "q_rank": qr,
        "call_us": round(t * 1e6, 2),
        "algorithmic_bytes": byts,
        "gbs": round(byts / t / 1e9, 1),
        "frac": round(byts / t / 1e9 / HBM_PEAK_GBS, 4),
    }


def prefill_figures(spec, seq_lens):
    """Algorithmic work of one naive-form prefill call: flops of the
    decompression GEMM (every cache row of a request through W_UK and W_UV)
    and of causal attention (query i of request b sees L_b - t_q + i + 1
    rows; q.k at width d_nope + d_rope, p.v at width d_v), and the bytes the
    call must move (cache rows, queries, weights, output, LSE).  The per-head
    K/V the first kernel writes for the second is not counted."""
    lens = [int(x) for x in seq_lens]
    H, T, e = spec.n_head, spec.t_q, 2
    vis = sum(sum(L - T + i + 1 for i in range(T)) for L in lens if L >= T)
    att = vis * H * 2 * (spec.d_nope + spec.d_rope + spec.d_v)
    dec = sum(max(L, 0) for L in lens) * H * (spec.d_nope + spec.d_v) * spec.kv_rank * 2
    n_q = len(lens) * T * H
    byts = (sum(max(L, 0) for L in lens) * spec.D * e + n_q * (spec.d_nope + spec.d_rope) * e
            + H * (spec.d_nope + spec.d_v) * spec.kv_rank * e + n_q * spec.d_v * e + n_q * 4)
    return {"attend_flops": att, "decompress_flops": dec, "bytes": byts}


def time_prefill(name: str = "glm52_prefill", reps: int = 10):
    """The naive-form prefill call (decompression GEMM + causal flash
    attention) timed on its own with HIP events on its stream."""
    import numpy as np
    import torch

    import mla_inputs as mi
    import mla_latent_cache_amd as mla

    spec = mi.SPECS[name]
    case = mi.make_case(spec)
    B, T, H = spec.batch, spec.t_q, spec.n_head
    dims = (spec.n_head, spec.d_nope, spec.d_rope, spec.d_v, spec.kv_rank)

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)

    qn = dev(case.q_nope).view(B, T, H, spec.d_nope)
    qp = dev(case.q_pe).view(B, T, H, spec.d_rope) if spec.d_rope else None
    wuk, wuv, kv = dev(case.w_uk), dev(case.w_uv), dev(case.kv)
    bt = torch.from_numpy(case.block_table).cuda()
    sl = torch.from_numpy(case.seq_lens).cuda()
    out = torch.empty(B, T, H, spec.d_v, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(B, T, H, dtype=torch.float32, device="cuda")
    ws = torch.empty(mla.mla_prefill_workspace_size(dims, B, spec.max_blocks), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def call():
        mla.mla_prefill_attention(dims, case.scale, qn, qp, wuk, wuv, kv, bt, sl, out, lse, ws, stream)

    for _ in range(3):
        call()
    if mla.mla_decode_status(ws, stream) != 0:
        raise RuntimeError("prefill benchmark: the call reported a data error")
    es = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in es:
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize()
    t = sum(a.elapsed_time(b) for a, b in es) / reps * 1e-3  # seconds
    f = prefill_figures(spec, case.seq_lens)
    flops = f["attend_flops"] + f["decompress_flops"]
    tflops = flops / t / 1e12
    return {
        "kernels": "prefill_decompress (per-head K_nope/V GEMM) + prefill_attend (causal flash attention)",
        "workload": f"{spec.name}: {H} heads, d_nope {spec.d_nope}, d_rope {spec.d_rope}, d_v {spec.d_v}, "
                    f"kv_rank {spec.kv_rank}, batch {B} x {int(case.seq_lens[0])} rows, t_q {T} new queries",
        "call_us": round(t * 1e6, 1),
        "attend_flops": f["attend_flops"],
        "decompress_flops": f["decompress_flops"],
        "algorithmic_bytes": f["bytes"],
        "bound": "mfma",
        "tflops": round(tflops, 1),
        "peak_tflops": BF16_PEAK_TFLOPS,
        "frac": round(tflops / BF16_PEAK_TFLOPS, 4),
    }


def decode_figures_only(figs):
    return {k: figs[k] for k in ("decode_bytes", "decode_flops", "kv_bytes", "tokens_heads")}


def settle(run_one, settle_ms: float) -> int:
    """Untimed steps until `settle_ms` of wall time has passed.  The first tens
    of milliseconds of sustained load after a pause run 15-25 % slower than the
    steady state on this part (the same kernels, graph-replayed or launched from
    the host), so the timed region starts after them.  Returns the step count."""
    import torch
    n = 0
    t_end = time.perf_counter() + settle_ms * 1e-3
    while time.perf_counter() < t_end:
        for _ in range(8):
            run_one(n)
            n += 1
        torch.cuda.synchronize()
    return n


def measure(name: str, steps: int, warmup: int, n_copies: int, num_splits: int, eager: bool, with_ev: bool = True,
            settle_ms: float = 0.0):
    """Time one workload: the whole step (absorb -> decode -> decompress, or
    the decode call alone when the absorbed queries are given) replayed from
    HIP graphs over `n_copies` input copies, and the decode call alone with
    HIP events on its stream.  Returns (record, case, copies, stream)."""
    import numpy as np
    import torch

    import mla_inputs as mi
    import mla_latent_cache_amd as mla

    spec = mi.SPECS[name]
    log(f"workload {spec.name}: generating inputs")
    case = mi.make_case(spec)
    figs = work_figures(spec, case.seq_lens)
    dims = (spec.n_head, spec.d_nope, spec.d_rope, spec.d_v, spec.kv_rank)
    B, T, H, D, R = spec.batch, spec.t_q, spec.n_head, spec.D, spec.kv_rank
    sdt = torch.bfloat16 if spec.dtype == "bf16" else torch.float32

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    copies = []
    for k in range(max(1, n_copies)):
        c = {"kv": dev(case.kv), "bt": torch.from_numpy(case.block_table).cuda(),
             "sl": torch.from_numpy(case.seq_lens).cuda()}
        if spec.q_given:
            c["q_abs"] = dev(case.q_abs)
        else:
            c.update(q_nope=dev(case.q_nope), q_pe=dev(case.q_pe) if spec.d_rope else None,
                     w_uk=dev(case.w_uk), w_uv=dev(case.w_uv),
                     q_abs=torch.empty(B, T, H, D, dtype=sdt, device="cuda"))
        c["out_lat"] = torch.empty(B, T, H, R, dtype=sdt, device="cuda")
        c["lse"] = torch.empty(B, T, H, dtype=torch.float32, device="cuda")
        if not spec.q_given:
            c["out"] = torch.empty(B * T, H, spec.d_v, dtype=sdt, device="cuda")
        copies.append(c)
    splits = mla.mla_decode_resolve_splits(dims, B, T, spec.max_blocks, num_splits)
    ws = torch.empty(mla.mla_decode_workspace_size(dims, B, T, spec.max_blocks, 16, num_splits),
                     dtype=torch.uint8, device="cuda")

    def step(c, ev=None):
        stream = torch.cuda.current_stream()
        if not spec.q_given:
            mla.mla_absorb_q(dims, c["q_nope"], c["q_pe"], c["w_uk"], c["q_abs"], stream)
        if ev is not None:
            ev[0].record(stream)
        mla.mla_decode_attention(dims, case.scale, c["q_abs"], c["kv"], c["bt"], c["sl"], c["out_lat"], c["lse"],
                                 ws, num_splits, stream)
        if ev is not None:
            ev[1].record(stream)
        if not spec.q_given:
            mla.mla_decompress_v(dims, c["out_lat"], c["w_uv"], c["out"], stream)

    log(f"{spec.name}: warmup {warmup} steps ({splits} ranges per query tile, {len(copies)} input copies)")
    for k in range(warmup):
        step(copies[k % len(copies)])
    torch.cuda.synchronize()
    status = mla.mla_decode_status(ws)
    if status:
        raise RuntimeError(f"{spec.name}: device data-error flags {status:#x}")

    # The step's kernels are captured in one HIP graph per input copy, as a
    # serving loop would launch them; the timed region replays them.  With
    # eager, every kernel is launched from the host.
    stream = torch.cuda.current_stream()
    graphs = []
    if not eager:
        cap = torch.cuda.Stream()
        for c in copies:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                step(c)
            graphs.append(g)
        for k in range(max(1, warmup)):
            graphs[k % len(graphs)].replay()
        torch.cuda.synchronize()
    if settle_ms > 0:
        n_settle = settle(lambda k: graphs[k % len(graphs)].replay() if graphs else step(copies[k % len(copies)]),
                          settle_ms)
        log(f"{spec.name}: {n_settle} untimed steps over {settle_ms:.0f} ms before the timed region")

    # Timed region: the whole step, K times.
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for k in range(steps):
        if graphs:
            graphs[k % len(graphs)].replay()
        else:
            step(copies[k % len(copies)])
    t1.record(stream)
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / steps

    # The decode call alone: HIP events on its stream around each call.
    ev_dec = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for k in range(steps):
        step(copies[k % len(copies)], ev_dec[k])
    torch.cuda.synchronize()
    dec_ms = sorted(a.elapsed_time(b) for a, b in ev_dec)
    dec_avg = sum(dec_ms) / len(dec_ms)
    log(f"{spec.name}: {ms_step * 1e3:.1f} us/step ({'host launches' if eager else 'HIP graph replay'}); "
        f"decode call avg {dec_avg * 1e3:.1f} us (min {dec_ms[0] * 1e3:.1f})")

    stage = {}
    if not spec.q_given:
        for nm in ("absorb", "decompress"):
            es = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(20)]
            for k, (a, b) in enumerate(es):
                c = copies[k % len(copies)]
                a.record(stream)
                if nm == "absorb":
                    mla.mla_absorb_q(dims, c["q_nope"], c["q_pe"], c["w_uk"], c["q_abs"], stream)
                else:
                    mla.mla_decompress_v(dims, c["out_lat"], c["w_uv"], c["out"], stream)
                b.record(stream)
            torch.cuda.synchronize()
            stage[nm] = sum(a.elapsed_time(b) for a, b in es) / len(es)
    stage["decode"] = dec_avg

    dec_s = dec_avg * 1e-3
    dec_gbs = figs["decode_bytes"] / dec_s / 1e9
    dec_tflops = figs["decode_flops"] / dec_s / 1e12
    rec = {
        "workload": f"{spec.name}: {H} heads, d_nope {spec.d_nope}, d_rope {spec.d_rope}, d_v {spec.d_v}, "
                    f"kv_rank {R}, batch {B} x t_q {T}, cache rows per request "
                    f"{'ragged' if spec.lengths == 'ragged' else int(case.seq_lens[0])}, block 16",
        "batch": B, "t_q": T, "seq_lens_total": int(np.maximum(case.seq_lens, 0).sum()),
        "ranges_per_query_tile": splits, "input_copies": len(copies),
        "step_us": round(ms_step * 1e3, 2),
        "step_launch": "host launches" if eager else "HIP graph replay",
        "step_bytes": figs["bytes"], "step_gbs": round(figs["bytes"] / (ms_step * 1e-3) / 1e9, 2),
        "stages_us": {k: round(v * 1e3, 2) for k, v in stage.items()},
        "decode_us": round(dec_avg * 1e3, 2), "decode_min_us": round(dec_ms[0] * 1e3, 2),
        "decode_bytes": figs["decode_bytes"], "decode_flops": figs["decode_flops"],
        "decode_traffic": measured_traffic(spec.name),
        "decode_gbs": round(dec_gbs, 2), "decode_hbm_frac": round(dec_gbs / HBM_PEAK_GBS, 4),
        "decode_tflops": round(dec_tflops, 2), "decode_mfma_frac": round(dec_tflops / BF16_PEAK_TFLOPS, 4),
        "bound": "mfma" if figs["decode_flops"] / figs["decode_bytes"] > BF16_PEAK_TFLOPS / HBM_PEAK_GBS * 1e3
                 else "hbm",
        "tokens_heads_per_s": round(figs["tokens_heads"] / (ms_step * 1e-3), 1),
    }
    rec["decode_roofline_frac"] = rec["decode_mfma_frac"] if rec["bound"] == "mfma" else rec["decode_hbm_frac"]
    return rec, figs, case, copies, stream


def single_thread_oracle():
    """The oracle on one host thread: the tiny f32 workload in full, and a
    seeded sample of 256 (request, query, head) items of the GLM-5.2 decode
    workload (absorbed form), each scaled to GB/s of its workload's
    algorithmic bytes."""
    import mla_inputs as mi
    import oracle

    out = {}
    prev = oracle.threads()
    oracle.set_threads(1)
    try:
        for name, items in (("tiny_f32", None), ("glm52_decode", 256)):
            spec = mi.SPECS[name]
            case = mi.make_case(spec)
            figs = work_figures(spec, case.seq_lens)
            rec = cpu_baseline(spec, case, figs, items if items is not None else 1 << 30)
            out[name] = {k: rec[k] for k in ("value", "unit", "cores", "sample", "tokens_heads_per_s", "seconds")}
    finally:
        oracle.set_threads(prev)
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-ms", type=float, default=250.0,
                    help="after the warmup steps, untimed steps for this much wall time before each timed region "
                         "(sustained load runs slower for its first tens of milliseconds)")
    ap.add_argument("--workload", default="dsv3_ragged")
    ap.add_argument("--extra-workloads", default="glm52_decode,glm52_causal_tq4,nope_long,nope_wide",
                    help="comma-separated workloads also timed and reported under 'workloads' ('' for none)")
    ap.add_argument("--copies", type=int, default=4, help="input copies cycled across steps")
    ap.add_argument("--num-splits", type=int, default=0, help="KV splits per request (0 = automatic)")
    ap.add_argument("--cpu-items", type=int, default=8192, help="oracle items for the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="skip the naive-form prefill measurement")
    ap.add_argument("--no-dcp", action="store_true", help="skip the context-parallel share measurement")
    ap.add_argument("--no-mlaprolog", action="store_true", help="skip the fused prolog measurement")
    ap.add_argument("--eager", action="store_true",
                    help="launch every kernel of a timed step from the host instead of replaying a HIP graph")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="after the timed region, copy this many MiB device-to-device 3 times (a kernel of known "
                         "traffic for scaling hardware byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported (the decode path "
              "runs on a single MI355X; nothing here opens a second device).", file=sys.stderr)
        return 2

    import torch

    import mla_inputs as mi
    import mla_latent_cache_amd as mla

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    mla.lib()  # fails loudly when the HIP library is missing
    torch.cuda.set_device(0)

    main_rec, figs, case, copies, stream = measure(args.workload, args.steps, args.warmup, args.copies,
                                                   args.num_splits, args.eager, settle_ms=args.settle_ms)
    spec = mi.SPECS[args.workload]
    dims = (spec.n_head, spec.d_nope, spec.d_rope, spec.d_v, spec.kv_rank)

    # Other workloads: each timed the same way (fewer input copies), reported as records.
    extras = {}
    extra_names = [w for w in args.extra_workloads.split(",") if w and w != args.workload]
    sub = {}
    for w in extra_names:
        rec, f2, c2, cp2, _ = measure(w, args.steps, args.warmup, min(args.copies, 2), args.num_splits, args.eager,
                                  settle_ms=args.settle_ms)
        extras[w] = rec
        s2 = mi.SPECS[w]
        if w == "glm52_decode":
            d2 = (s2.n_head, s2.d_nope, s2.d_rope, s2.d_v, s2.kv_rank)
            sub["prolog"] = time_prolog(s2, c2, d2, cp2[0]["kv"], stream)
            if not args.no_dcp:
                sub["dcp"] = time_dcp(s2, c2, d2, cp2[0]["q_abs"], stream)
            if not args.no_mlaprolog:
                sub["mlaprolog"] = time_mlaprolog(s2, c2, d2)
        del cp2
        torch.cuda.empty_cache()
    prefill = None if args.no_prefill else time_prefill()

    if args.copy_calibration_mb > 0:
        n = args.copy_calibration_mb * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: 3 x {args.copy_calibration_mb} MiB device-to-device")

    ms_step = main_rec["step_us"] * 1e-3
    value = figs["bytes"] / (ms_step * 1e-3) / 1e9
    bound = main_rec["bound"]
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": args.settle_ms,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.dtype,
        "data": "synthetic (seeded SplitMix64 normals; RMS-normalised latent rows; shuffled block tables)",
        "config": {k: main_rec[k] for k in ("workload", "batch", "t_q", "seq_lens_total", "ranges_per_query_tile",
                                            "input_copies")},
        "tflops": round(figs["flops"] / (ms_step * 1e-3) / 1e12, 3),
        "tokens_heads_per_s": main_rec["tokens_heads_per_s"],
        "step_launch": main_rec["step_launch"],
        "stages_us": main_rec["stages_us"],
        "roofline": {
            "kernel": "decode call (one C-ABI call: split-KV kernel + LSE merge)",
            "bound": bound,
            "achieved": main_rec["decode_gbs"] if bound == "hbm" else main_rec["decode_tflops"],
            "peak": HBM_PEAK_GBS if bound == "hbm" else BF16_PEAK_TFLOPS,
            "unit": "GB/s" if bound == "hbm" else "TFLOP/s",
            "frac": main_rec["decode_roofline_frac"],
            "traffic": measured_traffic(spec.name),
            "algorithmic_bytes_per_launch": figs["decode_bytes"],
            "algorithmic_flops_per_launch": figs["decode_flops"],
            "avg_launch_us": main_rec["decode_us"],
            "hbm_frac": main_rec["decode_hbm_frac"],
            "mfma_tflops": main_rec["decode_tflops"],
            "mfma_frac": main_rec["decode_mfma_frac"],
        },
        "workloads": extras,
        "prefill": prefill,
    }
    result.update(sub)
    if not args.no_cpu_baseline:
        log("cpu baseline: oracle on host cores")
        cb = cpu_baseline(spec, case, figs, args.cpu_items)
        log("cpu baseline: oracle on one host thread (tiny and GLM-5.2 sample)")
        cb["single_thread"] = single_thread_oracle()
        result["cpu_baseline"] = cb
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
