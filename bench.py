"""Benchmark of the causal-attention hot path on one MI355X.

One step = one pass of every kernel of the path over synthetic inputs:
  1. Llama-3-8B-shaped GQA causal prefill with RoPE (B=4, S=8192, 32 query / 8 KV heads of 128,
     theta 5e5): RoPE table + key rotation + the MFMA attention kernel;
  2. Llama-3-8B-shaped GQA KV-cache decode (B=64, one query each, contexts drawn in [1024, 8192],
     contiguous per-sequence caches of 8192 rows): split-KV kernel + split reduction;
  3. MLA-absorbed decode (B=32, 128 heads, one shared 576-dim row per token, context 4096,
     scale 1/sqrt(192)): MFMA kernel + split reduction.
Prefill is priced in algorithmic TFLOP/s (4*Dh FLOPs per unmasked (query, key) pair) against the
dense bf16 matrix peak; decode in algorithmic GB/s (each needed cache row once, plus q and out)
against HBM peak. The headline value is the mean of the two fractions, in percent.
The decode parts rotate over replicas of their caches (2 for the GQA decode, 4 for the MLA decode),
so each call reads rows that are not in the 256 MiB Infinity Cache. The roofline object prices the
prefill's attention kernel alone, timed by HIP events the library records around its launch on
the call's stream. The GPT-2-small-shaped prefill (Dh=64) is timed after the step as a component.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--only PART]
Prints one JSON line. `--extras` instead measures the widened rows (chunked prefill with RoPE + cache
append, RoPE variants, sliding window with sinks) on the same prefill shape, one JSON line each.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import synth  # noqa: E402
from causal_head_attention_gqa_amd import accounting as acc  # noqa: E402

METRIC = "causal prefill TFLOP/s + KV-decode HBM GB/s, as % of MI355X peak"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    # the chip takes ~20 steps after the process starts to reach its steady state (the prefill kernel
    # 2.04 -> 1.96 ms over them); 30 untimed steps take ~70 ms
    p.add_argument("--warmup", type=int, default=30)
    p.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing (profiling runs)")
    p.add_argument("--only", choices=["prefill", "decode", "mla"], default=None,
                   help="time a single part (profiling runs); the JSON line then reports that part")
    p.add_argument("--copy-probe", action="store_true",
                   help="run only a plain 1 GiB device-to-device copy (calibrates the HBM byte counters)")
    p.add_argument("--extras", action="store_true",
                   help="measure the widened rows instead (chunked prefill with cache append, sliding window "
                        "with sinks, RoPE variants): one JSON line each")
    return p.parse_args()


def copy_probe(torch, reps=5):
    """A copy kernel of known size: reads and writes exactly 1 GiB per launch."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n, "ms_per_copy": dt * 1e3,
                      "copy_gbs_read_plus_write": 2 * n / dt / 1e9}))


# ---------------------------------------------------------------------------------- inputs ----
def device_normal(torch, shape, seed):
    """N(0,1) drawn on the device (seeded), rounded to bf16 (round-to-nearest-even)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)


GQA_REPLICAS = 2  # 2 x 1.2 GB of touched cache rows per rotation
MLA_REPLICAS = 4  # 4 x 151 MB = 604 MB, over twice the 256 MiB Infinity Cache


def make_inputs(torch, attn):
    P, D, M = synth.LLAMA3_PREFILL, synth.LLAMA3_DECODE, synth.MLA_DECODE
    x = {}
    x["pq"] = device_normal(torch, (P.B, P.S, P.Nh, P.Dh), 1000 * P.wid + 0)
    x["pk"] = device_normal(torch, (P.B, P.S, P.Nkv, P.Dh), 1000 * P.wid + 1)
    x["pv"] = device_normal(torch, (P.B, P.S, P.Nkv, P.Dh), 1000 * P.wid + 2)
    x["pout"] = torch.empty_like(x["pq"])
    x["pws"] = torch.empty(max(1, attn.prefill_workspace_bytes(P.B, P.S, P.Nkv, P.Dh, P.rope_theta, attn.ATTN_BF16)),
                           dtype=torch.uint8, device="cuda")
    x["dq"] = device_normal(torch, (D.B, D.Nh, D.Dqk), 1000 * D.wid + 0)
    x["dk"] = [device_normal(torch, (D.B, D.max_ctx, D.Nkv, D.Dqk), 1000 * D.wid + 1 + 10 * r)
               for r in range(GQA_REPLICAS)]
    x["dv"] = [device_normal(torch, (D.B, D.max_ctx, D.Nkv, D.Dv), 1000 * D.wid + 2 + 10 * r)
               for r in range(GQA_REPLICAS)]
    x["dctx_np"] = D.ctx_lens()
    x["dctx"] = torch.as_tensor(x["dctx_np"], device="cuda")
    x["dout"] = torch.empty((D.B, D.Nh, D.Dv), dtype=torch.bfloat16, device="cuda")
    x["dws"] = torch.empty(attn.decode_workspace_bytes(D.B, D.Nh, D.Nkv, D.Dqk, D.Dv, D.max_ctx, attn.ATTN_BF16),
                           dtype=torch.uint8, device="cuda")
    x["mq"] = device_normal(torch, (M.B, M.Nh, M.Dqk), 1000 * M.wid + 0)
    x["mkv"] = [device_normal(torch, (M.B, M.max_ctx, 1, M.Dqk), 1000 * M.wid + 1 + 10 * r)
                for r in range(MLA_REPLICAS)]
    x["mctx_np"] = M.ctx_lens()
    x["mctx"] = torch.as_tensor(x["mctx_np"], device="cuda")
    x["mout"] = torch.empty((M.B, M.Nh, M.Dv), dtype=torch.bfloat16, device="cuda")
    x["mws"] = torch.empty(attn.decode_workspace_bytes(M.B, M.Nh, 1, M.Dqk, M.Dv, M.max_ctx, attn.ATTN_BF16),
                           dtype=torch.uint8, device="cuda")
    return x


# ----------------------------------------------------------------------------- cpu baseline ----
def cpu_baseline():
    """Time the fp64 oracle as it stands on a bounded sample of the same workloads (~10 s)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # noqa: BLE001
        threads = 1
    P, D, M = synth.LLAMA3_PREFILL, synth.LLAMA3_DECODE, synth.MLA_DECODE
    # prefill: all 8192 rows of query heads 0-7 of sequence 0
    hq = 8
    q = synth.as_f32(synth.normal(P.wid, 10, (1, P.S, hq, P.Dh), "bf16"), "bf16")
    k = synth.as_f32(synth.normal(P.wid, 11, (1, P.S, 1, P.Dh), "bf16"), "bf16")
    v = synth.as_f32(synth.normal(P.wid, 12, (1, P.S, 1, P.Dh), "bf16"), "bf16")
    rows = np.arange(P.S)
    tp = 0.0
    for h in range(hq):
        t0 = time.perf_counter()
        oracle.prefill_rows(q[:, :, h:h + 1], k, v, 0, 0, rows, rope_theta=P.rope_theta)
        tp += time.perf_counter() - t0
    p_flops = hq * acc.prefill_flops(1, P.S, 1, P.Dh, causal=True)
    # decode: every sequence of the GQA decode and of the MLA decode, one at a time
    td, tm = 0.0, 0.0
    ctx = D.ctx_lens()
    for b in range(D.B):
        c = int(ctx[b])
        dq = synth.as_f32(synth.normal(D.wid, 100 + 3 * b, (1, D.Nh, D.Dqk), "bf16"), "bf16")
        dk = synth.as_f32(synth.normal(D.wid, 101 + 3 * b, (1, c, D.Nkv, D.Dqk), "bf16"), "bf16")
        dv = synth.as_f32(synth.normal(D.wid, 102 + 3 * b, (1, c, D.Nkv, D.Dv), "bf16"), "bf16")
        t0 = time.perf_counter()
        oracle.decode(dq, dk, dv, np.array([c]))
        td += time.perf_counter() - t0
    d_bytes = acc.decode_bytes(ctx, D.B, D.Nh, D.Nkv, D.Dqk, D.Dv, 2)
    mctx = M.ctx_lens()
    for b in range(M.B):
        c = int(mctx[b])
        mq = synth.as_f32(synth.normal(M.wid, 100 + 2 * b, (1, M.Nh, M.Dqk), "bf16"), "bf16")
        mk = synth.as_f32(synth.normal(M.wid, 101 + 2 * b, (1, c, 1, M.Dqk), "bf16"), "bf16").astype(np.float64)
        t0 = time.perf_counter()
        oracle.decode(mq, mk, mk[..., :M.Dv], np.array([c]), scale=M.scale)
        tm += time.perf_counter() - t0
    m_bytes = acc.decode_bytes(mctx, M.B, M.Nh, 1, M.Dqk, M.Dv, 2, shared_row=True)
    p_tflops = p_flops / tp / 1e12
    d_gbs = (d_bytes + m_bytes) / (td + tm) / 1e9
    frac = 0.5 * (p_tflops / acc.PEAK_BF16_TFLOPS + d_gbs / acc.PEAK_HBM_GBS)
    return {
        "value": 100.0 * frac, "unit": "% of peak", "cores": int(threads), "kind": "oracle",
        "sample": (f"fp64 numpy oracle on the host: every row of query heads 0-7 of sequence 0 of the Llama-3-8B "
                   f"prefill ({tp:.1f} s, {p_tflops * 1e3:.2f} GFLOP/s algorithmic; the oracle materialises the "
                   f"full 8192x8192 score matrix, i.e. does twice the causal FLOPs it is credited with); all 64 "
                   f"sequences of the "
                   f"GQA decode ({td:.1f} s) and all 32 of the MLA decode ({tm:.1f} s): {d_gbs:.3f} GB/s "
                   f"algorithmic; {threads} BLAS threads; host {platform.machine()}, {os.cpu_count()} logical CPUs"),
        "prefill_tflops": p_tflops, "decode_gbs": d_gbs,
    }


def prefill_traffic():
    """HBM bytes per launch of the prefill kernel from the committed rocprofv3 counter record, or
    None when the kernel sources changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "prefill_bf16_llama3_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    h = hashlib.sha256()
    for f in rec["source_files"]:
        h.update((hashlib.sha256(open(os.path.join(ROOT, f), "rb").read()).hexdigest() + "  " + f + "\n").encode())
    if h.hexdigest() != rec["source_sha256"]:
        return None
    return int((rec["fetch_size_kib_per_dispatch"] * rec["fetch_scale"]
                + rec["write_size_kib_per_dispatch"] * rec["write_scale"]) * 1024)


# ---------------------------------------------------------------------------------- extras ----
def window_pairs(S: int, window: int, sinks: int) -> int:
    """Visible (query, key) pairs of causal attention with a window of `window` keys plus `sinks`."""
    p = np.arange(S, dtype=np.int64)
    inside = np.minimum(p + 1, window)
    extra = np.clip(np.minimum(sinks, p - window + 1), 0, None)
    return int((inside + extra).sum())


def run_extras(torch, attn, steps: int, warmup: int):
    """The Llama-3-8B-shaped prefill (B=4, S=8192, 32/8 heads of 128, RoPE 5e5) done the other ways the
    library offers, each priced by its own algorithmic FLOPs (or bytes for the cache append)."""
    P = synth.LLAMA3_PREFILL
    B, S, Nh, Nkv, Dh, theta = P.B, P.S, P.Nh, P.Nkv, P.Dh, P.rope_theta
    C = 2048  # chunk length of the chunked prefill
    q = device_normal(torch, (B, S, Nh, Dh), 1000 * P.wid + 0)
    k = device_normal(torch, (B, S, Nkv, Dh), 1000 * P.wid + 1)
    v = device_normal(torch, (B, S, Nkv, Dh), 1000 * P.wid + 2)
    qc = [q[:, c:c + C].contiguous() for c in range(0, S, C)]
    kc_ = [k[:, c:c + C].contiguous() for c in range(0, S, C)]
    vc_ = [v[:, c:c + C].contiguous() for c in range(0, S, C)]
    starts = [torch.full((B,), c, dtype=torch.int32, device="cuda") for c in range(0, S, C)]
    zero = torch.zeros((B,), dtype=torch.int32, device="cuda")
    kcache = torch.empty((B, S, Nkv, Dh), dtype=torch.bfloat16, device="cuda")
    vcache = torch.empty_like(kcache)
    out = torch.empty_like(q)
    outc = [torch.empty_like(t) for t in qc]
    ws = torch.empty(max(1, attn.prefill_cached_workspace_bytes(S, Dh, theta)), dtype=torch.uint8, device="cuda")
    pws = torch.empty(max(1, attn.prefill_workspace_bytes(B, S, Nkv, Dh, theta, attn.ATTN_BF16)),
                      dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(warmup):
            fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        torch.cuda.synchronize()
        for e0, e1 in ev:
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        return float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev]))

    flops_causal = acc.prefill_flops(B, S, Nh, Dh, causal=True)
    workload = f"Llama-3-8B GQA prefill B{B} S{S} Nh{Nh} Nkv{Nkv} Dh{Dh} RoPE{theta:g}"
    lines = []

    def emit(name, ms, work, unit, peak, extra, wl=None):
        rate = work / (ms * 1e-3) / (1e12 if unit == "TFLOP/s" else 1e9)
        lines.append({"extra": name, "workload": wl or workload, **extra, "ms": ms, "achieved": rate, "unit": unit,
                      "peak": peak, "frac": rate / peak})

    # whole-sequence prefill, as the reference point of the rows below
    ms_whole = timed(lambda: attn.prefill(q, k, v, rope_theta=theta, out=out, workspace=pws))
    emit("whole_prefill", ms_whole, flops_causal, "TFLOP/s", acc.PEAK_BF16_TFLOPS, {})

    # chunked prefill: per chunk, RoPE + append of its K/V to the cache, then its queries against the cache
    def appends(rope_dims=0, inter=False):
        for i in range(len(qc)):
            attn.kv_append(kc_[i], vc_[i], kcache, vcache, starts[i], rope_theta=theta, rope_dims=rope_dims,
                           interleaved=inter)

    def chunked(rope_dims=0, inter=False):
        for i in range(len(qc)):
            attn.kv_append(kc_[i], vc_[i], kcache, vcache, starts[i], rope_theta=theta, rope_dims=rope_dims,
                           interleaved=inter)
            attn.prefill_cached(qc[i], kcache, vcache, starts[i], rope_theta=theta, rope_dims=rope_dims,
                                rope_interleaved=inter, out=outc[i], workspace=ws)

    ms_chunk = timed(chunked)
    emit("chunked_prefill", ms_chunk, flops_causal, "TFLOP/s", acc.PEAK_BF16_TFLOPS,
         {"chunks": S // C, "chunk_len": C, "includes": "RoPE + cache append of each chunk"})
    ms_app = timed(appends)
    app_bytes = 2 * 2 * B * S * Nkv * Dh * 2  # K and V: read the new rows, write the cache rows
    emit("kv_append", ms_app / (S // C), app_bytes // (S // C), "GB/s", acc.PEAK_HBM_GBS,
         {"rows_per_call": B * C * Nkv, "note": "per call of one 2048-token chunk"})

    # RoPE variants on the same chunked prefill (q rotated in registers, keys at append)
    for name, rd, inter in (("rope_adjacent_pairs", 0, True), ("rope_partial_64", 64, False)):
        ms_v = timed(lambda rd=rd, inter=inter: chunked(rd, inter))
        emit(name, ms_v, flops_causal, "TFLOP/s", acc.PEAK_BF16_TFLOPS,
             {"chunks": S // C, "rope_dims": rd or Dh, "pairs": "adjacent" if inter else "half-split"})

    # sliding window with attention sinks over the whole sequence (cache filled beforehand)
    appends()
    torch.cuda.synchronize()
    W, sinks = 4096, 4
    pairs = window_pairs(S, W, sinks)
    ms_w = timed(lambda: attn.prefill_cached(q, kcache, vcache, zero, rope_theta=theta, window=W, sinks=sinks,
                                              out=out, workspace=ws))
    emit("sliding_window", ms_w, 4 * Dh * B * Nh * pairs, "TFLOP/s", acc.PEAK_BF16_TFLOPS,
         {"window": W, "sinks": sinks, "visible_pairs_per_head": pairs})
    del q, k, v, qc, kc_, vc_, kcache, vcache, out, outc, pws

    # MLA's non-absorbed prefill, DeepSeek-V3 shape: 128 heads, q/k 192 = 128 + 64 decoupled RoPE dims, v 128
    Mp = synth.MLA_PREFILL
    mq = device_normal(torch, (Mp.B, Mp.S, Mp.Nh, Mp.Dh), 1000 * Mp.wid + 0)
    mk = device_normal(torch, (Mp.B, Mp.S, Mp.Nkv, Mp.Dh), 1000 * Mp.wid + 1)
    mv = device_normal(torch, (Mp.B, Mp.S, Mp.Nkv, Mp.dv), 1000 * Mp.wid + 2)
    mo = torch.empty((Mp.B, Mp.S, Mp.Nh, Mp.dv), dtype=torch.bfloat16, device="cuda")
    mws = torch.empty(max(1, attn.prefill_mla_workspace_bytes(Mp.B, Mp.S, Mp.Nkv, Mp.rope_theta)), dtype=torch.uint8,
                      device="cuda")
    ms_m = timed(lambda: attn.prefill_mla(mq, mk, mv, rope_theta=Mp.rope_theta, out=mo, workspace=mws))
    emit("mla_prefill", ms_m, acc.prefill_flops(Mp.B, Mp.S, Mp.Nh, Mp.Dh, causal=True, Dv=Mp.dv), "TFLOP/s",
         acc.PEAK_BF16_TFLOPS, {"flop_per_pair": 2 * (Mp.Dh + Mp.dv), "includes": "k^R rotation pass"},
         wl=f"DeepSeek-V3 MLA non-absorbed prefill B{Mp.B} S{Mp.S} Nh{Mp.Nh} q/k {Mp.Dh} v {Mp.dv} RoPE{Mp.rope_theta:g}")
    del mq, mk, mv, mo, mws

    # MLA-absorbed decode with the decoupled q^R block rotated in-kernel at ctx-1 (the same workload as
    # the bench step's MLA part otherwise; cold-cache replicas as there)
    M = synth.MLA_DECODE
    rq = device_normal(torch, (M.B, M.Nh, M.Dqk), 1000 * M.wid + 0)
    rkv = [device_normal(torch, (M.B, M.max_ctx, 1, M.Dqk), 1000 * M.wid + 1 + 10 * r) for r in range(MLA_REPLICAS)]
    rctx_np = M.ctx_lens()
    rctx = torch.as_tensor(rctx_np, device="cuda")
    rout = torch.empty((M.B, M.Nh, M.Dv), dtype=torch.bfloat16, device="cuda")
    rws = torch.empty(attn.decode_workspace_bytes(M.B, M.Nh, 1, M.Dqk, M.Dv, M.max_ctx, attn.ATTN_BF16),
                      dtype=torch.uint8, device="cuda")
    rcalls = [0]

    def mla_rope():
        kv = rkv[rcalls[0] % MLA_REPLICAS]
        rcalls[0] += 1
        attn.decode(rq, kv, kv[..., :M.Dv], rctx, scale=M.scale, rope_theta=1e4, out=rout, workspace=rws)

    ms_r = timed(mla_rope)
    emit("mla_decode_rope", ms_r, acc.decode_bytes(rctx_np, M.B, M.Nh, 1, M.Dqk, M.Dv, 2, shared_row=True), "GB/s",
         acc.PEAK_HBM_GBS, {"rope_theta": 1e4, "includes": "q^R (dims 512..575) rotated in-kernel at ctx-1; merge"},
         wl=f"MLA-absorbed decode B{M.B} ctx{M.max_ctx} {M.Nh}x{M.Dqk}/{M.Dv}")
    for ln in lines:
        print(json.dumps(ln))


# ------------------------------------------------------------------------------------ main ----
def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this library runs on one GPU: every workload is one GPU's share; "
                                   "--gpus above 1 is not supported"}))
        sys.exit(2)
    import torch
    if args.copy_probe:
        copy_probe(torch)
        return
    if args.extras:
        import causal_head_attention_gqa_amd as attn
        run_extras(torch, attn, args.steps, args.warmup)
        return
    import causal_head_attention_gqa_amd as attn
    P, D, M = synth.LLAMA3_PREFILL, synth.LLAMA3_DECODE, synth.MLA_DECODE
    x = make_inputs(torch, attn)
    calls = {"decode": 0, "mla": 0}

    def run_prefill():
        attn.prefill(x["pq"], x["pk"], x["pv"], rope_theta=P.rope_theta, out=x["pout"], workspace=x["pws"])

    def run_decode():
        r = calls["decode"] % GQA_REPLICAS
        calls["decode"] += 1
        attn.decode(x["dq"], x["dk"][r], x["dv"][r], x["dctx"], out=x["dout"], workspace=x["dws"])

    def run_mla():
        r = calls["mla"] % MLA_REPLICAS
        calls["mla"] += 1
        attn.decode(x["mq"], x["mkv"][r], x["mkv"][r][..., :M.Dv], x["mctx"], scale=M.scale, out=x["mout"],
                    workspace=x["mws"])

    parts = [("prefill", run_prefill), ("decode", run_decode), ("mla", run_mla)]
    if args.only:
        parts = [p for p in parts if p[0] == args.only]
    stream = torch.cuda.current_stream()

    def new_events(n=2):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for e in evs:  # create the HIP events before any timed region
            e.record(stream)
        return evs

    def step(evs=None, kernel=False):
        """One pass of every part. evs[i] = (start, end): around part i's whole call, or with
        kernel=True around its main kernel alone (recorded by the library at the launch)."""
        for i, (_, fn) in enumerate(parts):
            if evs is None:
                fn()
            elif kernel:
                with attn.kernel_events(*evs[i]):
                    fn()
            else:
                evs[i][0].record(stream)
                fn()
                evs[i][1].record(stream)

    for _ in range(args.warmup):
        step()
    # the timed steps: one event pair around each part's call, nothing else added to the stream
    events = [[new_events() for _ in parts] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(events[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = {name: float(np.mean([events[s][i][0].elapsed_time(events[s][i][1]) for s in range(args.steps)]))
          for i, (name, _) in enumerate(parts)}
    # the same steps again, with the event pairs around each part's main kernel alone (roofline)
    kevents = [[new_events() for _ in parts] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for s in range(args.steps):
        step(kevents[s], kernel=True)
    torch.cuda.synchronize()
    kms = {name: float(np.mean([kevents[s][i][0].elapsed_time(kevents[s][i][1]) for s in range(args.steps)]))
           for i, (name, _) in enumerate(parts)}

    p_flops = acc.prefill_flops(P.B, P.S, P.Nh, P.Dh, causal=True)
    d_bytes = acc.decode_bytes(x["dctx_np"], D.B, D.Nh, D.Nkv, D.Dqk, D.Dv, 2)
    m_bytes = acc.decode_bytes(x["mctx_np"], M.B, M.Nh, 1, M.Dqk, M.Dv, 2, shared_row=True)
    comp = {}
    if "prefill" in ms:
        comp["prefill_tflops"] = p_flops / (ms["prefill"] * 1e-3) / 1e12
        comp["prefill_ms"] = ms["prefill"]
        comp["prefill_kernel_ms"] = kms["prefill"]
        comp["prefill_kernel_tflops"] = p_flops / (kms["prefill"] * 1e-3) / 1e12
    if "decode" in ms:
        comp["gqa_decode_gbs"] = d_bytes / (ms["decode"] * 1e-3) / 1e9
        comp["gqa_decode_ms"] = ms["decode"]
        comp["gqa_split_kernel_ms"] = kms["decode"]
    if "mla" in ms:
        comp["mla_decode_gbs"] = m_bytes / (ms["mla"] * 1e-3) / 1e9
        comp["mla_decode_tflops"] = acc.decode_flops(x["mctx_np"], M.Nh, M.Dqk, M.Dv) / (ms["mla"] * 1e-3) / 1e12
        comp["mla_decode_ms"] = ms["mla"]
        comp["mla_split_kernel_ms"] = kms["mla"]
    dec_ms = ms.get("decode", 0.0) + ms.get("mla", 0.0)
    dec_bytes = (d_bytes if "decode" in ms else 0) + (m_bytes if "mla" in ms else 0)
    fracs = []
    if "prefill" in ms:
        fracs.append(comp["prefill_tflops"] / acc.PEAK_BF16_TFLOPS)
    if dec_ms > 0:
        comp["decode_gbs"] = dec_bytes / (dec_ms * 1e-3) / 1e9
        fracs.append(comp["decode_gbs"] / acc.PEAK_HBM_GBS)
    value = 100.0 * float(np.mean(fracs))
    comp["decode_cache_replicas"] = {"gqa": GQA_REPLICAS, "mla": MLA_REPLICAS}

    if "prefill" in ms:
        # GPT-2-small-shaped prefill (B=8, S=1024, 12 heads of 64, no RoPE): 200 back-to-back calls,
        # kernel events around each, after the step's timed region
        G = synth.GPT2_PREFILL
        gq = device_normal(torch, (G.B, G.S, G.Nh, G.Dh), 1000 * G.wid + 0)
        gk = device_normal(torch, (G.B, G.S, G.Nkv, G.Dh), 1000 * G.wid + 1)
        gv = device_normal(torch, (G.B, G.S, G.Nkv, G.Dh), 1000 * G.wid + 2)
        gout = torch.empty_like(gq)
        for _ in range(5):
            attn.prefill(gq, gk, gv, out=gout)
        gev = [new_events() for _ in range(200)]
        torch.cuda.synchronize()
        for k0, k1 in gev:
            with attn.kernel_events(k0, k1):
                attn.prefill(gq, gk, gv, out=gout)
        torch.cuda.synchronize()
        g_ms = float(np.median([a_.elapsed_time(b_) for a_, b_ in gev]))
        g_flops = acc.prefill_flops(G.B, G.S, G.Nh, G.Dh, causal=True)
        comp["gpt2_prefill_kernel_ms"] = g_ms
        comp["gpt2_prefill_tflops"] = g_flops / (g_ms * 1e-3) / 1e12
        comp["gpt2_prefill_frac"] = comp["gpt2_prefill_tflops"] / acc.PEAK_BF16_TFLOPS

    if "prefill" in ms:
        roofline = {"kernel": "prefill_bf16_kernel<128,128,4,false,false> (Llama-3-8B GQA prefill; kernel alone, "
                              "HIP events around its launch)",
                    "bound": "mfma", "achieved": comp["prefill_kernel_tflops"], "peak": acc.PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": comp["prefill_kernel_tflops"] / acc.PEAK_BF16_TFLOPS,
                    "flops_per_launch": p_flops, "kernel_ms": kms["prefill"], "traffic": prefill_traffic()}
    else:
        name = args.only
        b = d_bytes if name == "decode" else m_bytes
        gbs = b / (kms[name] * 1e-3) / 1e9
        roofline = {"kernel": f"{name} decode split kernel (HIP events around its launch)", "bound": "hbm",
                    "achieved": gbs, "peak": acc.PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / acc.PEAK_HBM_GBS,
                    "kernel_ms": kms[name], "traffic": None}

    line = {
        "metric": METRIC, "value": value, "unit": "% of peak", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": wall * 1e3 / args.steps, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "Llama-3-8B GQA causal prefill B4 S8192 Nh32 Nkv8 Dh128 RoPE5e5 + Llama-3-8B GQA "
                               "decode B64 ctx~U[1024,8192] + MLA-absorbed decode B32 ctx4096 128x576/512",
                   "parts": [p[0] for p in parts]},
        "components": comp,
        "roofline": roofline,
        "cpu_baseline": None if args.no_cpu_baseline or args.only else cpu_baseline(),
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
