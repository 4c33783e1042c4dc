#!/usr/bin/env python3
"""Benchmark of the sink-attention hot path on one MI355X.

One step = one pass over every row of the hot path on synthetic inputs that
already sit in HBM:
  * causal prefill of the GPT-OSS-shaped workload (one 8192-token sequence,
    64 query / 8 KV heads, head_dim 64, bf16) -- sink_attn_prefill;
  * split-KV decode of 64 requests x 8192 cached tokens (64 / 8 heads, d 64,
    HND cache, 1024-token chunks) -- sink_attn_decode_split then
    sink_attn_merge_states.  Step i reads copy i % 4 of the K/V caches (4.3 GB
    per round of copies), so that no step finds its cache in the 256 MiB
    Infinity Cache.
All three kernels run back to back on torch's current stream; each launch is
bracketed by HIP events on that stream.  Before the warm-up steps the step
runs for at least --settle-ms of wall time (the shader clock takes some tens
of milliseconds of load to settle); `settle_ms` reports it.

Printed: ONE JSON line.  `value` is prefill TFLOP/s (algorithmic flops: 4*D
per visible causal (query, key) pair, i.e. 4*D*Hq*N(N+1)/2) over the prefill
kernel's mean event-timed duration; the `decode` object carries the decode
KV-read GB/s (K and V of every cached token read once per KV head) over the
split + merge duration, which `decode.roofline` compares with the HBM peak
(the split kernel alone beside it).  `roofline` compares the prefill kernel
with the bf16 dense MFMA peak.

After the timed steps (not part of them): `mfma_rate_reference` times a plain
loop of bf16 MFMAs on every SIMD over the prefill's own K data (and over
constant operands), and `roofline.frac_of_measured_mfma` is the prefill's rate
against it; `hbm_read_reference` times a plain streaming-read kernel
(libbenchprobes.so) and `decode.frac_of_measured_read`
relates the decode to it; `extra` holds the other workloads' lines -- the
head_dim 128 varlen prefill, chunked prefill, multi-token decode, decode over
FP8 caches and over 16-token pages (these three with the library's chunk
size, sink_attn_decode_split_size, and 1024-token chunks beside it), the
split-KV decode shape with the library's chunk size, KV-cache append, the
ragged long-context decode at B = 1, 8, 32, 128 (library's chunk size; B < 32
is latency bound and flagged so) and the one-launch decode
(sink_attn_decode_fused) beside split + merge; the ragged, one-launch and
append lines take device time from HIP-graph replay and cycle through copies
of their inputs so that each round of calls touches at least 4 GiB.

Last, the oracle leg (`cpu_baseline`, `parity`): the fp64 CPU oracle runs
every configuration's rows on this host's cores -- the tiny and the
GPT-OSS-shaped prefill, the split-KV decode, the ragged decode at each batch
size and the wide-GQA varlen prefill -- timed per configuration
(`cpu_baseline.per_config`, with the thread count and the CPU model), and the
same rows are the all-row parity check of the GPU outputs the bench produced.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import subprocess
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import gqa_attention_sinks_prefill_amd as sa  # noqa: E402
from gqa_attention_sinks_prefill_amd import workloads as wl  # noqa: E402

# MI355X published peaks (dense): bf16 MFMA 256 CU x 2.4 GHz x 4096 flop/clk/CU,
# HBM3E 8 TB/s.
PEAK_BF16_TFLOPS = 256 * 2.4e9 * 4096 / 1e12
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")


def log(msg: str) -> None:
    """One progress line on stderr per finished phase (the JSON line alone goes to stdout)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Hash of the library's kernel sources (the benchmark's reference kernels,
    *_probe.hip, are not part of it)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gqa_attention_sinks_prefill_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith("_probe.hip"):
            continue
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the kernel sources as they are now (else None)."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    ent = rec.get("kernels", {}).get(kernel)
    return None if ent is None else ent.get("hbm_bytes_per_launch")


def cpu_model() -> str:
    """The host CPU's model name as lscpu reports it, with its family / model /
    stepping numbers (a virtualised host may report only the brand), else
    /proc/cpuinfo's model name."""
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=20).stdout
        f = {}
        for ln in out.splitlines():
            if ":" in ln:
                key, val = ln.split(":", 1)
                f.setdefault(key.strip(), val.strip())
        if "Model name" in f:
            ids = ", ".join(f"{k.lower()} {f[k]}" for k in ("CPU family", "Model", "Stepping") if k in f)
            return f"{f['Model name']} ({ids})" if ids else f["Model name"]
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


BOUND = {"bound_max_abs": 2e-2, "bound_mean_abs": 2e-3, "bound_lse_abs": 4e-3}


def oracle_prefill_leg(inp, cfg, out_gpu, lse_gpu, seconds: float, seed: int = 0):
    """Time the fp64 oracle on a prefill workload's (token, head) rows, in a
    seeded random order and in chunks, until every row is done or `seconds`
    have passed; the same rows are the parity check of the GPU output."""
    import oracle   # test infrastructure: only the oracle leg of the benchmark uses it

    threads = oracle.default_threads()
    T, Hq, D = inp["q"].shape
    cu = inp["cu_seqlens"].numpy().astype(np.int64)
    order = np.random.default_rng(seed).permutation(T * Hq)
    rows_all = np.stack([order // Hq, order % Hq], 1)
    chunk = 16384
    flops, elapsed, done = 0.0, 0.0, 0
    max_err, sum_err, lse_err = 0.0, 0.0, 0.0
    out_cpu, lse_cpu = out_gpu.detach().cpu(), lse_gpu.detach().cpu()
    while done < len(rows_all) and elapsed < seconds:
        rows = rows_all[done:done + chunk]
        t0 = time.perf_counter()
        o, lse, _ = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["sinks"],
                                   inp["cu_seqlens"], causal=True, scale=cfg.scale,
                                   rows=rows, threads=threads)
        elapsed += time.perf_counter() - t0
        pos = rows[:, 0] - cu[np.searchsorted(cu, rows[:, 0], side="right") - 1]
        flops += float(np.sum(4.0 * D * (pos + 1)))
        t, h = torch.from_numpy(rows[:, 0]), torch.from_numpy(rows[:, 1])
        err = np.abs(out_cpu[t, h].double().numpy() - o)
        max_err = max(max_err, float(err.max()))
        sum_err += float(err.sum())
        fin = np.isfinite(lse)
        lse_err = max(lse_err, float(np.abs(lse_cpu[t, h].double().numpy()[fin] - lse[fin]).max(initial=0.0)))
        done += len(rows)
    full = done == len(rows_all)
    what = ("all" if full else f"{done} random") + f" of the {len(rows_all)} (token, head) rows"
    base = {"workload": cfg.name, "value": flops / elapsed / 1e12, "unit": "TFLOP/s",
            "cores": threads, "seconds": round(elapsed, 2),
            "sample": f"{what}, {flops:.3g} algorithmic flop in {elapsed:.1f} s, fp64 C + OpenMP"}
    parity = {"workload": cfg.name, "rows": int(done), "all_rows": bool(full), "max_abs": max_err,
              "mean_abs": sum_err / (done * D), "lse_max_abs": lse_err, **BOUND}
    parity["ok"] = bool(max_err <= 2e-2 and parity["mean_abs"] <= 2e-3 and lse_err <= 4e-3)
    return base, parity


def oracle_decode_leg(cpu_inp, name, out_gpu, lse_gpu, kv_bytes: float):
    """The fp64 oracle over every (request, head) row of a decode workload,
    timed (KV GB/s of the same algorithmic bytes as the GPU line), and the
    all-row parity check of the GPU output and lse."""
    import oracle   # test infrastructure: only the oracle leg of the benchmark uses it

    threads = oracle.default_threads()
    t0 = time.perf_counter()
    o, lse, _ = oracle.decode(cpu_inp["q"], cpu_inp["k_cache"], cpu_inp["v_cache"],
                              cpu_inp["seq_lens"], cpu_inp["sinks"], threads=threads)
    elapsed = time.perf_counter() - t0
    D = o.shape[1]
    got = out_gpu.detach().cpu().double().numpy().reshape(-1, D)
    err = np.abs(got - o)
    g_lse = lse_gpu.detach().cpu().double().numpy().reshape(-1)
    fin = np.isfinite(lse)
    lse_err = float(np.abs(g_lse[fin] - lse[fin]).max(initial=0.0))
    base = {"workload": name, "value": kv_bytes / elapsed / 1e9, "unit": "GB/s",
            "cores": threads, "seconds": round(elapsed, 2),
            "sample": f"all {o.shape[0]} (request, head) rows, fp64 C + OpenMP"}
    parity = {"workload": name, "rows": int(o.shape[0]), "all_rows": True,
              "max_abs": float(err.max()), "mean_abs": float(err.mean()),
              "lse_max_abs": lse_err, **BOUND}
    parity["ok"] = bool(parity["max_abs"] <= 2e-2 and parity["mean_abs"] <= 2e-3
                        and lse_err <= 4e-3 and np.array_equal(np.isneginf(g_lse), np.isneginf(lse)))
    return base, parity


def varlen_prefill_measurement(dev, stream, reps: int, keep: dict | None = None):
    """TFLOP/s of the wide-GQA varlen prefill (16 packed sequences of U[512, 6000]
    tokens, 64 q / 4 KV heads, head_dim 128, causal), event-timed like the main
    line.  With `keep`, one more call (with lse) leaves its inputs and outputs
    there for the oracle leg."""
    cfg = wl.VARLEN_PREFILL
    inp = wl.prefill_inputs(cfg)
    q, k, v = inp["q"].to(dev), inp["k"].to(dev), inp["v"].to(dev)
    sinks, cu = inp["sinks"].to(dev), inp["cu_seqlens"].to(dev)
    out = torch.empty_like(q)
    run = lambda: sa.sink_attn_prefill(q, k, v, sinks, cu, inp["max_seqlen"], causal=True,
                                       scale=cfg.scale, out=out, stream=stream)
    for _ in range(3):
        run()
    torch.cuda.synchronize()
    e = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
         for _ in range(reps)]
    for a, b in e:
        a.record(stream)
        run()
        b.record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in e]))
    flops = wl.prefill_flops(inp["seqlens"].tolist(), cfg.num_q_heads, cfg.head_dim)
    tf = flops / (ms * 1e-3) / 1e12
    if keep is not None:
        out.fill_(float("nan"))
        lse = torch.full((q.shape[0], q.shape[1]), float("nan"), device=dev)
        sa.sink_attn_prefill(q, k, v, sinks, cu, inp["max_seqlen"], causal=True,
                             scale=cfg.scale, out=out, lse=lse, stream=stream)
        torch.cuda.synchronize()
        keep.update(inp=inp, cfg=cfg, out=out.cpu(), lse=lse.cpu())
    return {"workload": cfg.name, "value": round(tf, 2), "unit": "TFLOP/s",
            "mean_launch_ms": round(ms, 4), "algorithmic_flop_per_launch": flops,
            "roofline": {"bound": "mfma", "peak": round(PEAK_BF16_TFLOPS, 1),
                         "frac": round(tf / PEAK_BF16_TFLOPS, 4)}}


def chunked_prefill_measurement(dev, stream, reps: int):
    """TFLOP/s of chunked prefill: 4 sequences of 8192 tokens, the last 2048 of
    each new (6144 cached keys before them), 64 q / 8 KV heads, d 64, causal."""
    cfg = wl.CHUNKED_PREFILL
    inp = wl.chunked_prefill_inputs(cfg, wl.CHUNK_LEN)
    q, k, v = inp["q"].to(dev), inp["k"].to(dev), inp["v"].to(dev)
    sinks = inp["sinks"].to(dev)
    cq, ck = inp["cu_seqlens_q"].to(dev), inp["cu_seqlens_k"].to(dev)
    out = torch.empty_like(q)
    run = lambda: sa.sink_attn_prefill_chunked(q, k, v, sinks, cq, ck, inp["max_seqlen_q"],
                                               causal=True, scale=cfg.scale, out=out,
                                               stream=stream)
    for _ in range(10):
        run()
    torch.cuda.synchronize()
    e = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
         for _ in range(reps)]
    for a, b in e:
        a.record(stream)
        run()
        b.record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in e]))
    flops = wl.chunked_prefill_flops(inp["seqlens_q"].tolist(), inp["seqlens_k"].tolist(),
                                     cfg.num_q_heads, cfg.head_dim)
    tf = flops / (ms * 1e-3) / 1e12
    return {"workload": cfg.name, "value": round(tf, 2), "unit": "TFLOP/s",
            "mean_launch_ms": round(ms, 4), "algorithmic_flop_per_launch": flops,
            "roofline": {"bound": "mfma", "peak": round(PEAK_BF16_TFLOPS, 1),
                         "frac": round(tf / PEAK_BF16_TFLOPS, 4)}}


def kv_append_measurement(dev, stream, reps: int):
    """GB/s (bytes read + written) of appending 1024 new tokens to each of 64
    requests' HND caches (8 KV heads, d 64, 8192 slots), token-major rows in;
    device time from graph replay, cycling through copies of the new rows and
    of the caches (one call moves 256 MiB)."""
    cfg = wl.KV_APPEND
    counts = [cfg["new"]] * cfg["batch"]
    inp = wl.kv_append_inputs(counts, cfg["max_ctx"], cfg["num_kv_heads"], cfg["head_dim"],
                              cfg["seed"])
    moved = 2.0 * 2 * sum(counts) * cfg["num_kv_heads"] * cfg["head_dim"] * 2   # K+V, read + write
    n = rotation(moved)
    kn, vn = inp["k_new"].to(dev), inp["v_new"].to(dev)
    cu, pos = inp["cu_seqlens_new"].to(dev), inp["cache_pos"].to(dev)
    shape = (cfg["batch"], cfg["num_kv_heads"], cfg["max_ctx"], cfg["head_dim"])
    sets = [(kn, vn, torch.zeros(shape, dtype=torch.bfloat16, device=dev),
             torch.zeros(shape, dtype=torch.bfloat16, device=dev))]
    sets += [(kn.clone(), vn.clone(), torch.zeros_like(sets[0][2]), torch.zeros_like(sets[0][3]))
             for _ in range(n - 1)]

    def run(s, i):
        a, b, kc, vc = sets[i % n]
        sa.sink_attn_kv_append(a, b, cu, pos, kc, vc, max_new=cfg["new"], stream=s)

    ms = graph_ms(run, stream, reps=max(3, reps // 2))
    gbs = moved / (ms * 1e-3) / 1e9
    del sets
    torch.cuda.empty_cache()
    return {"workload": cfg["name"], "value": round(gbs, 1), "unit": "GB/s",
            "metric": "KV-cache append GB/s (bytes read + written, graph replay)",
            "mean_ms": round(ms, 4), "algorithmic_bytes": moved, "copies_rotated": n,
            "roofline": {"bound": "hbm", "peak": PEAK_HBM_GBS, "frac": round(gbs / PEAK_HBM_GBS, 4)}}


def _decode_line(name, metric, kv, chosen, times, copies, extra=None):
    """One decode line: the value at the library's chunk size, 1024 beside it."""
    ms = times[chosen]
    gbs = kv / (ms * 1e-3) / 1e9
    line = {"workload": name, "value": round(gbs, 1), "unit": "GB/s", "metric": metric,
            "split_size": chosen, "mean_ms": round(ms, 4),
            "split1024_ms_same_run": round(times[1024], 4),
            "split1024_gbs": round(kv / (times[1024] * 1e-3) / 1e9, 1),
            "algorithmic_bytes_per_step": kv, "cache_copies_rotated": copies,
            "roofline": {"bound": "hbm", "peak": PEAK_HBM_GBS, "frac": round(gbs / PEAK_HBM_GBS, 4)}}
    line.update(extra or {})
    return line


def _partials(B, q_len, Hq, ns, D, dev):
    return (torch.empty(B, q_len, Hq, ns, D, device=dev), torch.empty(B, q_len, Hq, ns, device=dev),
            torch.empty(B, q_len, Hq, ns, device=dev))


def multi_decode_measurement(dev, stream, reps: int):
    """KV GB/s of multi-token decode (speculative / MTP verification): 64 requests x
    8192 cached tokens, the last 4 of them new, split decode + merge with the
    library's chunk size for these (equal) lengths, 1024-token chunks beside it;
    device time from graph replay over rotated cache copies."""
    cfg = wl.MTP_DECODE
    inp = wl.decode_inputs(cfg)
    q, lens, sinks = inp["q"].to(dev), inp["seq_lens"].to(dev), inp["sinks"].to(dev)
    B, q_len, Hq, D = q.shape
    kv = wl.decode_kv_bytes(inp["seq_lens"].tolist(), cfg.num_kv_heads, cfg.head_dim)
    n = rotation(kv)
    caches = [(inp["k_cache"].to(dev), inp["v_cache"].to(dev))]
    caches += [(caches[0][0].clone(), caches[0][1].clone()) for _ in range(n - 1)]
    out = torch.empty(B, q_len, Hq, D, dtype=torch.bfloat16, device=dev)
    chosen = sa.sink_attn_decode_split_size(B, cfg.max_ctx, Hq, cfg.num_kv_heads, D, q_len,
                                            seq_lens=inp["seq_lens"])
    times = {}
    for split in sorted({1024, chosen}):
        ns = -(-cfg.max_ctx // split)
        part = _partials(B, q_len, Hq, ns, D, dev)

        def run(s, i, split=split, ns=ns, part=part):
            kc, vc = caches[i % n]
            sa.sink_attn_decode_multi(q, kc, vc, lens, sinks, split, ns, scale=cfg.scale,
                                      out=out, partials=part, stream=s)
        times[split] = graph_ms(run, stream, reps=max(3, reps // 2))
        del part
    del caches
    torch.cuda.empty_cache()
    return _decode_line("mtp_decode_b64_q4_ctx8192_h64kv8_d64",
                        "multi-token decode KV GB/s (split + merge, graph replay)", kv, chosen,
                        times, n)


def fp8_decode_measurement(dev, stream, reps: int):
    """Decode over FP8 (E4M3) caches: 64 requests x 8192 tokens, 64 / 8 heads,
    d 64, split decode + merge with the library's chunk size (1024 beside it),
    graph replay over rotated cache copies.  GB/s of the one-byte codes read
    (half the bytes of the bf16 line for the same tokens)."""
    cfg = wl.FP8_DECODE
    inp = wl.fp8_decode_inputs(cfg)
    q, lens, sinks = inp["q"].to(dev), inp["seq_lens"].to(dev), inp["sinks"].to(dev)
    ks, vs = inp["k_scale"].to(dev), inp["v_scale"].to(dev)
    B, Hq, D = q.shape
    kv = wl.decode_kv_bytes_fp8(inp["seq_lens"].tolist(), cfg.num_kv_heads, cfg.head_dim)
    n = rotation(kv)
    caches = [(inp["k_cache"].to(dev), inp["v_cache"].to(dev))]
    caches += [(caches[0][0].clone(), caches[0][1].clone()) for _ in range(n - 1)]
    out = torch.empty(B, Hq, D, dtype=torch.bfloat16, device=dev)
    chosen = sa.sink_attn_decode_split_size(B, cfg.max_ctx, Hq, cfg.num_kv_heads, D,
                                            seq_lens=inp["seq_lens"])
    times = {}
    for split in sorted({1024, chosen}):
        ns = -(-cfg.max_ctx // split)
        part = _partials(B, 1, Hq, ns, D, dev)

        def run(s, i, split=split, ns=ns, part=part):
            kc, vc = caches[i % n]
            sa.sink_attn_decode_fp8(q, kc, vc, ks, vs, lens, sinks, split, ns, scale=cfg.scale,
                                    out=out, partials=part, stream=s)
        times[split] = graph_ms(run, stream, reps=max(3, reps // 2))
        del part
    del caches
    torch.cuda.empty_cache()
    return _decode_line("fp8_decode_b64_ctx8192_h64kv8_d64",
                        "decode FP8 KV GB/s (split + merge, graph replay)", kv, chosen, times, n)


def paged_decode_measurement(dev, stream, reps: int, page_size: int = 16):
    """Decode over a paged bf16 cache: the split-decode shape (64 x 8192, 64 / 8
    heads, d 64) in 16-token pages under a random block table (seeded), split
    decode + merge with the library's chunk size (capped at the 254 pages a
    chunk may span; 1024 beside it), graph replay over rotated page pools;
    GB/s of K/V bytes read."""
    cfg = wl.SPLIT_DECODE
    inp = wl.decode_inputs(cfg)
    B, Hkv, L, D = inp["k_cache"].shape
    per = L // page_size
    g = torch.Generator().manual_seed(9)
    perm = torch.randperm(B * per, generator=g).view(B, per).to(torch.int32)
    kv = wl.decode_kv_bytes(inp["seq_lens"].tolist(), cfg.num_kv_heads, cfg.head_dim)
    n = rotation(kv)
    # page p of request b holds its tokens p*P .. p*P+P-1 (one scatter on the GPU)
    kc, vc = inp["k_cache"].to(dev), inp["v_cache"].to(dev)
    kp = torch.empty(B * per, Hkv, page_size, D, dtype=torch.bfloat16, device=dev)
    vp = torch.empty_like(kp)
    idx = perm.view(-1).to(dev).long()
    kp[idx] = kc.view(B, Hkv, per, page_size, D).permute(0, 2, 1, 3, 4).reshape(B * per, Hkv, page_size, D)
    vp[idx] = vc.view(B, Hkv, per, page_size, D).permute(0, 2, 1, 3, 4).reshape(B * per, Hkv, page_size, D)
    del kc, vc
    pools = [(kp, vp)] + [(kp.clone(), vp.clone()) for _ in range(n - 1)]
    bt = perm.to(dev)
    q, lens, sinks = inp["q"].to(dev), inp["seq_lens"].to(dev), inp["sinks"].to(dev)
    Hq = q.shape[1]
    out = torch.empty(B, Hq, D, dtype=torch.bfloat16, device=dev)
    cap = 1 << ((254 * page_size).bit_length() - 1)      # largest power of two <= 254 pages
    chosen = min(cap, sa.sink_attn_decode_split_size(B, L, Hq, Hkv, D, seq_lens=inp["seq_lens"]))
    times = {}
    for split in sorted({1024, chosen}):
        ns = -(-L // split)
        part = _partials(B, 1, Hq, ns, D, dev)

        def run(s, i, split=split, ns=ns, part=part):
            k_, v_ = pools[i % n]
            sa.sink_attn_decode_paged(q, k_, v_, bt, lens, sinks, split, ns, scale=cfg.scale,
                                      out=out, partials=part, stream=s)
        times[split] = graph_ms(run, stream, reps=max(3, reps // 2))
        del part
    del pools, kp, vp
    torch.cuda.empty_cache()
    return _decode_line(f"paged_decode_b64_ctx8192_page{page_size}_h64kv8_d64",
                        "paged decode KV GB/s (split + merge, graph replay)", kv, chosen, times, n,
                        {"split_cap_pages": 254})


def library_split_decode_measurement(dev, stream, reps: int):
    """The split-KV decode shape (64 requests x 8192 tokens, 64 / 8 heads, d 64)
    through the length-aware split + merge with the library's chunk size for
    these equal lengths (1024-token chunks beside it), graph replay over rotated
    cache copies."""
    cfg = wl.SPLIT_DECODE
    chosen = sa.sink_attn_decode_split_size(cfg.batch, cfg.max_ctx, cfg.num_q_heads,
                                            cfg.num_kv_heads, cfg.head_dim,
                                            seq_lens=[cfg.ctx] * cfg.batch)
    x = _decode_buffers(cfg, dev, chosen)
    times = {chosen: graph_ms(_merged(cfg, x), stream, reps=max(3, reps // 2))}
    if chosen != 1024:
        B, Hq, D = x["q"].shape
        x1 = dict(x, split=1024, ns=cfg.num_splits,
                  part=tuple(t.view(B, Hq, *t.shape[3:]) for t in _partials(B, 1, Hq, cfg.num_splits, D, dev)))
        times[1024] = graph_ms(_merged(cfg, x1), stream, reps=max(3, reps // 2))
        del x1
    kv, n = x["kv"], len(x["caches"])
    del x
    torch.cuda.empty_cache()
    return _decode_line(cfg.name.replace("_split1024", "") + "_library_split",
                        "decode KV GB/s (length-aware split + merge, graph replay)", kv, chosen,
                        times, n)


def probes_lib():
    """The benchmark's reference kernels (libbenchprobes.so, built beside the library)."""
    import ctypes
    path = os.path.join(ROOT, "gqa_attention_sinks_prefill_amd", "libbenchprobes.so")
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: run `python -m gqa_attention_sinks_prefill_amd.build_native`")
    return ctypes.CDLL(path)


def hbm_read_reference(dev, stream, reps: int = 10):
    """GB/s of a plain streaming-read kernel (libbenchprobes.so): 4 GiB read
    once per launch, each workgroup a contiguous slice, non-temporal 16-byte
    loads."""
    import ctypes
    lib = probes_lib()
    lib.hbm_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                   ctypes.c_void_p, ctypes.c_void_p]
    nbytes, blocks = 4 << 30, 8192
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    out = torch.zeros(blocks, dtype=torch.int32, device=dev)
    sp = stream.cuda_stream
    run = lambda: lib.hbm_read_probe(buf.data_ptr(), nbytes, blocks, out.data_ptr(), sp)
    for _ in range(10):
        if run() != 0:
            raise RuntimeError("hbm_read_probe failed")
    torch.cuda.synchronize()
    e = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
         for _ in range(reps)]
    for a, b in e:
        a.record(stream)
        run()
        b.record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in e]))
    del buf
    return {"kernel": "hbm_read_probe (contiguous slices, non-temporal 16-byte loads, 8192 x 256 threads)",
            "bytes": nbytes, "value": round(nbytes / (ms * 1e-3) / 1e9, 1), "unit": "GB/s"}


def mfma_rate_reference(dev, stream, operands: torch.Tensor, reps: int = 5, iters: int = 40000):
    """TFLOP/s of a plain loop of independent bf16 32x32x16 MFMAs on every SIMD
    (libbenchprobes.so; 2 waves per SIMD), with operands read from `operands`
    (a bf16 tensor of the workload: they change from one MFMA to the next, as
    the prefill's do) and with all operands 1.0.  The chip holds a lower clock
    while its matrix units switch random data, so the first rate is the
    ceiling that power leaves for bf16 contractions over such inputs."""
    import ctypes
    lib = probes_lib()
    lib.mfma_rate_probe.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                    ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    blocks = 2 * cus
    out = torch.zeros(blocks, dtype=torch.int32, device=dev)
    sp = stream.cuda_stream
    flop = blocks * 4 * iters * 16 * 2 * 32 * 32 * 16
    res = {"kernel": f"mfma_rate_probe (v_mfma_f32_32x32x16_bf16 loop, {blocks} x 256 threads, "
                     f"{iters} x 16 MFMAs per wave)", "unit": "TFLOP/s"}
    for name, ptr, nbytes in (("workload_operands", operands.data_ptr(),
                               operands.numel() * operands.element_size()),
                              ("constant_operands", None, 0)):
        run = lambda: lib.mfma_rate_probe(ptr, nbytes, blocks, iters, out.data_ptr(), sp)
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 0.2:       # settle the clock under this load
            if run() != 0:
                raise RuntimeError("mfma_rate_probe failed")
            torch.cuda.synchronize()
        e = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(reps)]
        for a, b in e:
            a.record(stream)
            run()
            b.record(stream)
        torch.cuda.synchronize()
        ms = float(np.mean([a.elapsed_time(b) for a, b in e]))
        res[name] = round(flop / (ms * 1e-3) / 1e12, 1)
    res["value"] = res["workload_operands"]
    res["frac_of_peak"] = round(res["workload_operands"] / PEAK_BF16_TFLOPS, 4)
    return res


ROTATE_BYTES = 4 << 30


def rotation(touched_bytes: float, target: int = ROTATE_BYTES) -> int:
    """Copies of a call's inputs to cycle through so that one round of them
    touches >= `target` bytes (4 GiB, 16x the 256 MiB Infinity Cache): a timed
    call then finds its bytes in HBM, not left in that cache by the calls
    before it.  At most 20, the calls one timed graph holds."""
    return int(min(20, max(1, -(-int(target) // max(int(touched_bytes), 1)))))


def graph_ms(run, stream, calls: int = 20, reps: int = 10) -> float:
    """Mean device time of one call: `calls` calls captured in one HIP graph,
    replayed `reps` times between HIP events on `stream` (no host launch
    overhead inside the timed region -- what a serving loop that replays a
    captured step sees).  `run(s, i)` enqueues call i on stream s."""
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        for i in range(10):
            run(side, i)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cap = torch.cuda.current_stream()
        for i in range(calls):
            run(cap, i)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        graph.replay()
        torch.cuda.synchronize()
        e = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(reps)]
        for a, b in e:
            a.record(stream)
            graph.replay()
            b.record(stream)
        torch.cuda.synchronize()
    del graph
    return float(np.mean([a.elapsed_time(b) for a, b in e])) / calls


def _decode_buffers(cfg, dev, split=None):
    """Inputs of a decode workload on the GPU, with `rotation` copies of the
    caches, partials for chunks of `split` tokens (the config's by default),
    and the CPU inputs (for the oracle leg)."""
    d = wl.decode_inputs(cfg)
    q, kc, vc = d["q"].to(dev), d["k_cache"].to(dev), d["v_cache"].to(dev)
    B, Hq, D = q.shape
    split = cfg.split_size if split is None else split
    ns = -(-cfg.max_ctx // split)
    kv = wl.decode_kv_bytes(d["seq_lens"].tolist(), cfg.num_kv_heads, cfg.head_dim)
    n = rotation(kv)
    caches = [(kc, vc)] + [(kc.clone(), vc.clone()) for _ in range(n - 1)]
    return dict(q=q, caches=caches, lens=d["seq_lens"].to(dev), sinks=d["sinks"].to(dev), ns=ns,
                split=split,
                part=(torch.empty(B, Hq, ns, D, device=dev), torch.empty(B, Hq, ns, device=dev),
                      torch.empty(B, Hq, ns, device=dev)),
                out=torch.empty(B, Hq, D, dtype=torch.bfloat16, device=dev),
                lse=torch.empty(B, Hq, device=dev),
                counters=sa.decode_counters(B, Hq, kc.shape[1], 1, dev), kv=kv, cpu=d)


def _split_merge(cfg, x):
    def run(s, i):
        kc, vc = x["caches"][i % len(x["caches"])]
        sa.sink_attn_decode(x["q"], kc, vc, x["lens"], x["sinks"], x["split"], x["ns"],
                            scale=cfg.scale, out=x["out"], partials=x["part"], stream=s)
    return run


def _merged(cfg, x, lse=False):
    def run(s, i):
        kc, vc = x["caches"][i % len(x["caches"])]
        sa.sink_attn_decode_merged(x["q"], kc, vc, x["lens"], x["sinks"], x["split"], x["ns"],
                                   scale=cfg.scale, out=x["out"], partials=x["part"],
                                   lse=x["lse"] if lse else None, stream=s)
    return run


def _one_launch(cfg, x):
    def run(s, i):
        kc, vc = x["caches"][i % len(x["caches"])]
        sa.sink_attn_decode_fused(x["q"], kc, vc, x["lens"], x["sinks"], x["split"],
                                  x["ns"], scale=cfg.scale, counters=x["counters"],
                                  out=x["out"], partials=x["part"], stream=s)
    return run


def ragged_decode_measurement(dev, stream, batch: int, reps: int, keep: dict | None = None):
    """KV GB/s of ragged decode over contexts U[1024, 32768] (64 / 8 heads, d 64)
    through sink_attn_decode_merged (chunks past a request's end write no
    state; the merge stops at the last chunk with keys), with the chunk size
    sink_attn_decode_split_size picks for the shape; device time from graph
    replay.  Beside it: the same call with 1024-token chunks, and split decode
    + sink_attn_merge_states.  B = 1 and 8 are latency bound.  With `keep`,
    one more call (with lse) leaves the CPU inputs and the outputs there for
    the oracle leg."""
    cfg = wl.ragged_decode(batch)
    x = _decode_buffers(cfg, dev)
    split = sa.sink_attn_decode_split_size(batch, cfg.max_ctx, cfg.num_q_heads,
                                           cfg.num_kv_heads, cfg.head_dim,
                                           seq_lens=x["cpu"]["seq_lens"])
    if split != cfg.split_size:
        B, Hq, D = x["q"].shape
        ns = -(-cfg.max_ctx // split)
        x.update(split=split, ns=ns, part=(torch.empty(B, Hq, ns, D, device=dev),
                                           torch.empty(B, Hq, ns, device=dev),
                                           torch.empty(B, Hq, ns, device=dev)))
    reps = max(3, reps // 2)
    two = graph_ms(_split_merge(cfg, x), stream, reps=reps)
    ms = graph_ms(_merged(cfg, x), stream, reps=reps)
    line = {"workload": cfg.name, "unit": "GB/s",
            "metric": "decode KV GB/s (split + length-aware merge, graph replay)",
            "split_size": split, "mean_ms": round(ms, 4), "split_merge_ms_same_run": round(two, 4)}
    if split != cfg.split_size:
        B, Hq, D = x["q"].shape
        ns1 = cfg.num_splits
        x1024 = dict(x, split=cfg.split_size, ns=ns1,
                     part=(torch.empty(B, Hq, ns1, D, device=dev), torch.empty(B, Hq, ns1, device=dev),
                           torch.empty(B, Hq, ns1, device=dev)))
        line["split1024_ms_same_run"] = round(graph_ms(_merged(cfg, x1024), stream, reps=reps), 4)
        del x1024
    kv = x["kv"]
    gbs = kv / (ms * 1e-3) / 1e9
    line.update({"value": round(gbs, 1), "algorithmic_bytes_per_step": kv,
                 "cache_copies_rotated": len(x["caches"]), "latency_bound": batch < 32,
                 "roofline": {"bound": "hbm", "peak": PEAK_HBM_GBS,
                              "frac": round(gbs / PEAK_HBM_GBS, 4)}})
    if keep is not None:
        x["out"].fill_(float("nan"))
        x["lse"].fill_(float("nan"))
        _merged(cfg, x, lse=True)(stream, 0)
        torch.cuda.synchronize()
        keep.update(cpu=x["cpu"], name=cfg.name, out=x["out"].cpu(), lse=x["lse"].cpu(), kv=kv)
    del x
    torch.cuda.empty_cache()
    return line


def one_launch_decode_measurement(dev, stream, cfg, reps: int):
    """sink_attn_decode_fused (split decode whose last workgroup per slice
    merges) against split + merge, both from graph replay in the same run."""
    x = _decode_buffers(cfg, dev)
    reps = max(3, reps // 2)
    two = graph_ms(_split_merge(cfg, x), stream, reps=reps)
    one = graph_ms(_one_launch(cfg, x), stream, reps=reps)
    two = min(two, graph_ms(_split_merge(cfg, x), stream, reps=reps))
    one = min(one, graph_ms(_one_launch(cfg, x), stream, reps=reps))
    gbs = x["kv"] / (one * 1e-3) / 1e9
    kv = x["kv"]
    del x
    torch.cuda.empty_cache()
    return {"workload": cfg.name, "value": round(gbs, 1), "unit": "GB/s",
            "metric": "decode KV GB/s, one launch (graph replay)", "mean_ms": round(one, 4),
            "split_merge_ms_same_run": round(two, 4), "algorithmic_bytes_per_step": kv,
            "cache_copies_rotated": rotation(kv),
            "roofline": {"bound": "hbm", "peak": PEAK_HBM_GBS, "frac": round(gbs / PEAK_HBM_GBS, 4)}}


def copy_calibration(dev, reps: int):
    """A plain device-to-device copy of 1 GiB: reads and writes exactly 2^30
    bytes each, the reference that scales the HBM byte counters."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(max(1, reps)):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "reps": max(1, reps)}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=30, help="untimed steps before the timed ones")
    ap.add_argument("--settle-ms", type=float, default=400.0,
                    help="wall time of untimed steps run before the warm-up steps, whatever "
                         "--warmup says (the shader clock settles under some tens of ms of load)")
    ap.add_argument("--cpu-seconds", type=float, default=150.0,
                    help="host time budget of the oracle per prefill workload (0 disables the "
                         "oracle leg)")
    ap.add_argument("--only", choices=("all", "prefill", "decode", "varlen", "ragged", "mtp",
                                       "fp8", "paged", "read", "mfma"),
                    default="all",
                    help="launch only one part of the step, or only the head_dim 128 varlen "
                         "prefill / the B = 128 ragged decode / the multi-token decode / the "
                         "FP8-cache decode / the paged decode / the streaming-read or MFMA-rate "
                         "reference (for hardware-counter runs)")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the extra workloads' lines (and their oracle checks)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain 1 GiB device-to-device copy instead (scales HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)
    if args.copy_calibration:
        copy_calibration(dev, args.steps)
        return
    if args.only in ("varlen", "ragged", "mtp", "fp8", "paged", "read", "mfma"):
        stream = torch.cuda.current_stream()
        line = {"varlen": lambda: varlen_prefill_measurement(dev, stream, args.steps),
                "ragged": lambda: ragged_decode_measurement(dev, stream, 128, args.steps),
                "mtp": lambda: multi_decode_measurement(dev, stream, args.steps),
                "fp8": lambda: fp8_decode_measurement(dev, stream, args.steps),
                "paged": lambda: paged_decode_measurement(dev, stream, args.steps),
                "read": lambda: hbm_read_reference(dev, stream, max(3, args.steps)),
                "mfma": lambda: mfma_rate_reference(
                    dev, stream, wl.prefill_inputs(wl.GPTOSS_PREFILL)["k"].to(dev),
                    max(3, args.steps))}[args.only]()
        line["note"] = f"--only {args.only}: this workload alone"
        print(json.dumps(line), flush=True)
        return

    # ---- inputs, resident in HBM before timing ---------------------------------
    pcfg, dcfg = wl.GPTOSS_PREFILL, wl.SPLIT_DECODE
    run_p, run_d = args.only in ("all", "prefill"), args.only in ("all", "decode")
    pre = wl.prefill_inputs(pcfg) if run_p else wl.prefill_inputs(wl.TINY_PREFILL)
    dec = wl.decode_inputs(dcfg) if run_d else wl.decode_inputs(
        wl.DecodeConfig("unused", 1, 64, None, 64, 64, 8, 64, (-4.0, 4.0), 64, 0))
    q, k, v = pre["q"].to(dev), pre["k"].to(dev), pre["v"].to(dev)
    sinks_p, cu = pre["sinks"].to(dev), pre["cu_seqlens"].to(dev)
    out = torch.empty_like(q)
    dq, kc, vc = dec["q"].to(dev), dec["k_cache"].to(dev), dec["v_cache"].to(dev)
    lens, sinks_d = dec["seq_lens"].to(dev), dec["sinks"].to(dev)
    kv_bytes = wl.decode_kv_bytes(dec["seq_lens"].tolist(), dcfg.num_kv_heads, dcfg.head_dim)
    # copies of the caches, cycled through step by step (>= 4 GiB per round)
    caches = [(kc, vc)] + [(kc.clone(), vc.clone()) for _ in range(rotation(kv_bytes) - 1)]
    B, Hq, D = dq.shape
    ns = -(-kc.shape[2] // dcfg.split_size)
    po = torch.empty(B, Hq, ns, D, device=dev)
    pm = torch.empty(B, Hq, ns, device=dev)
    pd = torch.empty(B, Hq, ns, device=dev)
    dout = torch.empty(B, Hq, D, dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    log("inputs resident in HBM")

    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]

    def step(i, e=None, copy=None):
        kc_i, vc_i = caches[i % len(caches) if copy is None else copy]
        if e: e[0].record(stream)
        if run_p:
            sa.sink_attn_prefill(q, k, v, sinks_p, cu, pre["max_seqlen"], causal=True,
                                 scale=pcfg.scale, out=out, stream=stream)
        if e: e[1].record(stream)
        if run_d:
            sa.sink_attn_decode_split(dq, kc_i, vc_i, lens, sinks_d, dcfg.split_size, ns,
                                      scale=dcfg.scale, part_o=po, part_m=pm, part_d=pd,
                                      stream=stream)
        if e: e[2].record(stream)
        if run_d:
            sa.sink_attn_merge_states(po, pm, pd, out=dout, stream=stream)
        if e: e[3].record(stream)

    # ---- settle (wall-time bound), warm-up, timed steps ---------------------------
    t_settle, n_settle = time.perf_counter(), 0
    while True:
        step(n_settle)
        n_settle += 1
        if n_settle % 8 == 0:
            torch.cuda.synchronize()
            if (time.perf_counter() - t_settle) * 1e3 >= args.settle_ms:
                break
    settle_ms = (time.perf_counter() - t_settle) * 1e3
    log(f"settled: {n_settle} steps in {settle_ms:.0f} ms")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, ev[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log(f"{args.steps} timed steps done")

    pre_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    split_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    merge_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in ev]))
    flops = wl.prefill_flops(pre["seqlens"].tolist(), pcfg.num_q_heads, pcfg.head_dim)
    tflops = flops / (pre_ms * 1e-3) / 1e12
    dec_gbs = kv_bytes / ((split_ms + merge_ms) * 1e-3) / 1e9
    split_gbs = kv_bytes / (split_ms * 1e-3) / 1e9

    # the decode with one cache copy read over and over (for comparison only)
    single = None
    if run_d:
        es = [[torch.cuda.Event(enable_timing=True) for _ in range(4)]
              for _ in range(max(5, args.steps))]
        for i, e in enumerate(es):
            step(i, e, copy=0)
        torch.cuda.synchronize()
        one_ms = float(np.mean([e[1].elapsed_time(e[3]) for e in es]))
        single = {"ms": round(one_ms, 4), "value": round(kv_bytes / (one_ms * 1e-3) / 1e9, 1),
                  "unit": "GB/s",
                  "note": "split + merge re-reading one 1.07 GB cache copy every step "
                          "(part of it can stay in the Infinity Cache); not the reported value"}

    traffic_p = measured_traffic("prefill")
    traffic_d = measured_traffic("decode_split")
    res = {
        "metric": "sink-attn prefill TFLOP/s & decode KV GB/s, % of MI355X roofline",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": round(settle_ms, 1),
        "settle_steps": n_settle,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded randn / uniform inputs of the workload shapes; no weights)",
        "config": {"workload": pcfg.name, "decode_workload": dcfg.name,
                   "seq_len": 8192, "num_q_heads": 64, "num_kv_heads": 8, "head_dim": 64,
                   "causal": True, "decode_batch": dcfg.batch, "decode_ctx": dcfg.ctx,
                   "decode_split_size": dcfg.split_size,
                   "decode_cache_copies_rotated": len(caches), "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2),
                     "peak": round(PEAK_BF16_TFLOPS, 1), "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic_p, "kernel": "prefill_kernel<64,4,2>",
                     "algorithmic_flop_per_launch": flops, "mean_launch_ms": round(pre_ms, 4)},
        "decode": {"value": round(dec_gbs, 1), "unit": "GB/s",
                   "metric": "decode KV GB/s (split + merge)",
                   "ms": round(split_ms + merge_ms, 4), "split_ms": round(split_ms, 4),
                   "merge_ms": round(merge_ms, 4),
                   "roofline": {"bound": "hbm", "achieved": round(dec_gbs, 1),
                                "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                "frac": round(dec_gbs / PEAK_HBM_GBS, 4),
                                "kernels": "decode_split_kernel<64,1,4,false,false> + "
                                           "merge_rows_kernel<64>",
                                "algorithmic_bytes_per_step": kv_bytes,
                                "split_only": {"achieved": round(split_gbs, 1),
                                               "frac": round(split_gbs / PEAK_HBM_GBS, 4),
                                               "traffic": traffic_d}},
                   "single_cache_copy": single},
        "device": {"name": props.name, "compute_units": props.multi_processor_count,
                   "gcn_arch": getattr(props, "gcnArchName", "")},
    }
    oracle_on = args.cpu_seconds > 0
    keep_varlen = {} if oracle_on else None
    keep_ragged = {b: ({} if oracle_on else None) for b in wl.RAGGED_BATCHES}
    if run_p and not args.no_extra:
        r2, r4 = max(3, args.steps // 2), max(3, args.steps // 4)
        jobs = [lambda: varlen_prefill_measurement(dev, stream, r2, keep=keep_varlen),
                lambda: chunked_prefill_measurement(dev, stream, r2),
                lambda: multi_decode_measurement(dev, stream, r2),
                lambda: fp8_decode_measurement(dev, stream, r2),
                lambda: paged_decode_measurement(dev, stream, r2),
                lambda: library_split_decode_measurement(dev, stream, r2),
                lambda: kv_append_measurement(dev, stream, r2)]
        jobs += [lambda b=b: ragged_decode_measurement(dev, stream, b, r4, keep=keep_ragged[b])
                 for b in wl.RAGGED_BATCHES]
        jobs += [lambda c=c: one_launch_decode_measurement(dev, stream, c, r4)
                 for c in (wl.SPLIT_DECODE, wl.ragged_decode(1), wl.ragged_decode(128))]
        res["extra"] = []
        for job in jobs:
            res["extra"].append(job())
            log(f"extra line {res['extra'][-1]['workload']} done")
    if run_p and not args.no_extra:
        mref = mfma_rate_reference(dev, stream, k)
        res["mfma_rate_reference"] = mref
        res["roofline"]["frac_of_measured_mfma"] = round(tflops / mref["value"], 4)
        for line in res.get("extra", []):
            if line.get("roofline", {}).get("bound") == "mfma":
                line["roofline"]["frac_of_measured_mfma"] = round(line["value"] / mref["value"], 4)
        log("mfma rate reference done")
    if run_d and not args.no_extra:
        ref = hbm_read_reference(dev, stream)
        res["hbm_read_reference"] = ref
        res["decode"]["frac_of_measured_read"] = round(dec_gbs / ref["value"], 4)
        res["decode"]["roofline"]["split_only"]["frac_of_measured_read"] = round(
            split_gbs / ref["value"], 4)
    if args.only != "all":
        res["note"] = f"--only {args.only}: the other part of the step was not launched"

    # ---- oracle leg: CPU baseline per workload and all-row parity --------------
    res["cpu_baseline"] = None
    if oracle_on and run_p:
        import oracle   # test infrastructure: only this leg of the benchmark uses it
        per, parity = [], []
        lse = torch.empty(out.shape[0], out.shape[1], device=dev)
        sa.sink_attn_prefill(q, k, v, sinks_p, cu, pre["max_seqlen"], causal=True,
                             scale=pcfg.scale, out=out, lse=lse, stream=stream)
        torch.cuda.synchronize()
        b, p = oracle_prefill_leg(pre, pcfg, out, lse, args.cpu_seconds)
        per.append(b)
        parity.append(p)
        log(f"oracle {pcfg.name}: {b['seconds']} s")
        tiny = wl.prefill_inputs(wl.TINY_PREFILL)
        t_out = torch.empty(tiny["q"].shape, dtype=torch.bfloat16, device=dev)
        t_lse = torch.empty(tiny["q"].shape[:2], device=dev)
        sa.sink_attn_prefill(tiny["q"].to(dev), tiny["k"].to(dev), tiny["v"].to(dev),
                             tiny["sinks"].to(dev), tiny["cu_seqlens"].to(dev),
                             tiny["max_seqlen"], causal=True, scale=wl.TINY_PREFILL.scale,
                             out=t_out, lse=t_lse, stream=stream)
        torch.cuda.synchronize()
        b, p = oracle_prefill_leg(tiny, wl.TINY_PREFILL, t_out, t_lse, args.cpu_seconds)
        per.append(b)
        parity.append(p)
        if run_d:
            d_lse = torch.empty(B, Hq, device=dev)
            sa.sink_attn_merge_states(po, pm, pd, out=dout, lse=d_lse, stream=stream)
            torch.cuda.synchronize()
            b, p = oracle_decode_leg(dec, dcfg.name, dout, d_lse, kv_bytes)
            per.append(b)
            parity.append(p)
            log(f"oracle {dcfg.name}: {b['seconds']} s")
        for kr in keep_ragged.values():
            if kr:
                b, p = oracle_decode_leg(kr["cpu"], kr["name"], kr["out"], kr["lse"], kr["kv"])
                per.append(b)
                parity.append(p)
                log(f"oracle {kr['name']}: {b['seconds']} s")
                kr.clear()
        if keep_varlen:
            b, p = oracle_prefill_leg(keep_varlen["inp"], keep_varlen["cfg"], keep_varlen["out"],
                                      keep_varlen["lse"], args.cpu_seconds)
            per.append(b)
            parity.append(p)
            log(f"oracle {keep_varlen['cfg'].name}: {b['seconds']} s")
        head = dict(per[0])
        res["cpu_baseline"] = {"value": head["value"], "unit": head["unit"], "cores": head["cores"],
                               "kind": "oracle", "cpu_model": cpu_model(),
                               "sample": head["sample"] + f" ({pcfg.name})",
                               "per_config": per}
        res["parity"] = {"all_ok": all(p["ok"] for p in parity), "per_config": parity}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
