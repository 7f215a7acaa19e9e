#!/usr/bin/env python3
"""LRKV decode benchmark on one MI355X.

Workload: B = 8 requests of T = 4096 tokens, H = 16 heads, d_h = 128, r = 56, bf16 factored
paged cache (16-token pages, identity page table), one layer.  The cache is built on the
GPU by lrkv_append from X ~ N(0,1) and N(0, 1/fan_in) weights (synthetic inputs), then
replicated so that consecutive steps read different copies (more bytes than the 256 MB
Infinity Cache holds, so every step reads HBM).

One step = one decode step of the hot path: lrkv_append_pq (the 8 new tokens' rows
appended at position 4095 into the step's pool copy, and each query row's private queries
p = q B_K formed, in one launch), then lrkv_decode_pq of one query row per request over all
4096 positions.  Its output equals lrkv_append + lrkv_decode bit for bit (checked before the
timing); that path is timed too and reported beside it.  `value` = algorithmic cache bytes
per step (eq 9 of the LRKV notes: 2 b (sum of T) (d_h + H r)) / measured step time, in GB/s.

Printed: one JSON line on stdout; progress on stderr.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("LRKV decode: achieved HBM GB/s (% peak) + query-heads·tokens/s, B=8 T=4096")
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E peak, 8 TB/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "lrkv_decode_c1_traffic.json")


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


# the sources that decide the decode call's kernels and launches (the traffic record holds
# for them only)
DECODE_SOURCES = ("lrkv_api.hip", "lrkv_decode.hip", "lrkv_device.h", "lrkv_launch.h",
                  "lrkv_private.h")


def source_digest() -> str:
    csrc = os.path.join(ROOT, "factored_rank_kv_amd", "csrc")
    h = hashlib.sha256()
    for f in DECODE_SOURCES:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def traffic_record():
    """HBM bytes per decode call from the committed rocprofv3 counter runs, if they were taken
    on the current kernel sources; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_digest") != source_digest():
        return None
    return rec


def device_weights(w, dev):
    """bf16 codes on the device; the append weights (held [d][...]) in the output-major order
    lrkv_append reads ([...][d])."""
    import torch

    out = {}
    for k, v in w.items():
        if k in ("W_SK", "W_SV", "U_K", "U_V"):
            v = np.ascontiguousarray(v.reshape(v.shape[0], -1).T)
        out[k] = torch.from_numpy(bf16_codes(v).view(np.int16)).to(dev)
    return out


def bf16_codes(x):
    import synth

    return synth.to_bf16_bits(x)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--replicas", type=int, default=12,
                    help="pool copies rotated across steps (12 x 128 MiB = 1.5 GiB)")
    ap.add_argument("--chunk", type=int, default=0, help="chunk_tokens for lrkv_decode (0 = auto)")
    ap.add_argument("--graph", type=int, default=1, help="replay the step loop from a HIP graph")
    ap.add_argument("--cpu-baseline", type=int, default=1)
    ap.add_argument("--other-decodes", type=int, default=1,
                    help="also time decode on the ragged B=32 and the B=4 x 131072 workloads")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--prefill", type=int, default=1,
                    help="also time the B=4 x 8192 prefill (append + multi-query attention)")
    ap.add_argument("--rope", type=int, default=1,
                    help="also time the rotary decode (lrkv_decode_rope) on the same workload")
    ap.add_argument("--next-rows", type=int, default=1,
                    help="also time the key-norm and grouped decodes, the key-norm step of an "
                         "append and the page copy of a shared-prefix fork")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration runs)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): the LRKV decode "
              "path is built and timed on a single GPU", file=sys.stderr)
        sys.exit(2)

    import torch

    import factored_rank_kv_amd as F
    import synth

    dev = torch.device("cuda:0")
    work = synth.C1
    B, T, H, dh, r, d = work.B, work.lens[0], work.H, work.d_h, work.r, work.d
    lay = F.lrkv_layout(H, dh, r, work.page_size, F.LRKV_BF16)
    page_bytes = F.lrkv_page_bytes(lay)
    alg_bytes = 2 * 2 * B * T * (dh + H * r)  # eq 9, b = 2, N = 1 layer

    # ---------------- inputs (synthetic, seeded) ----------------
    t0 = time.time()
    w = synth.projection_weights(1, d, H, dh, r)
    wd = device_weights(w, dev)
    X = synth.activations(2, B * T, d)  # row b*T + j is request b, position j
    Xd = torch.from_numpy(bf16_codes(X).view(np.int16)).to(dev)
    del X
    q = synth.queries(3, B, 1, H, dh)
    qd = torch.from_numpy(bf16_codes(q).view(np.int16)).to(dev)
    table, num_pages = synth.page_assignment(0, [T] * B, work.page_size, permute=False)
    tab = torch.from_numpy(table).to(dev)
    lens = torch.full((B,), T, dtype=torch.int32, device=dev)
    log(f"inputs ready in {time.time() - t0:.1f}s; page {page_bytes} B, {num_pages} pages")

    # cache of the T-1 earlier tokens, built by lrkv_append (prefill of each prompt)
    pool0 = torch.zeros(num_pages * page_bytes, dtype=torch.uint8, device=dev)
    req_all = torch.arange(B, dtype=torch.int32, device=dev).repeat_interleave(T - 1)
    pos_all = torch.arange(T - 1, dtype=torch.int32, device=dev).repeat(B)
    rows_prev = (torch.arange(B, device=dev)[:, None] * T +
                 torch.arange(T - 1, device=dev)[None, :]).reshape(-1)
    X_prev = Xd[rows_prev].contiguous()
    F.lrkv_append(lay, X_prev, B * (T - 1), d, wd["W_SK"], wd["W_SV"], wd["U_K"], wd["U_V"],
                  req_all, pos_all, tab, table.shape[1], pool0, num_pages)
    del X_prev, req_all, pos_all
    X_new = Xd[torch.arange(B, device=dev) * T + (T - 1)].contiguous()
    req_new = torch.arange(B, dtype=torch.int32, device=dev)
    pos_new = torch.full((B,), T - 1, dtype=torch.int32, device=dev)
    pools = [pool0] + [pool0.clone() for _ in range(args.replicas - 1)]
    torch.cuda.synchronize()
    log(f"cache built and replicated x{args.replicas} "
        f"({args.replicas * pool0.numel() / 2**30:.2f} GiB)")

    ws_bytes = F.lrkv_decode_workspace_bytes(lay, B, 1, T, args.chunk)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    out = torch.empty((B, 1, H, dh), dtype=torch.int16, device=dev)

    def append(k):
        F.lrkv_append(lay, X_new, B, d, wd["W_SK"], wd["W_SV"], wd["U_K"], wd["U_V"], req_new,
                      pos_new, tab, table.shape[1], pools[k % len(pools)], num_pages)

    def decode(k):
        F.lrkv_decode(lay, qd, B, 1, wd["B_K"], wd["B_V"], pools[k % len(pools)], tab,
                      table.shape[1], lens, T, args.chunk, out, ws, ws_bytes)

    def step_plain(k):
        append(k)
        decode(k)

    # the private queries p = q B_K formed once per query row, with the append
    pq_bytes = F.lrkv_private_queries_bytes(lay, B, 1)
    pbuf = torch.empty(pq_bytes, dtype=torch.uint8, device=dev)

    def append_pq(k):
        F.lrkv_append_pq(lay, X_new, B, d, wd["W_SK"], wd["W_SV"], wd["U_K"], wd["U_V"], req_new,
                         pos_new, tab, table.shape[1], pools[k % len(pools)], num_pages, qd, B, 1,
                         wd["B_K"], pbuf, pq_bytes)

    def decode_pq(k):
        F.lrkv_decode_pq(lay, qd, pbuf, pq_bytes, B, 1, wd["B_V"], pools[k % len(pools)], tab,
                         table.shape[1], lens, T, args.chunk, out, ws, ws_bytes)

    def step(k):
        append_pq(k)
        decode_pq(k)

    # the two paths give the same bits
    step_plain(0)
    torch.cuda.synchronize()
    want = out.clone()
    out.fill_(-1)
    step(0)
    torch.cuda.synchronize()
    if not torch.equal(out, want):
        raise RuntimeError("lrkv_append_pq + lrkv_decode_pq differ from lrkv_append + lrkv_decode")
    del want

    stream = torch.cuda.current_stream()

    def timed(fn, n, use_graph):
        """Average ms per call of fn over exactly n calls (call k reads pool copy k mod the
        number of copies), HIP events on the launch stream around one graph replay."""
        if use_graph:
            g = torch.cuda.CUDAGraph()
            s = torch.cuda.Stream()
            s.wait_stream(stream)
            with torch.cuda.stream(s):
                fn(0)  # warm the capture stream
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=s):
                for k in range(n):
                    fn(k)
            torch.cuda.synchronize()
            g.replay()  # untimed: first replay uploads the graph
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            del g
            return e0.elapsed_time(e1) / n, n
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for k in range(n):
            fn(k)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n, n

    def per_call_us(fn, n):
        """Durations of n single calls, each between two HIP events on the launch stream.  A
        spin kernel first holds the stream while every call is enqueued, so the calls run back
        to back and no event pair spans host launch time."""
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        torch.cuda.synchronize()
        torch.cuda._sleep(200_000_000)  # ~0.1 s of spinning on one wavefront
        for k in range(n):
            evs[k].record(stream)
            fn(k)
        evs[n].record(stream)
        torch.cuda.synchronize()
        return np.array([evs[k].elapsed_time(evs[k + 1]) * 1e3 for k in range(n)])

    # ---------------- warmup + timed steps ----------------
    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    use_graph = bool(args.graph)
    ms_step, n_steps = timed(step, args.steps, use_graph)
    ms_decode, _ = timed(decode_pq, args.steps, use_graph)
    ms_append, _ = timed(append_pq, args.steps, use_graph)
    log(f"step {ms_step * 1e3:.2f} us (lrkv_decode_pq {ms_decode * 1e3:.2f} us, lrkv_append_pq "
        f"{ms_append * 1e3:.2f} us), graph={use_graph}, {n_steps} steps")
    ms_step_plain, _ = timed(step_plain, args.steps, use_graph)
    ms_decode_plain, _ = timed(decode, args.steps, use_graph)
    ms_append_plain, _ = timed(append, args.steps, use_graph)
    log(f"plain step {ms_step_plain * 1e3:.2f} us (lrkv_decode {ms_decode_plain * 1e3:.2f} us, "
        f"lrkv_append {ms_append_plain * 1e3:.2f} us)")
    calls = per_call_us(decode_pq, max(240, args.steps))
    pct = {p: float(np.percentile(calls, p)) for p in (10, 50, 90)}
    log(f"decode call by event pairs over {len(calls)} calls: p10 {pct[10]:.2f} p50 "
        f"{pct[50]:.2f} p90 {pct[90]:.2f} us")

    # achievable read bound: a plain streaming read (lrkv_read_probe) of the same bytes, on
    # the same rotating pool copies, best over a few grid sizes
    sink = torch.empty(2048 * 16, dtype=torch.uint8, device=dev)
    probe = {}
    for wg in (256, 512, 1024, 2048):
        def read_all(k, wg=wg):
            F.lrkv_read_probe(pools[k % len(pools)], alg_bytes, wg, sink)
        read_all(0)
        probe[wg] = timed(read_all, args.steps, use_graph)[0] * 1e3
    wg_best = min(probe, key=probe.get)
    read_us = probe[wg_best]
    log("read probe over the call's bytes: " +
        ", ".join(f"{wg} wg {us:.2f} us" for wg, us in probe.items()) +
        f"; decode call = {ms_decode * 1e3 / read_us:.3f} x the best read")

    if args.copy_probe:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        log(f"copy probe: 1 GiB copy {e0.elapsed_time(e1) / 10:.3f} ms = "
            f"{2 * (1 << 30) / (e0.elapsed_time(e1) / 10 * 1e-3) / 1e9:.0f} GB/s (read+write)")
        del src, dst

    step_s = ms_step * 1e-3
    dec_s = ms_decode * 1e-3
    value = alg_bytes / step_s / 1e9
    achieved = alg_bytes / dec_s / 1e9
    trec = traffic_record()
    roofline = {
        "bound": "hbm",
        "kernel": "lrkv_decode_pq call (decode_split_kernel with the private queries given + "
                  "merge_expand_kernel)",
        "achieved": round(achieved, 1),
        "peak": PEAK_HBM_GBS,
        "unit": "GB/s",
        "frac": round(achieved / PEAK_HBM_GBS, 4),
        "traffic": None if trec is None else trec["hbm_bytes_per_call"],
        "algorithmic_bytes": alg_bytes,
        "avg_call_us": round(ms_decode * 1e3, 3),
        "call_us_p10_p50_p90": [round(pct[10], 3), round(pct[50], 3), round(pct[90], 3)],
        "calls_in_distribution": int(len(calls)),
        "achieved_at_p50": round(alg_bytes / (pct[50] * 1e-6) / 1e9, 1),
        "read_probe": {"what": "plain streaming read of the same bytes (lrkv_read_probe)",
                       "us": round(read_us, 3), "workgroups": wg_best,
                       "GB/s": round(alg_bytes / (read_us * 1e-6) / 1e9, 1),
                       "frac": round(alg_bytes / (read_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                       "call_over_probe": round(ms_decode * 1e3 / read_us, 4)},
    }

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": n_steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "accumulate": "f32",
        "data": "synthetic",
        "config": {"workload": work.name, "B": B, "T": T, "H": H, "d_h": dh, "r": r, "d": d,
                   "page_size": work.page_size, "layout": "identity page table",
                   "step": "lrkv_append_pq (B new rows + the private queries, one launch) + "
                           "lrkv_decode_pq (q_len=1)",
                   "pool_replicas": len(pools), "chunk_tokens": args.chunk,
                   "hip_graph": use_graph},
        "pct_of_peak_hbm": round(100 * value / PEAK_HBM_GBS, 2),
        "query_head_tokens_per_s": round(H * B * T / step_s, 1),
        "query_heads_per_s": round(H * B / step_s, 1),
        "decode_only_gbps": round(achieved, 1),
        "append_us": round(ms_append * 1e3, 3),
        "plain_step": {"step": "lrkv_append + lrkv_decode (private queries formed in every "
                               "split workgroup)",
                       "step_us": round(ms_step_plain * 1e3, 3),
                       "decode_us": round(ms_decode_plain * 1e3, 3),
                       "append_us": round(ms_append_plain * 1e3, 3),
                       "GB/s": round(alg_bytes / (ms_step_plain * 1e-3) / 1e9, 1)},
        "roofline": roofline,
        "cpu_baseline": None,
    }

    if args.rope:
        # rotary decode (LRKV notes §8) on the same rotating pools and queries
        cs = torch.from_numpy(synth.rope_table(T, dh)).to(dev)
        rws = F.lrkv_decode_rope_workspace_bytes(lay, B, 1, T, 0)
        rws_t = torch.empty(rws, dtype=torch.uint8, device=dev)

        def rope_decode(k):
            F.lrkv_decode_rope(lay, qd, B, 1, wd["B_K"], wd["B_V"], pools[k % len(pools)], tab,
                               table.shape[1], lens, T, 0, cs, T, out, rws_t, rws)

        for k in range(5):
            rope_decode(k)
        ms_rope, n_rope = timed(rope_decode, 96, use_graph)
        rope_calls = per_call_us(rope_decode, 96)
        pairs = B * T * H
        # per (token, head): key block on MFMA 2 d_h r; turn + dot 4 d_h; values 2 (d_h + r) x 2
        fl_mfma = pairs * 2 * dh * r
        fl_valu = pairs * (4 * dh + 4 * (dh + r))
        table_bytes = T * dh * 4
        t_s = ms_rope * 1e-3
        terms = {"hbm": (alg_bytes + table_bytes) / (PEAK_HBM_GBS * 1e9),
                 "mfma": fl_mfma / (PEAK_BF16_TFLOPS * 1e12),
                 "alu": fl_valu / (PEAK_FP32_TFLOPS * 1e12)}
        bound = max(terms, key=terms.get)
        result["rope_decode"] = {
            "workload": work.name + "_rope", "call_us": round(ms_rope * 1e3, 3),
            "call_us_p10_p50_p90": [round(float(np.percentile(rope_calls, p)), 3)
                                    for p in (10, 50, 90)],
            "achieved_gbs": round(alg_bytes / t_s / 1e9, 1),
            "roofline": {"bound": bound, "terms_us": {k: round(v * 1e6, 3) for k, v in terms.items()},
                         "frac_of_bound": round(terms[bound] / t_s, 4),
                         "mfma_flop": fl_mfma, "valu_flop": fl_valu,
                         "bytes": alg_bytes + table_bytes},
        }
        log(f"rope decode: {ms_rope * 1e3:.2f} us per call ({alg_bytes / t_s / 1e9:.0f} GB/s), "
            f"bound {bound} {terms[bound] * 1e6:.2f} us")
        del rws_t

    if args.next_rows:
        result["next_rows"] = next_rows_bench(torch, F, dev, timed, per_call_us, use_graph, qd,
                                              wd, tab, table.shape[1], lens, B, T, H, dh, r,
                                              num_pages, req_new, pos_new, args.replicas)

    if args.prefill:
        result["prefill"] = prefill_bench(torch, F, synth, dev)
    if args.other_decodes:
        result["other_decodes"] = other_decodes(torch, F, synth, dev)

    if args.cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(work, w, args.cpu_seconds)

    print(json.dumps(result), flush=True)


PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3  # MI355X fp32 vector


def next_rows_bench(torch, F, dev, timed, per_call_us, use_graph, qd, wd, tab, max_pages, lens,
                    B, T, H, dh, r, num_pages, req_new, pos_new, replicas):
    """The rows after the hot path, on the B=8 x 4096 shape (pools of seeded random bf16 rows,
    rotated across calls as in the main loop; the values do not change the work):
    - decode over a key-norm layout (LRKV notes §8, RMSNorm): the pages carry one reciprocal
      per (head, slot) more;
    - the key-norm step of a decode-step append (8 rows);
    - decode over a grouped layout (LRKV notes §3: 32 heads, r = 32, 2 shared blocks);
    - the device part of a shared-prefix fork: whole-page copies (lrkv_copy_pages)."""
    out_rec = {}
    g = torch.Generator(device=dev)
    g.manual_seed(77)

    def rand_pools(nbytes):
        p0 = torch.randn(nbytes // 2, device=dev, generator=g).to(torch.bfloat16).view(torch.uint8)
        return [p0] + [p0.clone() for _ in range(replicas - 1)]

    def hbm_line(name, lay, q, BK, BV, n_heads, prepare=None, data_bytes=None, pq=False):
        pb = F.lrkv_page_bytes(lay)
        data_bytes = pb if data_bytes is None else data_bytes  # read per page (no padding)
        pools = rand_pools(num_pages * pb)
        if prepare is not None:  # fix up the first copy, then copy it to the others
            prepare(pools[0])
            for p_ in pools[1:]:
                p_.copy_(pools[0])
        ws_bytes = F.lrkv_decode_workspace_bytes(lay, B, 1, T, 0)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        o = torch.empty((B, 1, n_heads, dh), dtype=torch.int16, device=dev)
        if pq:  # the private queries formed once per query row beforehand (lrkv_decode_pq)
            pqb = F.lrkv_private_queries_bytes(lay, B, 1)
            pbuf = torch.empty(pqb, dtype=torch.uint8, device=dev)
            F.lrkv_private_queries(lay, q, B, 1, BK, pbuf, pqb)

        def call(k):
            if pq:
                F.lrkv_decode_pq(lay, q, pbuf, pqb, B, 1, BV, pools[k % len(pools)], tab, max_pages,
                                 lens, T, 0, o, ws, ws_bytes)
            else:
                F.lrkv_decode(lay, q, B, 1, BK, BV, pools[k % len(pools)], tab, max_pages, lens,
                              T, 0, o, ws, ws_bytes)

        for k in range(5):
            call(k)
        ms, _ = timed(call, 96, use_graph)
        calls = per_call_us(call, 96)
        nbytes = num_pages * data_bytes
        t_s = ms * 1e-3
        rec = {"call_us": round(ms * 1e3, 3),
               "call_us_p10_p50_p90": [round(float(np.percentile(calls, p)), 3) for p in (10, 50, 90)],
               "roofline": {"bound": "hbm", "achieved": round(nbytes / t_s / 1e9, 1),
                            "peak": PEAK_HBM_GBS, "unit": "GB/s",
                            "frac": round(nbytes / t_s / 1e9 / PEAK_HBM_GBS, 4),
                            "bytes": nbytes, "page_bytes": pb, "page_data_bytes": data_bytes}}
        log(f"{name}: {ms * 1e3:.2f} us per call, {nbytes / t_s / 1e9:.0f} GB/s "
            f"({100 * nbytes / t_s / 1e9 / PEAK_HBM_GBS:.1f} %)")
        del pools, ws
        return rec

    # control: the plain layout on the same kind of random rows
    lay_p = F.lrkv_layout(H, dh, r, 16, F.LRKV_BF16)
    out_rec["plain_decode_random_rows"] = hbm_line("plain decode, random rows", lay_p, qd,
                                                   wd["B_K"], wd["B_V"], H)
    # key-norm layout: same heads, rank and queries as the main workload
    lay_kn = F.lrkv_layout(H, dh, r, 16, F.LRKV_BF16, 1, 1)
    req_all = torch.arange(B, dtype=torch.int32, device=dev).repeat_interleave(T)
    pos_all = torch.arange(T, dtype=torch.int32, device=dev).repeat(B)

    def real_norms(pool):  # the reciprocals the key-norm step computes for these rows
        F.lrkv_key_norms(lay_kn, wd["B_K"], 1e-6, req_all, pos_all, B * T, tab, max_pages, pool,
                         num_pages)

    kn_data = 16 * 2 * (dh + H * r) * 2 + 16 * H * 2  # eq 9 per page + the reciprocals
    out_rec["key_norm_decode"] = hbm_line("key-norm decode", lay_kn, qd, wd["B_K"], wd["B_V"], H,
                                          prepare=real_norms, data_bytes=kn_data)
    out_rec["key_norm_decode"]["workload"] = "c1_bf16_b8_t4096_key_norm"
    out_rec["key_norm_decode_pq"] = hbm_line("key-norm decode, private queries given", lay_kn, qd,
                                             wd["B_K"], wd["B_V"], H, prepare=real_norms,
                                             data_bytes=kn_data, pq=True)
    out_rec["key_norm_decode_pq"]["workload"] = "c1_bf16_b8_t4096_key_norm"

    # the key-norm step of a decode-step append: 8 rows, every head
    pool_kn = torch.randn(num_pages * F.lrkv_page_bytes(lay_kn) // 2, device=dev,
                          generator=g).to(torch.bfloat16).view(torch.uint8)

    def norms(k):
        F.lrkv_key_norms(lay_kn, wd["B_K"], 1e-6, req_new, pos_new, B, tab, max_pages, pool_kn,
                         num_pages)

    for k in range(5):
        norms(k)
    ms_n, _ = timed(norms, 96, use_graph)
    out_rec["key_norm_step"] = {"rows": B, "call_us": round(ms_n * 1e3, 3)}
    log(f"key-norm step of an 8-row append: {ms_n * 1e3:.2f} us")
    del pool_kn

    # grouped layout: 32 heads, r = 32, two shared blocks
    Hg, rg = 32, 32
    lay_g = F.lrkv_layout(Hg, dh, rg, 16, F.LRKV_BF16, 0, 2)
    qg = torch.randn(B, 1, Hg, dh, device=dev, generator=g).to(torch.bfloat16).view(torch.int16)
    BKg = (torch.randn(Hg, dh, rg, device=dev, generator=g) / rg ** 0.5).to(torch.bfloat16).view(torch.int16)
    BVg = (torch.randn(Hg, dh, rg, device=dev, generator=g) / rg ** 0.5).to(torch.bfloat16).view(torch.int16)
    out_rec["grouped_decode"] = hbm_line("grouped decode (32 heads, r=32, 2 groups)", lay_g, qg,
                                         BKg, BVg, Hg)
    out_rec["grouped_decode"]["workload"] = "bf16_b8_t4096_h32_r32_g2"
    out_rec["grouped_decode_pq"] = hbm_line("grouped decode, private queries given", lay_g, qg,
                                            BKg, BVg, Hg, pq=True)
    out_rec["grouped_decode_pq"]["workload"] = "bf16_b8_t4096_h32_r32_g2"

    # page copies of a shared-prefix fork (copy on write), 256 pages of the main layout
    lay = F.lrkv_layout(H, dh, r, 16, F.LRKV_BF16)
    pb = F.lrkv_page_bytes(lay)
    n_cp = 256
    cp_pool = torch.empty(2 * n_cp * pb, dtype=torch.uint8, device=dev)
    src = torch.arange(n_cp, dtype=torch.int32, device=dev)
    dst = src + n_cp

    def copy(k):
        F.lrkv_copy_pages(lay, cp_pool, src, dst, n_cp)

    for k in range(5):
        copy(k)
    ms_c, _ = timed(copy, 96, use_graph)
    moved = 2 * n_cp * pb
    out_rec["prefix_page_copy"] = {
        "pages": n_cp, "call_us": round(ms_c * 1e3, 3),
        "roofline": {"bound": "hbm", "achieved": round(moved / (ms_c * 1e-3) / 1e9, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(moved / (ms_c * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                     "bytes": moved}}
    log(f"page copy, {n_cp} pages: {ms_c * 1e3:.2f} us ({moved / (ms_c * 1e-3) / 1e9:.0f} GB/s)")
    del cp_pool
    return out_rec


def prefill_bench(torch, F, synth, dev):
    """B=4 prompts of T=8192, d=2048, H=16, d_h=128, r=56: lrkv_append of all 32768 rows
    (the X [W_SK | W_SV | U_K | U_V] product on MFMA) into a permuted 2048-page pool, then
    lrkv_decode with q_len = 8192 (causal multi-query attention on MFMA).  Synthetic X,
    weights and Q (seeded draws, bf16)."""
    work = synth.C4
    B, T, H, dh, r, d = work.B, work.lens[0], work.H, work.d_h, work.r, work.d
    lay = F.lrkv_layout(H, dh, r, work.page_size, F.LRKV_BF16)
    n = B * T
    w = synth.projection_weights(41, d, H, dh, r)
    wd = device_weights(w, dev)
    g = torch.Generator(device=dev)
    g.manual_seed(42)
    X = torch.randn(n, d, device=dev, generator=g).to(torch.bfloat16).view(torch.int16)
    q = torch.randn(B, T, H, dh, device=dev, generator=g).to(torch.bfloat16).view(torch.int16)
    table, npg = synth.page_assignment(43, [T] * B, work.page_size, permute=True)
    tab = torch.from_numpy(table).to(dev)
    pool = torch.zeros(npg * F.lrkv_page_bytes(lay), dtype=torch.uint8, device=dev)
    req = torch.arange(B, dtype=torch.int32, device=dev).repeat_interleave(T)
    pos = torch.arange(T, dtype=torch.int32, device=dev).repeat(B)
    lens = torch.full((B,), T, dtype=torch.int32, device=dev)
    out = torch.empty(B, T, H, dh, dtype=torch.int16, device=dev)
    ws_bytes = F.lrkv_decode_workspace_bytes(lay, B, T, T, 0)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

    def append():
        F.lrkv_append(lay, X, n, d, wd["W_SK"], wd["W_SV"], wd["U_K"], wd["U_V"], req, pos, tab,
                      table.shape[1], pool, npg)

    def attend():
        F.lrkv_decode(lay, q, B, T, wd["B_K"], wd["B_V"], pool, tab, table.shape[1], lens, T, 0,
                      out, ws, ws_bytes)

    def ms_of(fn, reps):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    # the vendor library (hipBLASLt through torch.matmul) on the same plain product, X times
    # the stacked [d x (2 d_h + 2 H r)] weights, without the scatter into pages: context
    # for the append kernel.  After 20 untimed calls of each (the clocks settle), the two are
    # timed in alternation, seven rounds of 10 calls each, and each side reports its median
    # round, so that both see the same conditions.
    Xb = X.view(torch.bfloat16)
    Wcat = torch.randn(d, 2 * dh + 2 * H * r, device=dev, generator=g).to(torch.bfloat16)
    Yb = torch.empty(n, Wcat.shape[1], dtype=torch.bfloat16, device=dev)
    blas = lambda: torch.matmul(Xb, Wcat, out=Yb)
    for _ in range(20):
        append()
        blas()
    rounds_app, rounds_blas = [], []
    for _ in range(7):
        rounds_app.append(ms_of(append, 10))
        rounds_blas.append(ms_of(blas, 10))
    ms_app = sorted(rounds_app)[3]
    ms_blas = sorted(rounds_blas)[3]
    del Wcat, Yb
    ms_att = ms_of(attend, 10)
    fl_app = 2.0 * n * d * (2 * dh + 2 * H * r)
    pairs = B * T * (T + 1) / 2
    fl_att = pairs * H * 4 * (dh + r) + B * T * H * 4 * dh * r  # scores + values, p + expansion
    tf_app = fl_app / (ms_app * 1e-3) / 1e12
    tf_att = fl_att / (ms_att * 1e-3) / 1e12
    log(f"prefill: append {ms_app:.3f} ms ({tf_app:.0f} TFLOP/s; hipBLASLt plain product "
        f"{ms_blas:.3f} ms, ratio {ms_app / ms_blas:.3f}), attention {ms_att:.3f} ms "
        f"({tf_att:.0f} TFLOP/s)")
    return {
        "workload": work.name, "B": B, "T": T, "d": d,
        "append_ms": round(ms_app, 4), "append_tflops": round(tf_app, 1),
        "hipblaslt_plain_product_ms": round(ms_blas, 4),
        "append_rounds_ms": [round(x, 4) for x in rounds_app],
        "hipblaslt_rounds_ms": [round(x, 4) for x in rounds_blas],
        "append_over_hipblaslt": round(ms_app / ms_blas, 4),
        "attention_ms": round(ms_att, 4), "attention_tflops": round(tf_att, 1),
        "roofline_append": {"bound": "mfma", "achieved": round(tf_app, 1),
                            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                            "frac": round(tf_app / PEAK_BF16_TFLOPS, 4),
                            "flop": fl_app},
        "roofline_attention": {"bound": "mfma", "achieved": round(tf_att, 1),
                               "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                               "frac": round(tf_att / PEAK_BF16_TFLOPS, 4),
                               "flop": fl_att},
    }


def other_decodes(torch, F, synth, dev):
    """Single-query decode on the two large workloads, for context next to the headline B=8
    line: B=32 requests of ragged lengths (uniform in 512..32768, permuted pages) and B=4
    requests of 131072 tokens (H=32, r=32).  The cache holds N(0, 1) bf16 draws (the kernels
    do the same work whatever the values); each pool (about 2.2 and 2.4 GiB) is larger than
    the 256 MB Infinity Cache.  Reported at the automatic split size and, for the ragged
    batch, at 768-token chunks."""
    out = {}
    for work, chunks in ((synth.C2, (0, 768)), (synth.C3, (0,))):
        H, dh, r, B = work.H, work.d_h, work.r, work.B
        lay = F.lrkv_layout(H, dh, r, work.page_size, F.LRKV_BF16)
        lens = list(work.lens)
        table, npg = synth.page_assignment(5, lens, work.page_size, permute=True)
        g = torch.Generator(device=dev)
        g.manual_seed(7)
        pool = torch.randn(npg * F.lrkv_page_bytes(lay) // 2, device=dev, generator=g,
                           dtype=torch.bfloat16).view(torch.uint8)
        q = torch.randn(B, 1, H, dh, device=dev, generator=g).to(torch.bfloat16).view(torch.int16)
        BK = (torch.randn(H, dh, r, device=dev, generator=g) / r ** 0.5).to(torch.bfloat16)
        BV = (torch.randn(H, dh, r, device=dev, generator=g) / r ** 0.5).to(torch.bfloat16)
        tab = torch.from_numpy(table).to(dev)
        lt = torch.tensor(lens, dtype=torch.int32, device=dev)
        msl = max(lens)
        alg = 2 * 2 * sum(lens) * (dh + H * r)
        o = torch.empty(B, 1, H, dh, dtype=torch.int16, device=dev)
        pqb = F.lrkv_private_queries_bytes(lay, B, 1)
        pbuf = torch.empty(pqb, dtype=torch.uint8, device=dev)
        F.lrkv_private_queries(lay, q, B, 1, BK.view(torch.int16), pbuf, pqb)
        for ch, pq in [(c, False) for c in chunks] + [(0, True)]:
            n = F.lrkv_decode_workspace_bytes(lay, B, 1, msl, ch)
            ws = torch.empty(n, dtype=torch.uint8, device=dev)

            def call():
                if pq:  # the private queries formed once beforehand (lrkv_decode_pq)
                    F.lrkv_decode_pq(lay, q, pbuf, pqb, B, 1, BV.view(torch.int16), pool, tab,
                                     table.shape[1], lt, msl, ch, o, ws, n)
                else:
                    F.lrkv_decode(lay, q, B, 1, BK.view(torch.int16), BV.view(torch.int16), pool,
                                  tab, table.shape[1], lt, msl, ch, o, ws, n)

            for _ in range(3):
                call()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(20):
                call()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) / 20 * 1e3
            gbs = alg / us / 1e3
            key = work.name + ("" if ch == 0 else f"_chunk{ch}") + ("_pq" if pq else "")
            out[key] = {"call_us": round(us, 2), "algorithmic_bytes": alg,
                        "achieved_gbs": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBS, 4),
                        "chunk_tokens": ch}
            if pq:
                out[key]["private_queries"] = "formed once beforehand by lrkv_private_queries " \
                    "(in a decode step, beside the append), outside the timed calls"
            log(f"{key}: {us:.1f} us per call, {gbs:.0f} GB/s ({100 * gbs / PEAK_HBM_GBS:.1f} %)")
        del pool
        torch.cuda.empty_cache()
    return out


def cpu_baseline(work, weights, target_s):
    """The float64 oracle timed on the host: page walk, reconstruction of K_h and V_h, and
    textbook attention for a sample of the workload's requests.  Its input pool comes from
    the oracle's own Algorithm-1 append of the same synthetic rows (untimed)."""
    import oracle as O
    import synth

    L = O.Layout(work.H, work.d_h, work.r, work.page_size, O.BF16)
    n_req = 2
    T = work.lens[0]
    t0 = time.time()
    w64 = {k: O.bf16_bits_to_f64(bf16_codes(v)) for k, v in weights.items()}
    X = synth.activations(2, n_req * T, work.d)  # same rows as requests 0..n_req-1
    X64 = O.bf16_bits_to_f64(bf16_codes(X))
    table, npg = synth.page_assignment(0, [T] * n_req, work.page_size, permute=False)
    req = np.repeat(np.arange(n_req), T)
    pos = np.tile(np.arange(T), n_req)
    pool = O.append_reference(np.zeros(npg * O.page_bytes(L), np.uint8), L, X64, w64["W_SK"],
                              w64["W_SV"], w64["U_K"], w64["U_V"], req, pos, table)
    q64 = O.bf16_bits_to_f64(bf16_codes(synth.queries(3, work.B, 1, work.H, work.d_h)))[:n_req]
    log(f"cpu baseline: sample pool built in {time.time() - t0:.1f}s")
    passes = 0
    t_total = 0.0
    while t_total < target_s and passes < 100:
        t1 = time.perf_counter()
        O.decode_reference(L, q64, w64["B_K"], w64["B_V"], pool, table, [T] * n_req)
        t_total += time.perf_counter() - t1
        passes += 1
    per_pass = t_total / passes
    sample_bytes = 2 * 2 * n_req * T * (work.d_h + work.H * work.r)
    blas = blas_info()
    threads = blas.get("threads") or int(os.environ.get("OMP_NUM_THREADS") or os.cpu_count())
    log(f"cpu baseline: {passes} passes, {per_pass:.3f} s each ({blas})")
    return {
        "value": round(sample_bytes / per_pass / 1e9, 4),
        "unit": "GB/s",
        "cores": int(threads),
        "cpu_model": cpu_model(),
        "blas": blas,
        "kind": "oracle",
        "sample": (f"{n_req} of the {work.B} requests (T={T}, all {work.H} heads), float64 numpy "
                   f"oracle, {passes} timed passes ({t_total:.1f} s), same eq-9 bytes metric"),
        "query_head_tokens_per_s": round(work.H * n_req * T / per_pass, 1),
    }


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def blas_info() -> dict:
    """numpy's BLAS library and the threads it runs (threadpoolctl's report)."""
    try:
        import threadpoolctl

        for rec in threadpoolctl.threadpool_info():
            if rec.get("user_api") == "blas":
                return {"vendor": rec.get("internal_api"), "version": rec.get("version"),
                        "threads": rec.get("num_threads")}
    except Exception:  # the report is informational only
        pass
    return {}


if __name__ == "__main__":
    main()
