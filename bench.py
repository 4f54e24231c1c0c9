#!/usr/bin/env python3
"""Benchmark: F16-weight products on one MI355X, Llama-3-8B-shaped matrices.

One step is one pass of the whole hot path over one batch of synthetic input:

  decode (n = 1):  the eight GEMVs of the set (q, k, v, o, gate, up, down and
                   the 128256x4096 logits, vec_dot order), each taking its own
                   f32 activation column and rounding it to f16 (to_f16, same
                   code) inside the launch, as ONE f16wm_mat_vec_table launch
                   (the products are independent: every column is a seeded
                   input);
  prefill (n = 512): to_f16 of each 512-column activation block, then the
                   exact product of every matrix (tinyBLAS order, picked by
                   takes_sgemm) and the MFMA fp16 product of every matrix.

Inputs are seeded synthetic data (N(0,0.02) f16 weights, N(0,1) f32
activations) resident in HBM before the timed region.  The weight set is
1.49 GB, well above the 256 MB last-level cache, so each step streams it cold.

Prints ONE JSON line.  `value` is the decode GEMV throughput in GB/s:
algorithmic bytes of the set / the table launch's time (HIP events around it
in each timed step).  Beside it: the same products as the five dependent
launches a model's layer issues (eager and as a HIP graph), per-launch
distributions (median, p10, p90 over --dist launches), the n = 512 GEMM
throughputs ("gemm_n512", with the logits launch of each on its own), the
576x576 case, the 135M-shaped step, and the oracle timed on the host."""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_F16_PEAK_TFLOPS = 2516.6  # dense fp16 MFMA, 256 CUs x 2.4 GHz
MFMA_F32_PEAK_TFLOPS = 157.3  # dense fp32 MFMA (published): 256 CUs x 2.4 GHz x 256 flop/clk


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing leg")
    p.add_argument("--cpu-sample-rows", type=int, default=4,
                   help="the oracle's prefill sample is rows/N of every matrix")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="also run one plain 1 GiB device copy (reference for HBM byte counters)")
    p.add_argument("--dist", type=int, default=50,
                   help="launches per timing distribution (median, p10, p90)")
    return p.parse_args()


def cpu_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def source_hash(path: str) -> str:
    """Hash of a kernel source and of the headers beside it that it includes
    (quoted includes, followed), so a change to any of them shows."""
    h = hashlib.sha256()
    seen, todo = set(), [path]
    while todo:
        p = todo.pop(0)
        if p in seen or not os.path.exists(p):
            continue
        seen.add(p)
        text = open(p, "rb").read()
        h.update(os.path.basename(p).encode() + b"\0" + text)
        todo += [os.path.join(os.path.dirname(p), inc.decode()) for inc in re.findall(rb'#include "([^"]+)"', text)]
    return h.hexdigest()[:16]


def traffic_record(kernel_src: str):
    """HBM traffic per launch measured with rocprofv3 PMC counters, read from
    profiles/hbm_traffic.md (a fenced json block), valid only for the kernel
    source (and included headers) it was measured on."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.md")
    if not os.path.exists(path):
        return None
    m = re.search(r"```json\n(.*?)```", open(path).read(), re.S)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("source_sha") != source_hash(kernel_src):
        return None
    return rec


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU (--gpus %d requested): the products would shard by output rows "
              "across GPUs, which is not implemented." % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import f16_weight_matrix_amd as f16wm
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    f16wm.lib()

    S = dict(synth.LLAMA3_8B)
    S["logits"] = synth.LLAMA3_8B_LOGITS
    N = synth.PREFILL_N

    t0 = time.time()
    host_w = {m: synth.weight(synth.CFG_8B, 0, m, *S[m]) for m in S}
    W = {m: torch.from_numpy(w.view(np.int16)).to(dev).view(torch.float16) for m, w in host_w.items()}
    # decode activation columns (f32): attn-in, o-in, ffn-in, down-in, logits-in
    dec = synth.activation(synth.CFG_8B, 0, 0, 5, 14336)
    dec_k = {"attn": 4096, "o": 4096, "ffn": 4096, "down": 14336, "logits": 4096}
    X1 = {g: torch.from_numpy(dec[i, :dec_k[g]].copy()).to(dev) for i, g in enumerate(dec_k)}
    # prefill activation blocks (f32) [512][k]
    pre = synth.activation(synth.CFG_8B_PREFILL, 0, 0, N, 14336)
    XN = {g: torch.from_numpy(np.ascontiguousarray(pre[:, :dec_k[g]])).to(dev) for g in dec_k}
    AN = {g: torch.empty((N, dec_k[g]), dtype=torch.float16, device=dev) for g in dec_k}
    del pre
    O1 = {m: torch.empty(S[m][0], dtype=torch.float32, device=dev) for m in S}
    ON = {m: torch.empty((N, S[m][0]), dtype=torch.float32, device=dev) for m in S}
    OM = {m: torch.empty((N, S[m][0]), dtype=torch.float32, device=dev) for m in S}
    torch.cuda.synchronize()
    setup_s = time.time() - t0

    src_of = {"q": "attn", "k": "attn", "v": "attn", "o": "o", "gate": "ffn", "up": "ffn",
              "down": "down", "logits": "logits"}
    # algorithmic bytes per GEMV launch: weights (f16) + the f32 activation
    # column (rounded to f16 inside the launch) + outputs (f32)
    gemv_launches = [("qkv", ["q", "k", "v"], "attn"), ("o", ["o"], "o"), ("gateup", ["gate", "up"], "ffn"),
                     ("down", ["down"], "down"), ("logits", ["logits"], "logits")]

    def gemv_bytes(mats, g):
        k = dec_k[g]
        return sum(2 * S[m][0] * k + 4 * S[m][0] for m in mats) + 4 * k

    gemv_b = [gemv_bytes(ms, g) for _, ms, g in gemv_launches]
    decode_bytes = sum(gemv_b)
    flops_n512 = sum(2 * S[m][0] * S[m][1] * N for m in S)

    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    # The decode GEMV set as one table launch: the eight products, each with
    # its own f32 column (rounded inside the launch), are independent here
    # (every column is a seeded input), so f16wm_mat_vec_table runs them in
    # one launch.  In a forward pass the same call takes the products of one
    # dependency level.
    table = f16wm.VecTable([(W[m], X1[src_of[m]], O1[m]) for m in S])

    def decode_sequence():
        # the same products as a model's layer issues them: Q/K/V grouped, O,
        # gate/up grouped, down, logits (five launches)
        for name, mats, g in gemv_launches:
            if len(mats) > 1:
                f16wm.mat_vec_multi([W[m] for m in mats], X1[g], [O1[m] for m in mats])
            else:
                f16wm.mat_vec(W[mats[0]], X1[g], O1[mats[0]])

    def step(timed):
        e = [ev() for _ in range(4)] if timed else None
        if timed:
            e[0].record()
        table()
        if timed:
            e[1].record()
        # ---- prefill, n = 512, exact order (takes_sgemm holds for every shape);
        # Q/K/V and gate/up share their activation block: one launch each
        for g in dec_k:
            f16wm.to_f16(XN[g], AN[g])
        for _, mats, g in gemv_launches:
            f16wm.mat_mul_multi([W[m] for m in mats], AN[g], [ON[m] for m in mats])
        if timed:
            e[2].record()
        # ---- prefill, n = 512, MFMA fp16
        for _, mats, g in gemv_launches:
            f16wm.mat_mul_mfma_multi([W[m] for m in mats], AN[g], [OM[m] for m in mats])
        if timed:
            e[3].record()
        return e

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    if args.calibrate_copy:
        # a plain copy of known size: 1 GiB read + 1 GiB written
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    recs = []
    t_start = time.perf_counter()
    for _ in range(args.steps):
        recs.append(step(True))
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t_start

    K = args.steps
    dec_table_avg = sum(e[0].elapsed_time(e[1]) for e in recs) / K
    exact_avg = sum(e[1].elapsed_time(e[2]) for e in recs) / K
    mfma_avg = sum(e[2].elapsed_time(e[3]) for e in recs) / K
    value = decode_bytes / (dec_table_avg * 1e-3) / 1e9
    want = {m: O1[m].view(torch.int32).clone() for m in S}

    # Distribution of the table launch: NDIST launches, each between its own
    # pair of events (event overhead included; the roofline below uses
    # back-to-back launches instead).
    table_ms = per_launch_ms(torch, ev, table, args.dist)

    # The dependent five-launch sequence, eager and as a HIP graph (the
    # weight set is six times the last-level cache: every pass is cold).
    seq_ms = per_launch_ms(torch, ev, decode_sequence, args.dist)
    seq_same = all(torch.equal(O1[m].view(torch.int32), want[m]) for m in S)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        decode_sequence()
    torch.cuda.synchronize()
    graph_same = True
    for _ in range(2):
        for m in S:
            O1[m].fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        graph_same = graph_same and all(torch.equal(O1[m].view(torch.int32), want[m]) for m in S)
    seq_graph_ms = per_launch_ms(torch, ev, graph.replay, args.dist)
    del graph

    # Per-launch timings of the sequence's five launches (events between
    # launches: dispatch and event overhead included).
    gemv_ms = []
    for _ in range(K):
        ge = [(ev(), ev()) for _ in gemv_launches]
        for i, (name, mats, g) in enumerate(gemv_launches):
            ge[i][0].record()
            if len(mats) > 1:
                f16wm.mat_vec_multi([W[m] for m in mats], X1[g], [O1[m] for m in mats])
            else:
                f16wm.mat_vec(W[mats[0]], X1[g], O1[mats[0]])
            ge[i][1].record()
        gemv_ms.append(ge)
    torch.cuda.synchronize()
    gemv_ms = [[a.elapsed_time(b) for a, b in ge] for ge in gemv_ms]
    per_launch = {name: {"bytes": gemv_b[i], "avg_us": round(1e3 * sum(r[i] for r in gemv_ms) / K, 2),
                         "GB_s": round(gemv_b[i] / (sum(r[i] for r in gemv_ms) / K * 1e-3) / 1e9, 1)}
                  for i, (name, _, _) in enumerate(gemv_launches)}

    # Roofline of the kernel `value` measures: the table launch
    # (vec_dot_lds_table: every product of the set is k >= 4096, so one LDS
    # launch), K launches back to back between two HIP events on the stream
    # the library launches on (torch's current stream).
    tbl_ms = back_to_back_ms(torch, ev, table, max(K, 20))
    achieved = decode_bytes / (tbl_ms * 1e-3) / 1e9
    table_kernel = "vec_dot_lds_table<16, true, true>"
    rec = traffic_record(os.path.join(ROOT, "f16_weight_matrix_amd", "csrc", "vec_dot.hip"))
    traffic = rec.get("bytes_per_launch") if rec and rec.get("kernel") == table_kernel else None

    # The step's time-dominant kernel: the exact (tinyBLAS order) logits
    # product at n = 512, and the MFMA logits product, each timed alone.
    lo_flops = 2 * S["logits"][0] * S["logits"][1] * N
    exact_lo_ms = back_to_back_ms(torch, ev, lambda: f16wm.mat_mul(W["logits"], AN["logits"], ON["logits"]),
                                  max(4, K // 2))
    mfma_lo_ms = back_to_back_ms(torch, ev, lambda: f16wm.mat_mul_mfma(W["logits"], AN["logits"], OM["logits"]),
                                 max(K, 20))

    # C1: the 576x576 weight at n = 1 and n = 3 (launch-bound; parity case).
    c1 = c1_leg(f16wm, torch, np, synth, dev, ev, args.dist)

    # Next row beside the step: the embedding lookup of a 512-token micro-batch
    # from the tied 128256x4096 table (get_rows), timed on its own.
    ids = torch.from_numpy(np.random.default_rng(7).integers(0, S["logits"][0], N)).to(dev)
    emb = torch.empty((N, S["logits"][1]), dtype=torch.float32, device=dev)
    gr_ms = back_to_back_ms(torch, ev, lambda: f16wm.get_rows(W["logits"], ids, emb), 20)
    gr_graph_us = graph_per_launch_us(torch, [lambda: f16wm.get_rows(W["logits"], ids, emb)] * 20, 3)
    gr_bytes = N * S["logits"][1] * (2 + 4) + N * 8
    attn = attention_helpers_leg(f16wm, torch, np, synth, dev, ev)

    # the 135M-shaped sequences, as graphs (their own timing; inputs resident)
    small = smollm2_135m_leg(f16wm, torch, np, synth, dev, reps=max(2, args.steps))

    exact_tflops = flops_n512 / (exact_avg * 1e-3) / 1e12
    mfma_tflops = flops_n512 / (mfma_avg * 1e-3) / 1e12
    ex_lo_tf = lo_flops / (exact_lo_ms * 1e-3) / 1e12
    mf_lo_tf = lo_flops / (mfma_lo_ms * 1e-3) / 1e12

    mfma_acc = mfma_accuracy(torch, np, host_w, AN, OM, gemv_launches, S, N)
    out = {
        "metric": "F16 GEMV GB/s (n=1) and GEMM TFLOP/s (n=512), % of MI355X roofline",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(1e3 * wall_s / K, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic: seeded N(0,0.02) f16 weights, N(0,1) f32 activations",
        "config": {
            "workload": "Llama-3-8B-shaped F16 set (q/o 4096x4096, k/v 1024x4096, gate/up 14336x4096, "
                        "down 4096x14336, logits 128256x4096): the decode GEMV set at n=1 as one table launch of "
                        "its eight independent products (value), then prefill n=512 exact and MFMA",
            "arithmetic": "f16 weights and rounded f16 activations widened exactly, f32 FMA chains in the exact "
                          "ggml orders; the MFMA fast path multiplies fp16 into f32",
            "decode_bytes_per_step": decode_bytes,
            "prefill_flops_per_product_set": flops_n512,
            "parallelism": "single GPU",
        },
        "phases_ms": {"decode_table": round(dec_table_avg, 4),
                      "prefill_exact": round(exact_avg, 4), "prefill_mfma": round(mfma_avg, 4)},
        "decode_table_launch_ms": stats(table_ms),
        "decode_tokens_per_s_equivalent": round(1e3 / dec_table_avg, 1),
        "decode_sequence": {
            "what": "the same eight products as five dependent launches (Q/K/V grouped, O, gate/up grouped, down, "
                    "logits), as a model's layer issues them",
            "eager_ms": stats(seq_ms), "graph_ms": stats(seq_graph_ms),
            "GB_s_eager_median": round(decode_bytes / (stats(seq_ms)["median"] * 1e-3) / 1e9, 1),
            "GB_s_graph_median": round(decode_bytes / (stats(seq_graph_ms)["median"] * 1e-3) / 1e9, 1),
            "bits_equal_table": seq_same, "graph_bits_equal_table": graph_same,
            "per_launch": per_launch,
            "per_launch_note": "each launch between its own pair of HIP events: dispatch and event overhead "
                               "included (kernel durations: rocprofv3 kernel trace)"},
        "roofline": {
            "kernel": table_kernel + " (the whole 8B GEMV set in one launch, f32 columns rounded in staging, "
                      "vec_dot order)",
            "covers": "the kernel value measures; the step's time-dominant kernel is the exact logits GEMM, "
                      "whose roofline is gemm_n512.exact.logits_launch",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "avg_launch_us": round(tbl_ms * 1e3, 2),
            "algorithmic_bytes_per_launch": decode_bytes,
        },
        "gemm_n512": {
            "exact": {"kernel": "tinyblas_mfma (tinyBLAS order, one chain step per fp32 MFMA 32x32x1)",
                      "bound": "mfma", "achieved": round(exact_tflops, 2), "unit": "TFLOP/s",
                      "peak": MFMA_F32_PEAK_TFLOPS, "frac": round(exact_tflops / MFMA_F32_PEAK_TFLOPS, 4),
                      "logits_launch": {"kernel": "tinyblas_mfma<true, false> (128256x4096, n=512)",
                                        "avg_launch_us": round(exact_lo_ms * 1e3, 1), "flops": lo_flops,
                                        "achieved": round(ex_lo_tf, 2), "unit": "TFLOP/s",
                                        "peak": MFMA_F32_PEAK_TFLOPS,
                                        "frac": round(ex_lo_tf / MFMA_F32_PEAK_TFLOPS, 4)}},
            "mfma": {"kernel": "mfma_fast (fp16 MFMA)", "bound": "mfma",
                     "achieved": round(mfma_tflops, 1), "unit": "TFLOP/s",
                     "peak": MFMA_F16_PEAK_TFLOPS, "frac": round(mfma_tflops / MFMA_F16_PEAK_TFLOPS, 4),
                     "logits_launch": {"kernel": "mfma_fast<256, 256, 2, 4, 2> (128256x4096, n=512)",
                                       "avg_launch_us": round(mfma_lo_ms * 1e3, 1), "flops": lo_flops,
                                       "achieved": round(mf_lo_tf, 1), "unit": "TFLOP/s",
                                       "peak": MFMA_F16_PEAK_TFLOPS,
                                       "frac": round(mf_lo_tf / MFMA_F16_PEAK_TFLOPS, 4)},
                     "accuracy": mfma_acc},
        },
        "c1_576x576": c1,
        "smollm2_135m": small,
        "next_rows": dict({"get_rows_512x4096": {"avg_us": round(gr_ms * 1e3, 2), "graph_us": round(gr_graph_us, 2),
                                                 "bytes": gr_bytes,
                                                 "GB_s": round(gr_bytes / (gr_ms * 1e-3) / 1e9, 1),
                                                 "GB_s_graph": round(gr_bytes / (gr_graph_us * 1e-6) / 1e9, 1)}},
                          **attn),
        "setup_s": round(setup_s, 1),
    }

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(host_w, dec, dec_k, S, N, args.cpu_sample_rows, value, args.dist)

    print(json.dumps(out), flush=True)


def per_launch_ms(torch, ev, fn, n):
    """n calls of fn, each between its own pair of HIP events on the current
    stream; the list of durations in ms."""
    pairs = [(ev(), ev()) for _ in range(n)]
    for a, b in pairs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in pairs]


def mfma_accuracy(torch, np, host_w, AN, OM, launches, S, N, samples=1024, seed=7):
    """The fp16 MFMA products' error, reported apart from the exact orders:
    `samples` seeded (column, row) outputs per matrix of the last timed step
    against an fp64 dot product of the same f16 operands (the weights as
    drawn, the activation block as the GPU rounded it), computed here with
    numpy.  err_over_abs_sum is |y - ref| / sum |w * a| (the acceptance
    measure, 2e-3 allowed); max_rel_err is |y - ref| / |ref| over the
    samples with |ref| at least 1e-2 of the samples' rms."""
    rng = np.random.default_rng(seed)
    e_abs = e_rel = 0.0
    count = 0
    for _, mats, g in launches:
        a64 = AN[g].cpu().numpy().astype(np.float64)                    # [N][k]
        for m in mats:
            rows, k = S[m]
            r = rng.integers(0, rows, samples)
            c = rng.integers(0, N, samples)
            y = OM[m][torch.from_numpy(c).to(OM[m].device), torch.from_numpy(r).to(OM[m].device)]
            y = y.cpu().numpy().astype(np.float64)
            prod = host_w[m][r].view(np.float16).astype(np.float64) * a64[c]
            ref = prod.sum(axis=1)
            absum = np.abs(prod).sum(axis=1)
            err = np.abs(y - ref)
            e_abs = max(e_abs, float((err / np.maximum(absum, 1e-300)).max()))
            big = np.abs(ref) >= 1e-2 * np.sqrt(np.mean(ref * ref))
            if big.any():
                e_rel = max(e_rel, float((err[big] / np.abs(ref[big])).max()))
            count += samples
    return {"samples": count, "err_over_abs_sum": float("%.3g" % e_abs), "max_rel_err": float("%.3g" % e_rel),
            "tolerance": 2e-3, "reference": "fp64 dot products of the same f16 operands (numpy, in this script)"}


def graph_per_launch_us(torch, fns, reps):
    """The launches fns (each one call), captured once in a HIP graph and
    replayed reps times between two HIP events: microseconds per launch.
    GPU-side gaps between the launches are included, the host's dispatch of
    each launch is not (short kernels would otherwise measure Python)."""
    for fn in fns:
        fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for fn in fns:
            fn()
    torch.cuda.synchronize()
    g.replay()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    del g
    return a.elapsed_time(b) * 1e3 / (reps * len(fns))


def back_to_back_ms(torch, ev, fn, n):
    """Average ms per call of n calls issued back to back between two HIP
    events on the current stream."""
    fn()
    a, b = ev(), ev()
    a.record()
    for _ in range(n):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n


def stats(vals):
    """median, p10, p90 (nearest rank) and count of a list of durations (the
    unit of the list, rounded to 4 decimals)."""
    v = sorted(vals)
    q = lambda f: v[min(len(v) - 1, max(0, int(round(f * (len(v) - 1)))))]  # noqa: E731
    return {"median": round(q(0.5), 4), "p10": round(q(0.1), 4), "p90": round(q(0.9), 4), "n": len(v)}


def c1_leg(f16wm, torch, np, synth, dev, ev, n):
    """The 576x576 weight (seed 0) at n = 1 (vec_dot) and n = 3 (tinyBLAS),
    f32 columns rounded inside the launch: per-launch times (launch-bound)."""
    w, a = synth.c1()
    wd = torch.from_numpy(w.view(np.int16)).to(dev).view(torch.float16)
    ad = torch.from_numpy(a).to(dev)
    o1 = torch.empty(576, dtype=torch.float32, device=dev)
    o3 = torch.empty((3, 576), dtype=torch.float32, device=dev)
    t1 = per_launch_ms(torch, ev, lambda: f16wm.mat_vec(wd, ad[0], o1), n)
    t3 = per_launch_ms(torch, ev, lambda: f16wm.mat_mul(wd, ad, o3), n)
    return {"n1_mat_vec_us": {k: (round(v * 1e3, 2) if k != "n" else v) for k, v in stats(t1).items()},
            "n3_mat_mul_us": {k: (round(v * 1e3, 2) if k != "n" else v) for k, v in stats(t3).items()}}


def smollm2_135m_leg(f16wm, torch, np, synth, dev, reps):
    """The 135M-shaped workload as whole sequences: a decode step (30 layers x
    {Q/K/V grouped, O, gate/up grouped, down} + the tied 49152x576 logits = 121
    product launches, f32 columns rounded inside each launch) and an n = 512
    prefill pass (per layer four to_f16 roundings and four grouped products,
    exact order and fp16 MFMA), each captured once as a HIP graph.  The weights
    (30 distinct layers, 268,959,744 bytes) exist in COPIES device copies and
    a graph replay runs one pass per copy, so a pass never finds its weights
    in the 256 MB last-level cache.  The activations are fixed seeded inputs
    (in a model they come from the steps between the products, which are not
    part of this path).  Graph replays are checked bit for bit against the
    same sequence run eagerly."""
    S = dict(synth.SMOLLM2_135M)
    L = synth.SMOLLM2_135M_LAYERS
    LOG = synth.SMOLLM2_135M_LOGITS
    N = synth.PREFILL_N
    COPIES = 4
    host = {(l, m): synth.weight(synth.CFG_135M, l, m, *S[m]) for l in range(L) for m in S}
    host[(0, "logits")] = synth.weight(synth.CFG_135M, 0, "logits", *LOG)
    W0 = {key: torch.from_numpy(w.view(np.int16)).to(dev).view(torch.float16) for key, w in host.items()}
    Wc = [W0] + [{key: t.clone() for key, t in W0.items()} for _ in range(COPIES - 1)]
    weight_bytes = sum(2 * w.size for w in host.values())
    del host
    groups = [("qkv", ["q", "k", "v"], 576), ("o", ["o"], 576), ("gateup", ["gate", "up"], 576),
              ("down", ["down"], 1536)]
    # decode: one f32 column per layer and group, one for the logits
    X1 = {}
    for l in range(L):
        acts = synth.activation(synth.CFG_135M, l, 0, 4, 1536)
        for gi, (g, _, k) in enumerate(groups):
            X1[(l, g)] = torch.from_numpy(acts[gi, :k].copy()).to(dev)
    X1["logits"] = torch.from_numpy(synth.activation(synth.CFG_135M, L, 0, 1, 576)[0].copy()).to(dev)
    O1 = {(l, m): torch.empty(S[m][0], dtype=torch.float32, device=dev) for l in range(L) for m in S}
    O1["logits"] = torch.empty(LOG[0], dtype=torch.float32, device=dev)
    # prefill: one f32 block [512][k] per group, shared by the layers
    pre = synth.activation(synth.CFG_135M_PREFILL, 0, 0, N, 1536)
    XN = {g: torch.from_numpy(np.ascontiguousarray(pre[:, :k])).to(dev) for g, _, k in groups}
    AN = {g: torch.empty((N, k), dtype=torch.float16, device=dev) for g, _, k in groups}
    ON = {(l, m): torch.empty((N, S[m][0]), dtype=torch.float32, device=dev) for l in range(L) for m in S}
    ON["logits"] = torch.empty((N, LOG[0]), dtype=torch.float32, device=dev)

    def decode(W):
        for l in range(L):
            for g, mats, _ in groups:
                if len(mats) > 1:
                    f16wm.mat_vec_multi([W[(l, m)] for m in mats], X1[(l, g)], [O1[(l, m)] for m in mats])
                else:
                    f16wm.mat_vec(W[(l, mats[0])], X1[(l, g)], O1[(l, mats[0])])
        f16wm.mat_vec(W[(0, "logits")], X1["logits"], O1["logits"])

    def prefill(W, mfma):
        mm = f16wm.mat_mul_mfma_multi if mfma else f16wm.mat_mul_multi
        for l in range(L):
            for g, mats, _ in groups:
                f16wm.to_f16(XN[g], AN[g])
                mm([W[(l, m)] for m in mats], AN[g], [ON[(l, m)] for m in mats])
        f16wm.to_f16(XN["qkv"], AN["qkv"])
        mm([W[(0, "logits")]], AN["qkv"], [ON["logits"]])

    # the same decode products as tables (f16wm_mat_vec_table), one per weight
    # copy: 181 short-row products (two launches of at most 96) and 30 staged
    # ones (one launch)
    src = {"q": "qkv", "k": "qkv", "v": "qkv", "o": "o", "gate": "gateup", "up": "gateup", "down": "down"}
    tables = {id(W): f16wm.VecTable([(W[(l, m)], X1[(l, src[m])], O1[(l, m)]) for l in range(L) for m in S] +
                                    [(W[(0, "logits")], X1["logits"], O1["logits"])]) for W in Wc}

    dec_launches = 4 * L + 1
    dec_bytes = sum(2 * S[m][0] * S[m][1] + 4 * S[m][0] for m in S) * L + sum(4 * k for _, _, k in groups) * L \
        + 2 * LOG[0] * LOG[1] + 4 * LOG[0] + 4 * LOG[1]
    pre_flops = 2 * N * (sum(S[m][0] * S[m][1] for m in S) * L + LOG[0] * LOG[1])

    def snapshot(outs):
        return [t.view(torch.int32).clone() for t in outs]

    res = {}
    for name, fn, outs in (
            ("decode_step", lambda W: decode(W), [O1["logits"], O1[(L - 1, "down")], O1[(0, "q")]]),
            ("decode_table", lambda W: tables[id(W)](), [O1["logits"], O1[(L - 1, "down")], O1[(0, "q")]]),
            ("prefill_exact", lambda W: prefill(W, False), [ON["logits"], ON[(L - 1, "down")], ON[(0, "k")]]),
            ("prefill_mfma", lambda W: prefill(W, True), [ON["logits"], ON[(L - 1, "down")], ON[(0, "k")]])):
        for _ in range(2):
            for W in Wc:
                fn(W)
        torch.cuda.synchronize()
        want = snapshot(outs)
        # eager timing (Python issues every launch)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            for W in Wc:
                fn(W)
        e1.record()
        torch.cuda.synchronize()
        eager_us = e0.elapsed_time(e1) * 1e3 / (reps * COPIES)
        # one graph: one pass over each weight copy
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for W in Wc:
                fn(W)
        torch.cuda.synchronize()
        same = True
        for _ in range(2):                     # replays checked, eager work between them
            for t in outs:
                t.fill_(float("nan"))
            graph.replay()
            torch.cuda.synchronize()
            same = same and all(torch.equal(a, b) for a, b in zip(snapshot(outs), want))
            fn(Wc[0])
            torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        graph_us = e0.elapsed_time(e1) * 1e3 / (reps * COPIES)
        del graph
        r = {"graph_us": round(graph_us, 2), "eager_us": round(eager_us, 2), "graph_bits_equal_eager": same}
        if name.startswith("decode"):
            r.update({"launches": dec_launches if name == "decode_step" else 3, "bytes": dec_bytes,
                      "GB_s": round(dec_bytes / (graph_us * 1e-6) / 1e9, 1),
                      "steps_per_s": round(1e6 / graph_us, 1),
                      "tokens_per_s_equivalent": round(1e6 / graph_us, 1),
                      "tokens_per_s_note": "one decode step's weight stream per token (the products only)"})
            if name == "decode_table":
                r["what"] = ("the step's 211 products as one f16wm_mat_vec_table call (independent products: "
                             "every column is a seeded input; a model's layers depend on each other)")
        else:
            r.update({"launches": 2 * (4 * L + 1), "flops": pre_flops,
                      "TFLOP_s": round(pre_flops / (graph_us * 1e-6) / 1e12, 2)})
        res[name] = r
    res["weight_copies"] = COPIES
    res["weight_bytes_per_copy"] = weight_bytes
    return res


def attention_helpers_leg(f16wm, torch, np, synth, dev, ev):
    """The f16 attention helpers on an 8B-shaped layer (8 KV heads x 128, 32
    query heads): vec_dot_u16 scores over a 32768-position f16 K cache (64 MB,
    a quarter of the last-level cache: a fresh cache copy per launch keeps
    every launch cold), and mad / scale over the f16 V accumulators of 32768
    query rows (32 heads x 1024 tokens) of 128 elements (rotating over copies
    for the same reason).  Times are per launch of back-to-back launches
    between two HIP events, launch gaps included."""
    n_kv, n_kv_head, d, n_head = 32768, 8, 128, 32
    copies = 6
    kcs = [torch.from_numpy(synth.random_f16(90 + c, (n_kv, n_kv_head, d)).view(np.int16)).to(dev)
           .view(torch.float16) for c in range(copies)]
    q = torch.from_numpy(synth.random_f16(99, (n_head, d)).view(np.int16)).to(dev).view(torch.float16)
    out = torch.empty((n_head, n_kv), dtype=torch.float32, device=dev)
    for kc in kcs:
        f16wm.kq(kc, q, out)
    reps = 4
    e0, e1 = ev(), ev()
    e0.record()
    for _ in range(reps):
        for kc in kcs:
            f16wm.kq(kc, q, out)
    e1.record()
    torch.cuda.synchronize()
    kq_us = e0.elapsed_time(e1) * 1e3 / (reps * copies)
    kq_graph_us = graph_per_launch_us(torch, [lambda kc=kc: f16wm.kq(kc, q, out) for kc in kcs], reps)
    kq_bytes = 2 * n_kv * n_kv_head * d + 2 * n_head * d + 4 * n_head * n_kv
    del kcs
    # mad / scale rotate over 48 accumulator (and V) copies, 768 MB in all, so
    # no launch finds its 8 MB arrays in the last-level cache.
    nvec, n = 32768, 128
    acc0 = torch.from_numpy(synth.random_f16(100, (nvec, n)).view(np.int16)).to(dev).view(torch.float16)
    v0 = torch.from_numpy(synth.random_f16(101, (nvec, n)).view(np.int16)).to(dev).view(torch.float16)
    copies = 48
    accs = [acc0.clone() for _ in range(copies)]
    vs = [v0.clone() for _ in range(copies)]
    w = torch.rand(nvec, device=dev) * 0.01
    sc = torch.ones(nvec, device=dev)
    for acc, v in zip(accs, vs):
        f16wm.mad(acc, v, w)
        f16wm.scale(acc, sc)
    reps = 2
    e0, e1, e2 = ev(), ev(), ev()
    e0.record()
    for _ in range(reps):
        for acc, v in zip(accs, vs):
            f16wm.mad(acc, v, w)
    e1.record()
    for _ in range(reps):
        for acc in accs:
            f16wm.scale(acc, sc)
    e2.record()
    torch.cuda.synchronize()
    mad_us = e0.elapsed_time(e1) * 1e3 / (reps * copies)
    scale_us = e1.elapsed_time(e2) * 1e3 / (reps * copies)
    mad_graph_us = graph_per_launch_us(torch, [lambda acc=acc, v=v: f16wm.mad(acc, v, w) for acc, v in zip(accs, vs)], reps)
    scale_graph_us = graph_per_launch_us(torch, [lambda acc=acc: f16wm.scale(acc, sc) for acc in accs], reps)
    del accs, vs
    mad_bytes = nvec * n * 6 + nvec * 4
    scale_bytes = nvec * n * 4 + nvec * 4
    return {
        "kq_32768x8x128_32heads": {"avg_us": round(kq_us, 2), "graph_us": round(kq_graph_us, 2), "bytes": kq_bytes,
                                   "GB_s": round(kq_bytes / (kq_us * 1e-6) / 1e9, 1),
                                   "GB_s_graph": round(kq_bytes / (kq_graph_us * 1e-6) / 1e9, 1)},
        "mad_32768x128": {"avg_us": round(mad_us, 2), "graph_us": round(mad_graph_us, 2), "bytes": mad_bytes,
                          "GB_s": round(mad_bytes / (mad_us * 1e-6) / 1e9, 1),
                          "GB_s_graph": round(mad_bytes / (mad_graph_us * 1e-6) / 1e9, 1)},
        "scale_32768x128": {"avg_us": round(scale_us, 2), "graph_us": round(scale_graph_us, 2), "bytes": scale_bytes,
                            "GB_s": round(scale_bytes / (scale_us * 1e-6) / 1e9, 1),
                            "GB_s_graph": round(scale_bytes / (scale_graph_us * 1e-6) / 1e9, 1)},
        "timing_note": ("avg_us: eager launches back to back between two HIP events (the host's dispatch of each "
                        "launch included once it is slower than the kernel); graph_us: the same launches replayed "
                        "as one HIP graph"),
    }


def host_cpus():
    """What the host offers: os.cpu_count(), the CPUs this process may run
    on, and `nproc`."""
    import subprocess
    try:
        aff = len(os.sched_getaffinity(0))
    except AttributeError:
        aff = None
    try:
        nproc = int(subprocess.run(["nproc"], capture_output=True, text=True, timeout=10).stdout.strip())
    except Exception:  # noqa: BLE001 - reported as unknown
        nproc = None
    return {"os_cpu_count": os.cpu_count(), "affinity": aff, "nproc": nproc}


def cpu_baseline(host_w, dec, dec_k, S, N, sample_div, gpu_value, ndist):
    """The oracle as it stands, on the host cores: the full decode GEMV set
    (same inputs), repeated until about 5 s have passed, and the exact
    n = 512 products on the first rows/N rows of every matrix (about 8 s at
    N = 4 on 16 cores), both on the CPUs this process may use up to 16 (one
    GPU's share of a shared host); and the 576x576 case on one thread,
    ndist times (median, p10, p90)."""
    import numpy as np

    import oracle
    import synth

    orc = oracle.default()
    T = cpu_threads()
    src = {"q": "attn", "k": "attn", "v": "attn", "o": "o", "gate": "ffn", "up": "ffn", "down": "down",
           "logits": "logits"}
    step_bytes = sum(4 * k for k in dec_k.values())    # the f32 columns
    for m, w in host_w.items():
        step_bytes += 2 * w.shape[0] * dec_k[src[m]] + 4 * w.shape[0]
    reps = 0
    t = time.perf_counter()
    while reps < 3 or time.perf_counter() - t < 5.0:
        a16 = {g: orc.to_f16(dec[i, :dec_k[g]]) for i, g in enumerate(dec_k)}
        for m, w in host_w.items():
            orc.mat_vec(w, a16[src[m]], threads=T)
        reps += 1
    dt_gemv = time.perf_counter() - t
    nbytes = reps * step_bytes
    pre = synth.activation(synth.CFG_8B_PREFILL, 0, 0, N, 14336)
    flops = 0
    t = time.perf_counter()
    for m, w in host_w.items():
        k = dec_k[src[m]]
        rows = max(4, (w.shape[0] // sample_div) // 4 * 4)
        orc.mat_mul(w[:rows], orc.to_f16(pre[:, :k]), threads=T)
        flops += 2 * rows * k * N
    dt_mm = time.perf_counter() - t
    # the 576x576 case on one thread
    w1, a1 = synth.c1()
    t1, t3 = [], []
    for _ in range(ndist):
        t = time.perf_counter()
        a16 = orc.to_f16(a1)
        orc.mat_vec(w1, a16[0], threads=1)
        t1.append((time.perf_counter() - t) * 1e6)
        t = time.perf_counter()
        orc.mat_mul(w1, orc.to_f16(a1), threads=1)
        t3.append((time.perf_counter() - t) * 1e6)
    c1_bytes = 2 * 576 * 576 + 4 * 576 + 4 * 576
    us = lambda v: {k: (round(x, 1) if k != "n" else x) for k, x in stats(v).items()}  # noqa: E731
    return {
        "value": round(nbytes / dt_gemv / 1e9, 3),
        "unit": "GB/s",
        "cores": T,
        "kind": "oracle",
        "sample": "decode: the full 8B GEMV set %d times (%d bytes each, %.2f s); prefill exact: the first 1/%d "
                  "of the rows of every matrix at n=512 (%.3g FLOP, %.2f s); 576x576 at n=1 and n=3 on one "
                  "thread, %d times each" % (reps, step_bytes, dt_gemv, sample_div, flops, dt_mm, ndist),
        "host": dict(host_cpus(), threads_used=T,
                     note="oracle threads = the CPUs this process may use, at most 16 (one GPU's share)"),
        "gemm_exact_tflops": round(flops / dt_mm / 1e12, 5),
        "c1_576x576_single_thread": {"n1_mat_vec_us": us(t1), "n3_mat_mul_us": us(t3),
                                     "n1_GB_s_median": round(c1_bytes / stats(t1)["median"] / 1e3, 3)},
        "gpu_over_cpu": round(gpu_value / (nbytes / dt_gemv / 1e9), 1),
    }


if __name__ == "__main__":
    main()
