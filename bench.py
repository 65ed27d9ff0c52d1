#!/usr/bin/env python3
"""Throughput of the CSA decode hot path at 1M-token context on one MI355X.

One step = one decode pass of a CSA layer over a batch of 8 sequences at
position 1,048,575 (1,048,576-token context, 262,144 compressed blocks per
sequence): compress the block the new token completes (KV and MXFP4 indexer
key), score every block with the MXFP4 lightning indexer, select the top 2048,
and attend over them plus a 128-token window with 64 heads on the shared
512-wide latent.  Inputs are seeded synthetic data already resident in HBM.

Six independent input sets are cycled so that consecutive steps never find
their working set (~90 MB per step) in the 256 MB MALL.  The timed region runs
exactly K steps as HIP graph replays: one graph holds one step per input set,
back to back (as a decode loop captures many layers' steps in one graph, so a
graph launch is not paid per step), replayed K // sets times, and single-step
graphs run the remainder; every step keeps all of its kernels, so nothing is
skipped.  The per-launch duration of the dominant
kernel (the MXFP4 indexer) is measured with HIP events on the launch stream
in a separate eager pass queued behind a backlog, so host launch gaps do not
enter it.  The CPU oracle is timed on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
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

METRIC = "CSA/HCA decode tokens/s at 1M ctx on 1 GPU; achieved HBM TB/s vs peak"
HBM_PEAK_GBS = 8000.0
KEY_BYTES = 34  # MXFP4 indexer key: 64 e2m1 codes (32 B) + 2 e8m0 scales
CAND_SLICE, CAND_PER_SLICE, CAND_BYTES, META_BYTES = 1024, 32, 8, 16  # fused indexer's slice candidates
INDEX_KERNEL = {"fused": "index_mxfp4_kernel<4, true>", "two-stage": "index_mxfp4_kernel<4, false>"}
PMC_SUMMARY = os.path.join(ROOT, "profiles", "index_mxfp4_csa_decode_1m_b8_pmc.txt")
INDEX_SOURCES = [os.path.join(ROOT, "long_context_attention_04_amd", "csrc", f)
                 for f in ("index.hip", "select.h", "common.h", "compress_block.h", "kernels.h")]  # the indexer kernel's code


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="csa_decode_1m_b8")
    ap.add_argument("--sets", type=int, default=6)
    ap.add_argument("--no-graph", action="store_true", help="time plain launches instead of graph replays")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--select", choices=("fused", "two-stage"), default="fused",
                    help="index+top-k as one fused call or as scores then selection")
    ap.add_argument("--cpu-seqs", type=int, default=8, help="sequences in the oracle's timed sample")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="repeat the oracle sample up to this long")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MiB",
                    help="also run one plain device copy of this size (a known-size reference for HBM counters)")
    return ap.parse_args()


def compress_bytes(layer) -> int:
    """The step's compressions: m raw KV rows (bf16) and m raw indexer-key rows (fp32) read per
    sequence, one KV entry (bf16) and one MXFP4 indexer key written."""
    return layer.B * (layer.m * (layer.D * 2 + layer.dI * 4) + layer.D * 2 + KEY_BYTES)


def algorithmic_bytes(layer) -> dict:
    """Bytes the method must move once per step (stored operands read once + outputs written once)."""
    B, N, k, W, H, D = layer.B, layer.n_cap, layer.k, layer.W, layer.H, layer.D
    keys = B * N * KEY_BYTES
    gather = B * (k + W) * D * 2
    q_out = B * H * D * 2 + B * H * D * 4 + B * H * 4
    small = B * k * 4 + B * layer.HI * (layer.dI * 4 + 4)
    comp = compress_bytes(layer)
    return {"keys": keys, "gather": gather, "q_out": q_out, "small": small, "compress": comp,
            "total": keys + gather + q_out + small + comp}


def backlog(torch, ms=15.0):
    """Queue ~ms of GPU work so the launches enqueued after it run back to back and their
    events time the GPU, not the host's launch gaps."""
    try:
        torch.cuda._sleep(int(ms * 1e-3 * 2.4e9))  # bounded spin (clock cycles)
        return None
    except Exception:  # pragma: no cover - fall back to plain memory traffic
        x = torch.empty(1 << 26, dtype=torch.float32, device="cuda")
        for _ in range(int(ms * 4)):
            x.fill_(1.0)
        return x


def launch_us(torch, layers, reps, launch) -> float:
    """Mean duration of one library call (`launch(layer)`): `reps` calls queued back to back
    behind a backlog on the stream they are launched on (torch's current stream), bracketed
    by two HIP events, so neither host launch gaps nor per-call event records enter it."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    keep = backlog(torch)
    e0.record()
    for i in range(reps):
        launch(layers[i % len(layers)])
    e1.record()
    torch.cuda.synchronize()
    del keep
    return float(e0.elapsed_time(e1) * 1e3 / reps)


def index_launch_bytes(layer, fused: bool) -> int:
    """Algorithmic bytes of one indexer launch: every key read once, the query and head weights,
    the scores written once, and (fused) the slices' candidates and metadata written once and the
    step's compressions (their raw rows read, the new KV entry and indexer key written)."""
    B, N = layer.B, layer.n_cap
    nbytes = B * N * KEY_BYTES + B * layer.HI * (layer.dI * 4 + 4) + B * N * 4
    if fused:
        ns = (N + CAND_SLICE - 1) // CAND_SLICE
        nbytes += B * ns * (CAND_PER_SLICE * CAND_BYTES + META_BYTES)
        nbytes += compress_bytes(layer)
    return nbytes


def stage_us(torch, layers, reps) -> dict:
    names = list(layers[0].stage_names)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(reps)]
    torch.cuda.synchronize()
    keep = backlog(torch)
    for i in range(reps):
        layers[i % len(layers)].step(marks=lambda j, i=i: ev[i][j].record())
    torch.cuda.synchronize()
    del keep
    out = {}
    for j, nm in enumerate(names):
        out[nm] = round(float(np.mean([ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(reps)]) * 1e3), 2)
    return out


def source_hash() -> str:
    h = hashlib.sha256()
    for f in INDEX_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def pmc_traffic(kernel_launch_bytes) -> dict | None:
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it matches the source."""
    if not os.path.exists(PMC_SUMMARY):
        return None
    txt = open(PMC_SUMMARY).read()
    src_hash = source_hash()
    vals = {}
    for line in txt.splitlines():
        if "=" in line and not line.startswith("#"):
            k_, v_ = line.split("=", 1)
            vals[k_.strip()] = v_.strip()
    if vals.get("source_sha256_16") != src_hash:
        return None
    try:
        return {"fetch_bytes": float(vals["fetch_bytes_per_launch"]), "write_bytes": float(vals["write_bytes_per_launch"]),
                "total": float(vals["fetch_bytes_per_launch"]) + float(vals["write_bytes_per_launch"])}
    except KeyError:
        return None


def cpu_baseline(torch, layer, n_seq, seconds) -> dict:
    """The oracle, as it stands, on the first n_seq sequences of one step (bounded sample),
    repeated until about `seconds` of CPU time (at most 8 repetitions)."""
    total, reps = 0.0, 0
    while reps < 8 and (reps == 0 or total < seconds):
        r = _cpu_sample(torch, layer, n_seq)
        total += r["seconds"]
        reps += 1
    r["value"] = round(n_seq * reps / total, 3)
    r["seconds"] = round(total, 3)
    r["sample"] += f", repeated {reps}x"
    return r


def _cpu_sample(torch, layer, n_seq) -> dict:
    import oracle
    from oracle import formats as OF
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
    L = layer
    sel = list(range(n_seq))
    t = L.host["t"][sel]
    base = L.host["raw_base"][sel]
    # ---- fetch inputs (device -> host marshalling, not timed)
    raw_kv = L.raw_kv.data[sel].double().cpu().numpy()
    raw_ik = L.raw_ik.data[sel].double().cpu().numpy()
    z_kv = L.z_kv.cpu().numpy().astype(np.float64)
    z_ik = L.z_ik.cpu().numpy().astype(np.float64)
    kc = L.k_idx.data[sel].cpu().numpy()
    ks = L.k_idx.scale[sel].cpu().numpy()
    q = L.q.data[sel].double().cpu().numpy()
    qi = L.q_idx.data[sel].cpu().numpy()
    w = L.w[sel].cpu().numpy().astype(np.float64)
    N = L.n_cap
    elapsed = 0.0
    # ---- timed: compress the new block, quantise, score, select
    t0 = time.perf_counter()
    first = np.full(n_seq, N - 1)
    new_kv = oracle.compress(raw_kv, base, z_kv, L.m, first, np.ones(n_seq))
    new_ik = oracle.compress(raw_ik, base, z_ik, L.m, first, np.ones(n_seq))
    kc = kc.copy()
    ks = ks.copy()
    for b in range(n_seq):
        c_, s_ = OF.quantize_mxfp4(new_ik[b][1].astype(np.float32))
        kc[b, N - 1], ks[b, N - 1] = c_[0], s_[0]
    kv_deq = OF.dequantize_mxfp4(kc, ks)
    qc, qs = OF.quantize_mxfp4(qi)
    q_deq = OF.dequantize_mxfp4(qc, qs)
    scores = oracle.index_scores(q_deq, w, kv_deq, t, L.m, n_cap=N)
    idx = oracle.topk(scores, t, L.m, L.k)
    elapsed += time.perf_counter() - t0
    # ---- fetch the rows the oracle selected (marshalling, not timed)
    rows = []
    for b in range(n_seq):
        ii = torch.as_tensor(idx[b, 0][idx[b, 0] >= 0], device="cuda")
        rows.append(L.kv_cmp.data[b].index_select(0, ii).double().cpu().numpy())
    # ---- timed: attention over the selection + window
    t0 = time.perf_counter()
    for b in range(n_seq):
        r_ = rows[b]
        j_new = np.where(idx[b, 0] == N - 1)[0]
        if j_new.size:  # the block this step produced comes from the oracle's own compressor
            r_[j_new[0]] = OF.round_bf16(new_kv[b][1][0].astype(np.float32))
        compact = np.arange(r_.shape[0])[None, None]
        oracle.csa_sparse_attn(q[b:b + 1], r_[None], compact, raw_kv[b:b + 1], base[b:b + 1], L.W, t[b:b + 1],
                               L.scale)
    elapsed += time.perf_counter() - t0
    return {"value": round(n_seq / elapsed, 3), "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{n_seq} of {L.B} sequences of one step (compress new block, MXFP4 quantise, "
                      f"index {N} blocks, top-{L.k}, attention over {L.k}+{L.W} entries), fp64 numpy",
            "seconds": elapsed}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the hot path shards by sequence with no collectives; see DESIGN.md)", file=sys.stderr)
        sys.exit(2)
    import torch

    import long_context_attention_04_amd as csa  # noqa: F401  (fails loudly when libcsa.so is missing)
    from long_context_attention_04_amd import workloads

    torch.cuda.set_device(0)
    name = args.workload
    wl = __import__("synth").WORKLOADS[name]
    if wl.kind != "csa_decode":
        print(f"bench.py times the CSA decode workloads; {name} is covered by the parity tests", file=sys.stderr)
        sys.exit(2)
    layers = [workloads.build(name, salt=s) for s in range(args.sets)]
    for layer in layers:
        layer.fused_select = args.select == "fused"
    torch.cuda.synchronize()

    # ---- eager warm-up (also validates every stage once)
    for i in range(max(args.warmup, 1)):
        layers[i % len(layers)].step()
    torch.cuda.synchronize()

    graphs = []
    if not args.no_graph:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for layer in layers:
                layer.step()  # warm the capture stream
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        for layer in layers:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                layer.step()
            graphs.append(g)
        cycle = torch.cuda.CUDAGraph()  # one step per input set, back to back
        with torch.cuda.graph(cycle):
            for layer in layers:
                layer.step()
        for i in range(args.warmup):
            graphs[i % len(graphs)].replay()
        cycle.replay()
        torch.cuda.synchronize()

    # ---- timed region: exactly K steps
    K = args.steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if graphs:
        for _ in range(K // len(layers)):
            cycle.replay()
        for i in range(K % len(layers)):
            graphs[i].replay()
    else:
        for i in range(K):
            layers[i % len(layers)].step()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms = dt * 1e3 / K
    tok_s = layers[0].B / (dt / K)

    # ---- dominant kernel: event-timed launches, and the stage breakdown
    fused = args.select == "fused"
    # the dominant kernel: the indexer (with the slices' candidate selection when fused), one launch
    if fused:
        idx_us = launch_us(torch, layers, max(K, 20), lambda layer: layer.compress_index_topk(1))
    else:
        idx_us = launch_us(torch, layers, max(K, 20), lambda layer: layer.index())
    attn_us = launch_us(torch, layers, max(K, 20), lambda layer: layer.attend())
    stages = stage_us(torch, layers, max(K // 2, 10))
    ab = algorithmic_bytes(layers[0])
    launch_bytes = index_launch_bytes(layers[0], fused)
    achieved = launch_bytes / (idx_us * 1e-6) / 1e9
    traffic = pmc_traffic(launch_bytes)
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic["total"] if traffic else None,
            "kernel": INDEX_KERNEL[args.select], "kernel_us": round(idx_us, 2), "bytes_per_launch": launch_bytes}
    res = {
        "metric": METRIC, "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16+mxfp4", "data": "synthetic",
        "config": {"workload": name, "batch": wl.batch, "context": wl.extra["context"], "heads": wl.heads,
                   "latent_dim": wl.dim, "idx_heads": wl.idx_heads, "idx_dim": wl.idx_dim, "topk": wl.topk,
                   "window": wl.window, "m": wl.m, "kv": wl.kv_dtype, "indexer": wl.idx_dtype,
                   "timing": f"graph of {len(layers)} steps" if graphs else "eager", "input_sets": args.sets},
        "hbm_tb_s_step": round(ab["total"] / (dt / K) / 1e12, 3),
        "algorithmic_bytes_per_step": ab["total"],
        "stages_us_eager": stages,
        "attention_call_us": round(attn_us, 2),  # csa_sparse_attn: split kernel + merge kernel
        "roofline": roof,
    }
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        res["copy_calibration_bytes"] = n
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(torch, layers[0], args.cpu_seqs, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
