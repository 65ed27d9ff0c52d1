#!/usr/bin/env python3
"""Throughput of the CSA / HCA attention hot path on one MI355X.

Default workload (the headline): one decode step of a CSA layer over a batch of
8 sequences at position 1,048,575 (1,048,576-token context, 262,144 compressed
blocks each): compress the block the new token completes (KV entry and MXFP4
indexer key), score every block with the MXFP4 lightning indexer, select the top
2048, and attend over them plus a 128-token window with 64 heads on the shared
512-wide latent (--kv mxfp4: FP4 KV caching of the compressed entries).
--workload picks another: the 2048-query CSA or HCA prefill chunk over a 64k
context (MFMA-bound), HCA decode at batch 64, the hybrid CSA + HCA layer pair at
batch 32 (--kv bf16 or fp8), or a CSA2 group of layers sharing one cache and one
top-k at 1M context.  Inputs are seeded synthetic data already resident in HBM.

Timed region: exactly K steps, bracketed by synchronizations.  Several
independent input sets are cycled so consecutive steps do not find their working
set in the 256 MB MALL; one HIP graph holds one step per input set, back to back
(as a decode loop captures many layers' steps in one graph), replayed K // sets
times, single-step graphs run the remainder; every step keeps all of its
kernels.  Events around each cycle replay give the per-step median, p10 and p90;
the same K steps launched eagerly behind a GPU backlog give the eager figure.

Roofline: the dominant kernel's algorithmic bytes (or flops) per launch -- the
operands the method must read once and the outputs it writes once; workspace and
score round trips excluded and reported separately -- over its mean launch
duration, from K launches queued back to back behind a backlog on the launch
stream between two HIP events.  Peaks: 8 TB/s HBM, 2.5 PFLOP/s dense bf16 MFMA;
the measured streaming-read ceiling (csa_stream_read over 2 GiB) is reported
beside them.  The oracle is timed on a bounded sample on the host's cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--kv bf16|fp8|mxfp4]
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

METRIC = "CSA/HCA decode tokens/s at 1M ctx on 1 GPU; achieved HBM TB/s vs peak"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
KEY_BYTES = 34  # MXFP4 indexer key: 64 e2m1 codes (32 B) + 2 e8m0 scales
SLICE, SLICE_SLOTS, SLOT_BYTES, META_BYTES = 1024, 32, 8, 16  # fused indexer's slice lists
PMC_SUMMARY = os.path.join(ROOT, "profiles", "index_mxfp4_csa_decode_1m_b8_pmc.txt")
# the sources the dominant kernel of the headline workload is built from (the counter
# summary is valid only for the build it was taken from)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=120)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="csa_decode_1m_b8")
    ap.add_argument("--kv", choices=("bf16", "fp8", "mxfp4"), default=None,
                    help="KV format: hybrid pair bf16 (default) | fp8; 1M decode bf16 (default) | mxfp4 "
                         "(FP4 KV caching); CSA2 group mxfp4 (default) | bf16")
    ap.add_argument("--sets", type=int, default=6)
    ap.add_argument("--no-graph", action="store_true", help="time plain launches instead of graph replays")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the streaming-read ceiling")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="repeat the oracle sample up to this long")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MiB",
                    help="also run one plain device copy of this size (a known-size reference for HBM counters)")
    return ap.parse_args()


# ============================================================================ timing helpers


def backlog(torch, ms=15.0):
    """Queue ~ms of GPU work so launches enqueued after it run back to back and their
    events time the GPU, not the host's launch gaps."""
    torch.cuda._sleep(int(ms * 1e-3 * 2.4e9))  # bounded spin (clock cycles)


def launch_us(torch, n, reps, launch) -> float:
    """Mean duration of one library call launch(i % n): reps calls queued back to back behind a
    backlog on torch's current stream (the stream they are launched on), between two events."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    backlog(torch)
    e0.record()
    for i in range(reps):
        launch(i % n)
    e1.record()
    torch.cuda.synchronize()
    return float(e0.elapsed_time(e1) * 1e3 / reps)


def projection_timings(torch, rows=8, d_model=4096, rank=1024, HI=8, dI=64, H=64, dh=128, D=512, sets=40) -> dict:
    """The projections either side of the decode step, timed alone at batch `rows`: the
    indexer query (c = W_dq h, q_I = W_uq c, w = W_w h) and the MLA absorbed query and
    output up-projection.  Each is bound by its bf16 weight stream; `sets` weight copies
    rotate so that the weights come from HBM, not the last-level cache."""
    import long_context_attention_04_amd as csa
    dev, bf = "cuda", torch.bfloat16

    def rnd(*shape):
        return (torch.randn(*shape, device=dev) / np.sqrt(shape[-1])).to(bf)

    res = {}
    # indexer query
    h = rnd(rows, 1, d_model)
    W = [(rnd(1, rank, d_model), rnd(1, HI * dI, rank), rnd(1, HI, d_model)) for _ in range(sets)]
    qi = torch.empty(rows, 1, HI, dI, device=dev)
    w = torch.empty(rows, 1, HI, device=dev)
    ws = torch.empty(csa.csa_index_query_workspace_size(rows, 1, d_model, rank, HI, dI), dtype=torch.uint8, device=dev)
    D3 = [[csa.desc(x, csa.BF16) for x in ws3] for ws3 in W]
    hd, qd = csa.desc(h, csa.BF16), csa.desc(qi, csa.F32)
    us = launch_us(torch, sets, 4 * sets, lambda i: csa.csa_index_query(hd, *D3[i], rows, 1, d_model, rank, HI, dI, qd,
                                                                        w, ws, ws.numel()))
    nb = 2 * (rank * d_model + HI * dI * rank + HI * d_model) + rows * (2 * d_model + 4 * HI * dI + 4 * HI)
    res["index_query"] = {"us": round(us, 2), "bytes": nb, "gb_s": round(nb / us * 1e-3, 1),
                          "shape": f"rows {rows}, d_model {d_model}, rank {rank}, {HI} x {dI}"}
    # MLA absorbed query and output up-projection
    q = rnd(rows, H, dh)
    Wk = [rnd(H, D, dh) for _ in range(sets)]
    Wv = [rnd(H, dh, D) for _ in range(sets)]
    ql = torch.empty(rows, H, D, dtype=bf, device=dev)
    ol = torch.randn(rows, H, D, device=dev)
    o = torch.empty(rows, H, dh, dtype=bf, device=dev)
    wq = torch.empty(max(csa.csa_latent_query_workspace_size(rows, H, dh, D), 1), dtype=torch.uint8, device=dev)
    wo = torch.empty(max(csa.csa_latent_output_workspace_size(rows, H, dh, D), 1), dtype=torch.uint8, device=dev)
    us = launch_us(torch, sets, 4 * sets, lambda i: csa.csa_latent_query(q, Wk[i], rows, H, dh, D, ql, wq, wq.numel()))
    nb = 2 * H * D * dh + rows * H * (2 * dh + 2 * D)
    res["latent_query"] = {"us": round(us, 2), "bytes": nb, "gb_s": round(nb / us * 1e-3, 1),
                           "shape": f"rows {rows}, {H} heads of {dh} onto {D}"}
    us = launch_us(torch, sets, 4 * sets, lambda i: csa.csa_latent_output(ol, Wv[i], rows, H, dh, D, o, csa.BF16, wo,
                                                                           wo.numel()))
    nb = 2 * H * D * dh + rows * H * (4 * D + 2 * dh)
    res["latent_output"] = {"us": round(us, 2), "bytes": nb, "gb_s": round(nb / us * 1e-3, 1),
                            "shape": f"rows {rows}, {H} heads: {D} -> {dh}"}
    for v in res.values():
        v["frac"] = round(v["gb_s"] / HBM_PEAK_GBS, 4)
    return res


def stream_ceiling(torch) -> dict:
    """HBM streaming-read ceiling: csa_stream_read over 2 GiB, best of 5."""
    from long_context_attention_04_amd import csa_stream_read, csa_stream_read_sink_size
    nbytes = 2 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sink = torch.empty(csa_stream_read_sink_size(), dtype=torch.uint8, device="cuda")
    times = []
    for _ in range(6):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        csa_stream_read(buf, nbytes, sink)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e-3)
    del buf
    best = min(times[1:])
    return {"gb_s": round(nbytes / best / 1e9, 1), "bytes": nbytes, "frac_of_peak": round(nbytes / best / 1e9 /
                                                                                         HBM_PEAK_GBS, 4),
            "kernel": "stream_read_kernel (csa_stream_read), best of 5"}


def pmc_traffic():
    """HBM bytes per launch of the headline's dominant kernel from the committed rocprofv3 counter
    summary, when it was taken from the kernel's current sources (its source hash matches; else None)."""
    if not os.path.exists(PMC_SUMMARY):
        return None
    vals = {}
    for line in open(PMC_SUMMARY).read().splitlines():
        if "=" in line and not line.startswith("#"):
            k_, v_ = line.split("=", 1)
            vals[k_.strip()] = v_.strip()
    from long_context_attention_04_amd.rocprof_summary import source_hash
    if vals.get("source_sha256_16") != source_hash(quiet=True):
        return None
    try:
        return float(vals["fetch_bytes_per_launch"]) + float(vals["write_bytes_per_launch"])
    except KeyError:
        return None


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


def time_oracle(sample, seconds, units) -> dict:
    """Run sample() (returns a description) repeatedly until `seconds` of wall time have passed;
    units = work units (tokens) per call."""
    total, reps, desc = 0.0, 0, ""
    while reps == 0 or total < seconds:
        t0 = time.perf_counter()
        desc = sample()
        total += time.perf_counter() - t0
        reps += 1
    return {"value": round(units * reps / total, 3), "unit": "tokens/s", "cores": blas_threads(),
            "cpu_count": os.cpu_count(), "kind": "oracle", "sample": f"{desc}, fp64 numpy, repeated {reps}x",
            "seconds": round(total, 3)}


# ============================================================================ workloads


class CsaDecode:
    """The headline: CSA decode at 1M context, batch 8, MXFP4 indexer (fused index+top-k)."""

    def __init__(self, name, sets, torch, kv="bf16"):
        from long_context_attention_04_amd import workloads
        import synth
        self.wl = synth.WORKLOADS[name]
        self.layers = [workloads.build(name, salt=s, kv_fmt=kv) for s in range(sets)]
        L = self.layers[0]
        self.tokens = L.B
        B, N, k, W, H, D = L.B, L.n_cap, L.k, L.W, L.H, L.D
        row = D * 2 if kv == "bf16" else D // 2 + D // 32  # stored bytes per KV row (MXFP4: codes + scales)
        comp = B * (L.m * (row + L.dI * 4) + row + KEY_BYTES)  # the step's compressions
        qw = B * L.HI * (L.dI * 4 + 4)
        self.bytes = {"keys": B * N * KEY_BYTES, "gather": B * (k + W) * row,
                      "q_out_lse": B * H * D * 2 + B * H * D * 4 + B * H * 4, "idx": B * k * 4, "q_idx_w": qw,
                      "compress": comp}
        ns = (N + SLICE - 1) // SLICE
        self.excluded = {"slice_lists": B * ns * (SLICE_SLOTS * SLOT_BYTES + META_BYTES),
                         "attention_split_partials": 2 * B * 8 * H * (D + 2) * 4}
        self.dominant = {"kernel": "index_mxfp4_kernel<4, true> (csa_compress_index_topk part 1)",
                         "bound": "hbm", "work": self.bytes["keys"] + qw + comp,
                         "work_note": "keys read once + q_idx and w + the step's compressions"}
        self.dtype = "bf16+mxfp4"
        self.kv = kv
        wl = self.wl
        self.config = {"workload": name, "batch": wl.batch, "context": wl.extra["context"], "heads": wl.heads,
                       "latent_dim": wl.dim, "idx_heads": wl.idx_heads, "idx_dim": wl.idx_dim, "topk": wl.topk,
                       "window": wl.window, "m": wl.m, "kv": kv, "indexer": wl.idx_dtype}
        self.metric = METRIC
        self.torch = torch

    def step(self, i):
        self.layers[i].step()

    def dominant_launch(self, i):
        self.layers[i].compress_index_topk(1)

    def extra_timings(self):
        L = self.layers
        return {"attention_call_us": round(launch_us(self.torch, len(L), 40, lambda i: L[i].attend()), 2),
                "index_topk_call_us": round(launch_us(self.torch, len(L), 40,
                                                      lambda i: L[i].compress_index_topk(3)), 2),
                "projections": projection_timings(self.torch, rows=L[0].B)}

    def traffic(self):
        return pmc_traffic()

    def cpu_baseline(self, seconds):
        import oracle
        from oracle import formats as OF
        torch, L = self.torch, self.layers[0]
        n_seq = L.B
        t = L.host["t"]
        base = L.host["raw_base"]
        raw_kv = L.raw_kv.data.double().cpu().numpy()
        raw_ik = L.raw_ik.data.double().cpu().numpy()
        z_kv = L.z_kv.cpu().numpy().astype(np.float64)
        z_ik = L.z_ik.cpu().numpy().astype(np.float64)
        kc0 = L.k_idx.data.cpu().numpy()
        ks0 = L.k_idx.scale.cpu().numpy()
        q = L.q.data.double().cpu().numpy()
        qi = L.q_idx.data.cpu().numpy()
        w = L.w.cpu().numpy().astype(np.float64)
        N = L.n_cap
        # the rows any selection could need are fetched up front (marshalling, not timed): the
        # oracle's own selection is recomputed inside the timed sample
        kv_rows = {}

        def sample():
            first = np.full(n_seq, N - 1)
            new_kv = oracle.compress(raw_kv, base, z_kv, L.m, first, np.ones(n_seq))
            new_ik = oracle.compress(raw_ik, base, z_ik, L.m, first, np.ones(n_seq))
            kc, ks = kc0.copy(), ks0.copy()
            for b in range(n_seq):
                c_, s_ = OF.quantize_mxfp4(new_ik[b][1].astype(np.float32))
                kc[b, N - 1], ks[b, N - 1] = c_[0], s_[0]
            qc, qs = OF.quantize_mxfp4(qi)
            scores = oracle.index_scores(OF.dequantize_mxfp4(qc, qs), w, OF.dequantize_mxfp4(kc, ks), t, L.m,
                                         n_cap=N)
            idx = oracle.topk(scores, t, L.m, L.k)
            for b in range(n_seq):
                sel = idx[b, 0][idx[b, 0] >= 0]
                key = (b, sel.tobytes())
                if key not in kv_rows:  # device -> host marshalling of the selected rows
                    kv_rows[key] = L.kv_cmp.data[b].index_select(0, torch.as_tensor(sel, device="cuda")).double() \
                        .cpu().numpy()
                rows = kv_rows[key].copy()
                rows[sel == N - 1] = OF.round_bf16(new_kv[b][1][0].astype(np.float32))
                oracle.csa_sparse_attn(q[b:b + 1], rows[None], np.arange(rows.shape[0])[None, None],
                                       raw_kv[b:b + 1], base[b:b + 1], L.W, t[b:b + 1], L.scale)
            return (f"all {n_seq} sequences of one step: compress the new block, MXFP4-quantise, index {N} blocks, "
                    f"top-{L.k}, attention over {L.k}+{L.W} entries")

        sample()  # warm the marshalling cache (device reads are not oracle work)
        return time_oracle(sample, seconds, n_seq)


class Csa2Decode:
    """CSA2 cross-layer reuse: a group of layers sharing one compressed cache (MXFP4 entries
    by default, bf16 window rows) and one top-k at 1M context, batch 8.  A step is the
    group's decode step: compress + index + top-k once, then one attention per layer."""

    def __init__(self, name, sets, torch, kv="mxfp4"):
        from long_context_attention_04_amd import workloads
        import synth
        self.wl = wl = synth.WORKLOADS[name]
        self.layers = [workloads.build(name, salt=s, kv_fmt=kv) for s in range(sets)]
        G = self.layers[0]
        L = G.base
        nl = G.layers
        self.tokens = L.B
        B, N, k, W, H, D = L.B, L.n_cap, L.k, L.W, L.H, L.D
        row = D * 2 if kv == "bf16" else D // 2 + D // 32
        comp = B * (L.m * (D * 2 + L.dI * 4) + row + KEY_BYTES)
        qw = B * L.HI * (L.dI * 4 + 4)
        self.bytes = {"keys": B * N * KEY_BYTES, "q_idx_w": qw, "compress": comp, "idx": B * k * 4,
                      "gather_per_layer_x_layers": nl * B * (k * row + W * D * 2),
                      "q_out_lse_x_layers": nl * B * H * (D * 2 + D * 4 + 4)}
        self.excluded = {"attention_split_partials": nl * 2 * B * 8 * H * (D + 2) * 4}
        self.dominant = {"kernel": "index_mxfp4_kernel<4, true> (csa_compress_index_topk part 1)",
                         "bound": "hbm", "work": self.bytes["keys"] + qw + comp,
                         "work_note": "keys read once + q_idx and w + the step's compressions (once per group)"}
        self.dtype = f"{kv}+mxfp4"
        self.config = {"workload": name, "batch": wl.batch, "context": wl.extra["context"], "layers": nl,
                       "heads": wl.heads, "latent_dim": wl.dim, "idx_heads": wl.idx_heads, "idx_dim": wl.idx_dim,
                       "topk": wl.topk, "window": wl.window, "m": wl.m, "kv": kv, "indexer": wl.idx_dtype}
        self.metric = (f"CSA2 layer-group decode tokens/s ({nl} layers sharing one cache and top-k, 1M ctx, "
                       "batch 8) on 1 GPU")
        self.torch = torch

    def step(self, i):
        self.layers[i].step()

    def dominant_launch(self, i):
        self.layers[i].base.compress_index_topk(1)

    def extra_timings(self):
        G = self.layers
        att = launch_us(self.torch, len(G), 40, lambda i: G[i].attend_layer(1))
        sel = launch_us(self.torch, len(G), 40, lambda i: G[i].base.compress_index_topk(3))
        return {"attention_call_us": round(att, 2), "index_topk_call_us": round(sel, 2)}

    def traffic(self):
        return None

    def cpu_baseline(self, seconds):
        import oracle
        from oracle import formats as OF
        G = self.layers[0]
        L, n_seq = G.base, 2
        t = L.host["t"]
        base = L.host["raw_base"]
        raw_kv = L.raw_kv.data.double().cpu().numpy()
        idx = L.idx.cpu().numpy()  # the shared selection (the oracle's selection is timed in the 1M decode line)
        qs = [L.q.data.double().cpu().numpy()] + [q.data.double().cpu().numpy() for q in G.q]
        data = []
        for b in range(n_seq):
            sel = self.torch.as_tensor(idx[b, 0], device="cuda")
            c = L.kv_cmp.data[b].index_select(0, sel).cpu().numpy()
            sc = L.kv_cmp.scale[b].index_select(0, sel).cpu().numpy()
            data.append((c, sc))

        def sample():
            for b, (c, sc) in enumerate(data):
                rows = OF.dequantize_mxfp4(c, sc)[None]
                for q in qs:
                    oracle.csa_sparse_attn(q[b:b + 1], rows, np.arange(L.k)[None, None], raw_kv[b:b + 1],
                                           base[b:b + 1], L.W, t[b:b + 1], L.scale)
            return (f"{n_seq} of {L.B} sequences: dequantise the {L.k} shared MXFP4 rows, attention for each of the "
                    f"{G.layers} layers (selection not included)")

        return time_oracle(sample, seconds, n_seq)


class CsaPrefill:
    """The prefill chunk: 2048 queries over a 64k context, bf16 indexer (MFMA-bound)."""

    def __init__(self, name, sets, torch):
        from long_context_attention_04_amd import workloads
        import synth
        self.wl = wl = synth.WORKLOADS[name]
        self.layers = [workloads.build(name, salt=s) for s in range(sets)]
        L = self.layers[0]
        self.tokens = L.B * L.tq
        pos = L.host["t"]
        vis = (pos + 1) // L.m
        flops = int(np.sum(vis)) * 2 * L.HI * L.dI * L.B
        self.dominant = {"kernel": "index_bf16_tile_kernel (csa_index_scores)", "bound": "mfma", "work": flops,
                         "work_note": "2 * H_I * d_I flops per visible (query, block) pair, causal"}
        self.bytes = {"keys": L.B * L.n_cap * L.dI * 2, "q_idx_w": L.B * L.tq * L.HI * (L.dI * 2 + 4),
                      "gather_unique": L.B * L.n_cap * L.D * 2,
                      "q_out_lse": L.B * L.tq * L.H * (L.D * 2 + L.D * 4 + 4), "idx": L.B * L.tq * L.k * 4}
        self.excluded = {"scores": L.B * L.tq * L.n_cap * 4}
        self.dtype = "bf16"
        self.config = {"workload": name, "batch": wl.batch, "queries": wl.tq, "context": wl.extra["context"],
                       "heads": wl.heads, "latent_dim": wl.dim, "idx_heads": wl.idx_heads, "idx_dim": wl.idx_dim,
                       "topk": wl.topk, "window": wl.window, "m": wl.m, "kv": wl.kv_dtype, "indexer": wl.idx_dtype}
        self.metric = "CSA prefill chunk tokens/s (2048 queries over 64k ctx) on 1 GPU; indexer TFLOP/s vs bf16 MFMA peak"
        self.torch = torch

    def step(self, i):
        self.layers[i].step()

    def dominant_launch(self, i):
        self.layers[i].index()

    def extra_timings(self):
        L = self.layers
        return {"topk_call_us": round(launch_us(self.torch, len(L), 10, lambda i: L[i].topk()), 2),
                "attention_call_us": round(launch_us(self.torch, len(L), 10, lambda i: L[i].attend()), 2)}

    def traffic(self):
        return None

    def cpu_baseline(self, seconds):
        import oracle
        L = self.layers[0]
        ctx, m, nq = self.wl.extra["context"], L.m, 4
        raw_kv = L.raw_kv.data[0].double().cpu().numpy()
        kv_c = L.kv_cmp.data[0].double().cpu().numpy()
        k_c = L.k_idx.data[0].double().cpu().numpy()
        q = L.q.data[0].double().cpu().numpy()
        qi = L.q_idx.data[0].double().cpu().numpy()
        w = L.w[0].cpu().numpy().astype(np.float64)
        rows = np.linspace(0, L.tq - 1, nq).astype(int)

        def sample():
            for tq in rows:
                t = np.array([[ctx + tq]])
                sc = oracle.index_scores(qi[None, tq:tq + 1], w[None, tq:tq + 1], k_c[None], t, m, n_cap=L.n_cap)
                idx = oracle.topk(sc, t, m, L.k)
                oracle.csa_sparse_attn(q[None, tq:tq + 1], kv_c[None], idx, raw_kv[None], [0], L.W, t, L.scale)
            return f"{nq} of {L.tq} chunk queries (index {L.n_cap} blocks, top-{L.k}, attention over {L.k}+{L.W})"

        return time_oracle(sample, seconds, nq)


class HcaDecode:
    """HCA decode, batch 64, contexts of 64k-128k tokens: dense attention over the heavily
    compressed entries plus the window."""

    def __init__(self, name, sets, torch):
        from long_context_attention_04_amd import workloads
        import synth
        self.wl = wl = synth.WORKLOADS[name]
        self.layers = [workloads.build(name, salt=s) for s in range(sets)]
        L = self.layers[0]
        self.tokens = L.B
        vis = L.host["vis"]
        gather = int(np.sum(vis + L.W)) * L.D * 2
        q_out = L.B * L.H * (L.D * 2 + L.D * 4 + 4)
        self.bytes = {"entries": gather, "q_out_lse": q_out}
        self.excluded = {"attention_split_partials": 2 * L.B * 4 * L.H * (L.D + 2) * 4}  # HCA decode: four splits
        self.dominant = {"kernel": "attn_chunk_kernel<bf16, 4, 128, 2 head groups> + attn_merge_kernel (hca_attn)", "bound": "hbm",
                         "work": gather + q_out, "work_note": "visible compressed rows + window rows + q, out, lse"}
        self.dtype = "bf16"
        self.config = {"workload": name, "batch": wl.batch, "context": f"U[{wl.extra['len_lo']}, {wl.extra['len_hi']}]",
                       "heads": wl.heads, "latent_dim": wl.dim, "m_hc": wl.m_hc, "window": wl.window,
                       "kv": wl.kv_dtype}
        self.metric = "HCA decode tokens/s (batch 64, 64k-128k ctx) on 1 GPU; achieved HBM TB/s vs peak"
        self.torch = torch

    def step(self, i):
        self.layers[i].step()

    def dominant_launch(self, i):
        self.layers[i].attend()

    def extra_timings(self):
        return {}

    def traffic(self):
        return None

    def cpu_baseline(self, seconds):
        import oracle
        L, n_seq = self.layers[0], 8
        data = []
        for b in range(n_seq):
            vis = int(L.host["vis"][b])
            data.append((L.q.data[b:b + 1].double().cpu().numpy(), L.kv_hc.data[b, :vis].double().cpu().numpy(),
                         L.raw_kv.data[b:b + 1].double().cpu().numpy()))

        def sample():
            for b, (q, kv, raw) in enumerate(data):
                oracle.hca_attn(q, kv[None], L.m_hc, raw, L.host["raw_base"][b:b + 1], L.W, L.host["t"][b:b + 1],
                                L.scale)
            return f"{n_seq} of {L.B} sequences (dense attention over their visible blocks + {L.W} window rows)"

        return time_oracle(sample, seconds, n_seq)


class HcaPrefill:
    """HCA prefill: a 2048-query chunk over a 64k context; the step compresses the 16 blocks
    the chunk completes, then every query attends densely over its visible blocks and its
    window (MFMA-bound)."""

    def __init__(self, name, sets, torch):
        from long_context_attention_04_amd import workloads
        import synth
        self.wl = wl = synth.WORKLOADS[name]
        self.layers = [workloads.build(name, salt=s) for s in range(sets)]
        L = self.layers[0]
        self.tokens = L.B * L.tq
        t = L.host["t"]
        entries = int(np.sum((t + 1) // L.m_hc + np.minimum(L.W, t + 1)))
        flops = entries * L.H * 4 * L.D
        self.dominant = {"kernel": "attn_chunk_kernel (hca_attn)", "bound": "mfma", "work": flops,
                         "work_note": "4 * D flops per (query, head, visible entry): QK^T and PV, causal"}
        nb = L.max_blocks
        self.bytes = {"entries_unique": L.B * L.n_cap * L.D * 2, "window_raw": L.B * (L.W + L.tq) * L.D * 2,
                      "compress": L.B * nb * L.D * 2, "q_out_lse": L.B * L.tq * L.H * (L.D * 2 + L.D * 4 + 4)}
        self.excluded = {}
        self.dtype = "bf16"
        self.config = {"workload": name, "batch": wl.batch, "queries": wl.tq, "context": wl.extra["context"],
                       "heads": wl.heads, "latent_dim": wl.dim, "m_hc": wl.m_hc, "window": wl.window,
                       "kv": wl.kv_dtype}
        self.metric = "HCA prefill chunk tokens/s (2048 queries over 64k ctx) on 1 GPU; attention TFLOP/s vs bf16 MFMA peak"
        self.torch = torch

    def step(self, i):
        self.layers[i].step()

    def dominant_launch(self, i):
        self.layers[i].attend()

    def extra_timings(self):
        L = self.layers
        return {"compress_call_us": round(launch_us(self.torch, len(L), 10, lambda i: L[i].compress()), 2)}

    def traffic(self):
        return None

    def cpu_baseline(self, seconds):
        import oracle
        L, nq = self.layers[0], 4
        raw = L.raw_kv.data.double().cpu().numpy()
        kv0 = L.kv_hc.data.double().cpu().numpy()
        q = L.q.data.double().cpu().numpy()
        z = L.z_hc.cpu().numpy().astype(np.float64)
        base, n0, nb = L.host["raw_base"], L.host["n0"], L.max_blocks
        rows = np.linspace(0, L.tq - 1, nq).astype(int)

        def sample():
            kv = kv0.copy()
            blocks = oracle.compress(raw, base, z, L.m_hc, [n0], [nb])[0][1]
            kv[0, n0:n0 + nb] = blocks
            for r in rows:
                oracle.hca_attn(q[:, r:r + 1], kv, L.m_hc, raw, base, L.W, L.host["t"][:, r:r + 1], L.scale)
            return f"compress the chunk's {nb} blocks + {nq} of {L.tq} chunk queries (dense over their visible blocks)"

        return time_oracle(sample, seconds, nq)


class HybridDecode:
    """The hybrid layer pair: a CSA layer (bf16 indexer, top-1024) and an HCA layer, batch 32,
    262k contexts, bf16 or fp8 KV; each step first compresses the blocks the new token completes."""

    def __init__(self, name, sets, torch, kv):
        from long_context_attention_04_amd import workloads
        import synth
        self.wl = wl = synth.WORKLOADS[name]
        self.pairs = [workloads.build(name, kv_fmt=kv, salt=s) for s in range(sets)]
        C, Hh = self.pairs[0]
        self.tokens = C.B
        t = C.host["t"][:, 0]
        vc = (t + 1) // C.m
        vh = (t + 1) // Hh.m_hc
        eb = 2 if kv == "bf16" else 1
        keys = int(np.sum(vc)) * C.dI * 2
        self.bytes = {"csa_keys": keys, "csa_gather": C.B * (C.k + C.W) * C.D * eb,
                      "hca_entries": int(np.sum(vh + Hh.W)) * Hh.D * eb,
                      "q_out_lse": 2 * C.B * C.H * (C.D * 2 + C.D * 4 + 4), "idx": C.B * C.k * 4,
                      "q_idx_w": C.B * C.HI * (C.dI * 2 + 4)}
        self.excluded = {"scores": C.B * C.n_cap * 4}
        self.dominant = {"kernel": "index_bf16_kernel (csa_index_scores, CSA layer)", "bound": "hbm",
                         "work": keys + self.bytes["q_idx_w"], "work_note": "visible bf16 keys + q_idx and w"}
        self.dtype = kv
        self.config = {"workload": name, "batch": wl.batch, "context": f"{wl.extra['context']}+U[0, {wl.extra['tail_hi']}]",
                       "heads": wl.heads, "latent_dim": wl.dim, "m": wl.m, "m_hc": wl.m_hc, "topk": wl.topk,
                       "window": wl.window, "kv": kv, "indexer": wl.idx_dtype}
        self.metric = f"hybrid CSA+HCA layer-pair decode tokens/s (batch 32, 262k ctx, {kv} KV) on 1 GPU; HBM TB/s vs peak"
        self.torch = torch

    def step(self, i):
        C, Hh = self.pairs[i]
        C.step()
        Hh.step()

    def dominant_launch(self, i):
        self.pairs[i][0].index()

    def extra_timings(self):
        P = self.pairs
        return {"csa_attention_call_us": round(launch_us(self.torch, len(P), 20, lambda i: P[i][0].attend()), 2),
                "hca_attention_call_us": round(launch_us(self.torch, len(P), 20, lambda i: P[i][1].attend()), 2),
                "csa_topk_call_us": round(launch_us(self.torch, len(P), 20, lambda i: P[i][0].topk()), 2)}

    def traffic(self):
        return None

    def cpu_baseline(self, seconds):
        import oracle
        from oracle import formats as OF
        C, Hh = self.pairs[0]
        n_seq = 4

        def values(st, b, rows):  # stored rows as values (bf16 cast, or e4m3 codes times row scales)
            if st.scale is None:
                return st.data[b, rows].double().cpu().numpy()
            return OF.dequantize_fp8_rows(st.data[b, rows].cpu().numpy(), st.scale[b, rows].cpu().numpy())

        data = []
        for b in range(n_seq):
            t = int(C.host["t"][b, 0])
            vc, vh = (t + 1) // C.m, (t + 1) // Hh.m_hc
            data.append((t, C.q_idx.data[b:b + 1].double().cpu().numpy(), C.w[b:b + 1].cpu().numpy().astype(np.float64),
                         C.k_idx.data[b, :vc].double().cpu().numpy(), C.q.data[b:b + 1].double().cpu().numpy(),
                         Hh.q.data[b:b + 1].double().cpu().numpy(), values(Hh.kv_hc, b, slice(0, vh)),
                         values(C.raw_kv, b, slice(None))[None]))

        def sample():
            for b, (t, qi, w, kc, q, qh, kh, raw) in enumerate(data):
                tt = np.array([[t]])
                sc = oracle.index_scores(qi, w, kc[None], tt, C.m, n_cap=kc.shape[0])
                oracle.topk(sc, tt, C.m, C.k)
                oracle.hca_attn(qh, kh[None], Hh.m_hc, raw, C.host["raw_base"][b:b + 1], Hh.W, tt, Hh.scale)
            return f"{n_seq} of {C.B} sequences (CSA index {C.n_cap} blocks + top-{C.k}, HCA attention)"

        return time_oracle(sample, seconds, n_seq)


def make_job(args, torch):
    import synth
    kind = synth.WORKLOADS[args.workload].kind
    if kind == "csa_decode" and args.workload == "csa_decode_1m_b8":
        if args.kv == "fp8":
            print("the 1M decode runs with bf16 or mxfp4 KV", file=sys.stderr)
            sys.exit(2)
        return CsaDecode(args.workload, args.sets, torch, args.kv or "bf16")
    if kind == "csa2_decode":
        if args.kv == "fp8":
            print("CSA2 runs with mxfp4 or bf16 KV", file=sys.stderr)
            sys.exit(2)
        return Csa2Decode(args.workload, args.sets, torch, args.kv or "mxfp4")
    if kind == "csa_prefill":
        return CsaPrefill(args.workload, min(args.sets, 3), torch)
    if kind == "hca_decode":
        return HcaDecode(args.workload, args.sets, torch)
    if kind == "hca_prefill":
        return HcaPrefill(args.workload, min(args.sets, 3), torch)
    if kind == "hybrid_decode":
        if args.kv == "mxfp4":
            print("the hybrid pair runs with bf16 or fp8 KV", file=sys.stderr)
            sys.exit(2)
        return HybridDecode(args.workload, min(args.sets, 4), torch, args.kv or "bf16")
    print(f"bench.py times the 1M decode, prefill, HCA and hybrid workloads; {args.workload} is covered by the "
          "parity tests", file=sys.stderr)
    sys.exit(2)


# ============================================================================ main


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the hot path shards by sequence with no collectives; see DESIGN.md)", file=sys.stderr)
        sys.exit(2)
    import torch

    import long_context_attention_04_amd as csa  # noqa: F401  (fails loudly when libcsa.so is missing)

    torch.cuda.set_device(0)
    job = make_job(args, torch)
    nsets = len(job.layers) if hasattr(job, "layers") else len(job.pairs)
    torch.cuda.synchronize()

    # ---- eager warm-up (also validates every stage once)
    for i in range(max(args.warmup, 1)):
        job.step(i % nsets)
    torch.cuda.synchronize()

    cycle, singles = None, []
    if not args.no_graph:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for i in range(nsets):
                job.step(i)  # warm the capture stream
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        for i in range(nsets):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                job.step(i)
            singles.append(g)
        cycle = torch.cuda.CUDAGraph()  # one step per input set, back to back
        with torch.cuda.graph(cycle):
            for i in range(nsets):
                job.step(i)
        for i in range(args.warmup):
            singles[i % nsets].replay()
        cycle.replay()
        torch.cuda.synchronize()

    # ---- timed region: exactly K steps
    K = args.steps
    n_cycles = K // nsets if cycle is not None else 0
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n_cycles + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if cycle is not None:
        ev[0].record()
        for c in range(n_cycles):
            cycle.replay()
            ev[c + 1].record()
        for i in range(K % nsets):
            singles[i].replay()
    else:
        for i in range(K):
            job.step(i % nsets)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    step_us = dt * 1e6 / K
    if n_cycles:
        per = np.array([ev[c].elapsed_time(ev[c + 1]) * 1e3 / nsets for c in range(n_cycles)])
        dist = {"median": round(float(np.median(per)), 2), "p10": round(float(np.percentile(per, 10)), 2),
                "p90": round(float(np.percentile(per, 90)), 2), "samples": int(n_cycles),
                "sample": f"one graph replay of {nsets} steps / {nsets}"}
    else:
        dist = None
    eager_us = launch_us(torch, nsets, K, job.step)

    # ---- dominant kernel, roofline, ceiling
    dom_us = launch_us(torch, nsets, max(K, 20), job.dominant_launch)
    d = job.dominant
    if d["bound"] == "mfma":
        achieved = d["work"] / (dom_us * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / BF16_PEAK_TFLOPS, 4), "traffic": None}
    else:
        achieved = d["work"] / (dom_us * 1e-6) / 1e9
        traffic = job.traffic()
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic}
    roof.update({"kernel": d["kernel"], "kernel_us": round(dom_us, 2), "work_per_launch": d["work"],
                 "work_note": d["work_note"]})
    ceiling = None if args.no_ceiling else stream_ceiling(torch)
    if ceiling and roof["bound"] == "hbm":
        roof["frac_of_ceiling"] = round(roof["achieved"] / ceiling["gb_s"], 4)
    step_bytes = sum(job.bytes.values())
    res = {
        "metric": job.metric, "value": round(job.tokens * K / dt, 1), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(step_us * 1e-3, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": job.dtype, "data": "synthetic",
        "config": dict(job.config, timing=f"graph of {nsets} steps" if cycle is not None else "eager",
                       input_sets=nsets),
        "step_us": dist, "eager_step_us": round(eager_us, 2),
        "hbm_tb_s_step": round(step_bytes / (step_us * 1e-6) / 1e12, 3),
        "algorithmic_bytes_per_step": step_bytes, "algorithmic_bytes": job.bytes,
        "excluded_bytes_per_step": job.excluded,
        "roofline": roof, "stream_read_ceiling": ceiling,
    }
    res.update(job.extra_timings())
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)  # one elementwise kernel: reads n bytes, writes n bytes
        torch.cuda.synchronize()
        res["copy_calibration_bytes"] = n
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = job.cpu_baseline(args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
