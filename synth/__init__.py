"""Seeded synthetic inputs for the CSA / HCA hot path.

This module only draws random numbers and describes workload sizes; it holds
none of the method's arithmetic (no merging, scoring, selection, softmax or
quantisation).  Both the CPU oracle's tests and the HIP path's tests and bench
draw their inputs from here, so both sides see identical inputs.

Generator: numpy PCG64 seeded with SeedSequence([0xC5A, workload id,
crc32(tensor name)]); normals are drawn with ``standard_normal(dtype=float32)``.
Activations (raw KV rows, raw indexer keys, latent queries, indexer queries and
head weights, compressor logits) are plain N(0, 1).  Tensors too large to draw
on the host in reasonable time (the two > 1 GiB compressed caches) are drawn on
the device with torch's seeded generator instead; see ``device_normal``.
"""
from __future__ import annotations

import zlib
from dataclasses import dataclass, field

import numpy as np

SEED_ROOT = 0xC5A


@dataclass(frozen=True)
class Workload:
    """Sizes of one workload.  `kind` says which stages run."""

    name: str
    wid: int
    kind: str  # "csa_decode" | "csa2_decode" | "csa_prefill" | "hca_decode" | "hca_prefill" | "hybrid_decode"
    batch: int
    tq: int
    heads: int
    dim: int
    window: int
    kv_dtype: str
    m: int = 4
    m_hc: int = 128
    idx_heads: int = 0
    idx_dim: int = 0
    topk: int = 0
    idx_dtype: str = "f32"
    notes: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def scale(self) -> float:
        # softmax scale 1/sqrt(128): every workload has query heads of dim 128
        return 1.0 / np.sqrt(128.0)


WORKLOADS = {
    w.name: w
    for w in [
        Workload(
            name="csa_decode_tiny_4k", wid=1, kind="csa_decode", batch=1, tq=1,
            heads=16, dim=128, window=64, kv_dtype="f32", m=4, idx_heads=4, idx_dim=32,
            topk=32, idx_dtype="f32",
            notes="1 query at position 4095 over 4096 raw tokens; fp32 throughout",
            extra={"context": 4096},
        ),
        Workload(
            name="csa_prefill_2k_on_64k", wid=2, kind="csa_prefill", batch=1, tq=2048,
            heads=64, dim=512, window=128, kv_dtype="bf16", m=4, idx_heads=8, idx_dim=64,
            topk=512, idx_dtype="bf16",
            notes="2048 new queries at positions 65536..67583 over a 65536-token context",
            extra={"context": 65536},
        ),
        Workload(
            name="hca_decode_b64_128k", wid=3, kind="hca_decode", batch=64, tq=1,
            heads=64, dim=512, window=128, kv_dtype="bf16", m_hc=128,
            notes="per-sequence context lengths uniform in [65536, 131072]",
            extra={"len_lo": 65536, "len_hi": 131072},
        ),
        Workload(
            name="csa_decode_1m_b8", wid=4, kind="csa_decode", batch=8, tq=1,
            heads=64, dim=512, window=128, kv_dtype="bf16", m=4, idx_heads=8, idx_dim=64,
            topk=2048, idx_dtype="mxfp4",
            notes="1 query per sequence at position 1048575 over 1048576 raw tokens",
            extra={"context": 1048576},
        ),
        Workload(
            name="hybrid_decode_b32_256k", wid=5, kind="hybrid_decode", batch=32, tq=1,
            heads=64, dim=512, window=128, kv_dtype="bf16", m=4, m_hc=128, idx_heads=8,
            idx_dim=64, topk=1024, idx_dtype="bf16",
            notes="262144 + tail tokens, tail uniform in [0, 127]; bf16 or fp8 e4m3 KV",
            extra={"context": 262144, "tail_hi": 127},
        ),
        Workload(
            name="csa2_decode_1m_b8", wid=7, kind="csa2_decode", batch=8, tq=1,
            heads=64, dim=512, window=128, kv_dtype="mxfp4", m=4, idx_heads=8, idx_dim=64,
            topk=2048, idx_dtype="mxfp4",
            notes="a group of 2 layers sharing one compressed cache (MXFP4 entries, bf16 window) and "
                  "one top-k; each layer attends with its own query; 1M context as the 1M decode",
            extra={"context": 1048576, "layers": 2},
        ),
        Workload(
            name="hca_prefill_2k_on_64k", wid=6, kind="hca_prefill", batch=1, tq=2048,
            heads=64, dim=512, window=128, kv_dtype="bf16", m_hc=128,
            notes="2048 new queries at positions 65536..67583 over a 65536-token context; the chunk "
                  "completes 16 heavily compressed blocks, which the step compresses",
            extra={"context": 65536},
        ),
    ]
}


def seed_for(w: Workload | int, name: str, salt: int = 0) -> np.random.SeedSequence:
    wid = w.wid if isinstance(w, Workload) else int(w)
    return np.random.SeedSequence([SEED_ROOT, wid, zlib.crc32(name.encode()), int(salt)])


def rng(w: Workload | int, name: str, salt: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed_for(w, name, salt)))


def normal(w: Workload | int, name: str, shape, salt: int = 0) -> np.ndarray:
    """N(0, 1) float32 of the given shape."""
    return rng(w, name, salt).standard_normal(size=tuple(shape), dtype=np.float32)


def integers(w: Workload | int, name: str, lo: int, hi: int, size, salt: int = 0) -> np.ndarray:
    """Uniform integers in [lo, hi] (both ends included)."""
    return rng(w, name, salt).integers(lo, hi, size=size, endpoint=True).astype(np.int64)


def device_seed(w: Workload | int, name: str, salt: int = 0) -> int:
    """A 63-bit seed for torch's device generator, derived from the same seed sequence."""
    return int(seed_for(w, name, salt).generate_state(2, dtype=np.uint32).astype(np.uint64)
               .view(np.uint64)[0] & np.uint64(0x7FFFFFFFFFFFFFFF))


def device_normal(w: Workload | int, name: str, shape, device, dtype=None, salt: int = 0,
                  chunk_rows: int = 1 << 16):
    """N(0, 1) drawn on `device` by torch's seeded generator, stored as `dtype`.

    Drawn in fp32 chunks along the leading dims and cast chunk by chunk (the cast
    is a storage conversion done by torch), so peak extra memory stays small.
    """
    import torch

    dtype = dtype or torch.float32
    g = torch.Generator(device=device)
    g.manual_seed(device_seed(w, name, salt))
    out = torch.empty(tuple(shape), dtype=dtype, device=device)
    flat = out.view(-1, shape[-1])
    for r0 in range(0, flat.shape[0], chunk_rows):
        r1 = min(flat.shape[0], r0 + chunk_rows)
        flat[r0:r1] = torch.randn((r1 - r0, shape[-1]), generator=g, device=device,
                                  dtype=torch.float32).to(dtype)
    return out
