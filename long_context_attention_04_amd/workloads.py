"""Device-side workloads and step runners built on the C ABI.

A *step* is one decode (or prefill-chunk) pass of an attention layer: first
the compressor merges any block completed by the new token(s), then the
lightning indexer scores the compressed blocks, top-k selects them and sparse
attention runs over the selection plus the sliding window (CSA); HCA attends
densely over its heavily compressed blocks plus the window.  Every stage is a
call into libcsa; this module only allocates device memory (torch), fills it
from the seeded generators in ``synth`` and orders the calls.

Inputs are synthetic (see synth): N(0, 1) raw rows, latent queries, indexer
queries, head weights and compressor logits.  Compressed caches of the 1M and
262k contexts are drawn directly (N(0, 1) rows, MXFP4/bf16 keys quantised by
the library), except the blocks a step completes, which the step itself
produces with the compressor.  Cache rows beyond a sequence's visible blocks
are filled with NaN so a stray read shows up in the output.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

import synth

from . import (BF16, F32, FP8_E4M3, MXFP4, csa_attn_workspace_size, csa_compress, csa_compress_index_topk,
               csa_compress_jobs,
               csa_index_scores, csa_index_topk, csa_index_topk_part, csa_index_topk_workspace_size, csa_quantize_fp8, csa_quantize_mxfp4, csa_sparse_attn,
               csa_topk, csa_topk_workspace_size, desc, hca_attn)

DEV = "cuda"


def _i32(x):
    return torch.as_tensor(np.asarray(x, dtype=np.int32), device=DEV)


def _f32(x):
    return torch.as_tensor(np.asarray(x, dtype=np.float32), device=DEV)


def _bf16(x):
    return torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).to(DEV)


def quantize_mxfp4_rows(x: torch.Tensor):
    """[..., n] fp32 device tensor -> (codes [..., n/2] u8, scales [..., n/32] u8) via the library."""
    rows = x.numel() // x.shape[-1]
    codes = torch.empty(x.shape[:-1] + (x.shape[-1] // 2,), dtype=torch.uint8, device=DEV)
    scales = torch.empty(x.shape[:-1] + (x.shape[-1] // 32,), dtype=torch.uint8, device=DEV)
    csa_quantize_mxfp4(x.contiguous(), rows, x.shape[-1], codes, scales)
    return codes, scales


def quantize_fp8_rows(x: torch.Tensor):
    rows = x.numel() // x.shape[-1]
    codes = torch.empty(x.shape, dtype=torch.uint8, device=DEV)
    scale = torch.empty(x.shape[:-1], dtype=torch.float32, device=DEV)
    csa_quantize_fp8(x.contiguous(), rows, x.shape[-1], codes, scale)
    return codes, scale


@dataclass
class Stored:
    """A stored [B, rows, dim] tensor in one of the library formats."""

    data: torch.Tensor
    dtype: int
    scale: torch.Tensor | None = None

    def desc(self):
        return desc(self.data, self.dtype, self.scale)


def store(x: torch.Tensor, fmt: str) -> Stored:
    """fp32 [B, rows, dim] device tensor -> stored format (bf16 cast by torch; fp8/MXFP4 by the library)."""
    if fmt == "f32":
        return Stored(x.contiguous(), F32)
    if fmt == "bf16":
        return Stored(x.to(torch.bfloat16).contiguous(), BF16)
    if fmt == "fp8":
        c, s = quantize_fp8_rows(x)
        return Stored(c, FP8_E4M3, s)
    if fmt == "mxfp4":
        c, s = quantize_mxfp4_rows(x)
        return Stored(c, MXFP4, s)
    raise ValueError(fmt)


def empty_stored(B, rows, dim, fmt) -> Stored:
    if fmt == "f32":
        return Stored(torch.full((B, rows, dim), float("nan"), device=DEV), F32)
    if fmt == "bf16":
        return Stored(torch.full((B, rows, dim), float("nan"), dtype=torch.bfloat16, device=DEV), BF16)
    if fmt == "fp8":
        return Stored(torch.full((B, rows, dim), 0x7F, dtype=torch.uint8, device=DEV), FP8_E4M3,
                      torch.ones((B, rows), device=DEV))
    if fmt == "mxfp4":
        return Stored(torch.zeros((B, rows, dim // 2), dtype=torch.uint8, device=DEV), MXFP4,
                      torch.full((B, rows, dim // 32), 0xFF, dtype=torch.uint8, device=DEV))
    raise ValueError(fmt)


# ============================================================================ CSA layer state


@dataclass
class CsaLayer:
    """State of one CSA layer for a batch of sequences, plus one step's inputs."""

    B: int
    tq: int
    m: int
    H: int
    D: int
    HI: int
    dI: int
    k: int
    W: int
    n_cap: int
    scale: float
    kv_cmp: Stored            # [B, n_cap, D]
    k_idx: Stored             # [B, n_cap, dI]
    raw_kv: Stored            # [B, R, D]   raw rows (window + blocks to compress)
    raw_ik: Stored            # [B, R, dI]  raw indexer keys
    raw_base: torch.Tensor    # [B] int32
    z_kv: torch.Tensor        # [m] f32
    z_ik: torch.Tensor        # [m] f32
    q: Stored                 # [B, tq, H, D]
    q_idx: Stored             # [B, tq, HI, dI]
    w: torch.Tensor           # [B, tq, HI] f32
    q_pos: torch.Tensor       # [B, tq] int32
    blk_first: torch.Tensor   # [B] int32 blocks this step completes
    blk_count: torch.Tensor   # [B] int32
    max_blocks: int
    scores: torch.Tensor = None
    idx: torch.Tensor = None
    out: torch.Tensor = None
    lse: torch.Tensor = None
    ws_topk: torch.Tensor = None
    ws_itk: torch.Tensor = None
    ws_attn: torch.Tensor = None
    host: dict = field(default_factory=dict)  # host copies of small inputs (positions etc.)

    def alloc_outputs(self):
        B, tq = self.B, self.tq
        self.scores = torch.empty((B, tq, self.n_cap), dtype=torch.float32, device=DEV)
        self.idx = torch.empty((B, tq, self.k), dtype=torch.int32, device=DEV)
        self.out = torch.empty((B, tq, self.H, self.D), dtype=torch.float32, device=DEV)
        self.lse = torch.empty((B, tq, self.H), dtype=torch.float32, device=DEV)
        n = csa_topk_workspace_size(B, tq, self.n_cap, self.k)
        self.ws_topk = torch.empty(max(n, 1), dtype=torch.uint8, device=DEV)
        n = csa_index_topk_workspace_size(B, tq, self.n_cap, self.k, scores_kept=False)  # fits either use
        self.ws_itk = torch.empty(max(n, 1), dtype=torch.uint8, device=DEV)
        n = csa_attn_workspace_size(B, tq, self.H, self.D, self.k + self.W)
        self.ws_attn = torch.empty(max(n, 1), dtype=torch.uint8, device=DEV)

    # --- stages -------------------------------------------------------------
    def compress_kv(self, stream=None):
        csa_compress(self.raw_kv.desc(), self.raw_base, self.z_kv, self.m, self.D, self.blk_first, self.blk_count,
                     self.max_blocks, self.B, self.kv_cmp.desc(), stream)

    def compress_keys(self, stream=None):
        csa_compress(self.raw_ik.desc(), self.raw_base, self.z_ik, self.m, self.dI, self.blk_first, self.blk_count,
                     self.max_blocks, self.B, self.k_idx.desc(), stream)

    def kv_job(self):
        return (self.raw_kv.desc(), self.raw_base, self.z_kv, self.m, self.D, self.blk_first, self.blk_count,
                self.max_blocks, self.B, self.kv_cmp.desc())

    def key_job(self):
        return (self.raw_ik.desc(), self.raw_base, self.z_ik, self.m, self.dI, self.blk_first, self.blk_count,
                self.max_blocks, self.B, self.k_idx.desc())

    def compress(self, stream=None):
        """Both compressions of the step (KV and indexer key) in one launch."""
        csa_compress_jobs([self.kv_job(), self.key_job()], stream)

    def compress_index_topk(self, part=3, stream=None):
        """compress, then index_topk (or one part of it), the compressions inside the indexer
        launch where the shapes allow."""
        csa_compress_index_topk(self.kv_job(), self.key_job(), self.q_idx.desc(), self.w, self.k_idx.desc(),
                                self.q_pos, self.B, self.tq, self.HI, self.dI, self.m, self.n_cap, self.k,
                                self._scores(), self.idx, self.ws_itk, self.ws_itk.numel(), part, stream)

    def index(self, stream=None):
        csa_index_scores(self.q_idx.desc(), self.w, self.k_idx.desc(), self.q_pos, self.B, self.tq, self.HI, self.dI,
                         self.m, self.n_cap, self.scores, stream)

    def topk(self, stream=None):
        csa_topk(self.scores, self.q_pos, self.B, self.tq, self.n_cap, self.m, self.k, self.idx, self.ws_topk,
                 self.ws_topk.numel(), stream)

    def index_topk(self, stream=None):
        csa_index_topk(self.q_idx.desc(), self.w, self.k_idx.desc(), self.q_pos, self.B, self.tq, self.HI, self.dI,
                       self.m, self.n_cap, self.k, self._scores(), self.idx, self.ws_itk, self.ws_itk.numel(), stream)

    def index_topk_part(self, part, stream=None):
        """Part 1 (scores + slice candidates) or part 2 (selection) of index_topk."""
        csa_index_topk_part(self.q_idx.desc(), self.w, self.k_idx.desc(), self.q_pos, self.B, self.tq, self.HI,
                            self.dI, self.m, self.n_cap, self.k, self._scores(), self.idx, self.ws_itk,
                            self.ws_itk.numel(), part, stream)

    def attend(self, stream=None):
        csa_sparse_attn(self.q.desc(), self.kv_cmp.desc(), self.idx, self.k, self.raw_kv.desc(), self.raw_base,
                        self.W, self.q_pos, self.B, self.tq, self.H, self.D, self.scale, self.out, self.lse,
                        self.ws_attn, self.ws_attn.numel(), stream)

    stage_names = ("compress", "index+topk", "attention")
    fused_select = True  # score and select with csa_index_topk (else csa_index_scores, then csa_topk)
    fused_compress = True  # with fused_select: the compressions run inside the indexer launch
    keep_scores = False  # with fused_select: also return every score (in self.scores)

    def _scores(self):
        return self.scores if self.keep_scores else None

    def select(self, stream=None):
        if self.fused_select:
            self.index_topk(stream)
        else:
            self.index(stream)
            self.topk(stream)

    def step(self, stream=None, marks=None):
        """One pass of the CSA hot path (compress the new blocks, score and select the
        top-k, attend).  `marks(i)` is called between stages; with the compressions
        inside the indexer launch, the compress stage is empty and index+topk holds them."""
        if self.fused_select and self.fused_compress:
            stages = (lambda st: None, lambda st: self.compress_index_topk(3, st), self.attend)
        else:
            stages = (self.compress, self.select, self.attend)
        for i, stage in enumerate(stages):
            if marks:
                marks(i)
            stage(stream)
        if marks:
            marks(len(self.stage_names))


@dataclass
class HcaLayer:
    B: int
    tq: int
    m_hc: int
    H: int
    D: int
    W: int
    n_cap: int
    scale: float
    kv_hc: Stored
    raw_kv: Stored
    raw_base: torch.Tensor
    z_hc: torch.Tensor
    q: Stored
    q_pos: torch.Tensor
    blk_first: torch.Tensor
    blk_count: torch.Tensor
    max_blocks: int
    out: torch.Tensor = None
    lse: torch.Tensor = None
    ws_attn: torch.Tensor = None
    host: dict = field(default_factory=dict)

    def alloc_outputs(self):
        self.out = torch.empty((self.B, self.tq, self.H, self.D), dtype=torch.float32, device=DEV)
        self.lse = torch.empty((self.B, self.tq, self.H), dtype=torch.float32, device=DEV)
        n = csa_attn_workspace_size(self.B, self.tq, self.H, self.D, self.n_cap + self.W)
        self.ws_attn = torch.empty(max(n, 1), dtype=torch.uint8, device=DEV)

    def compress(self, stream=None):
        csa_compress(self.raw_kv.desc(), self.raw_base, self.z_hc, self.m_hc, self.D, self.blk_first, self.blk_count,
                     self.max_blocks, self.B, self.kv_hc.desc(), stream)

    def attend(self, stream=None):
        hca_attn(self.q.desc(), self.kv_hc.desc(), self.m_hc, self.n_cap, self.raw_kv.desc(), self.raw_base, self.W,
                 self.q_pos, self.B, self.tq, self.H, self.D, self.scale, self.out, self.lse, self.ws_attn,
                 self.ws_attn.numel(), stream)

    def step(self, stream=None, marks=None):
        for i, stage in enumerate((self.compress, self.attend)):
            if marks:
                marks(i)
            stage(stream)
        if marks:
            marks(2)


# ============================================================================ builders


def _poison_beyond(st: Stored, visible: np.ndarray):
    """NaN-fill rows at or beyond each sequence's visible count (bf16/f32 only)."""
    if st.dtype not in (F32, BF16):
        return
    for b, v in enumerate(visible):
        st.data[b, int(v):] = float("nan")


def build_csa_decode(wl: synth.Workload, salt: int = 0, kv_fmt: str | None = None) -> CsaLayer:
    """A CSA decode step at position L-1 over a context of L tokens (L % m == 0, so the
    step completes block L/m - 1).  Blocks before it are drawn directly for contexts
    beyond 64k tokens and produced by the compressor from raw rows otherwise.  kv_fmt
    overrides the workload's KV format (e.g. "mxfp4": FP4 KV caching of the compressed
    entries and the window rows)."""
    B, m, H, D, HI, dI, k, W = wl.batch, wl.m, wl.heads, wl.dim, wl.idx_heads, wl.idx_dim, wl.topk, wl.window
    L = wl.extra["context"]
    N = L // m
    t = L - 1
    direct = L > 65536
    R = W if direct else L                       # raw rows kept on the device
    base = L - R
    raw_kv = torch.as_tensor(synth.normal(wl, "raw_kv", (B, R, D), salt), device=DEV) if not direct else \
        synth.device_normal(wl, "raw_kv", (B, R, D), DEV, salt=salt)
    raw_ik = torch.as_tensor(synth.normal(wl, "raw_ik", (B, R, dI), salt), device=DEV) if not direct else \
        synth.device_normal(wl, "raw_ik", (B, R, dI), DEV, salt=salt)
    kv_fmt = kv_fmt or wl.kv_dtype
    ik_fmt = wl.idx_dtype
    raw_kv_s = store(raw_kv, "bf16" if kv_fmt == "mxfp4" else kv_fmt)  # MXFP4 caches keep bf16 raw rows
    raw_ik_s = Stored(raw_ik.contiguous(), F32)
    z_kv = _f32(synth.normal(wl, "z_kv", (m,), salt))
    z_ik = _f32(synth.normal(wl, "z_ik", (m,), salt))
    raw_base = _i32(np.full(B, base))
    if direct:
        kv_cmp = Stored(synth.device_normal(wl, "kv_cmp", (B, N, D), DEV, dtype=torch.bfloat16, salt=salt), BF16) \
            if kv_fmt == "bf16" else store(synth.device_normal(wl, "kv_cmp", (B, N, D), DEV, salt=salt), kv_fmt)
        kraw = synth.device_normal(wl, "k_idx", (B, N, dI), DEV, salt=salt)
        k_idx = store(kraw, ik_fmt)
        del kraw
        # the block this step completes is produced by the step's compressor
        if k_idx.dtype == MXFP4:
            k_idx.data[:, N - 1] = 0
            k_idx.scale[:, N - 1] = 0xFF
        else:
            k_idx.data[:, N - 1] = float("nan")
        if kv_cmp.dtype in (F32, BF16):
            kv_cmp.data[:, N - 1] = float("nan")
        elif kv_cmp.dtype == MXFP4:
            kv_cmp.scale[:, N - 1] = 0xFF  # NaN scale until the step compresses the block
    else:
        kv_cmp = empty_stored(B, N, D, kv_fmt)
        k_idx = empty_stored(B, N, dI, ik_fmt)
        first = _i32(np.zeros(B))
        cnt = _i32(np.full(B, N - 1))
        csa_compress(raw_kv_s.desc(), raw_base, z_kv, m, D, first, cnt, N - 1, B, kv_cmp.desc())
        csa_compress(raw_ik_s.desc(), raw_base, z_ik, m, dI, first, cnt, N - 1, B, k_idx.desc())
    q_raw = synth.normal(wl, "q", (B, 1, H, D), salt)
    q = Stored(_f32(q_raw), F32) if kv_fmt == "f32" else Stored(_bf16(q_raw), BF16)
    qi = synth.normal(wl, "q_idx", (B, 1, HI, dI), salt)
    q_idx = Stored(_f32(qi), F32) if ik_fmt in ("f32", "mxfp4") else Stored(_bf16(qi), BF16)
    w = _f32(synth.normal(wl, "w_idx", (B, 1, HI), salt))
    layer = CsaLayer(B=B, tq=1, m=m, H=H, D=D, HI=HI, dI=dI, k=k, W=W, n_cap=N, scale=wl.scale, kv_cmp=kv_cmp,
                     k_idx=k_idx, raw_kv=raw_kv_s, raw_ik=raw_ik_s, raw_base=raw_base, z_kv=z_kv, z_ik=z_ik, q=q,
                     q_idx=q_idx, w=w, q_pos=_i32(np.full((B, 1), t)), blk_first=_i32(np.full(B, N - 1)),
                     blk_count=_i32(np.ones(B)), max_blocks=1)
    layer.host = {"t": np.full((B, 1), t), "raw_base": np.full(B, base), "L": L, "direct": direct}
    layer.alloc_outputs()
    return layer


@dataclass
class Csa2Group:
    """CSA2 cross-layer reuse: a group of layers sharing one compressed cache and one
    top-k selection.  The group's step compresses the new block and selects once (with
    the first layer's indexer query), then every layer attends over the shared entries
    with its own query; layer 0 is an ordinary CSA layer."""

    base: CsaLayer
    q: list          # per layer l >= 1: Stored [B, tq, H, D]
    out: list        # per layer l >= 1: [B, tq, H, D] f32
    lse: list
    ws_attn: list

    @property
    def layers(self):
        return 1 + len(self.q)

    def attend_layer(self, l, stream=None):
        L = self.base
        if l == 0:
            L.attend(stream)
            return
        csa_sparse_attn(self.q[l - 1].desc(), L.kv_cmp.desc(), L.idx, L.k, L.raw_kv.desc(), L.raw_base, L.W, L.q_pos,
                        L.B, L.tq, L.H, L.D, L.scale, self.out[l - 1], self.lse[l - 1], self.ws_attn[l - 1],
                        self.ws_attn[l - 1].numel(), stream)

    def attend(self, stream=None):
        for l in range(self.layers):
            self.attend_layer(l, stream)

    def step(self, stream=None, marks=None):
        L = self.base
        if marks:
            marks(0)
        L.compress_index_topk(3, stream)
        if marks:
            marks(1)
        self.attend(stream)
        if marks:
            marks(2)


def build_csa2_decode(wl: synth.Workload, salt: int = 0, kv_fmt: str | None = None) -> Csa2Group:
    """The 1M decode's layer state (cache, indexer, window) shared by `layers` layers; the
    layers after the first draw their own queries."""
    base = build_csa_decode(wl, salt, kv_fmt)
    n = wl.extra["layers"]
    B, H, D = base.B, base.H, base.D
    qs = [Stored(_bf16(synth.normal(wl, f"q_layer{l}", (B, 1, H, D), salt)), BF16) for l in range(1, n)]
    outs = [torch.empty((B, 1, H, D), dtype=torch.float32, device=DEV) for _ in range(1, n)]
    lses = [torch.empty((B, 1, H), dtype=torch.float32, device=DEV) for _ in range(1, n)]
    nws = csa_attn_workspace_size(B, 1, H, D, base.k + base.W)
    wss = [torch.empty(max(nws, 1), dtype=torch.uint8, device=DEV) for _ in range(1, n)]
    return Csa2Group(base=base, q=qs, out=outs, lse=lses, ws_attn=wss)


def build_csa_prefill(wl: synth.Workload, salt: int = 0) -> CsaLayer:
    """A prefill chunk of Tq queries at positions L .. L+Tq-1 over an L-token context;
    the chunk completes Tq/m new blocks, which the step compresses."""
    B, m, H, D, HI, dI, k, W, Tq = wl.batch, wl.m, wl.heads, wl.dim, wl.idx_heads, wl.idx_dim, wl.topk, \
        wl.window, wl.tq
    L = wl.extra["context"]
    T = L + Tq
    N = T // m
    raw_kv = store(torch.as_tensor(synth.normal(wl, "raw_kv", (B, T, D), salt), device=DEV), wl.kv_dtype)
    raw_ik = store(torch.as_tensor(synth.normal(wl, "raw_ik", (B, T, dI), salt), device=DEV), wl.idx_dtype)
    z_kv = _f32(synth.normal(wl, "z_kv", (m,), salt))
    z_ik = _f32(synth.normal(wl, "z_ik", (m,), salt))
    raw_base = _i32(np.zeros(B))
    kv_cmp = empty_stored(B, N, D, wl.kv_dtype)
    k_idx = empty_stored(B, N, dI, wl.idx_dtype)
    n_prefix = L // m
    csa_compress(raw_kv.desc(), raw_base, z_kv, m, D, _i32(np.zeros(B)), _i32(np.full(B, n_prefix)), n_prefix, B,
                 kv_cmp.desc())
    csa_compress(raw_ik.desc(), raw_base, z_ik, m, dI, _i32(np.zeros(B)), _i32(np.full(B, n_prefix)), n_prefix, B,
                 k_idx.desc())
    q = Stored(_bf16(synth.normal(wl, "q", (B, Tq, H, D), salt)), BF16)
    q_idx = Stored(_bf16(synth.normal(wl, "q_idx", (B, Tq, HI, dI), salt)), BF16)
    w = _f32(synth.normal(wl, "w_idx", (B, Tq, HI), salt))
    pos = L + np.arange(Tq)[None].repeat(B, 0)
    layer = CsaLayer(B=B, tq=Tq, m=m, H=H, D=D, HI=HI, dI=dI, k=k, W=W, n_cap=N, scale=wl.scale, kv_cmp=kv_cmp,
                     k_idx=k_idx, raw_kv=raw_kv, raw_ik=raw_ik, raw_base=raw_base, z_kv=z_kv, z_ik=z_ik, q=q,
                     q_idx=q_idx, w=w, q_pos=_i32(pos), blk_first=_i32(np.full(B, n_prefix)),
                     blk_count=_i32(np.full(B, N - n_prefix)), max_blocks=N - n_prefix)
    layer.host = {"t": pos, "raw_base": np.zeros(B, np.int64), "L": L}
    layer.alloc_outputs()
    return layer


def build_hca_decode(wl: synth.Workload, salt: int = 0) -> HcaLayer:
    """HCA decode: sequence b has L_b tokens, the query sits at t_b = L_b - 1; all complete
    heavily-compressed blocks are drawn directly (rows beyond them are NaN)."""
    B, H, D, W, mh = wl.batch, wl.heads, wl.dim, wl.window, wl.m_hc
    Lb = synth.integers(wl, "lengths", wl.extra["len_lo"], wl.extra["len_hi"], B, salt)
    t = Lb - 1
    ncap = int(wl.extra["len_hi"] // mh)
    kv = Stored(synth.device_normal(wl, "kv_hc", (B, ncap, D), DEV, dtype=torch.bfloat16, salt=salt), BF16)
    vis = (t + 1) // mh
    _poison_beyond(kv, vis)
    raw = store(synth.device_normal(wl, "raw_kv", (B, W, D), DEV, salt=salt), wl.kv_dtype)
    base = t - W + 1
    q = Stored(_bf16(synth.normal(wl, "q", (B, 1, H, D), salt)), BF16)
    layer = HcaLayer(B=B, tq=1, m_hc=mh, H=H, D=D, W=W, n_cap=ncap, scale=wl.scale, kv_hc=kv, raw_kv=raw,
                     raw_base=_i32(base), z_hc=_f32(synth.normal(wl, "z_hc", (mh,), salt)), q=q,
                     q_pos=_i32(t[:, None]), blk_first=_i32(np.zeros(B)), blk_count=_i32(np.zeros(B)), max_blocks=0)
    layer.host = {"t": t[:, None], "raw_base": base, "vis": vis}
    layer.alloc_outputs()
    return layer


def build_hca_prefill(wl: synth.Workload, salt: int = 0) -> HcaLayer:
    """HCA prefill: a chunk of Tq queries at positions L .. L+Tq-1 over an L-token context.
    The L/m_hc blocks before the chunk are drawn directly; the Tq/m_hc blocks the chunk
    completes are compressed by the step (block j is visible to query t once 128j+127 <= t).
    Raw rows kept: positions L-W .. L+Tq-1 (every query's window and the chunk's blocks)."""
    B, H, D, W, mh, Tq = wl.batch, wl.heads, wl.dim, wl.window, wl.m_hc, wl.tq
    L = wl.extra["context"]
    n0 = L // mh
    N = (L + Tq) // mh
    rbase = L - W
    raw = store(synth.device_normal(wl, "raw_kv", (B, W + Tq, D), DEV, salt=salt), wl.kv_dtype)
    kv = Stored(synth.device_normal(wl, "kv_hc", (B, N, D), DEV, dtype=torch.bfloat16, salt=salt), BF16)
    kv.data[:, n0:] = float("nan")  # written by the step's compression
    pos = L + np.arange(Tq)[None].repeat(B, 0)
    q = Stored(_bf16(synth.normal(wl, "q", (B, Tq, H, D), salt)), BF16)
    layer = HcaLayer(B=B, tq=Tq, m_hc=mh, H=H, D=D, W=W, n_cap=N, scale=wl.scale, kv_hc=kv, raw_kv=raw,
                     raw_base=_i32(np.full(B, rbase)), z_hc=_f32(synth.normal(wl, "z_hc", (mh,), salt)), q=q,
                     q_pos=_i32(pos), blk_first=_i32(np.full(B, n0)), blk_count=_i32(np.full(B, N - n0)),
                     max_blocks=N - n0)
    layer.host = {"t": pos, "raw_base": np.full(B, rbase), "n0": n0, "L": L}
    layer.alloc_outputs()
    return layer


def build_hybrid_decode(wl: synth.Workload, kv_fmt: str = "bf16", salt: int = 0):
    """A CSA layer and an HCA layer decoding one new token per sequence at t_b = L_b over
    L_b = 262144 + tail_b tokens.  The step first compresses the CSA block ((t_b+1) % 4 == 0)
    and the HCA block ((t_b+1) % 128 == 0) the new token completes; blocks completed
    earlier in the tail come from the compressor at setup, the rest are drawn directly."""
    B, H, D, W, m, mh, HI, dI, k = wl.batch, wl.heads, wl.dim, wl.window, wl.m, wl.m_hc, wl.idx_heads, \
        wl.idx_dim, wl.topk
    base_ctx = wl.extra["context"]
    tail = synth.integers(wl, "tail", 0, wl.extra["tail_hi"], B, salt)
    t = base_ctx + tail                       # position of the new token
    N = (base_ctx + mh) // m                  # CSA capacity: every block up to position base_ctx + 127
    NH = (base_ctx + mh) // mh
    R = 2 * mh                                # raw rows kept: positions base_ctx - mh .. base_ctx + mh - 1
    rbase = np.full(B, base_ctx - mh)
    raw_kv_f = synth.device_normal(wl, "raw_kv", (B, R, D), DEV, salt=salt)
    raw_kv = store(raw_kv_f, kv_fmt)
    raw_ik = Stored(synth.device_normal(wl, "raw_ik", (B, R, dI), DEV, salt=salt), F32)
    z_kv = _f32(synth.normal(wl, "z_kv", (m,), salt))
    z_ik = _f32(synth.normal(wl, "z_ik", (m,), salt))
    z_hc = _f32(synth.normal(wl, "z_hc", (mh,), salt))
    n0 = base_ctx // m                        # CSA blocks drawn directly
    nh0 = base_ctx // mh                      # HCA blocks drawn directly
    kv_c = store(synth.device_normal(wl, "kv_cmp", (B, N, D), DEV, salt=salt), kv_fmt) if kv_fmt == "fp8" else \
        Stored(synth.device_normal(wl, "kv_cmp", (B, N, D), DEV, dtype=torch.bfloat16, salt=salt), BF16)
    k_idx = Stored(synth.device_normal(wl, "k_idx", (B, N, dI), DEV, dtype=torch.bfloat16, salt=salt), BF16)
    kv_h = store(synth.device_normal(wl, "kv_hc", (B, NH, D), DEV, salt=salt), kv_fmt) if kv_fmt == "fp8" else \
        Stored(synth.device_normal(wl, "kv_hc", (B, NH, D), DEV, dtype=torch.bfloat16, salt=salt), BF16)
    # rows not drawn directly start poisoned (NaN, or the e4m3 NaN code) until compressed
    for st, first in ((kv_c, n0), (k_idx, n0), (kv_h, nh0)):
        if st.dtype == FP8_E4M3:
            st.data[:, first:] = 0x7F
        else:
            st.data[:, first:] = float("nan")
    # setup: tail blocks completed before the new token (positions <= t_b - 1)
    done_c = t // m - n0                      # blocks n0 .. t//m - 1 are complete before t
    csa_compress(raw_kv.desc(), _i32(rbase), z_kv, m, D, _i32(np.full(B, n0)), _i32(done_c), int(done_c.max()), B,
                 kv_c.desc())
    csa_compress(raw_ik.desc(), _i32(rbase), z_ik, m, dI, _i32(np.full(B, n0)), _i32(done_c), int(done_c.max()), B,
                 Stored(k_idx.data, BF16).desc())
    # blocks the new token completes
    c_cnt = ((t + 1) % m == 0).astype(np.int64)
    h_cnt = ((t + 1) % mh == 0).astype(np.int64)
    csa = CsaLayer(B=B, tq=1, m=m, H=H, D=D, HI=HI, dI=dI, k=k, W=W, n_cap=N, scale=wl.scale, kv_cmp=kv_c,
                   k_idx=k_idx, raw_kv=raw_kv, raw_ik=raw_ik, raw_base=_i32(rbase), z_kv=z_kv, z_ik=z_ik,
                   q=Stored(_bf16(synth.normal(wl, "q_csa", (B, 1, H, D), salt)), BF16),
                   q_idx=Stored(_bf16(synth.normal(wl, "q_idx", (B, 1, HI, dI), salt)), BF16),
                   w=_f32(synth.normal(wl, "w_idx", (B, 1, HI), salt)), q_pos=_i32(t[:, None]),
                   blk_first=_i32((t + 1) // m - 1), blk_count=_i32(c_cnt), max_blocks=1)
    hca = HcaLayer(B=B, tq=1, m_hc=mh, H=H, D=D, W=W, n_cap=NH, scale=wl.scale, kv_hc=kv_h, raw_kv=raw_kv,
                   raw_base=_i32(rbase), z_hc=z_hc, q=Stored(_bf16(synth.normal(wl, "q_hca", (B, 1, H, D), salt)),
                                                            BF16),
                   q_pos=_i32(t[:, None]), blk_first=_i32((t + 1) // mh - 1), blk_count=_i32(h_cnt), max_blocks=1)
    csa.host = {"t": t[:, None], "raw_base": rbase, "n0": n0, "tail": tail}
    hca.host = {"t": t[:, None], "raw_base": rbase, "nh0": nh0}
    csa.alloc_outputs()
    hca.alloc_outputs()
    return csa, hca


def build(name: str, salt: int = 0, kv_fmt: str | None = None):
    wl = synth.WORKLOADS[name]
    if wl.kind == "csa_decode":
        return build_csa_decode(wl, salt, kv_fmt)
    if wl.kind == "csa2_decode":
        return build_csa2_decode(wl, salt, kv_fmt)
    if wl.kind == "csa_prefill":
        return build_csa_prefill(wl, salt)
    if wl.kind == "hca_decode":
        return build_hca_decode(wl, salt)
    if wl.kind == "hca_prefill":
        return build_hca_prefill(wl, salt)
    if wl.kind == "hybrid_decode":
        return build_hybrid_decode(wl, kv_fmt or wl.kv_dtype, salt)
    raise ValueError(name)
