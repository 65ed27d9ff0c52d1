"""Stage-by-stage parity of the HIP path against the CPU oracle.

Each stage gets its inputs from the seeded generators (never from another HIP
stage), runs through the C ABI, and is compared with the oracle fed the same
stored values: bit-exact for codes and indices, within the stated tolerance
for floating point (max over output rows of ||err||_inf / ||ref||_inf).
Sizes span several tiles plus a ragged tail.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import formats as OF
from tests.gpu_helpers import down, row_rel_err, sorted_unique_choice, up, up_bf16, workspace

pytestmark = pytest.mark.gpu

TEST_WID = 100  # seed namespace of these stage tests


def _rng(name, salt=0):
    return synth.rng(TEST_WID, name, salt)


# ----------------------------------------------------------------------------- quantisers


def _awkward_f32(rows, cols, seed_name):
    r = _rng(seed_name)
    x = r.standard_normal((rows, cols)).astype(np.float32) * np.exp2(r.integers(-20, 20, (rows, 1))).astype(np.float32)
    x[0] = 0.0                                   # an all-zero row / blocks
    x[1, :32] = np.float32(1e-40)                # subnormal block
    x[2, :8] = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], np.float32)  # e2m1 midpoints (amax 6 -> e=0)
    x[3, ::7] = -0.0
    return x


def test_quantize_mxfp4_bit_exact(gpu_lib):
    csa = gpu_lib
    x = _awkward_f32(257, 128, "mx")
    codes = torch.empty((257, 64), dtype=torch.uint8, device="cuda")
    scales = torch.empty((257, 4), dtype=torch.uint8, device="cuda")
    csa.csa_quantize_mxfp4(up(x), 257, 128, codes, scales)
    want_c, want_s = OF.quantize_mxfp4(x)
    np.testing.assert_array_equal(down(scales), want_s)
    np.testing.assert_array_equal(down(codes), want_c)


def test_quantize_fp8_bit_exact(gpu_lib):
    csa = gpu_lib
    x = _awkward_f32(300, 512, "fp8")
    codes = torch.empty((300, 512), dtype=torch.uint8, device="cuda")
    rs = torch.empty((300,), dtype=torch.float32, device="cuda")
    csa.csa_quantize_fp8(up(x), 300, 512, codes, rs)
    want_c, want_s = OF.quantize_fp8_rows(x)
    np.testing.assert_array_equal(down(rs), want_s)
    np.testing.assert_array_equal(down(codes), want_c)


# ----------------------------------------------------------------------------- compression


@pytest.mark.parametrize("m,dim,in_dt,out_dt", [
    (4, 128, "f32", "f32"), (4, 512, "bf16", "bf16"), (128, 512, "bf16", "bf16"),
    (4, 64, "f32", "mxfp4"), (4, 512, "bf16", "fp8"), (128, 512, "fp8", "fp8"), (1, 96, "f32", "f32"),
    (16, 256, "bf16", "bf16"), (17, 64, "f32", "f32"),  # both sides of the per-thread weight path
])
def test_compress(gpu_lib, m, dim, in_dt, out_dt):
    csa = gpu_lib
    B, R = 3, 8 * m + 5
    r = _rng(f"cmp{m}{dim}{in_dt}{out_dt}")
    x = r.standard_normal((B, R, dim)).astype(np.float32)
    z = r.standard_normal(m).astype(np.float32)
    raw_base = np.array([0, 3 * m, 5 * m], dtype=np.int32)            # raw row 0 holds this position
    first = np.array([0, 3, 6], dtype=np.int32)
    count = np.array([8, 4, 0], dtype=np.int32)                       # ragged, one empty
    ncap = 12
    if in_dt == "f32":
        raw_t, raw_v = up(x), x.astype(np.float64)
        raw = csa.desc(raw_t, csa.F32)
    elif in_dt == "bf16":
        raw_t, raw_v = up_bf16(x)
        raw = csa.desc(raw_t, csa.BF16)
    else:
        c, s = OF.quantize_fp8_rows(x.reshape(-1, dim))
        raw_t, raw_s = up(c.reshape(B, R, dim)), up(s.reshape(B, R))
        raw_v = OF.dequantize_fp8_rows(c, s).reshape(B, R, dim)
        raw = csa.desc(raw_t, csa.FP8_E4M3, raw_s)
    if out_dt == "f32":
        out_t = torch.full((B, ncap, dim), float("nan"), device="cuda")
        out = csa.desc(out_t, csa.F32)
    elif out_dt == "bf16":
        out_t = torch.full((B, ncap, dim), float("nan"), device="cuda", dtype=torch.bfloat16)
        out = csa.desc(out_t, csa.BF16)
    elif out_dt == "fp8":
        out_t = torch.zeros((B, ncap, dim), dtype=torch.uint8, device="cuda")
        out_s = torch.zeros((B, ncap), device="cuda")
        out = csa.desc(out_t, csa.FP8_E4M3, out_s)
    else:
        out_t = torch.zeros((B, ncap, dim // 2), dtype=torch.uint8, device="cuda")
        out_s = torch.zeros((B, ncap, dim // 32), dtype=torch.uint8, device="cuda")
        out = csa.desc(out_t, csa.MXFP4, out_s)
    csa.csa_compress(raw, up(raw_base), up(z), m, dim, up(first), up(count), 8, B, out)
    want = oracle.compress(raw_v, raw_base, z.astype(np.float64), m, first, count)
    for b in range(B):
        j0, rows = want[b]
        if rows.shape[0] == 0:
            continue
        sl = slice(j0, j0 + rows.shape[0])
        if out_dt == "f32":
            got = down(out_t)[b, sl]
            assert row_rel_err(got, rows) < 1e-5
        elif out_dt == "bf16":
            got = down(out_t)[b, sl]
            # one bf16 rounding of an fp32-accumulated value: within one bf16 ulp, plus the fp32
            # merge's own error (weights and fma chain), at most (2m + 4) * 2^-24 * max_r |x_r|
            r0 = j0 * m - raw_base[b]
            xmax = np.abs(raw_v[b, r0:r0 + rows.shape[0] * m].reshape(rows.shape[0], m, dim)).max(axis=1)
            assert np.all(np.abs(got - rows) <= np.abs(rows) * 2.0 ** -7 + (2 * m + 4) * 2.0 ** -24 * xmax)
        elif out_dt == "fp8":
            codes, sc = down(out_t)[b, sl], down(out_s)[b, sl]
            got = OF.dequantize_fp8_rows(codes, sc)
            # the row scale follows the row maximum; each element within one e4m3 step
            amax = np.abs(rows).max(axis=1)
            np.testing.assert_allclose(sc, amax / 448.0, rtol=1e-5)
            assert np.all(np.abs(got - rows) <= np.maximum(np.abs(rows) * 2.0 ** -3, sc[:, None] * 2.0 ** -9) + 1e-30)
        else:
            codes, sc = down(out_t)[b, sl], down(out_s)[b, sl]
            got = OF.dequantize_mxfp4(codes, sc)
            # re-quantising the oracle's value must land within one code of the GPU's
            wc, ws = OF.quantize_mxfp4(rows.astype(np.float32))
            assert np.all(np.abs(sc.astype(int) - ws.astype(int)) <= 1)
            step = np.repeat(np.exp2(sc.astype(np.float64) - 127), 32, axis=1)
            assert np.all(np.abs(got - rows) <= 2 * step + 1e-30)
    # rows outside the requested blocks are untouched
    if out_dt == "f32":
        assert np.all(np.isnan(down(out_t)[2]))


def test_compress_jobs_match_single_calls(gpu_lib):
    """One csa_compress_jobs launch == the same jobs as separate csa_compress calls, bit for bit
    (every variant of the combined kernel: three input formats, 1/2/4 columns per thread, a
    wide-row job that takes a launch of its own, and an empty job)."""
    csa = gpu_lib
    B = 3
    r = _rng("cjobs")
    specs = [(4, 512, "bf16", csa.BF16), (4, 64, "f32", csa.MXFP4), (16, 1024, "fp8", csa.FP8_E4M3),
             (2, 200, "f32", csa.F32), (4, 2048, "bf16", csa.BF16), (3, 96, "fp8", csa.BF16)]
    jobs_a, jobs_b, outs = [], [], []
    for (m, dim, in_dt, out_dt) in specs:
        R = 6 * m + 3
        x = r.standard_normal((B, R, dim)).astype(np.float32)
        if in_dt == "f32":
            raw = csa.desc(up(x), csa.F32)
        elif in_dt == "bf16":
            raw = csa.desc(up_bf16(x)[0], csa.BF16)
        else:
            c, s_ = OF.quantize_fp8_rows(x.reshape(-1, dim))
            raw = csa.desc(up(c.reshape(B, R, dim)), csa.FP8_E4M3, up(s_.reshape(B, R)))
        z = up(r.standard_normal(m).astype(np.float32))
        base = up(np.array([0, m, 2 * m], np.int32))
        first = up(np.array([0, 2, 1], np.int32))
        count = up(np.array([5, 3, 0], np.int32))
        pair = []
        for _ in range(2):
            if out_dt == csa.MXFP4:
                o = (torch.zeros((B, 8, dim // 2), dtype=torch.uint8, device="cuda"),
                     torch.zeros((B, 8, dim // 32), dtype=torch.uint8, device="cuda"))
            elif out_dt == csa.FP8_E4M3:
                o = (torch.zeros((B, 8, dim), dtype=torch.uint8, device="cuda"), torch.zeros((B, 8), device="cuda"))
            elif out_dt == csa.BF16:
                o = (torch.zeros((B, 8, dim), dtype=torch.bfloat16, device="cuda"), None)
            else:
                o = (torch.zeros((B, 8, dim), device="cuda"), None)
            pair.append(o)
        outs.append(pair)
        args = (raw, base, z, m, dim, first, count, 5, B)
        jobs_a.append(args + (csa.desc(pair[0][0], out_dt, pair[0][1]),))
        jobs_b.append(args + (csa.desc(pair[1][0], out_dt, pair[1][1]),))
    for i in range(0, len(specs), 3):  # at most four jobs per call
        csa.csa_compress_jobs(jobs_a[i:i + 3])
    for j in jobs_b:
        csa.csa_compress(*j)
    torch.cuda.synchronize()
    for pair in outs:
        for ta, tb in zip(pair[0], pair[1]):
            if ta is not None:
                assert torch.equal(ta.view(torch.uint8) if ta.dtype == torch.bfloat16 else ta,
                                   tb.view(torch.uint8) if tb.dtype == torch.bfloat16 else tb)


# ----------------------------------------------------------------------------- indexer


def _index_case(name, B, Tq, HI, dI, N, m, kfmt):
    r = _rng(name)
    q = r.standard_normal((B, Tq, HI, dI)).astype(np.float32)
    w = r.standard_normal((B, Tq, HI)).astype(np.float32)
    kraw = r.standard_normal((B, N, dI)).astype(np.float32)
    # ragged visibility: positions spread over [0, N*m) plus the full cache
    pos = r.integers(0, N * m, (B, Tq)).astype(np.int32)
    pos[0, 0] = N * m - 1
    return q, w, kraw, pos


@pytest.mark.parametrize("B,Tq,HI,dI,N,kfmt", [
    (1, 1, 4, 32, 1024, "f32"), (2, 3, 4, 32, 777, "f32"),
    (2, 1, 8, 64, 5000, "bf16"), (1, 37, 8, 64, 3000, "bf16"),
    (2, 150, 8, 64, 5000, "bf16"),  # many queries: the 72-query tile kernel, ragged query and key tails
    (1, 40, 8, 64, 777, "bf16"),  # tile kernel, rows not 16-byte aligned (scalar score stores)
    (3, 1, 8, 64, 9000, "mxfp4"), (2, 5, 8, 64, 4100, "mxfp4"), (1, 1, 32, 64, 700, "mxfp4"),
])
def test_index_scores(gpu_lib, B, Tq, HI, dI, N, kfmt):
    csa = gpu_lib
    m = 4
    q, w, kraw, pos = _index_case(f"idx{B}{Tq}{HI}{N}{kfmt}", B, Tq, HI, dI, N, m, kfmt)
    if kfmt == "f32":
        qt, qv = up(q), q.astype(np.float64)
        kt, kv = up(kraw), kraw.astype(np.float64)
        qd, kd = csa.desc(qt, csa.F32), csa.desc(kt, csa.F32)
    elif kfmt == "bf16":
        qt, qv = up_bf16(q)
        kt, kv = up_bf16(kraw)
        qd, kd = csa.desc(qt, csa.BF16), csa.desc(kt, csa.BF16)
    else:
        qt = up(q)
        qc, qs = OF.quantize_mxfp4(q)
        qv = OF.dequantize_mxfp4(qc, qs)
        kc, ks = OF.quantize_mxfp4(kraw)
        kv = OF.dequantize_mxfp4(kc, ks)
        kt, kst = up(kc), up(ks)
        qd, kd = csa.desc(qt, csa.F32), csa.desc(kt, csa.MXFP4, kst)
    scores = torch.full((B, Tq, N), float("nan"), device="cuda")
    csa.csa_index_scores(qd, up(w), kd, up(pos), B, Tq, HI, dI, m, N, scores)
    got = down(scores)
    want = oracle.index_scores(qv, w.astype(np.float64), kv, pos, m, n_cap=N)
    inf = np.isinf(want)
    np.testing.assert_array_equal(np.isinf(got), inf)
    assert not np.any(np.isnan(got))
    fin_w = np.where(inf, 0.0, want)
    fin_g = np.where(inf, 0.0, got)
    assert row_rel_err(fin_g, fin_w) < 2e-6


# ----------------------------------------------------------------------------- top-k


@pytest.mark.parametrize("B,Tq,N,k,mode", [
    (1, 1, 1024, 32, "normal"), (2, 4, 16896, 512, "normal"), (1, 3, 5000, 512, "ties"),
    (2, 2, 3000, 100, "short"), (2, 1, 40000, 2048, "normal"), (1, 2, 70000, 1024, "ties"),
    (1, 1, 30000, 700, "equal"), (3, 1, 262144, 2048, "normal"),
    (4, 2, 65536, 2048, "partial"), (3, 1, 262144, 2048, "partial"),
    (1, 2, 70000, 1024, "extreme"), (2, 1, 262144, 2048, "extreme"), (1, 1, 16000, 512, "extreme"),
    (1, 2, 70000, 1024, "tiny"), (2, 1, 262144, 2048, "narrow"),
    (2, 1, 262144, 2048, "hot2"), (1, 2, 70000, 1024, "hot2"), (1, 1, 262144, 2048, "hot12"),
    # rows of <= 20,480 keys with k <= 4,096: the register-resident kernel
    (1, 2, 12000, 700, "equal"), (1, 2, 20000, 1024, "tiny"), (2, 1, 9000, 300, "narrow"),
    (2, 2, 16896, 512, "partial"), (1, 1, 20480, 2048, "extreme"),
    (1, 2, 9000, 5000, "normal"),  # k > 4,096: the LDS kernel
    # more rows than resident register-path workgroups (two per CU): some walk two rows;
    # rows of 16-byte multiples and (777) of odd length
    (2, 300, 9000, 300, "normal"), (1, 300, 777, 100, "ties"),
])
def test_topk_exact(gpu_lib, B, Tq, N, k, mode):
    csa = gpu_lib
    m = 4
    r = _rng(f"topk{B}{Tq}{N}{k}{mode}")
    if mode == "ties":
        s = r.integers(-20, 20, (B, Tq, N)).astype(np.float32)
        s[s == 0] = np.where(r.random(int((s == 0).sum())) < 0.5, -0.0, 0.0).astype(np.float32)
    elif mode in ("hot2", "hot12"):
        # 1024-key slices holding far more than their 32 listed keys of the row's top-k:
        # two (each re-read in full from the scores) or twelve (the whole row reselected)
        s = r.standard_normal((B, Tq, N)).astype(np.float32)
        hot = (5, N // 4096) if mode == "hot2" else tuple(3 + 5 * i for i in range(12))
        for sl in hot:
            s[..., sl * 1024:(sl + 1) * 1024] += 3.0
    elif mode == "equal":
        s = np.zeros((B, Tq, N), np.float32)
    elif mode == "extreme":  # infinities and near-overflow magnitudes among normal scores
        s = r.standard_normal((B, Tq, N)).astype(np.float32)
        hit = r.random((B, Tq, N))
        s[hit < 0.002] = np.inf
        s[(hit >= 0.002) & (hit < 0.004)] = -np.inf
        s[(hit >= 0.004) & (hit < 0.006)] = 3e38
        s[(hit >= 0.006) & (hit < 0.008)] = -3e38
    elif mode == "tiny":  # subnormal scores: a score span too small to divide by
        s = (r.integers(-6, 6, (B, Tq, N)) * 1e-45).astype(np.float32)
    elif mode == "narrow":  # distinct scores packed into a few ulps around 1
        s = (1.0 + r.integers(0, 4000, (B, Tq, N)) * np.float32(2.0 ** -23)).astype(np.float32)
    else:
        s = r.standard_normal((B, Tq, N)).astype(np.float32)
    pos = np.full((B, Tq), N * m - 1, np.int32)
    if mode == "short":
        pos[:, 0] = 4 * 40 - 1  # only 40 visible < k: padding
        pos[-1, -1] = 4 * 100 - 1  # exactly k visible
    elif mode == "partial":
        # rows that see only part of the cache: their few slices hold fewer candidates
        # than k (and one holds just over k), so the selection must fall back to the row
        pos[:, 0] = r.integers(k * m + 4, (N // 8) * m, B)
        pos[0, 0] = (k + 1) * m - 1
    elif Tq > 1:
        pos[0, 1] = (N // 2) * m + 2  # a shorter row
    idx = torch.full((B, Tq, k), -7, dtype=torch.int32, device="cuda")
    ws = workspace(csa.csa_topk_workspace_size(B, Tq, N, k))
    csa.csa_topk(up(s), up(pos), B, Tq, N, m, k, idx, ws, ws.numel())
    got = down(idx)
    want = oracle.topk(s.astype(np.float64), pos, m, k)
    np.testing.assert_array_equal(got, want)


# ----------------------------------------------------------------------------- indexer query


def _index_query_bounds(hv, wdq, wuq, ww, HI, dI):
    """Elementwise error bounds of the library's arithmetic against the fp64 oracle:
    fp32 sums of exact bf16 products (gamma_K = K u / (1 - K u), u = 2^-24, any
    summation order), c rounded to bf16 (unit roundoff 2^-8: 8 significant bits) before the
    second product."""
    u = 2.0 ** -24
    d, r = hv.shape[-1], wdq.shape[0]
    gd, gr = d * u / (1 - d * u), r * u / (1 - r * u)
    c = hv @ wdq.T
    A = np.abs(hv) @ np.abs(wdq).T
    bc = 2.0 ** -8 * (np.abs(c) + gd * A) + gd * A
    bq = bc @ np.abs(wuq).T + gr * ((np.abs(c) + bc) @ np.abs(wuq).T)
    bw = gd * (np.abs(hv) @ np.abs(ww).T)
    return bq.reshape(hv.shape[:-1] + (HI, dI)), bw


@pytest.mark.parametrize("B,Tq,d,r,HI,dI,fmt", [
    (1, 1, 4096, 1024, 4, 32, "f32"),     # the 4k decode's indexer shape (4 heads of 32)
    (1, 2048, 4096, 1024, 8, 64, "bf16"),  # the 2k prefill chunk (8 heads of 64)
    (8, 1, 4096, 1024, 8, 64, "f32"),     # the 1M decode batch
    (3, 5, 96, 64, 2, 16, "f32"),         # ragged: K below one 128-chunk, rows in a partial tile
    (2, 40, 160, 96, 3, 8, "bf16"),       # K tails in both products, 80 rows (one split)
])
def test_index_query(gpu_lib, B, Tq, d, r, HI, dI, fmt):
    """csa_index_query against the oracle within the derived fp32 / bf16 bounds, and
    bitwise batch invariance (one row alone gives the same bits)."""
    csa = gpu_lib
    rg = _rng(f"iq{B}{Tq}{d}{r}{HI}{dI}{fmt}")
    h = rg.standard_normal((B, Tq, d)).astype(np.float32)
    ht, hv = up_bf16(h)
    wdq_t, wdq = up_bf16((rg.standard_normal((r, d)) / np.sqrt(d)).astype(np.float32))
    wuq_t, wuq = up_bf16((rg.standard_normal((HI * dI, r)) / np.sqrt(r)).astype(np.float32))
    ww_t, ww = up_bf16((rg.standard_normal((HI, d)) / np.sqrt(d)).astype(np.float32))
    # weights are passed as [1, rows, cols]: stride_row is their row pitch
    W = [csa.desc(x.unsqueeze(0), csa.BF16) for x in (wdq_t, wuq_t, ww_t)]

    def run(hsel, nb):
        qdt = torch.float32 if fmt == "f32" else torch.bfloat16
        q = torch.full((nb, Tq, HI, dI), float("nan"), dtype=qdt, device="cuda")
        w = torch.full((nb, Tq, HI), float("nan"), device="cuda")
        ws = workspace(csa.csa_index_query_workspace_size(nb, Tq, d, r, HI, dI))
        ws.fill_(0xA5)  # contents on entry do not matter
        csa.csa_index_query(csa.desc(hsel, csa.BF16), W[0], W[1], W[2], nb, Tq, d, r, HI, dI,
                            csa.desc(q, csa.F32 if fmt == "f32" else csa.BF16), w, ws, ws.numel())
        return down(q), down(w)

    q, w = run(ht, B)
    want_q, want_w = oracle.index_query(hv, wdq, wuq, ww, HI, dI)
    bq, bw = _index_query_bounds(hv, wdq, wuq, ww, HI, dI)
    if fmt == "bf16":
        bq = bq + 2.0 ** -8 * (np.abs(want_q) + bq)
    assert np.all(np.isfinite(q)) and np.all(np.isfinite(w))
    assert np.all(np.abs(q - want_q) <= bq * 1.001), np.max(np.abs(q - want_q) / bq)
    assert np.all(np.abs(w - want_w) <= bw * 1.001), np.max(np.abs(w - want_w) / bw)
    # one sequence alone: the same bits (the K sums do not depend on the number of rows)
    q1, w1 = run(ht[B - 1:B].contiguous(), 1)
    np.testing.assert_array_equal(q1[0], q[B - 1])
    np.testing.assert_array_equal(w1[0], w[B - 1])


# ----------------------------------------------------------------------------- MLA projections


@pytest.mark.parametrize("rows,H,dh,D", [
    (8, 64, 128, 512),    # the 1M decode batch: 64 heads of 128 onto the 512-wide latent
    (2048, 2, 128, 512),  # a prefill chunk's rows (one split per tile)
    (70, 4, 96, 160),     # ragged: K tails below and above one 128-chunk, rows in a partial tile
    (1, 3, 32, 64),
])
def test_latent_projections(gpu_lib, rows, H, dh, D):
    """csa_latent_query / csa_latent_output against the oracle within derived bounds (fp32
    sums of exact bf16 products: gamma_K = K u / (1 - K u), u = 2^-24; bf16 outputs add
    half an ulp, at most 2^-8 relative; o_lat = hi + lo to 2^-16 relative, and the
    hi and lo magnitudes add up to at most (1 + 2^-7) |o_lat|), and bitwise
    batch invariance (a few rows alone give the same bits)."""
    csa = gpu_lib
    rg = _rng(f"lat{rows}{H}{dh}{D}")
    qt, qv = up_bf16(rg.standard_normal((rows, H, dh)).astype(np.float32))
    wuk_t, wuk = up_bf16((rg.standard_normal((H, dh, D)) / np.sqrt(dh)).astype(np.float32))
    wuv_t, wuv = up_bf16((rg.standard_normal((H, dh, D)) / np.sqrt(D)).astype(np.float32))
    o_lat = rg.standard_normal((rows, H, D)).astype(np.float32)
    o_t = up(o_lat)
    wuk_tt = wuk_t.transpose(1, 2).contiguous()  # [H, D, dh]: the absorbed form's row layout

    def gamma(k):
        return k * 2.0 ** -24 / (1 - k * 2.0 ** -24)

    def query(qsel, n):
        out = torch.full((n, H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
        ws = workspace(csa.csa_latent_query_workspace_size(n, H, dh, D))
        ws.fill_(0xA5)
        csa.csa_latent_query(qsel, wuk_tt, n, H, dh, D, out, ws, ws.numel())
        return down(out)

    def output(osel, n, dt):
        out = torch.full((n, H, dh), float("nan"), dtype=torch.float32 if dt == csa.F32 else torch.bfloat16,
                         device="cuda")
        ws = workspace(csa.csa_latent_output_workspace_size(n, H, dh, D))
        ws.fill_(0xA5)
        csa.csa_latent_output(osel, wuv_t, n, H, dh, D, out, dt, ws, ws.numel())
        return down(out)

    got = query(qt, rows)
    want = oracle.latent_query(qv, wuk)
    b = gamma(dh) * oracle.latent_query(np.abs(qv), np.abs(wuk))
    b = b + 2.0 ** -8 * (np.abs(want) + b)
    assert np.all(np.isfinite(got))
    assert np.all(np.abs(got - want) <= b * 1.001), np.max(np.abs(got - want) / b)
    want_o = oracle.latent_output(o_lat, wuv)
    bo = (2.0 ** -16 + gamma(2 * D) * (1 + 2.0 ** -7)) * oracle.latent_output(np.abs(o_lat), np.abs(wuv))
    got_o = output(o_t, rows, csa.F32)
    assert np.all(np.isfinite(got_o))
    assert np.all(np.abs(got_o - want_o) <= bo * 1.001), np.max(np.abs(got_o - want_o) / bo)
    got_ob = output(o_t, rows, csa.BF16)
    bob = bo + 2.0 ** -8 * (np.abs(want_o) + bo)
    assert np.all(np.abs(got_ob - want_o) <= bob * 1.001), np.max(np.abs(got_ob - want_o) / bob)
    # a few rows alone: the same bits whatever the number of rows (and the split of K)
    r0, n = rows // 2, min(3, rows - rows // 2)
    np.testing.assert_array_equal(query(qt[r0:r0 + n].contiguous(), n), got[r0:r0 + n])
    np.testing.assert_array_equal(output(o_t[r0:r0 + n].contiguous(), n, csa.F32), got_o[r0:r0 + n])


# ----------------------------------------------------------------------------- fused index + top-k


@pytest.mark.parametrize("B,Tq,HI,N,k,mode", [
    (2, 1, 8, 65536, 2048, "normal"),
    (3, 1, 8, 262144, 2048, "normal"),   # the 1M-context decode shape
    (2, 2, 32, 40000, 1024, "normal"),   # 32 heads, ragged last slice
    (2, 1, 8, 65536, 2048, "cluster"),   # one slice holds most top scores: the exact fallback runs
    (1, 1, 8, 30000, 512, "equal"),      # all scores equal: the lowest indices win
    (2, 1, 8, 65536, 2048, "few"),       # 40 distinct keys: many copies of the slices' 32nd score
    (2, 3, 8, 40000, 2048, "short"),     # some rows see at most k blocks
    (3, 2, 8, 262144, 2048, "partial"),  # rows seeing a fraction of the cache: few candidates
    # long rows whose slice lists cannot decide: two slices hold most top scores (those two
    # are rescored), twelve do (the row is rescored), ties everywhere (the row is rescored)
    (2, 1, 8, 262144, 2048, "cluster2"),
    (2, 1, 32, 150000, 1024, "cluster2"),
    (1, 2, 8, 262144, 2048, "cluster12"),
    (1, 1, 8, 262144, 2048, "equal"),
    (2, 1, 8, 262144, 2048, "few"),
])
def test_index_topk_fused(gpu_lib, B, Tq, HI, N, k, mode):
    """csa_index_topk == csa_index_scores then csa_topk, bit for bit (scores and idx),
    and idx == the oracle's top-k of those scores."""
    csa = gpu_lib
    m, dI = 4, 64
    r = _rng(f"itk{B}{Tq}{HI}{N}{k}{mode}")
    q = r.standard_normal((B, Tq, HI, dI)).astype(np.float32)
    w = r.standard_normal((B, Tq, HI)).astype(np.float32)
    pos = r.integers(N * m // 2, N * m, (B, Tq)).astype(np.int32)
    pos[0, 0] = N * m - 1
    gen = torch.Generator(device="cuda")
    gen.manual_seed(int(r.integers(1 << 31)))
    kraw = torch.randn((B, N, dI), generator=gen, device="cuda")
    if mode == "cluster":
        w = np.abs(w)
        kraw[:, 5 * 1024:6 * 1024] = 3.0 * up(q[:, 0, 0])[:, None, :]
    elif mode in ("cluster2", "cluster12"):
        w = np.abs(w)
        hot = (5, N // 4096) if mode == "cluster2" else tuple(3 + 5 * i for i in range(12))
        qv = up(q[:, 0, 0])[:, None, :]
        for sl in hot:
            noise = torch.randn((B, 1024, dI), generator=gen, device="cuda")
            kraw[:, sl * 1024:(sl + 1) * 1024] = 3.0 * qv + 0.5 * noise
    elif mode == "equal":
        kraw[:] = kraw[:, :1]
    elif mode == "few":
        pick = torch.as_tensor(r.integers(0, 40, N), device="cuda").long()
        kraw[:] = kraw[:, pick]
    elif mode == "short":
        pos[1, :] = r.integers(0, k * m // 2, Tq)
    elif mode == "partial":
        pos[:, 1] = r.integers(k * m + 4, (N // 16) * m, B)
    kc = torch.empty((B, N, dI // 2), dtype=torch.uint8, device="cuda")
    ks = torch.empty((B, N, dI // 32), dtype=torch.uint8, device="cuda")
    csa.csa_quantize_mxfp4(kraw, B * N, dI, kc, ks)
    qd, kd = csa.desc(up(q), csa.F32), csa.desc(kc, csa.MXFP4, ks)
    wt, pt = up(w), up(pos)
    s1 = torch.full((B, Tq, N), float("nan"), device="cuda")
    i1 = torch.full((B, Tq, k), -7, dtype=torch.int32, device="cuda")
    csa.csa_index_scores(qd, wt, kd, pt, B, Tq, HI, dI, m, N, s1)
    ws1 = workspace(csa.csa_topk_workspace_size(B, Tq, N, k))
    csa.csa_topk(s1, pt, B, Tq, N, m, k, i1, ws1, ws1.numel())
    s2 = torch.full((B, Tq, N), float("nan"), device="cuda")
    i2 = torch.full((B, Tq, k), -7, dtype=torch.int32, device="cuda")
    ws2 = workspace(csa.csa_index_topk_workspace_size(B, Tq, N, k))
    csa.csa_index_topk(qd, wt, kd, pt, B, Tq, HI, dI, m, N, k, s2, i2, ws2, ws2.numel())
    assert torch.equal(s1, s2)
    np.testing.assert_array_equal(down(i2), down(i1))
    # the same call in two parts (scores + candidates, then selection)
    s3 = torch.full((B, Tq, N), float("nan"), device="cuda")
    i3 = torch.full((B, Tq, k), -7, dtype=torch.int32, device="cuda")
    ws3 = workspace(csa.csa_index_topk_workspace_size(B, Tq, N, k))
    csa.csa_index_topk_part(qd, wt, kd, pt, B, Tq, HI, dI, m, N, k, s3, None, ws3, ws3.numel(), 1)
    csa.csa_index_topk_part(qd, wt, kd, pt, B, Tq, HI, dI, m, N, k, s3, i3, ws3, ws3.numel(), 2)
    assert torch.equal(s3, s2)
    np.testing.assert_array_equal(down(i3), down(i2))
    np.testing.assert_array_equal(down(i2), oracle.topk(down(s2).astype(np.float64), pos, m, k))
    # no scores kept: the same selection, in one call and in two parts (rows the lists cannot
    # decide are selected from scores the call keeps in its workspace or recomputes there)
    ws4 = workspace(csa.csa_index_topk_workspace_size(B, Tq, N, k, scores_kept=False))
    for parts in ((3,), (1, 2)):
        ws4.fill_(0xA5)  # contents on entry do not matter
        i4 = torch.full((B, Tq, k), -7, dtype=torch.int32, device="cuda")
        for part in parts:
            csa.csa_index_topk_part(qd, wt, kd, pt, B, Tq, HI, dI, m, N, k, None, i4 if part & 2 else None, ws4,
                                    ws4.numel(), part)
        np.testing.assert_array_equal(down(i4), down(i2))


# ----------------------------------------------------------------------------- attention


def _attn_inputs(name, B, Tq, H, D, N, R, kv_fmt):
    r = _rng(name)
    q = r.standard_normal((B, Tq, H, D)).astype(np.float32)
    kvc = r.standard_normal((B, N, D)).astype(np.float32)
    raw = r.standard_normal((B, R, D)).astype(np.float32)
    return r, q, kvc, raw


def _store_kv(csa, x, fmt):
    B, N, D = x.shape
    if fmt == "f32":
        return csa.desc(up(x), csa.F32), x.astype(np.float64), None
    if fmt == "bf16":
        t, v = up_bf16(x)
        return csa.desc(t, csa.BF16), v, t
    if fmt == "fp4":  # MXFP4 codes and block scales as the oracle's quantiser writes them
        c, s = OF.quantize_mxfp4(x)
        t, st = up(c), up(s)
        return csa.desc(t, csa.MXFP4, st), OF.dequantize_mxfp4(c, s), (t, st)
    c, s = OF.quantize_fp8_rows(x.reshape(-1, D))
    t, st = up(c.reshape(B, N, D)), up(s.reshape(B, N))
    return csa.desc(t, csa.FP8_E4M3, st), OF.dequantize_fp8_rows(c, s).reshape(B, N, D), (t, st)


@pytest.mark.parametrize("B,Tq,H,D,k,W,fmt,tol", [
    (1, 1, 16, 128, 32, 64, "f32", 1e-5),
    (2, 1, 64, 512, 300, 128, "bf16", 2e-3),   # several splits + ragged tail
    (3, 1, 64, 512, 40, 7, "bf16", 2e-3),
    (1, 6, 32, 512, 100, 50, "bf16", 2e-3),    # several queries, one split each
    (2, 1, 48, 512, 520, 128, "fp8", 5e-3),
    (2, 1, 64, 512, 300, 128, "fp4", 2e-3),    # MXFP4 cache: several splits + ragged tail
    (2, 5, 32, 512, 100, 50, "fp4", 2e-3),     # MXFP4, several queries (chunked many-query kernel)
    (2, 1, 16, 512, 17, 1, "bf16", 2e-3),
    (1, 5, 48, 512, 64, 32, "bf16", 2e-3),     # 48 heads, several queries (three head groups)
    (2, 3, 64, 512, 200, 64, "fp8", 5e-3),
    (2, 9, 64, 512, 300, 128, "bf16", 2e-3),   # several queries, 64 heads: two head groups, four 107-entry chunks
    (1, 4, 16, 512, 90, 20, "bf16", 2e-3),     # several queries, one head group
])
def test_csa_sparse_attn(gpu_lib, B, Tq, H, D, k, W, fmt, tol):
    csa = gpu_lib
    m, N = 4, 4096
    R = 1024
    r, q, kvc, raw = _attn_inputs(f"csa{B}{Tq}{H}{k}{W}{fmt}", B, Tq, H, D, N, R, fmt)
    # consecutive positions per sequence (a prefill chunk when Tq > 1); sequence 0 starts
    # early, so it has few visible blocks (k slots padded with -1) and a short window
    start = r.integers(N * m // 2, N * m - Tq, B)
    start[0] = 3 + (W if W < 8 else 0)
    pos = (start[:, None] + np.arange(Tq)[None]).astype(np.int32)
    raw_base = np.maximum(0, pos[:, 0] - W - 5).astype(np.int32)
    assert all(int(pos[b].max()) - raw_base[b] < R for b in range(B))
    idx = np.stack([[sorted_unique_choice(r, oracle.visible_blocks(int(pos[b, t]), m), k) for t in range(Tq)]
                    for b in range(B)])
    qd = csa.desc(up(q), csa.F32) if fmt == "f32" else csa.desc(up_bf16(q)[0], csa.BF16)
    qv = q.astype(np.float64) if fmt == "f32" else up_bf16(q)[1]
    kvd, kvv, _ = _store_kv(csa, kvc, fmt)
    rawd, rawv, _ = _store_kv(csa, raw, "bf16" if fmt == "fp4" else fmt)  # MXFP4 caches take bf16 raw rows
    out = torch.full((B, Tq, H, D), float("nan"), device="cuda")
    lse = torch.full((B, Tq, H), float("nan"), device="cuda")
    ws = workspace(csa.csa_attn_workspace_size(B, Tq, H, D, k + W))
    scale = 1 / np.sqrt(128)
    csa.csa_sparse_attn(qd, kvd, up(idx.astype(np.int32)), k, rawd, up(raw_base), W, up(pos), B, Tq, H, D, scale,
                        out, lse, ws, ws.numel())
    want, want_lse = oracle.csa_sparse_attn(qv, kvv, idx, rawv, raw_base, W, pos, scale)
    assert row_rel_err(down(out), want) < tol
    assert np.max(np.abs(down(lse) - want_lse)) < tol


@pytest.mark.parametrize("B,Tq,H,mhc,ncap,W,fmt,tol", [
    (4, 1, 64, 128, 40, 128, "bf16", 2e-3),
    (3, 1, 64, 16, 700, 33, "bf16", 2e-3),
    (2, 1, 32, 128, 20, 128, "fp8", 5e-3),
    # prefill chunks: consecutive queries, blocks completing inside the chunk
    (2, 37, 64, 16, 90, 128, "bf16", 2e-3),
    (1, 200, 64, 8, 300, 33, "bf16", 2e-3),
    (2, 70, 32, 16, 60, 20, "fp8", 5e-3),
    (3, 1, 64, 16, 700, 33, "fp4", 2e-3),
    (1, 40, 64, 16, 90, 128, "fp4", 2e-3),
])
def test_hca_attn(gpu_lib, B, Tq, H, mhc, ncap, W, fmt, tol):
    csa = gpu_lib
    D = 512
    R = 512
    r, q, kvh, raw = _attn_inputs(f"hca{B}{Tq}{H}{mhc}{ncap}{fmt}", B, Tq, H, D, ncap, R, fmt)
    if Tq == 1:
        pos = r.integers(mhc * ncap // 2, mhc * ncap, (B, Tq)).astype(np.int32)
        pos[0, 0] = mhc - 2  # no complete block yet: window only
    else:  # a chunk of consecutive positions per sequence; sequence 0's chunk starts at 0
        p0 = r.integers(mhc * ncap // 2, mhc * ncap - Tq, B)
        p0[0] = 0
        pos = (p0[:, None] + np.arange(Tq)[None]).astype(np.int32)
    assert R >= W + Tq + 3
    raw_base = np.maximum(0, pos[:, 0] - W - 3).astype(np.int32)
    qd, qv = csa.desc(up_bf16(q)[0], csa.BF16), up_bf16(q)[1]
    kvd, kvv, _ = _store_kv(csa, kvh, fmt)
    rawd, rawv, _ = _store_kv(csa, raw, "bf16" if fmt == "fp4" else fmt)  # MXFP4 caches take bf16 raw rows
    out = torch.full((B, Tq, H, D), float("nan"), device="cuda")
    lse = torch.full((B, Tq, H), float("nan"), device="cuda")
    ws = workspace(csa.csa_attn_workspace_size(B, Tq, H, D, ncap + W))
    scale = 1 / np.sqrt(128)
    csa.hca_attn(qd, kvd, mhc, ncap, rawd, up(raw_base), W, up(pos), B, Tq, H, D, scale, out, lse, ws, ws.numel())
    want, want_lse = oracle.hca_attn(qv, kvv, mhc, rawv, raw_base, W, pos, scale)
    assert row_rel_err(down(out), want) < tol
    assert np.max(np.abs(down(lse) - want_lse)) < tol


def test_attention_deterministic_and_batch_invariant(gpu_lib):
    """Same inputs give bitwise the same outputs, and a sequence's result does not
    depend on the other sequences in the batch."""
    csa = gpu_lib
    B, H, D, N, k, W, m = 4, 64, 512, 2048, 600, 128, 4
    r, q, kvc, raw = _attn_inputs("det", B, 1, H, D, N, 512, "bf16")
    pos = np.full((B, 1), N * m - 1, np.int32)
    raw_base = (pos[:, 0] - 300).astype(np.int32)
    idx = np.stack([[sorted_unique_choice(r, N, k)] for _ in range(B)]).astype(np.int32)
    qt = up_bf16(q)[0]
    kt = up_bf16(kvc)[0]
    rt = up_bf16(raw)[0]

    def run(sel):
        nb = len(sel)
        out = torch.empty((nb, 1, H, D), device="cuda")
        lse = torch.empty((nb, 1, H), device="cuda")
        ws = workspace(csa.csa_attn_workspace_size(nb, 1, H, D, k + W))
        qs, ks, rs = qt[sel].contiguous(), kt[sel].contiguous(), rt[sel].contiguous()
        csa.csa_sparse_attn(csa.desc(qs, csa.BF16), csa.desc(ks, csa.BF16), up(idx[sel]), k, csa.desc(rs, csa.BF16),
                            up(raw_base[sel]), W, up(pos[sel]), nb, 1, H, D, 0.088, out, lse, ws, ws.numel())
        return down(out), down(lse)

    a = run([0, 1, 2, 3])
    b = run([0, 1, 2, 3])
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    for i in range(B):
        s = run([i])
        assert np.array_equal(s[0][0], a[0][i]) and np.array_equal(s[1][0], a[1][i])


@pytest.mark.parametrize("kv_fmt,ik_fmt,tq,N,k,first", [
    ("bf16", "f32", 1, 24000, 512, (1023, 5000, 7000)),       # short rows: selected from their scores
    ("fp8", "bf16", 1, 24000, 512, (1023, 5000, 7000)),
    ("bf16", "f32", 2, 24000, 512, (1023, 5000, 7000)),       # compressions in a launch of their own
    ("bf16", "f32", 1, 131072, 1024, (1023, 90000, 131071)),  # long rows: slice lists and the merge
])
def test_compress_index_topk_matches_separate_calls(gpu_lib, kv_fmt, ik_fmt, tq, N, k, first):
    """csa_compress_index_topk == csa_compress_jobs then csa_index_topk_part, bit for bit: the
    stored KV entries and indexer keys, the scores and the selection -- with new blocks on a
    slice boundary, a sequence completing none, either part alone, and (tq=2) the shapes that
    run the compressions in a launch of their own."""
    csa = gpu_lib
    B, HI, dI, D, m, R = 3, 8, 64, 512, 4, 16
    r = _rng(f"cit{kv_fmt}{ik_fmt}{tq}{N}")
    first = np.array(first, np.int32)  # blocks 1023 and 1024 sit in two slices
    count = np.array([2, 1, 0], np.int32)
    count[-1] = 1 if first[-1] == N - 1 else 0  # the last block of the cache completed this step
    raw_base = (m * first - m).astype(np.int32)
    end = m * (first + count) - 1  # the token completing the last new block
    pos = np.stack([end - (tq - 1 - t) for t in range(tq)], axis=1).astype(np.int32)
    kraw = torch.as_tensor(r.standard_normal((B, N, dI)).astype(np.float32), device="cuda")
    kc0 = torch.empty((B, N, dI // 2), dtype=torch.uint8, device="cuda")
    ks0 = torch.empty((B, N, dI // 32), dtype=torch.uint8, device="cuda")
    csa.csa_quantize_mxfp4(kraw, B * N, dI, kc0, ks0)
    xi = r.standard_normal((B, R, dI)).astype(np.float32)
    raw_ik = csa.desc(up(xi), csa.F32) if ik_fmt == "f32" else csa.desc(up_bf16(xi)[0], csa.BF16)
    xk = r.standard_normal((B, R, D)).astype(np.float32)
    if kv_fmt == "bf16":
        raw_kv = csa.desc(up_bf16(xk)[0], csa.BF16)
        kv0 = (torch.as_tensor(r.standard_normal((B, N, D)).astype(np.float32), device="cuda").to(torch.bfloat16),
               None)
    else:
        c_, s_ = OF.quantize_fp8_rows(xk.reshape(-1, D))
        raw_kv = csa.desc(up(c_.reshape(B, R, D)), csa.FP8_E4M3, up(s_.reshape(B, R)))
        kv0 = (torch.randint(0, 120, (B, N, D), dtype=torch.uint8, device="cuda"), torch.rand((B, N), device="cuda"))
    z_kv = up(r.standard_normal(m).astype(np.float32))
    z_ik = up(r.standard_normal(m).astype(np.float32))
    q = up(r.standard_normal((B, tq, HI, dI)).astype(np.float32))
    w = up(r.standard_normal((B, tq, HI)).astype(np.float32))
    dpos, dbase, dfirst, dcount = up(pos), up(raw_base), up(first), up(count)
    kv_dt = csa.BF16 if kv_fmt == "bf16" else csa.FP8_E4M3

    def state():
        kc, ks = kc0.clone(), ks0.clone()
        kv = (kv0[0].clone(), None if kv0[1] is None else kv0[1].clone())
        return kc, ks, kv

    def jobs(kc, ks, kv):
        kvj = (raw_kv, dbase, z_kv, m, D, dfirst, dcount, 2, B, csa.desc(kv[0], kv_dt, kv[1]))
        kyj = (raw_ik, dbase, z_ik, m, dI, dfirst, dcount, 2, B, csa.desc(kc, csa.MXFP4, ks))
        return kvj, kyj

    def outputs():
        return (torch.full((B, tq, N), float("nan"), device="cuda"),
                torch.full((B, tq, k), -7, dtype=torch.int32, device="cuda"),
                workspace(csa.csa_index_topk_workspace_size(B, tq, N, k, scores_kept=False)))

    def bits(kc, ks, kv, sc, ix):
        kvb = kv[0].view(torch.uint8) if kv[0].dtype == torch.bfloat16 else kv[0]
        return [kc, ks, kvb] + ([kv[1]] if kv[1] is not None else []) + [sc.view(torch.int32), ix]

    # reference: the compressions, then the indexer with selection
    kc, ks, kv = state()
    sc, ix, ws = outputs()
    kvj, kyj = jobs(kc, ks, kv)
    csa.csa_compress_jobs([kvj, kyj])
    csa.csa_index_topk_part(csa.desc(q, csa.F32), w, csa.desc(kc, csa.MXFP4, ks), dpos, B, tq, HI, dI, m, N, k, sc,
                            ix, ws, ws.numel(), 3)
    want = bits(kc, ks, kv, sc, ix)
    for parts in ((3,), (1, 2)):
        kc, ks, kv = state()
        sc, ix, ws = outputs()
        kvj, kyj = jobs(kc, ks, kv)
        for part in parts:
            csa.csa_compress_index_topk(kvj, kyj, csa.desc(q, csa.F32), w, csa.desc(kc, csa.MXFP4, ks), dpos, B, tq,
                                        HI, dI, m, N, k, sc, ix, ws, ws.numel(), part)
        got = bits(kc, ks, kv, sc, ix)
        for a_, b_ in zip(want, got):
            assert torch.equal(a_, b_)
    # without scores: the same stored entries and selection
    for parts in ((3,), (1, 2)):
        kc, ks, kv = state()
        _, ix, ws = outputs()
        kvj, kyj = jobs(kc, ks, kv)
        for part in parts:
            csa.csa_compress_index_topk(kvj, kyj, csa.desc(q, csa.F32), w, csa.desc(kc, csa.MXFP4, ks), dpos, B, tq,
                                        HI, dI, m, N, k, None, ix if part & 2 else None, ws, ws.numel(), part)
        got = bits(kc, ks, kv, want[-2].view(torch.float32), ix)
        for a_, b_ in zip(want, got):
            assert torch.equal(a_, b_)
    # the new keys did change (the comparison is not of untouched tensors)
    assert not torch.equal(kc[0, 1023], kc0[0, 1023]) or not torch.equal(ks[0, 1023], ks0[0, 1023])


def test_attention_workspace_reuse(gpu_lib):
    """One workspace serves a sequence of CSA and HCA calls with different split
    layouts, each giving the results of a call with a fresh workspace."""
    csa = gpu_lib
    B, H, D, N, k, W, m, mhc, ncap = 3, 64, 512, 2048, 600, 128, 4, 16, 700
    r, q, kvc, raw = _attn_inputs("wsreuse", B, 1, H, D, N, 512, "bf16")
    pos = np.full((B, 1), N * m - 1, np.int32)
    pos[1, 0] = N * m // 3
    raw_base = (pos[:, 0] - 300).astype(np.int32)
    idx = np.stack([[sorted_unique_choice(r, oracle.visible_blocks(int(pos[b, 0]), m), k)] for b in range(B)])
    idx = idx.astype(np.int32)
    kvh = r.standard_normal((B, ncap, D)).astype(np.float32)
    qt, kt, rt, ht = up_bf16(q)[0], up_bf16(kvc)[0], up_bf16(raw)[0], up_bf16(kvh)[0]
    n_csa = csa.csa_attn_workspace_size(B, 1, H, D, k + W)
    n_hca = csa.csa_attn_workspace_size(B, 1, H, D, ncap + W)
    assert n_csa > 0 and n_hca > 0  # both calls split their lists

    def call(kind, qq, ws):
        out = torch.empty((B, 1, H, D), device="cuda")
        lse = torch.empty((B, 1, H), device="cuda")
        if kind == "csa":
            csa.csa_sparse_attn(csa.desc(qq, csa.BF16), csa.desc(kt, csa.BF16), up(idx), k, csa.desc(rt, csa.BF16),
                                up(raw_base), W, up(pos), B, 1, H, D, 0.088, out, lse, ws, ws.numel())
        else:
            hpos = np.minimum(pos, mhc * ncap - 1).astype(np.int32)
            csa.hca_attn(csa.desc(qq, csa.BF16), csa.desc(ht, csa.BF16), mhc, ncap, csa.desc(rt, csa.BF16),
                         up(raw_base), W, up(hpos), B, 1, H, D, 0.088, out, lse, ws, ws.numel())
        return down(out), down(lse)

    shared = workspace(max(n_csa, n_hca))
    q2 = (qt.float() * 0.5).to(torch.bfloat16)
    for kind, qq in (("csa", qt), ("hca", qt), ("csa", q2), ("hca", q2), ("csa", qt)):
        got = call(kind, qq, shared)
        n = n_csa if kind == "csa" else n_hca
        fresh = call(kind, qq, workspace(n))
        assert np.array_equal(got[0], fresh[0]) and np.array_equal(got[1], fresh[1])


def test_attention_fp8_zero_row_is_an_entry(gpu_lib):
    """An all-zero fp8 row has row scale 0; it is still an entry of the softmax (logit 0,
    contributes a zero vector), not an empty slot."""
    csa = gpu_lib
    B, Tq, H, D, k, W, m, N = 1, 1, 16, 512, 24, 4, 4, 256
    r, q, kvc, raw = _attn_inputs("fp8zero", B, Tq, H, D, N, 64, "fp8")
    q *= 0.05  # small logits, so the zero rows carry visible weight
    idx = np.sort(r.choice(N, k, replace=False)).astype(np.int32)[None, None]
    kvc[0, idx[0, 0, :5]] = 0.0  # five selected rows are exactly zero
    pos = np.array([[N * m - 1]], np.int32)
    raw_base = np.array([N * m - 40], np.int32)
    qd, qv = csa.desc(up_bf16(q)[0], csa.BF16), up_bf16(q)[1]
    kvd, kvv, (_, kv_scale) = _store_kv(csa, kvc, "fp8")
    kv_scale[0, torch.as_tensor(idx[0, 0, :5]).long().cuda()] = 0.0  # a zero scale: the row is still zero
    rawd, rawv, _ = _store_kv(csa, raw, "fp8")
    out = torch.full((B, Tq, H, D), float("nan"), device="cuda")
    lse = torch.full((B, Tq, H), float("nan"), device="cuda")
    ws = workspace(csa.csa_attn_workspace_size(B, Tq, H, D, k + W))
    scale = 1 / np.sqrt(128)
    csa.csa_sparse_attn(qd, kvd, up(idx), k, rawd, up(raw_base), W, up(pos), B, Tq, H, D, scale, out, lse, ws,
                        ws.numel())
    want, want_lse = oracle.csa_sparse_attn(qv, kvv, idx, rawv, raw_base, W, pos, scale)
    assert row_rel_err(down(out), want) < 5e-3
    assert np.max(np.abs(down(lse) - want_lse)) < 5e-3
