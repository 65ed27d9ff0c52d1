"""csa_sparse_attn_noalloc (the allocation-free sparse attention: its split partials
live in a static device array) against csa_sparse_attn with a caller workspace, on
the same inputs: two calls in a row, the second on a smaller input, so the second
runs on scratch that still holds the first call's partials.  Same kernels and
splits on both sides, so the outputs must agree bit for bit; the small case is also
checked against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_helpers import down, row_rel_err, sorted_unique_choice, up, up_bf16, workspace

pytestmark = pytest.mark.gpu

WID = 101  # seed namespace of this test
H, D, M = 64, 512, 4


def _case(csa, name, B, k, W, N):
    r = synth.rng(WID, name)
    q = r.standard_normal((B, 1, H, D)).astype(np.float32)
    kvc = r.standard_normal((B, N, D)).astype(np.float32)
    R = W + 64
    raw = r.standard_normal((B, R, D)).astype(np.float32)
    pos = r.integers(N * M // 2, N * M, (B, 1)).astype(np.int32)
    raw_base = np.maximum(0, pos[:, 0] - W - 3).astype(np.int32)
    idx = np.stack([[sorted_unique_choice(r, oracle.visible_blocks(int(pos[b, 0]), M), k)] for b in range(B)])
    qt, qv = up_bf16(q)
    kt, kv = up_bf16(kvc)
    rt, rv = up_bf16(raw)
    return dict(B=B, k=k, W=W, q=csa.desc(qt, csa.BF16), kv=csa.desc(kt, csa.BF16), raw=csa.desc(rt, csa.BF16),
                idx=up(idx.astype(np.int32)), raw_base=up(raw_base), pos=up(pos), keep=(qt, kt, rt),
                host=(qv, kv, idx, rv, raw_base, pos))


def _run(csa, c, noalloc):
    B, k, W = c["B"], c["k"], c["W"]
    out = torch.full((B, 1, H, D), float("nan"), device="cuda")
    lse = torch.full((B, 1, H), float("nan"), device="cuda")
    args = (c["q"], c["kv"], c["idx"], k, c["raw"], c["raw_base"], W, c["pos"], B, 1, H, D, 0.0625, out, lse)
    if noalloc:
        csa.csa_sparse_attn_noalloc(*args)
    else:
        ws = workspace(csa.csa_attn_workspace_size(B, 1, H, D, k + W))
        csa.csa_sparse_attn(*args, ws, ws.numel())
    return down(out), down(lse)


def test_noalloc_matches_workspace_entry_point(gpu_lib):
    csa = gpu_lib
    big = _case(csa, "big", B=8, k=2048, W=128, N=16384)  # the 1M-context decode's attention shape
    small = _case(csa, "small", B=3, k=600, W=64, N=2048)
    assert 0 < csa.csa_attn_workspace_size(3, 1, H, D, 664) < csa.csa_attn_workspace_size(8, 1, H, D, 2176)
    assert csa.csa_attn_workspace_size(8, 1, H, D, 2176) <= csa.CSA_NOALLOC_SCRATCH_BYTES
    for c in (big, small):
        got = _run(csa, c, noalloc=True)
        want = _run(csa, c, noalloc=False)
        assert np.isfinite(got[0]).all() and np.isfinite(got[1]).all()
        np.testing.assert_array_equal(got[0], want[0])
        np.testing.assert_array_equal(got[1], want[1])
    qv, kv, idx, rv, raw_base, pos = small["host"]
    ref, ref_lse = oracle.csa_sparse_attn(qv, kv, idx, rv, raw_base, small["W"], pos, 0.0625)
    got = _run(csa, small, noalloc=True)
    assert row_rel_err(got[0], ref) < 2e-3
    assert np.max(np.abs(got[1] - ref_lse)) < 2e-3


def test_noalloc_rejects_what_exceeds_its_scratch(gpu_lib):
    csa = gpu_lib
    # real buffers of the rejected shape: 64 rows x 8 splits x 64 heads x 514 floats of
    # partials exceed the static array
    B = 64
    c = _case(csa, "reject", B=B, k=2048, W=128, N=1024)
    assert csa.csa_attn_workspace_size(B, 1, H, D, 2048 + 128) > csa.CSA_NOALLOC_SCRATCH_BYTES
    out = torch.full((B, 1, H, D), float("nan"), device="cuda")
    with pytest.raises(csa.CsaError) as ei:
        csa.csa_sparse_attn_noalloc(c["q"], c["kv"], c["idx"], 2048, c["raw"], c["raw_base"], 128, c["pos"], B, 1, H,
                                    D, 0.0625, out, None)
    assert ei.value.status == 5  # CSA_ERR_WORKSPACE, before any launch
    torch.cuda.synchronize()
    assert torch.isnan(out).all()
