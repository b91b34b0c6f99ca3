"""The one-launch selection of short rows (at most 4096 columns: one workgroup per row
ranks its row from order keys held in LDS) against the oracle's selection rule on the
same fp32 values. Cases: random rows of several lengths (not all multiples of 4), every
candidate equal (the whole row one tie group), signed zeros next to -inf and NaN
entries, fewer candidates than the fill, the plain top-K of the HI block stage
(causal = 0), candidate maps whose entries ascend and do not (the fill then sorted in
LDS) with per-token context lengths, and the workspace: a dirty one is not read and is
left clean.
"""
import numpy as np
import pytest
import torch

import long_context_sparse_07_amd as L
from oracle import lsa_oracle as O

pytestmark = pytest.mark.gpu


def _want_causal(scores64, pos, p, K, S, W):
    """Selection rule of one causal row: forced set, then the fill over the finite,
    visible, non-forced candidates (scores64[i] belongs to position pos[i])."""
    F = O.forced_positions(p, S, W)
    ok = np.isfinite(scores64) & (pos >= 0) & (pos <= p) & ~np.isin(pos, F)
    fill = O.top_fill(pos[ok], scores64[ok], K - F.size)
    return O.pad_sorted(np.concatenate([F, fill]), K)


def _rows(rows, K, S, W, causal=True):
    R, N = rows.shape
    sc = torch.from_numpy(np.ascontiguousarray(rows, dtype=np.float32)).cuda().view(R, 1, N)
    got = L.lsa_select(sc, K, S, W, causal=causal).cpu().numpy()[:, 0]
    for i in range(R):
        s = rows[i].astype(np.float32).astype(np.float64)
        if causal:
            want = _want_causal(s, np.arange(N), N - 1, K, S, W)
        else:
            ok = np.isfinite(s)
            want = O.pad_sorted(O.top_fill(np.arange(N)[ok], s[ok], K), K)
        assert np.array_equal(got[i], want), f"row {i} (N={N}): {np.count_nonzero(got[i] != want)} entries differ"


@pytest.mark.parametrize("N", [4096, 4093, 1000, 65])
def test_random_rows(N):
    rng = np.random.default_rng(900 + N)
    _rows(rng.standard_normal((6, N)).astype(np.float32), 512, 16, 64)


def test_whole_row_one_tie_group():
    _rows(np.zeros((3, 4096), np.float32), 2048, 64, 512)
    _rows(np.full((2, 4000), 1.5, np.float32), 1000, 0, 0)


def test_signed_zeros_inf_nan_and_few_candidates():
    rng = np.random.default_rng(905)
    N = 4000
    row = np.where(rng.random(N) < 0.5, np.float32(0.0), np.float32(-0.0)).astype(np.float32)
    hot = rng.choice(np.arange(16, N - 64), 100, replace=False)
    row[hot] = rng.random(100).astype(np.float32) + 0.5
    row[rng.choice(np.arange(16, N - 64), 300, replace=False)] = -np.inf
    row[rng.choice(np.arange(16, N - 64), 50, replace=False)] = np.nan
    few = np.full(N, -np.inf, np.float32)
    few[rng.choice(np.arange(16, N - 64), 80, replace=False)] = rng.standard_normal(80).astype(np.float32)
    _rows(np.stack([row, few]), 512, 16, 64)


def test_block_stage_plain_top_k():
    rng = np.random.default_rng(906)
    rows = rng.standard_normal((4, 4096)).astype(np.float32)
    rows[1, rng.choice(4096, 3000, replace=False)] = -np.inf  # fewer finite blocks than asked... still > K
    rows[2, :] = 0.25                                        # all equal: the lowest block indices win
    _rows(rows, 256, 0, 0, causal=False)
    _rows(rows, 4096, 0, 0, causal=False)                    # K = every column


@pytest.mark.parametrize("order", ["ascending", "shuffled"])
def test_candidate_map(order):
    rng = np.random.default_rng(907 if order == "ascending" else 908)
    B, T, N, bs, n_keep, K, S, W = 2, 3, 8192, 64, 48, 640, 16, 64
    nblk = N // bs
    kept = np.full((B, T, n_keep), -1, np.int32)
    for b in range(B):
        for t in range(T):
            blocks = rng.choice(nblk, n_keep - 5, replace=False)
            kept[b, t, : blocks.size] = np.sort(blocks) if order == "ascending" else blocks
            if order == "shuffled":
                kept[b, t] = rng.permutation(kept[b, t])  # -1 entries anywhere
    ctx = np.array([N, N - 700], np.int32)
    scores = rng.standard_normal((B, T, n_keep * bs)).astype(np.float32)
    idx = L.lsa_select(torch.from_numpy(scores).cuda(), K, S, W, N=N, ctx_len=torch.from_numpy(ctx).cuda(),
                       kept=torch.from_numpy(kept).cuda(), block_size=bs).cpu().numpy()
    cols = np.arange(n_keep * bs)
    for b in range(B):
        for t in range(T):
            p = int(ctx[b]) - T + t
            blk = kept[b, t][cols // bs]
            pos = np.where((blk >= 0) & (blk < nblk), blk * bs + cols % bs, -1)
            want = _want_causal(scores[b, t].astype(np.float64), pos, p, K, S, W)
            assert np.array_equal(idx[b, t], want), f"{order} {b},{t}"


def test_dirty_workspace_is_not_read_and_left_clean():
    rng = np.random.default_rng(909)
    R, N, K = 5, 3000, 256
    rows = rng.standard_normal((R, N)).astype(np.float32)
    sc = torch.from_numpy(rows).cuda().view(R, 1, N)
    want = L.lsa_select(sc, K, 16, 64).cpu()
    nbytes = L.lsa_select_workspace_bytes(sc, K, 16, 64)
    ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")
    idx = torch.empty((R, 1, K), dtype=torch.int32, device="cuda")
    d = L.SelectDesc(B=R, T=1, N=N, scores=sc.data_ptr(), n_cols=N, K=K, sink=16, window=64, causal=1,
                     idx=idx.data_ptr(), workspace_state=L.LSA_WS_PRIMED)  # a wrong claim: not read
    assert L.lib().lsa_select(d, ws.data_ptr(), nbytes, torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    assert torch.equal(idx.cpu(), want)
    hist = ws[: R * 2048 * 4].view(torch.int32)
    assert int(hist.abs().sum()) == 0, "histogram not left at zero"
    ctr = ws[R * 2048 * 4: R * 2048 * 4 + R * 16 * 4].view(torch.int32)  # (R * 8192 is a multiple of 256)
    assert int(ctr.abs().sum()) == 0, "counters not left at zero"
