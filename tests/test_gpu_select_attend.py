"""The fused chain lsa_select_attend (the attention kernel finishes the selection, each
workgroup the part of the index list it attends over) against the two separate calls
lsa_select + lsa_attend on the same inputs: the index list, the attention output and
the log-sum-exp must be bit-identical. The separate calls are pinned to the oracle
elsewhere; one case here also checks the fused index list against the oracle directly.
The chain runs its fused kernel only for more than 48 query heads per KV head in one
layer (MLA here); for the other shapes the call runs the selection's resolve kernel and
the plain attention, which these cases check through the same entry point.

Cases: MLA (64 heads, 32-head blocks), 64 query heads on one 128-wide KV head (the
four-wave fused kernel of 128-wide rows) and GQA / MQA kernels (one wave); several
layers and KV heads sharing one selection row; one split and many; fp32 output with one
split (the kernel's early exit); the row bitmap in LDS and, for a long GQA row, in the
workspace; ties ranked by radix passes and from the workspace copy of the tie list; a
tie list that overflowed (the row is rescanned); rows with fewer candidates than the
fill, short contexts (everything forced) and padding; the primed chain
(lsa_index_select_attend). Each fused call leaves the selection workspace clean, which
the next call in the same test relies on.
"""
import numpy as np
import pytest
import torch

import long_context_sparse_07_amd as L
from test_gpu_select import _oracle_select
from synth import config, make_inputs
from gpu_harness import upload

pytestmark = pytest.mark.gpu


def _bf16(rng, shape, scale=1.0):
    return torch.from_numpy((rng.standard_normal(shape) * scale).astype(np.float32)).to(torch.bfloat16).cuda()


def _kv(rng, layers, B, N, Hq, Hkv, mla, T=1):
    if mla:
        q = _bf16(rng, (layers, B, T, Hq, 576), 576 ** -0.5)
        k = _bf16(rng, (layers, B, N, 1, 576))
        return q, k, None, 576 ** -0.5
    q = _bf16(rng, (layers, B, T, Hq, 128), 128 ** -0.5)
    k = _bf16(rng, (layers, B, N, Hkv, 128))
    v = _bf16(rng, (layers, B, N, Hkv, 128))
    return q, k, v, 128 ** -0.5


def _both(scores, K, S, W, q, k, v, scale, *, ctx_len=None, n_splits=0, out_dtype=None, causal=True, repeat=2):
    """Separate calls, then the fused chain `repeat` times, then the separate selection
    again (on the workspace the fused chain left clean); everything must agree."""
    idx0 = L.lsa_select(scores, K, S, W, ctx_len=ctx_len, causal=causal)
    out0, lse0 = L.lsa_attend(q, k, v, idx0, scale, n_splits=n_splits, out_dtype=out_dtype)
    for _ in range(repeat):
        idx1, out1, lse1 = L.lsa_select_attend(scores, K, S, W, q, k, v, scale, ctx_len=ctx_len, n_splits=n_splits,
                                               out_dtype=out_dtype, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(idx1, idx0), f"{int((idx1 != idx0).sum())} index entries differ"
        assert torch.equal(out1.view(torch.int16) if out1.dtype == torch.bfloat16 else out1,
                           out0.view(torch.int16) if out0.dtype == torch.bfloat16 else out0)
        assert torch.equal(lse1, lse0)
    idx2 = L.lsa_select(scores, K, S, W, ctx_len=ctx_len, causal=causal)
    assert torch.equal(idx2, idx0)
    return idx0


def _scores(rows):
    R, N = rows.shape
    return torch.from_numpy(np.ascontiguousarray(rows, dtype=np.float32)).cuda().view(R, 1, N)


@pytest.mark.parametrize("N,K,S,W,splits", [
    (9000, 512, 32, 128, 0), (5003, 2048, 64, 512, 0), (131072, 2048, 64, 512, 32), (4096, 256, 16, 64, 3),
])
def test_mla_random_rows(N, K, S, W, splits):
    rng = np.random.default_rng(100 + N % 97)
    B = 3
    rows = rng.standard_normal((B, N)).astype(np.float32)
    q, k, v, scale = _kv(rng, 1, B, N, 64, 1, True)
    idx = _both(_scores(rows), K, S, W, q, k, v, scale, n_splits=splits)
    if N == 9000:  # the fused index list against the oracle itself
        got = idx.cpu().numpy()[:, 0]
        for i in range(B):
            assert np.array_equal(got[i], _oracle_select(rows[i], K, S, W)), f"row {i}"


def test_mla_fp32_single_split():
    rng = np.random.default_rng(201)
    rows = rng.standard_normal((2, 6000)).astype(np.float32)
    q, k, v, scale = _kv(rng, 1, 2, 6000, 64, 1, True)
    _both(_scores(rows), 512, 16, 64, q, k, v, scale, n_splits=1, out_dtype=torch.float32)


@pytest.mark.parametrize("Hq,Hkv,layers,T", [(16, 1, 1, 4), (32, 4, 3, 1), (32, 1, 2, 2)])
def test_gqa_layers_and_kv_heads_share_rows(Hq, Hkv, layers, T):
    rng = np.random.default_rng(300 + Hq + Hkv + layers)
    B, N, K = 2, 7000, 512
    sc = torch.from_numpy(rng.standard_normal((B, T, N)).astype(np.float32)).cuda()
    q, k, v, scale = _kv(rng, layers, B, N, Hq, Hkv, False, T=T)
    _both(sc, K, 32, 128, q, k, v, scale)


def test_gqa_long_row_bitmap_in_workspace():
    # 300000 columns: the row bitmap does not fit beside the one-wave kernel's tile ring
    rng = np.random.default_rng(400)
    rows = rng.standard_normal((2, 300000)).astype(np.float32)
    q, k, v, scale = _kv(rng, 1, 2, 300000, 16, 1, False)
    _both(_scores(rows), 2048, 64, 512, q, k, v, scale)


def test_many_equal_scores():
    # radix passes over the tie list (3000 equal scores), and the workspace copy of the
    # tie list (10000 equal scores in a 40000-column row)
    rng = np.random.default_rng(500)
    rows = []
    for N, hot, eq in ((40000, 600, 3000), (40000, 500, 10000)):
        row = (rng.standard_normal(N) * 0.01 - 5.0).astype(np.float32)
        pos = rng.permutation(np.arange(16, N - 64))
        row[pos[:hot]] = 10.0 + rng.random(hot).astype(np.float32)
        row[pos[hot:hot + eq]] = 2.0
        rows.append(row)
    rows = np.stack(rows)
    for mla in (True, False):
        q, k, v, scale = _kv(rng, 1, 2, 40000, 64 if mla else 16, 1, mla)
        _both(_scores(rows), 2048, 16, 64, q, k, v, scale)


@pytest.mark.parametrize("mla", [False, True])
def test_tie_list_overflow_rescans_row(mla):
    # 2048 rows x 16384 columns: the per-row tie list holds 8192 entries; row 7 has
    # 10000 equal scores in its threshold bin (MLA: the fused kernel rescans the row)
    rng = np.random.default_rng(600)
    T, N = 2048, 16384
    rows = rng.standard_normal((T, N)).astype(np.float32)
    hot = 7
    rows[hot] = (rng.standard_normal(N) * 0.01 - 5.0).astype(np.float32)
    pos = rng.permutation(np.arange(16, N - 2048 - 64))
    rows[hot, pos[:500]] = 3.0 + rng.random(500).astype(np.float32)
    rows[hot, pos[500:10500]] = 2.0
    sc = torch.from_numpy(rows).cuda().view(1, T, N)
    q, k, v, scale = _kv(rng, 1, 1, N, 64 if mla else 16, 1, mla, T=T)
    _both(sc, 2048, 16, 64, q, k, v, scale, repeat=1)


def test_degenerate_rows():
    # per-sequence contexts: 40 (everything forced, padding), 700 (fewer candidates than
    # the fill after -inf masking), 5000 (random); plain top-K (causal = 0) too
    rng = np.random.default_rng(700)
    B, N = 3, 5000
    rows = rng.standard_normal((B, N)).astype(np.float32)
    rows[1, rng.choice(np.arange(100, 600), 450, replace=False)] = -np.inf
    ctx = torch.tensor([40, 700, 5000], dtype=torch.int32).cuda()
    q, k, v, scale = _kv(rng, 1, B, N, 64, 1, True)
    _both(_scores(rows), 512, 32, 128, q, k, v, scale, ctx_len=ctx)
    _both(_scores(rows), 512, 0, 0, q, k, v, scale, causal=False)


def test_primed_chain_equals_separate_calls():
    cfg = config(2, B=2, N=9000, K=512, S=32, W=128)
    inp = make_inputs(cfg)
    d = upload(inp)
    rng = np.random.default_rng(800)
    q, k, v, scale = _kv(rng, 1, cfg.B, cfg.N, 64, 1, True)
    sc, idx = L.lsa_index_select(d["qI"], d["w"], d["kI"], cfg.K, cfg.S, cfg.W, k_scale=d["kI_scale"],
                                 ctx_len=d["ctx_len"])
    out, lse = L.lsa_attend(q, k, v, idx, scale)
    for _ in range(2):
        sc2, idx2, out2, lse2 = L.lsa_index_select_attend(d["qI"], d["w"], d["kI"], cfg.K, cfg.S, cfg.W, q, k, v,
                                                          scale, k_scale=d["kI_scale"], ctx_len=d["ctx_len"])
        assert torch.equal(sc2, sc)
        assert torch.equal(idx2, idx)
        assert torch.equal(out2.view(torch.int16), out.view(torch.int16))
        assert torch.equal(lse2, lse)


@pytest.mark.parametrize("mla", [True, False])
def test_shared_selection_for_draft_tokens(mla):
    # one index row per sequence for T = 4 draft tokens (reading R29): each token attends
    # over the entries at or before its own position; equal, bit for bit, to per-token
    # rows with the later entries padded out, and to the oracle within the attention bound
    from gpu_harness import check_attn
    from oracle import lsa_oracle as O
    rng = np.random.default_rng(900 + mla)
    B, T, N, K = 2, 4, 5000, 512
    ctx = np.array([N, N - 37], np.int32)
    q, k, v, scale = _kv(rng, 1, B, N, 64 if mla else 16, 1, mla, T=T)
    shared = np.full((B, K), -1, np.int32)
    for b in range(B):
        p_last = int(ctx[b]) - 1
        win = np.arange(p_last - 5, p_last + 1)                      # the last draft positions
        rest = np.sort(rng.choice(p_last - 5, K - 20 - win.size, replace=False))
        row = np.concatenate([rest, win])
        shared[b, :row.size] = row
    per_tok = np.stack([O.shared_selection_rows(shared[b], int(ctx[b]), T) for b in range(B)]).astype(np.int32)
    o1, l1 = L.lsa_attend(q, k, v, torch.from_numpy(shared).cuda(), scale, shared=True,
                          ctx_len=torch.from_numpy(ctx).cuda())
    o0, l0 = L.lsa_attend(q, k, v, torch.from_numpy(per_tok).cuda(), scale)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o0.view(torch.int16)) and torch.equal(l1, l0)
    qf = q.float().cpu().numpy().astype(np.float64)
    kf = k.float().cpu().numpy().astype(np.float64)
    vf = kf[..., :512] if mla else v.float().cpu().numpy().astype(np.float64)
    of = o1.float().cpu().numpy()
    for b in range(B):
        for t in range(T):
            want, _ = O.attend(qf[0, b, t], kf[0, b], vf[0, b], per_tok[b, t], scale)
            check_attn(of[0, b, t], want, f"shared b={b} t={t}")


def test_mla_long_row_bitmap_in_workspace():
    # 600000 columns: the fused kernel's row bitmap (18750 words, laid out for 256
    # threads) no longer fits beside the tile ring and lives in the selection workspace
    g = torch.Generator(device="cuda").manual_seed(410)
    N = 600000
    sc = torch.randn((1, 1, N), device="cuda", generator=g)
    q = (torch.randn((1, 1, 1, 64, 576), device="cuda", generator=g) * 576 ** -0.5).to(torch.bfloat16)
    k = torch.randn((1, 1, N, 1, 576), device="cuda", generator=g).to(torch.bfloat16)
    _both(sc, 2048, 64, 512, q, k, None, 576 ** -0.5)


@pytest.mark.parametrize("N,splits,ties", [(9000, 0, False), (9000, 1, False), (9000, 5, True), (600000, 0, False)])
def test_gqa_64_heads_per_kv_head_fused_kernel(N, splits, ties):
    # 64 query heads on one 128-wide KV head: the chain runs the four-wave fused kernel of
    # 128-wide rows (the 32-head kernel is for MLA rows); one split and several, the row
    # bitmap in LDS and (600000 columns) in the workspace, a threshold bin of equal scores
    rng = np.random.default_rng(700 + N % 97 + splits)
    rows = rng.standard_normal((2, N)).astype(np.float32)
    if ties:
        rows[1] = (rng.standard_normal(N) * 0.01 - 5.0).astype(np.float32)
        pos = rng.permutation(np.arange(16, N - 600))
        rows[1, pos[:300]] = 3.0 + rng.random(300).astype(np.float32)
        rows[1, pos[300:3300]] = 2.0
    q, k, v, scale = _kv(rng, 1, 2, N, 64, 1, False)
    _both(_scores(rows), 1024, 32, 128, q, k, v, scale, n_splits=splits)
