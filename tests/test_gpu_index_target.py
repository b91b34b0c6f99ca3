"""lsa_index_target on the GPU against the oracle's indexer_target and indexer_kl (reading
R30).

Inputs are seeded: bf16 q and K rows, sorted index rows with -1 padding (one row with no
valid entry), fp32 indexer scores, and the log-sum-exp of the oracle's float64 forward
rounded to fp32 (the form lsa_attend stores). The GPU computes q . K with exact bf16
products and fp32 sums, then exp and the head mean in fp32; the oracle in float64.
Tolerance, from that arithmetic: target and gradient within 2e-6 absolute (entries are
probabilities, at most 1; fp32 rounding of a 576-long dot scaled by softmax_scale, then
of exp and a 64-term mean), the loss within 1e-5 relative. Two calls give the same bits.
Cases: MLA and GQA with padded rows and a row with no valid entry, and the 128K MLA
decode shape (8 sequences, 2048 selected rows each).
"""
import numpy as np
import pytest
import torch

import long_context_sparse_07_amd as L
from oracle import lsa_oracle as O

pytestmark = pytest.mark.gpu


def _bits(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def _f64(t):
    return t.to(torch.float32).numpy().astype(np.float64)


@pytest.mark.parametrize("mla", [True, False])
def test_index_target_matches_oracle(mla):
    rng = np.random.default_rng(80 + mla)
    B, T, N, K = 2, 3, 3000, 200
    Hq, Hkv, dqk = (64, 1, 576) if mla else (32, 4, 128)
    q = _bits(rng.standard_normal((B, T, Hq, dqk)) / np.sqrt(dqk))
    k = _bits(rng.standard_normal((B, N, Hkv, dqk)))
    idx = np.full((B, T, K), -1, np.int32)
    for b in range(B):
        for t in range(T):
            nv = [200, 150, 0][t] if b == 1 else [200, 77, 1][t]
            if nv:
                idx[b, t, :nv] = np.sort(rng.choice(N, nv, replace=False))
    scores = (rng.standard_normal((B, T, N)) * 2.0).astype(np.float32)
    tau = dqk ** -0.5
    qf, kf = _f64(q), _f64(k)
    lse = np.zeros((B, T, Hq))
    for b in range(B):
        for t in range(T):
            _, lse[b, t] = O.attend(qf[b, t], kf[b], kf[b], idx[b, t], tau)
    lse32 = lse.astype(np.float32)
    args = (q.cuda(), k.cuda(), torch.from_numpy(idx).cuda(), tau, torch.from_numpy(lse32).cuda(),
            torch.from_numpy(scores).cuda())
    tg, gr, ls = L.lsa_index_target(*args)
    tg2, gr2, ls2 = L.lsa_index_target(*args)
    torch.cuda.synchronize()
    assert torch.equal(tg, tg2) and torch.equal(gr, gr2) and torch.equal(ls, ls2)
    tg, gr, ls = tg.cpu().numpy(), gr.cpu().numpy(), ls.cpu().numpy()
    for b in range(B):
        for t in range(T):
            want_t = O.indexer_target(qf[b, t], kf[b], idx[b, t], tau, lse32[b, t].astype(np.float64))
            valid = idx[b, t] >= 0
            sc_sel = np.where(valid, scores[b, t][np.maximum(idx[b, t], 0)], 0.0).astype(np.float64)
            want_l, want_g = O.indexer_kl(want_t, sc_sel, valid)
            assert np.max(np.abs(tg[b, t] - want_t)) < 2e-6, (b, t)
            assert np.max(np.abs(gr[b, t] - want_g)) < 2e-6, (b, t)
            assert abs(ls[b, t] - want_l) <= 1e-5 * max(abs(want_l), 1.0), (b, t, ls[b, t], want_l)
            if not valid.any():
                assert not tg[b, t].any() and not gr[b, t].any() and ls[b, t] == 0
            else:
                assert abs(tg[b, t].sum() - 1.0) < 1e-4


def test_index_target_128k_mla_decode_shape():
    # 8 sequences of 131072 cached rows, one query token each, 2048 selected rows, 64 MLA
    # heads (the shape the benchmark times); the oracle reads the selected rows only
    rng = np.random.default_rng(82)
    B, N, K, Hq = 8, 131072, 2048, 64
    idx = np.stack([np.sort(rng.choice(N, K, replace=False)) for _ in range(B)]).astype(np.int32)[:, None, :]
    q = _bits(rng.standard_normal((B, 1, Hq, 576)) / 24.0)
    sel_rows = _bits(rng.standard_normal((B, K, 1, 576)))
    k = torch.zeros((B, N, 1, 576), dtype=torch.bfloat16)
    for b in range(B):
        k[b, idx[b, 0]] = sel_rows[b]
    scores = (rng.standard_normal((B, 1, N)) * 2.0).astype(np.float32)
    tau = 576 ** -0.5
    qf, ks = _f64(q), _f64(sel_rows)
    local = np.arange(K)
    lse = np.stack([O.attend(qf[b, 0], ks[b], ks[b], local, tau)[1] for b in range(B)]).astype(np.float32)[:, None]
    tg, gr, ls = L.lsa_index_target(q.cuda(), k.cuda(), torch.from_numpy(idx).cuda(), tau,
                                    torch.from_numpy(lse).cuda(), torch.from_numpy(scores).cuda())
    torch.cuda.synchronize()
    tg, gr, ls = tg.cpu().numpy(), gr.cpu().numpy(), ls.cpu().numpy()
    for b in range(B):
        want_t = O.indexer_target(qf[b, 0], ks[b], local, tau, lse[b, 0].astype(np.float64))
        want_l, want_g = O.indexer_kl(want_t, scores[b, 0][idx[b, 0]].astype(np.float64), np.ones(K, bool))
        assert np.max(np.abs(tg[b, 0] - want_t)) < 2e-6, b
        assert np.max(np.abs(gr[b, 0] - want_g)) < 2e-6, b
        assert abs(ls[b, 0] - want_l) <= 1e-5 * max(abs(want_l), 1.0), b
