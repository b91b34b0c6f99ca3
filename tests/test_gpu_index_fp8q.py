"""The fp8-query indexer (reading R27) on the GPU against the oracle.

Each query row is quantised on both sides in fp32 with the same steps (scale = max(amax,
1e-12) / 448, correctly rounded divisions, round to nearest even), so the codes agree;
the scores then differ only by the arithmetic of the contraction. Tolerance, from that
arithmetic: the matrix unit adds the 64 products of one 32x32x64 fp8 instruction with a
truncated alignment (measured on MI355X: error up to 2^-11.4 of the largest product of
the instruction); allowing 2^-10 per instruction, a 128-long dot (two instructions) of
head h with key s errs by at most 2^-9 * max_d |c_q[h,d] c_k[s,d]| (the codes' largest
product), so a score errs by at most k_scale[s] * 2^-9 * sum_h |w_h s_q,h| *
max_d |c_q[h,d] c_k[s,d]|, plus fp32 rounding of the epilogue (1e-5 of the row's largest
score). Scores are checked against the cheaper bound with 448^2 in place of the largest
product (no code exceeds 448). The selection band is the exact bound: it is computed
from each candidate's own code products for the candidates whose score lies within the
cheaper bound's band of the m-th score (the others are decided the same way under either
bound), and membership may differ from the oracle's only inside it.

Cases: 64 heads (two row blocks, one query per workgroup), the prefill kernel (64
queries, four query groups sharing each key tile), 32 heads, 16/8/4 heads (several
queries per row block), the HI fine stage through a kept map, per-sequence context
lengths, the primed index -> select chain, and the full 128K decode and 4096-token
prefill workloads (sampled rows for the prefill).
"""
import numpy as np
import pytest
import torch

import long_context_sparse_07_amd as L
from oracle import lsa_oracle as O
from synth import config, make_inputs
from gpu_harness import upload, check_band

pytestmark = pytest.mark.gpu

E8 = 2.0 ** -9 * 448.0 * 448.0


def _score_tol(qI_bits, w, kscale):
    """Per-column tolerance of one query's scores (see the module docstring)."""
    q = O.decode_bf16(qI_bits).astype(np.float32)
    _, sq = O.quantize_key_rows(q)
    return kscale.astype(np.float64) * E8 * float(np.sum(np.abs(w.astype(np.float64) * sq)))


def _band_rtol(qI_bits, w, k_codes, kscale, C, want, m):
    """Selection band (relative to |tau|, the m-th largest oracle score among the
    candidates C) from the candidates' own code products (see the module docstring)."""
    tau = np.sort(want[C])[::-1][min(m, C.size) - 1]
    loose = _score_tol(qI_bits, w, kscale[C])
    near = C[np.abs(want[C] - tau) <= 2.0 * float(np.max(loose)) + 1e-4 * abs(tau)]
    q = O.decode_bf16(qI_bits).astype(np.float32)
    cq, sq = O.quantize_key_rows(q)
    aq = np.abs(O.decode_e4m3fn(cq))                        # [H, D] query codes
    ak = np.abs(O.decode_e4m3fn(k_codes[near]))             # [n, D] key codes
    mx = np.max(aq[None, :, :] * ak[:, None, :], axis=2)    # [n, H] largest product per head
    ws = np.abs(w.astype(np.float64) * sq.astype(np.float64))
    tol = kscale[near].astype(np.float64) * 2.0 ** -9 * (mx @ ws)
    return 2.0 * float(np.max(tol)) / max(abs(tau), 1e-30) + 1e-4, 2.0 * float(np.max(loose)) / max(abs(tau), 1e-30)


def _check_row(g, want, tol, what):
    fin = np.isfinite(want)
    assert np.array_equal(np.isfinite(g), fin), f"{what}: masking differs"
    if not fin.any():
        return 0.0
    slack = 1e-5 * np.max(np.abs(want[fin]))
    err = np.abs(g[fin].astype(np.float64) - want[fin])
    assert np.all(err <= tol[fin] + slack), f"{what}: error {np.max(err - tol[fin]):.3e} above the bound"
    return float(np.max(err) / max(np.max(np.abs(want[fin])), 1e-30))


def _cfg(cid, **kw):
    return config(cid, q_fp8=True, **kw)


CASES = {
    "h64_decode": _cfg(2, B=2, N=6000, K=512, S=32, W=128),
    "h64_prefill": _cfg(4, B=1, N=3000, T=64, K=256, S=16, W=64),
    "h32_decode": _cfg(5, B=2, N=5000, K=512, S=32, W=128, layers=1),
    "h16": _cfg(2, B=1, N=3000, T=4, H_I=16, K=256, S=16, W=64),
    "h8": _cfg(2, B=1, N=2500, T=4, H_I=8, K=256, S=16, W=64),
    "h4": _cfg(2, B=2, N=2100, T=8, H_I=4, K=256, S=16, W=64),
}


@pytest.mark.parametrize("name", list(CASES))
def test_fp8_query_scores_and_selection(name):
    cfg = CASES[name]
    inp = make_inputs(cfg, with_kv=False)
    rng = np.random.default_rng(7)
    inp["ctx_len"] = np.array([cfg.N - int(rng.integers(0, 300)) * (b % 2) for b in range(cfg.B)], np.int32)
    d = upload(inp)
    sc = L.lsa_index(d["qI"], d["w"], d["kI"], k_scale=d["kI_scale"], ctx_len=d["ctx_len"], q_fp8=True)
    sc2, idx = L.lsa_index_select(d["qI"], d["w"], d["kI"], cfg.K, cfg.S, cfg.W, k_scale=d["kI_scale"],
                                  ctx_len=d["ctx_len"], q_fp8=True)
    torch.cuda.synchronize()
    assert torch.equal(sc2, sc)  # the primed chain writes the same scores
    g, gi = sc.cpu().numpy(), idx.cpu().numpy()
    ora = O.reference_step(inp, with_attend=False)
    P = O.query_positions(inp["ctx_len"], cfg.T)
    worst = 0.0
    for b in range(cfg.B):
        for t in range(cfg.T):
            p = int(P[b, t])
            want = ora["scores"][(b, t)]
            tol = _score_tol(inp["qI"][b, t], inp["w"][b, t], inp["kI_scale"][b][: p + 1])
            worst = max(worst, _check_row(g[b, t, : p + 1], want, tol, f"{name} {b},{t}"))
            assert np.all(np.isneginf(g[b, t, p + 1:]))
            F = O.forced_positions(p, cfg.S, cfg.W)
            C = np.setdiff1d(np.arange(p + 1), F)
            if C.size:
                m = cfg.K - F.size
                rtol, _ = _band_rtol(inp["qI"][b, t], inp["w"][b, t], inp["kI"][b], inp["kI_scale"][b], C, want, m)
                check_band(gi[b, t], C, want[C], F, cfg.K, rtol=rtol, what=f"{name} {b},{t}")
    print(f"{name}: largest score error {worst:.2e} of the row maximum")


def test_fp8_query_hi_fine_stage():
    cfg = _cfg(2, B=1, N=8192, T=2, K=512, S=32, W=128, hi=True, Bs=64, n_keep=24)
    inp = make_inputs(cfg, with_kv=False)
    d = upload(inp)
    kbar = L.lsa_block_means(d["kI"], cfg.Bs, k_scale=d["kI_scale"])
    cs = L.lsa_index(d["qI"], d["w"], kbar, mode=L.LSA_INDEX_BLOCKS, N=cfg.N, ctx_len=d["ctx_len"],
                     block_size=cfg.Bs, sink=cfg.S, window=cfg.W)
    kept = L.lsa_select(cs, cfg.n_keep, 0, 0, causal=False)
    fs = L.lsa_index(d["qI"], d["w"], d["kI"], k_scale=d["kI_scale"], kept=kept, block_size=cfg.Bs,
                     ctx_len=d["ctx_len"], q_fp8=True)
    torch.cuda.synchronize()
    g, kp = fs.cpu().numpy(), kept.cpu().numpy()
    keys = O.index_keys_f64(inp["kI"][0], inp["kI_scale"][0])
    P = O.query_positions(inp["ctx_len"], cfg.T)
    for t in range(cfg.T):
        p = int(P[0, t])
        q = O.index_query_f64(inp["qI"][0, t], True)
        w = inp["w"][0, t].astype(np.float64)
        cols = np.arange(cfg.n_keep * cfg.Bs)
        blk = kp[0, t][cols // cfg.Bs]
        pos = np.where(blk >= 0, blk * cfg.Bs + cols % cfg.Bs, -1)
        want = np.full(cols.size, -np.inf)
        ok = (pos >= 0) & (pos <= p)
        want[ok] = O.indexer_scores_at(q, w, keys[pos[ok]])
        tol = np.zeros(cols.size)
        tol[ok] = _score_tol(inp["qI"][0, t], inp["w"][0, t], inp["kI_scale"][0][pos[ok]])
        _check_row(g[0, t], want, tol, f"hi t={t}")


@pytest.mark.parametrize("cid", [2, 4])
def test_fp8_query_full_size_sampled(cid):
    # the 128K decode (8 sequences, every row) and the 4096-token prefill after 256K keys
    # (sampled rows) at their full sizes, in the launch configuration the benchmark times
    cfg = config(cid, q_fp8=True)
    inp = make_inputs(cfg, with_kv=False)
    d = upload(inp)
    sc, idx = L.lsa_index_select(d["qI"], d["w"], d["kI"], cfg.K, cfg.S, cfg.W, k_scale=d["kI_scale"],
                                 ctx_len=d["ctx_len"], q_fp8=True)
    torch.cuda.synchronize()
    if cid == 4:
        rng = np.random.default_rng(4040)
        rows = [(0, t) for t in sorted({0, 63, 64, 4095, *rng.integers(0, cfg.T, size=5).tolist()})]
    else:
        rows = [(b, 0) for b in range(cfg.B)]
    ora = O.reference_step(inp, rows=rows, with_attend=False)
    P = O.query_positions(inp["ctx_len"], cfg.T)
    for b, t in rows:
        p = int(P[b, t])
        g = sc[b, t, : p + 1].cpu().numpy()
        want = ora["scores"][(b, t)]
        tol = _score_tol(inp["qI"][b, t], inp["w"][b, t], inp["kI_scale"][b][: p + 1])
        err = _check_row(g, want, tol, f"c{cid} {b},{t}")
        F = O.forced_positions(p, cfg.S, cfg.W)
        C = np.setdiff1d(np.arange(p + 1), F)
        m = cfg.K - F.size
        rtol, rtol_loose = _band_rtol(inp["qI"][b, t], inp["w"][b, t], inp["kI"][b], inp["kI_scale"][b], C, want, m)
        check_band(idx[b, t].cpu().numpy(), C, want[C], F, cfg.K, rtol=rtol, what=f"c{cid} {b},{t}")
        print(f"c{cid} {b},{t}: score error {err:.2e} of the row maximum, selection band {rtol:.2e} "
              f"(448^2 bound: {rtol_loose:.2e})")
