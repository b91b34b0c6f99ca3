"""Helpers for the GPU parity tests: upload seeded inputs, run the HIP path through the
C ABI binding, and compare with the CPU oracle.

Data flows one way only: synth -> (oracle, GPU). Oracle results may be uploaded as
inputs of a later GPU stage (stage-wise checks); GPU results are never fed to the
oracle.
"""
from __future__ import annotations

import numpy as np
import torch

import long_context_sparse_07_amd as L
from oracle import lsa_oracle as O

ATT_MAX_ABS = 2e-2   # attention output tolerance (bf16 inputs, fp32 accumulation)
ATT_MEAN_ABS = 2e-3
BAND_RTOL = 1e-4     # selection: membership may differ only within 1e-4 of the m-th score


def _bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def upload(inp: dict) -> dict:
    cfg = inp["cfg"]
    d = {"cfg": cfg}
    d["qI"] = _bf16(inp["qI"])
    d["w"] = torch.from_numpy(inp["w"]).cuda()
    if cfg.k_fp8:
        d["kI"] = torch.from_numpy(inp["kI"]).cuda().view(torch.float8_e4m3fn)
        d["kI_scale"] = torch.from_numpy(inp["kI_scale"]).cuda()
    else:
        d["kI"] = _bf16(inp["kI"])
        d["kI_scale"] = None
    d["ctx_len"] = torch.from_numpy(inp["ctx_len"]).cuda()
    if "q" in inp:
        d["q"] = _bf16(inp["q"])
        d["k"] = _bf16(inp["k"])
        d["v"] = _bf16(inp["v"]) if inp["v"] is not None else None
    return d


def gpu_index_select(d: dict) -> dict:
    """index -> select on the GPU (flat, or HI coarse + fine)."""
    cfg = d["cfg"]
    r = {}
    if cfg.hi:
        kbar = L.lsa_block_means(d["kI"], cfg.Bs, k_scale=d["kI_scale"])
        cs = L.lsa_index(d["qI"], d["w"], kbar, mode=L.LSA_INDEX_BLOCKS, N=cfg.N, ctx_len=d["ctx_len"],
                         block_size=cfg.Bs, sink=cfg.S, window=cfg.W)
        kept = L.lsa_select(cs, cfg.n_keep, 0, 0, causal=False)
        fs = L.lsa_index(d["qI"], d["w"], d["kI"], k_scale=d["kI_scale"], kept=kept, block_size=cfg.Bs,
                         ctx_len=d["ctx_len"])
        idx = L.lsa_select(fs, cfg.K, cfg.S, cfg.W, N=cfg.N, ctx_len=d["ctx_len"], kept=kept, block_size=cfg.Bs)
        r.update(kbar=kbar, cscores=cs, kept=kept, fscores=fs, idx=idx)
    else:
        sc = L.lsa_index(d["qI"], d["w"], d["kI"], k_scale=d["kI_scale"], ctx_len=d["ctx_len"])
        idx = L.lsa_select(sc, cfg.K, cfg.S, cfg.W, ctx_len=d["ctx_len"])
        r.update(scores=sc, idx=idx)
    return r


def gpu_attend(d: dict, idx: torch.Tensor, **kw):
    cfg = d["cfg"]
    return L.lsa_attend(d["q"], d["k"], d["v"], idx, cfg.tau, **kw)


# ----------------------------------------------------------------------------- checks

def check_scores(gpu_row: np.ndarray, ora_row: np.ndarray, what=""):
    """Diagnostic agreement of fp32 GPU scores with float64 oracle scores."""
    g = gpu_row.astype(np.float64)
    fin = np.isfinite(ora_row)
    assert np.array_equal(np.isfinite(g[: len(ora_row)]), fin), f"{what}: masking differs"
    if fin.any():
        scale = max(np.max(np.abs(ora_row[fin])), 1e-30)
        err = np.max(np.abs(g[: len(ora_row)][fin] - ora_row[fin])) / scale
        assert err < 1e-4, f"{what}: score error {err:.2e} of the row maximum"
    return True


def check_band(gpu_idx: np.ndarray, pos: np.ndarray, sc: np.ndarray, forced: np.ndarray, K: int,
               rtol=BAND_RTOL, what=""):
    """Selection parity: forced set present, count right, sorted, and fill membership
    identical to the oracle's except for candidates within rtol of the m-th score."""
    g = np.asarray(gpu_idx, dtype=np.int64)
    valid = g[g >= 0]
    assert np.all(g[len(valid):] == -1), f"{what}: -1 padding not at the tail"
    assert np.all(np.diff(valid) > 0), f"{what}: not ascending/unique"
    F = set(forced.tolist())
    m = K - len(F)
    assert F <= set(valid.tolist()), f"{what}: forced set missing"
    fill = set(valid.tolist()) - F
    cand = dict(zip(pos.tolist(), sc.tolist()))
    assert fill <= set(cand), f"{what}: selected a non-candidate"
    want = min(m, len(cand))
    assert len(fill) == want, f"{what}: fill {len(fill)} != {want}"
    if len(cand) <= m or m == 0:
        return 0
    s_sorted = np.sort(sc)[::-1]
    tau = s_sorted[m - 1]
    band = max(rtol * abs(tau), 1e-12 * float(np.max(np.abs(sc))))
    must = {p for p, s in cand.items() if s > tau + band}
    never = {p for p, s in cand.items() if s < tau - band}
    assert must <= fill, f"{what}: {len(must - fill)} candidates above the band not selected"
    assert not (fill & never), f"{what}: {len(fill & never)} candidates below the band selected"
    exact_fill = set(O.top_fill(pos, sc, m).tolist())
    return len(fill ^ exact_fill) // 2          # band swaps (informational)


def check_attn(gpu: np.ndarray, ora: np.ndarray, what=""):
    err = np.abs(gpu.astype(np.float64) - ora)
    assert err.max() <= ATT_MAX_ABS, f"{what}: max abs err {err.max():.3e}"
    assert err.mean() <= ATT_MEAN_ABS, f"{what}: mean abs err {err.mean():.3e}"
    return err.max(), err.mean()


def oracle_rows(inp, rows):
    return O.reference_step(inp, rows=rows)


def check_topm_all_rows(scores: torch.Tensor, idx: torch.Tensor, ctx_len, T: int, K: int, S: int, W: int,
                        chunk: int = 64, what=""):
    """Properties of the selection that hold at any size, checked on every row on the GPU
    (torch ops as test infrastructure): idx ascending and unique with -1 only at the tail,
    the sink [0,S) and window [p-W+1, p] present, nothing selected outside them and the
    candidates, and the fill exactly the top m = K - |forced| candidates of the GPU's own
    fp32 scores by (score descending, position ascending). Returns the number of rows."""
    B, Tq, N = scores.shape
    dev = scores.device
    pos = torch.arange(N, device=dev)
    ctx = [int(c) for c in (ctx_len.tolist() if hasattr(ctx_len, "tolist") else ctx_len)]
    rows = 0
    for b in range(B):
        for t0 in range(0, Tq, chunk):
            t1 = min(Tq, t0 + chunk)
            sc = scores[b, t0:t1]
            ix = idx[b, t0:t1].long()
            p = torch.tensor([ctx[b] - T + t for t in range(t0, t1)], device=dev)[:, None]
            valid = ix >= 0
            nv = valid.sum(dim=1)
            ar = torch.arange(K, device=dev)[None, :]
            assert torch.equal(valid, ar < nv[:, None]), f"{what}: -1 padding not at the tail"
            d = ix[:, 1:] - ix[:, :-1]
            assert bool(((d > 0) | ~valid[:, 1:]).all()), f"{what}: not ascending/unique"
            sel = torch.zeros_like(sc, dtype=torch.bool)
            sel.scatter_(1, torch.where(valid, ix, torch.zeros_like(ix)), valid)
            sink_end = torch.clamp(p + 1, max=S)
            win_lo = torch.maximum(sink_end, p - W + 1) if W > 0 else p + 1
            vis = pos[None, :] <= p
            forced = vis & ((pos[None, :] < sink_end) | (pos[None, :] >= win_lo))
            cand = vis & ~forced & torch.isfinite(sc)
            assert bool((sel[forced]).all()), f"{what}: forced set missing"
            assert not bool((sel & ~forced & ~cand).any()), f"{what}: selected a non-candidate"
            fill = sel & cand
            m = K - forced.sum(dim=1)
            want_n = torch.minimum(m, cand.sum(dim=1))
            assert torch.equal(fill.sum(dim=1), want_n), f"{what}: fill count"
            inf = torch.tensor(float("inf"), device=dev)
            smin = torch.where(fill, sc, inf).min(dim=1).values[:, None]
            out = cand & ~fill
            assert not bool((out & (sc > smin)).any()), f"{what}: a higher candidate was left out"
            tmax = torch.where(fill & (sc == smin), pos[None, :], torch.full_like(pos[None, :], -1)).max(dim=1).values
            assert not bool((out & (sc == smin) & (pos[None, :] < tmax[:, None])).any()), f"{what}: tie-break"
            rows += t1 - t0
    return rows
