"""Float64 numpy oracle of the LSA hot path (index -> select -> attend).

TEST INFRASTRUCTURE ONLY: used by tests/, the smoke check and the benchmark's
CPU baseline; never by the product path.  Shares no code with the HIP library.

Sources (page title, section):
  [P3]  "LongCat-2.0: how Meituan trained a 1.6T coding model without Nvidia GPUs"
        (molayo1419.me), section "The sparse attention problem at 1M tokens":
        LSA extends DeepSeek Sparse Attention with Streaming-aware Indexing (SI),
        Cross-Layer Indexing (CLI) and Hierarchical Indexing (HI); MTP extension.
  [P5]  "LongCat-Flash-Lite-Sparse" summary (aitrends.kr), sections "Good to know"
        and "Technical features": SI splits the selection budget into a fixed sink
        and a local sliding window; CLI reuses one index result in several adjacent
        layers; HI retrieves coarse candidate blocks, then selects fine tokens inside
        them, and can be switched on at inference without retraining.
  [P1]  "LongCat-2.0" summary (aitrends.kr), "Technical features": LSA avoids full
        attention over all token pairs and attends over a selected set.

Readings where the pages are silent (the pages give no formula at all):
  R1  indexer score I[t,s] = sum_h w[t,h] * ReLU(q[t,h] . k[s])  (DSA-style);
      fp8 keys are dequantised k = scale[s] * e4m3fn(byte).
  R3  the budget K includes sink and window; the rest is filled by top-k.
  R4  sink = positions [0, S); window = the W positions ending at p_t inclusive.
  R5  sink/window overlap is a union; fill = K - |forced|.
  R6  ties: the lower position wins (blocks: the lower block index wins).
  R7  output ascending, padded with -1.
  R9  HI ranks only complete, causally visible blocks holding at least one
      non-forced candidate; candidates of an incomplete visible block are always
      kept (empty whenever W >= block size - 1).
  R10 coarse block score = max over heads of w * ReLU(q . mean key of the block).
  R11 query t of T sits at p_t = ctx_len - T + t.
  R2/R16 one selection per query token shared by all heads; query head hq reads
      KV head hq // (Hq/Hkv).
  R15 MLA: one latent row per token; K = the whole row, V = its first d_v columns.
  R12 fp8 keys: per token scale = max(max|k|, 1e-12)/448, bytes = e4m3fn(clamp(k/scale)),
      round to nearest even, float32 arithmetic.
  R25 cache append: new tokens go to positions pos0 + t; a block's HI summary is the mean
      of its dequantised keys, brought up to date when the block's last row is written.
  R27 fp8-query indexer (an option of the token scores, fp8 keys only): each (token,
      head) query row is quantised as R12 quantises a key row, and the score is R1's
      with the dequantised rows.
  R28 backward of the sparse attention (training; [P3] describes LSA as trained, and
      its operators as deterministic): the gradient of the attention of R2/R16 with
      respect to q, K and V over the selected rows only, the selection held fixed;
      it takes the forward's output and log-sum-exp as inputs (D = dO . O and
      P = exp(z - lse)), and gradients of one row from several queries add up.
  R29 shared selection for draft tokens (MTP, [P3]): one index row per sequence serves
      its T query tokens; token t uses only the entries at positions <= its own p_t (R11),
      so no token attends to a later position.
  R30 indexer distillation target (training the indexer, DSA-style, which [P3] says LSA
      extends): for a query token, the target over its selected positions is the
      attention distribution averaged over the query heads; the indexer's distribution
      is the softmax of its scores over the same positions; the loss is KL(target ||
      indexer) and its gradient with respect to the scores is indexer - target (the
      target is held fixed).
"""
from __future__ import annotations

import numpy as np

NEG_INF = -np.inf


# ----------------------------------------------------------------------------- O1 decode

def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact: bf16 is the top half of an fp32)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def decode_e4m3fn(codes: np.ndarray) -> np.ndarray:
    """OCP fp8 E4M3 ("fn": no infinities) bytes -> float64, from the format definition.

    sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 is
    subnormal m * 2^-9; S.1111.111 is NaN; largest finite value 448.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = (1.0 + m / 8.0) * np.exp2(e - 7.0)
    sub = m * 2.0 ** -9
    val = np.where(e == 0, sub, normal)
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return np.where(sign == 1, -val, val)


def index_query_f64(qI_bits: np.ndarray, fp8_query: bool = False) -> np.ndarray:
    """Indexer query rows (bf16 bits [..., D]) -> float64 (R1).

    fp8_query (reading R27; the indexer the pages' LSA extends runs its contraction in
    fp8, [P3] "The sparse attention problem at 1M tokens"): every row (one token, one
    head) is quantised by R12's procedure, codes c and scale s_q, and enters the score
    as s_q * e4m3fn(c). Since ReLU(s x) = s ReLU(x) for s > 0, the score equals
    scale_k[s] * sum_h (w[h] * s_q[h]) * ReLU(c_h . c_k), the form an fp8 x fp8
    contraction computes.
    """
    q = decode_bf16(qI_bits)
    if not fp8_query:
        return q
    codes, scale = quantize_key_rows(q.astype(np.float32))
    return decode_e4m3fn(codes) * scale.astype(np.float64)[..., None]


def index_keys_f64(kI: np.ndarray, kI_scale) -> np.ndarray:
    """Indexer-key cache -> float64 keys: bf16 bits, or fp8 bytes times the per-token scale (R1)."""
    if kI_scale is None:
        return decode_bf16(kI)
    return decode_e4m3fn(kI) * np.asarray(kI_scale, dtype=np.float64)[..., None]


# ----------------------------------------------------------------------------- cache append
# The write side of a decode step. SI's window ends at the current token (reading R4), so a
# step's new rows are in the caches before it runs; HI's coarse pass reads one summary per
# block [P5 "technical features", third bullet], kept current as blocks fill (reading R25:
# a block's summary is the mean of its dequantised keys, written when its last row is).

def encode_e4m3fn(x: np.ndarray) -> np.ndarray:
    """Values -> OCP e4m3fn bytes: the nearest finite value of the format (magnitudes above
    448 take 448), ties to the code with an even mantissa; the sign bit follows the sign of
    x (-0.0 included). From the format definition: the candidates are the decoded
    non-negative finite codes 0x00..0x7E, which increase with the code."""
    x = np.asarray(x, dtype=np.float64)
    table = decode_e4m3fn(np.arange(0x7F, dtype=np.uint8))
    a = np.minimum(np.abs(x), table[-1])
    hi = np.clip(np.searchsorted(table, a, side="left"), 0, 0x7E)  # first value >= a
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = a - table[lo], table[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return code | (np.signbit(x).astype(np.uint8) << np.uint8(7))


def quantize_key_rows(k32: np.ndarray):
    """Reading R12 for one row per token, in float32 arithmetic (the precision the pages'
    fp8 caches are written in): scale = max(max|k|, 1e-12) / 448, bytes =
    e4m3fn(clamp(k / scale, +-448)). Returns (bytes uint8 [n, D], scale float32 [n])."""
    k32 = np.asarray(k32, dtype=np.float32)
    amax = np.max(np.abs(k32), axis=-1)
    scale = np.maximum(amax, np.float32(1e-12)) / np.float32(448.0)
    y = np.clip(k32 / scale[..., None], np.float32(-448.0), np.float32(448.0))
    return encode_e4m3fn(y), scale.astype(np.float32)


def cache_append(caches: dict, k_new32: np.ndarray, rows_new: list, pos0: np.ndarray, fp8: bool):
    """Write T new tokens per sequence at positions pos0[b] + t (positions outside [0, N)
    are skipped). caches: 'k' (uint8 fp8 codes or uint16 bf16 bits [B, N, D]), 'scale'
    (float32 [B, N], fp8 only), 'rows' (list of uint16 arrays [B, N, E]). k_new32: the new
    keys as float32 [B, T, D] (bf16 values); rows_new: uint16 [B, T, E] per row set.
    Returns the list of (b, position) written."""
    B, T, _ = k_new32.shape
    N = caches["k"].shape[1]
    written = []
    for b in range(B):
        for t in range(T):
            s = int(pos0[b]) + t
            if not 0 <= s < N:
                continue
            if fp8:
                code, sc = quantize_key_rows(k_new32[b, t][None])
                caches["k"][b, s] = code[0]
                caches["scale"][b, s] = sc[0]
            else:
                caches["k"][b, s] = (np.asarray(k_new32[b, t], np.float32).view(np.uint32) >> 16).astype(np.uint16)
            for rc, rn in zip(caches["rows"], rows_new):
                rc[b, s] = rn[b, t]
            written.append((b, s))
    return written


def completed_blocks(written, Bs: int, n_blocks: int):
    """Blocks whose last row was written: (b, j) with (s + 1) % Bs == 0, j = s // Bs < n_blocks."""
    return sorted({(b, s // Bs) for b, s in written if (s + 1) % Bs == 0 and s // Bs < n_blocks})


# ----------------------------------------------------------------------------- O2 positions

def query_positions(ctx_len: np.ndarray, T: int) -> np.ndarray:
    """p[b, t] = ctx_len[b] - T + t  (R11: the T queries are the last T visible rows)."""
    ctx = np.asarray(ctx_len, dtype=np.int64)
    return ctx[:, None] - T + np.arange(T, dtype=np.int64)[None, :]


# ----------------------------------------------------------------------------- O3 indexer

def indexer_scores(q: np.ndarray, w: np.ndarray, keys: np.ndarray, p: int) -> np.ndarray:
    """Token scores of one query token over keys[0:n] (R1, DSA-style indexer named in [P3]).

    q [H, D], w [H], keys [n, D] (float64).  I[s] = sum_h w[h] * max(0, q[h] . keys[s]).
    Positions s > p are not visible: -inf.
    """
    dots = keys @ np.asarray(q, dtype=np.float64).T            # [n, H]
    score = np.maximum(dots, 0.0) @ np.asarray(w, dtype=np.float64)
    n = keys.shape[0]
    if p + 1 < n:
        score = score.copy()
        score[p + 1:] = NEG_INF
    return score


def indexer_scores_at(q, w, keys_rows: np.ndarray) -> np.ndarray:
    """The same score for an explicit list of key rows (used on HI fine candidates)."""
    dots = keys_rows @ np.asarray(q, dtype=np.float64).T
    return np.maximum(dots, 0.0) @ np.asarray(w, dtype=np.float64)


# ----------------------------------------------------------------------------- O4-O6 SI select

def forced_positions(p: int, S: int, W: int) -> np.ndarray:
    """SI forced set [P5 'technical features', first bullet; R4, R5]:
    sink [0, S) and window [p-W+1, p], both clipped to [0, p], as a union."""
    sink = np.arange(0, min(S, p + 1), dtype=np.int64)
    win = np.arange(max(0, p - W + 1), p + 1, dtype=np.int64) if W > 0 else np.zeros(0, np.int64)
    return np.union1d(sink, win)


def top_fill(cand_pos: np.ndarray, cand_score: np.ndarray, m: int) -> np.ndarray:
    """The first m candidates in (score descending, position ascending) order (R6).
    All candidates when there are no more than m of them."""
    cand_pos = np.asarray(cand_pos, dtype=np.int64)
    if cand_pos.size <= m:
        return cand_pos
    order = np.lexsort((cand_pos, -np.asarray(cand_score, dtype=np.float64)))
    return cand_pos[order[:m]]


def pad_sorted(sel: np.ndarray, K: int) -> np.ndarray:
    """Ascending positions padded with -1 to length K (R7)."""
    out = np.full(K, -1, dtype=np.int64)
    s = np.sort(np.asarray(sel, dtype=np.int64))
    out[: s.size] = s
    return out


def select_tokens(scores: np.ndarray, p: int, K: int, S: int, W: int) -> np.ndarray:
    """Flat SI selection of one query token [P5 'good to know' and 'technical features'; R3-R7].

    scores [n] over positions 0..n-1 (-inf beyond p).  Forced F = sink U window;
    candidates C = [0, p] minus F; fill m = K - |F| from C by (score desc, pos asc).
    """
    if S + W > K:
        raise ValueError("sink + window exceed the budget")
    F = forced_positions(p, S, W)
    allpos = np.arange(p + 1, dtype=np.int64)
    C = np.setdiff1d(allpos, F, assume_unique=True)
    fill = top_fill(C, scores[C], K - F.size)
    return pad_sorted(np.concatenate([F, fill]), K)


# ----------------------------------------------------------------------------- O7 HI

def block_means(keys: np.ndarray, Bs: int, n_blocks: int) -> np.ndarray:
    """Mean key of each complete block j < n_blocks: (1/Bs) sum_{s in block j} k[s]
    [P3 HI paragraph: a fast block-level pass; R10].  keys [>= n_blocks*Bs, D] float64."""
    return keys[: n_blocks * Bs].reshape(n_blocks, Bs, keys.shape[1]).mean(axis=1)


def eligible_blocks(p: int, S: int, W: int, Bs: int, n_blocks: int) -> np.ndarray:
    """R9: complete, causally visible blocks (j*Bs + Bs - 1 <= p) that contain at least
    one non-forced candidate position."""
    F = forced_positions(p, S, W)
    n_vis = min(n_blocks, (p + 1) // Bs)
    ok = np.zeros(n_blocks, dtype=bool)
    for j in range(n_vis):
        lo, hi = j * Bs, j * Bs + Bs
        n_forced = np.count_nonzero((F >= lo) & (F < hi))
        ok[j] = n_forced < Bs
    return ok


def coarse_block_scores(q, w, kbar: np.ndarray, p: int, S: int, W: int, Bs: int) -> np.ndarray:
    """c[j] = max_h w[h] * ReLU(q[h] . kbar[j]) over eligible blocks, -inf elsewhere (R9, R10)."""
    dots = kbar @ np.asarray(q, dtype=np.float64).T                       # [NB, H]
    c = np.max(np.asarray(w, dtype=np.float64)[None, :] * np.maximum(dots, 0.0), axis=1)
    ok = eligible_blocks(p, S, W, Bs, kbar.shape[0])
    return np.where(ok, c, NEG_INF)


def keep_blocks(c: np.ndarray, n_keep: int) -> np.ndarray:
    """Coarse stage of HI [P5 'technical features', third bullet]: the n_keep eligible
    blocks with the highest coarse score, lower block index first on ties; ascending,
    -1 padded."""
    j = np.nonzero(np.isfinite(c))[0]
    kept = top_fill(j, c[j], n_keep)
    return pad_sorted(kept, n_keep)


def hi_candidates(p: int, S: int, W: int, Bs: int, kept: np.ndarray) -> np.ndarray:
    """Fine candidates C' = C restricted to the kept blocks, plus the candidates of the
    incomplete visible block (R9)."""
    F = forced_positions(p, S, W)
    kept = kept[kept >= 0]
    inside = (kept[:, None] * Bs + np.arange(Bs)[None, :]).reshape(-1)
    tail_lo = ((p + 1) // Bs) * Bs
    tail = np.arange(tail_lo, p + 1, dtype=np.int64)
    pool = np.union1d(inside, tail)
    pool = pool[pool <= p]
    return np.setdiff1d(pool, F, assume_unique=False)


def select_tokens_hi(q, w, keys: np.ndarray, kbar: np.ndarray, p: int, K: int, S: int,
                     W: int, Bs: int, n_keep: int):
    """Two-stage HI selection of one query token: coarse blocks, then fine top-k inside
    the kept blocks, plus the SI forced set.  Returns (idx [K], kept [n_keep],
    fine candidate positions, their scores)."""
    c = coarse_block_scores(q, w, kbar, p, S, W, Bs)
    kept = keep_blocks(c, n_keep)
    cand = hi_candidates(p, S, W, Bs, kept)
    sc = indexer_scores_at(q, w, keys[cand]) if cand.size else np.zeros(0)
    F = forced_positions(p, S, W)
    fill = top_fill(cand, sc, K - F.size)
    return pad_sorted(np.concatenate([F, fill]), K), kept, cand, sc


def select_fine_given_kept(q, w, keys, kept, p, K, S, W, Bs):
    """Fine stage alone, for a given kept list (stage-wise checking of a GPU kept list)."""
    cand = hi_candidates(p, S, W, Bs, np.asarray(kept))
    sc = indexer_scores_at(q, w, keys[cand]) if cand.size else np.zeros(0)
    F = forced_positions(p, S, W)
    fill = top_fill(cand, sc, K - F.size)
    return pad_sorted(np.concatenate([F, fill]), K), cand, sc


# ----------------------------------------------------------------------------- O8 attention

def attend(q: np.ndarray, k_rows: np.ndarray, v_rows: np.ndarray, idx: np.ndarray, tau: float):
    """Softmax attention of one query token over the selected rows only [P1 'technical
    features': no attention over all token pairs; R2, R16].

    q [Hq, d_qk]; k_rows [N, Hkv, d_qk]; v_rows [N, Hkv, d_v] (float64); idx [K] with
    -1 padding.  z_s = tau * q[hq] . K[s, hq // g]; o = sum_s softmax(z)_s V[s, hq // g];
    lse = log sum_s exp(z_s).  Returns (o [Hq, d_v], lse [Hq]).
    """
    sel = np.asarray(idx, dtype=np.int64)
    sel = sel[sel >= 0]
    Hq = q.shape[0]
    Hkv = k_rows.shape[1]
    g = Hq // Hkv
    o = np.zeros((Hq, v_rows.shape[2]))
    lse = np.full(Hq, NEG_INF)
    if sel.size == 0:
        return o, lse
    for kvh in range(Hkv):
        Ks = k_rows[sel, kvh, :]                       # [n, d_qk]
        Vs = v_rows[sel, kvh, :]                       # [n, d_v]
        qs = q[kvh * g:(kvh + 1) * g]                  # [g, d_qk]
        z = tau * (qs @ Ks.T)                          # [g, n]
        zmax = z.max(axis=1, keepdims=True)
        e = np.exp(z - zmax)
        den = e.sum(axis=1, keepdims=True)
        o[kvh * g:(kvh + 1) * g] = (e @ Vs) / den
        lse[kvh * g:(kvh + 1) * g] = (zmax + np.log(den))[:, 0]
    return o, lse


def attend_backward(q, k_rows, v_rows, idx, tau, out, lse, dout):
    """Gradient of attend() for one query token (R28): the selection is a fixed input.

    q [Hq, d_qk], k_rows [N, Hkv, d_qk], v_rows [N, Hkv, d_v], idx [K] (-1 padding), out
    [Hq, d_v] and lse [Hq] from the forward, dout [Hq, d_v]; float64 throughout. With
    z_s = tau q . K_s, P_s = exp(z_s - lse), dP_s = dout . V_s, D = dout . out and
    dS_s = P_s (dP_s - D) (the softmax Jacobian applied to dP):
      dq = tau sum_s dS_s K_s;  dK_s = tau sum_h dS_s q_h;  dV_s = sum_h P_s dout_h
    where the KV sums run over the query heads of that KV head.
    Returns (dq [Hq, d_qk], dK [N, Hkv, d_qk], dV [N, Hkv, d_v]); rows not selected are 0.
    """
    sel = np.asarray(idx, dtype=np.int64)
    sel = sel[sel >= 0]
    Hq, dqk = q.shape
    N, Hkv = k_rows.shape[0], k_rows.shape[1]
    g = Hq // Hkv
    dq = np.zeros((Hq, dqk))
    dK = np.zeros((N, Hkv, dqk))
    dV = np.zeros((N, Hkv, v_rows.shape[2]))
    if sel.size == 0:
        return dq, dK, dV
    for kvh in range(Hkv):
        hs = slice(kvh * g, (kvh + 1) * g)
        Ks, Vs = k_rows[sel, kvh, :], v_rows[sel, kvh, :]       # [n, d]
        P = np.exp(tau * (q[hs] @ Ks.T) - lse[hs, None])         # [g, n]
        dP = dout[hs] @ Vs.T                                     # [g, n]
        D = np.sum(dout[hs] * out[hs], axis=1, keepdims=True)    # [g, 1]
        dS = P * (dP - D)
        dq[hs] = tau * (dS @ Ks)
        dK[sel, kvh, :] = tau * (dS.T @ q[hs])
        dV[sel, kvh, :] = P.T @ dout[hs]
    return dq, dK, dV


def mla_row_grad(dK, dV):
    """R15 under R28: an MLA latent row is both K and (its first d_v columns) V, so its
    gradient is dK plus dV on the first d_v columns."""
    d = dK.copy()
    d[..., : dV.shape[-1]] += dV
    return d


def indexer_target(q, k_rows, idx, tau, lse):
    """R30 target of one query token: p[j] = (1/Hq) sum_h exp(tau q_h . K[idx[j], kvh(h)] -
    lse_h) for valid entries j of idx (0 for padding). q [Hq, d_qk], k_rows [N, Hkv, d_qk],
    lse [Hq] from the forward. Returns float64 [K]."""
    idx = np.asarray(idx, dtype=np.int64)
    Hq, Hkv = q.shape[0], k_rows.shape[1]
    g = Hq // Hkv
    p = np.zeros(idx.size)
    ok = idx >= 0
    if not ok.any():
        return p
    sel = idx[ok]
    acc = np.zeros(sel.size)
    for h in range(Hq):
        z = tau * (k_rows[sel, h // g, :] @ q[h])
        acc += np.exp(z - lse[h])
    p[ok] = acc / Hq
    return p


def indexer_kl(target, scores_sel, valid):
    """R30 loss and gradient of one query token: u = softmax of the indexer scores over
    the valid entries; loss = sum_j target_j (log target_j - log u_j) over target_j > 0;
    d loss / d score_j = u_j - target_j (0 at invalid entries). Returns (loss, grad [K])."""
    target = np.asarray(target, dtype=np.float64)
    sc = np.asarray(scores_sel, dtype=np.float64)
    valid = np.asarray(valid, dtype=bool)
    grad = np.zeros(sc.size)
    if not valid.any():
        return 0.0, grad
    m = np.max(sc[valid])
    e = np.exp(sc[valid] - m)
    logu = (sc[valid] - m) - np.log(e.sum())
    u = np.exp(logu)
    t = target[valid]
    pos = t > 0
    loss = float(np.sum(t[pos] * (np.log(t[pos]) - logu[pos])))
    grad[valid] = u - t
    return loss, grad


def shared_selection_rows(idx_row, ctx: int, T: int) -> np.ndarray:
    """R29: the per-token index rows of one shared selection. Token t sits at
    p_t = ctx - T + t (R11) and keeps the entries s <= p_t; the rest become -1 (the
    entries ascend, so the kept ones stay first). Returns int64 [T, K]."""
    row = np.asarray(idx_row, dtype=np.int64)
    out = np.empty((T, row.size), dtype=np.int64)
    for t in range(T):
        p = ctx - T + t
        keep = row[(row >= 0) & (row <= p)]
        out[t] = -1
        out[t, : keep.size] = keep
    return out


def mla_kv(rows: np.ndarray, d_v: int):
    """R15: MLA latent rows [N, 1, d_qk] -> (K rows, V rows = first d_v columns)."""
    return rows, rows[..., :d_v]


# ----------------------------------------------------------------------------- pipeline

def reference_step(inp: dict, rows=None, layers=None, with_attend: bool = True) -> dict:
    """Run the whole path for the (b, t) pairs in ``rows`` (default: all).

    CLI [P3 CLI paragraph; P5 'technical features', second bullet]: the selection is
    computed once per query token and reused by every layer; each layer attends with
    its own q/K/V.  Returns dict with per-row idx (and kept for HI), out [L][...],
    lse [L][...], plus flat scores (non-HI) keyed by (b, t).
    """
    cfg = inp["cfg"]
    B, T = cfg.B, cfg.T
    P = query_positions(inp["ctx_len"], T)
    if rows is None:
        rows = [(b, t) for b in range(B) for t in range(T)]
    L = cfg.layers if layers is None else layers
    if cfg.hi and getattr(cfg, "q_fp8", False):
        raise NotImplementedError("R27 covers the token scores; the coarse block pass keeps bf16 queries")
    res = {"idx": {}, "kept": {}, "scores": {}, "cand": {}, "out": {}, "lse": {}}
    by_b = {}
    for b, t in rows:
        by_b.setdefault(b, []).append(t)
    for b, ts in by_b.items():
        keys = index_keys_f64(inp["kI"][b], None if inp["kI_scale"] is None else inp["kI_scale"][b])
        kbar = block_means(keys, cfg.Bs, int(inp["ctx_len"][b]) // cfg.Bs) if cfg.hi else None
        kv = {}
        for t in ts:
            p = int(P[b, t])
            qI = index_query_f64(inp["qI"][b, t], getattr(cfg, "q_fp8", False))
            w = np.asarray(inp["w"][b, t], dtype=np.float64)
            if cfg.hi:
                idx, kept, cand, sc = select_tokens_hi(qI, w, keys, kbar, p, cfg.K, cfg.S,
                                                       cfg.W, cfg.Bs, cfg.n_keep)
                res["kept"][(b, t)] = kept
                res["cand"][(b, t)] = (cand, sc)
            else:
                sc = indexer_scores(qI, w, keys[: p + 1], p)
                idx = select_tokens(sc, p, cfg.K, cfg.S, cfg.W)
                res["scores"][(b, t)] = sc
            res["idx"][(b, t)] = idx
            if not with_attend:
                continue
            for layer in range(L):
                if layer not in kv:
                    kv[layer] = _layer_kv(inp, cfg, layer, b)
                k_rows, v_rows = kv[layer]
                q = decode_bf16(inp["q"][layer, b, t])
                o, lse = attend(q, k_rows, v_rows, idx, cfg.tau)
                res["out"][(layer, b, t)] = o
                res["lse"][(layer, b, t)] = lse
    return res


class _LazyRows:
    """Decode KV rows on first access (full caches at 1M context are large in float64).

    rows[sel, h, :] decodes the selected rows of head h; rows[..., cols] (a column slice)
    returns the same lazy rows restricted to those columns, so that mla_kv can take the
    value columns of latent rows without decoding the whole cache."""

    def __init__(self, bits: np.ndarray, cols: slice = slice(None)):
        self.bits = bits
        self.cols = cols
        n = len(range(*cols.indices(bits.shape[-1])))
        self.shape = bits.shape[:-1] + (n,)

    def __getitem__(self, key):
        if isinstance(key, tuple) and len(key) == 2 and key[0] is Ellipsis and isinstance(key[1], slice):
            if self.cols != slice(None):
                raise NotImplementedError("one column slice of the raw rows")
            return _LazyRows(self.bits, key[1])
        sel, h, sl = key
        rows = decode_bf16(self.bits[sel, h, :])[..., self.cols]
        return rows[..., sl]


def _layer_kv(inp, cfg, layer, b):
    if cfg.mla:
        return mla_kv(_LazyRows(inp["k"][layer, b]), cfg.d_v)
    return _LazyRows(inp["k"][layer, b]), _LazyRows(inp["v"][layer, b])
