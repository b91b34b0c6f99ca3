"""Planted mistakes in the oracle (CPU only) must each be caught by a pin.

Each mutant replaces one oracle step with a plausible wrong version (dropped term,
wrong sign or index, off-by-one window, reversed tie-break, wrong reduction, wrong
head mapping) and runs the pins that should fail on it.
"""
import numpy as np
import pytest

from oracle import lsa_oracle as O
import test_oracle_pins as pins


def _run_pins(names):
    """True when at least one named pin fails."""
    for name in names:
        fn = getattr(pins, name)
        try:
            if name in ("test_indexer_matches_brute_force", "test_selection_matches_rank_counting",
                        "test_selection_invariants", "test_hi_matches_brute_force",
                        "test_budget_covers_context_equals_dense_causal",
                        "test_hi_all_blocks_kept_equals_flat",
                        "test_selection_without_forced_is_lexsort_and_partition",
                        "test_fine_given_all_eligible_kept_equals_flat"):
                for seed in range(4):
                    fn(seed)
            elif name == "test_attention_backward_matches_autograd":
                fn(6, 1, 24, 16, True)  # the MLA case (one latent row is both K and V)
                fn(8, 2, 16, 16, False)
            else:
                fn()
        except (AssertionError, ValueError, IndexError):
            return True
    return False


ALL = ["test_golden_hand_worked_flat_and_hi", "test_indexer_single_head_is_relu_dot",
       "test_indexer_matches_brute_force", "test_selection_invariants",
       "test_selection_matches_rank_counting", "test_selection_without_forced_is_lexsort_and_partition",
       "test_hi_matches_brute_force", "test_hi_all_blocks_kept_equals_flat",
       "test_budget_covers_context_equals_dense_causal", "test_attention_closed_forms",
       "test_attention_permutation_invariant_and_gqa_mapping", "test_e4m3fn_matches_torch_all_codes",
       "test_fp8_query_worked_example", "test_fp8_query_exact_for_representable_rows",
       "test_fp8_query_error_bound_rows_and_scaling", "test_fp8_query_score_is_the_fp8_contraction",
       "test_attention_backward_finite_differences", "test_attention_backward_closed_forms",
       "test_query_positions_hand_worked", "test_reference_step_positions_are_causal_prefixes",
       "test_reference_step_mla_one_selected_row_is_its_value_prefix", "test_reference_step_mla_dense_matches_sdpa",
       "test_fine_given_all_eligible_kept_equals_flat", "test_fine_given_kept_hand_worked",
       "test_e4m3fn_encode_round_trips_every_finite_code", "test_e4m3fn_encode_ties_to_even_and_saturation",
       "test_quantize_key_rows_scale_and_extremes", "test_cache_append_positions_rows_and_completed_blocks",
       "test_hi_recovers_planted_blocks", "test_attention_backward_matches_autograd",
       "test_shared_selection_rows_worked_example", "test_indexer_target_is_head_mean_of_attention",
       "test_indexer_kl_zero_minimum_and_finite_differences", "test_hi_candidates_hand_worked",
       "test_bf16_decode_matches_torch", "test_fp8_dequant_scale_multiplies"]


def _no_relu(q, w, keys, p):
    s = (keys @ q.T) @ w
    s = s.copy()
    s[p + 1:] = -np.inf
    return s


def _max_heads(q, w, keys, p):
    s = np.max(np.maximum(keys @ q.T, 0.0) * w[None, :], axis=1)
    s = s.copy()
    s[p + 1:] = -np.inf
    return s


def _window_exclusive(p, S, W):
    sink = np.arange(0, min(S, p + 1))
    win = np.arange(max(0, p - W), p) if W > 0 else np.zeros(0, np.int64)
    return np.union1d(sink, win).astype(np.int64)


def _ties_high(cand_pos, cand_score, m):
    cand_pos = np.asarray(cand_pos, dtype=np.int64)
    if cand_pos.size <= m:
        return cand_pos
    order = np.lexsort((-cand_pos, -np.asarray(cand_score)))
    return cand_pos[order[:m]]


def _coarse_sum(q, w, kbar, p, S, W, Bs):
    c = np.sum(w[None, :] * np.maximum(kbar @ q.T, 0.0), axis=1)
    ok = O.eligible_blocks(p, S, W, Bs, kbar.shape[0])
    return np.where(ok, c, -np.inf)


def _eligible_all(p, S, W, Bs, n_blocks):
    ok = np.zeros(n_blocks, dtype=bool)
    ok[: min(n_blocks, (p + 1) // Bs)] = True
    return ok


_real_attend = O.attend


def _attend_no_tau(q, k_rows, v_rows, idx, tau):
    return _real_attend(q, k_rows, v_rows, idx, 1.0)


def _attend_modulo_heads(q, k_rows, v_rows, idx, tau):
    Hq, Hkv = q.shape[0], k_rows.shape[1]
    o = np.zeros((Hq, v_rows.shape[2]))
    lse = np.zeros(Hq)
    for hq in range(Hq):
        oo, ll = _real_attend(q[hq:hq + 1], k_rows[:, hq % Hkv:hq % Hkv + 1],
                              v_rows[:, hq % Hkv:hq % Hkv + 1], idx, tau)
        o[hq], lse[hq] = oo[0], ll[0]
    return o, lse


def _e4m3_bias8(codes):
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    e, m = (c >> 3) & 0xF, c & 7
    val = np.where(e == 0, m * 2.0 ** -9, (1 + m / 8) * np.exp2(e - 8.0))
    return np.where((c >> 7) == 1, -val, val)


def _query_no_scale(qI_bits, fp8_query=False):
    q = O.decode_bf16(qI_bits)
    if not fp8_query:
        return q
    codes, _ = O.quantize_key_rows(q.astype(np.float32))
    return O.decode_e4m3fn(codes)


def _query_shared_scale(qI_bits, fp8_query=False):
    # one scale for the whole query (all heads) instead of one per row
    q = O.decode_bf16(qI_bits)
    if not fp8_query:
        return q
    s = np.float32(max(np.abs(q).max(), 1e-12)) / np.float32(448.0)
    y = np.clip(q.astype(np.float32) / s, -448.0, 448.0)
    return O.decode_e4m3fn(O.encode_e4m3fn(y)) * np.float64(s)


_real_bwd = O.attend_backward


def _bwd_no_delta(q, k_rows, v_rows, idx, tau, out, lse, dout):
    # the softmax Jacobian without its rank-one term (D = 0)
    return _real_bwd(q, k_rows, v_rows, idx, tau, np.zeros_like(out), lse, dout)


def _bwd_dk_without_tau(q, k_rows, v_rows, idx, tau, out, lse, dout):
    dq, dK, dV = _real_bwd(q, k_rows, v_rows, idx, tau, out, lse, dout)
    return dq, dK / tau, dV


def _positions_reversed(ctx_len, T):
    # token t at ctx - 1 - t: the right set of positions in the wrong token order
    ctx = np.asarray(ctx_len, dtype=np.int64)
    return ctx[:, None] - 1 - np.arange(T, dtype=np.int64)[None, :]


def _mla_value_last_columns(rows, d_v):
    # V taken from the last d_v columns of the latent row instead of the first
    return rows, rows[..., rows.shape[-1] - d_v:]


_real_fine = O.select_fine_given_kept


def _fine_block_offset(q, w, keys, kept, p, K, S, W, Bs):
    # kept block j read as the block after it
    kept = np.asarray(kept)
    return _real_fine(q, w, keys, np.where(kept >= 0, kept + 1, kept), p, K, S, W, Bs)


_real_table = O.decode_e4m3fn


def _e4m3_encode_truncate(x):
    # magnitudes rounded toward zero instead of to the nearest code
    x = np.asarray(x, dtype=np.float64)
    table = _real_table(np.arange(0x7F, dtype=np.uint8))
    a = np.minimum(np.abs(x), table[-1])
    code = np.clip(np.searchsorted(table, a, side="right") - 1, 0, 0x7E).astype(np.uint8)
    return code | (np.signbit(x).astype(np.uint8) << np.uint8(7))


_real_encode = O.encode_e4m3fn


def _quantize_scale_240(k32):
    # the scale taken against 240 (the e4m3fnuz maximum) instead of 448
    k32 = np.asarray(k32, dtype=np.float32)
    scale = np.maximum(np.max(np.abs(k32), axis=-1), np.float32(1e-12)) / np.float32(240.0)
    y = np.clip(k32 / scale[..., None], np.float32(-448.0), np.float32(448.0))
    return _real_encode(y), scale.astype(np.float32)


_real_append = O.cache_append


def _append_one_late(caches, k_new32, rows_new, pos0, fp8):
    # token t written at pos0 + t + 1
    return _real_append(caches, k_new32, rows_new, np.asarray(pos0) + 1, fp8)


def _completed_first_row(written, Bs, n_blocks):
    # a block counted complete when its first row is written
    return sorted({(b, s // Bs) for b, s in written if s % Bs == 0 and s // Bs < n_blocks})


_real_keep = O.keep_blocks


def _keep_one_fewer(c, n_keep):
    # one block fewer than n_keep kept (the last one dropped)
    kept = _real_keep(c, n_keep)
    n = int(np.count_nonzero(kept >= 0))
    if n:
        kept = kept.copy()
        kept[n - 1] = -1
    return kept


_real_hi_cand = O.hi_candidates


def _hi_cand_no_tail(p, S, W, Bs, kept):
    # the incomplete visible block's candidates left out
    c = _real_hi_cand(p, S, W, Bs, kept)
    return c[c < ((p + 1) // Bs) * Bs]


def _mla_grad_without_dv(dK, dV):
    # the value part of the latent row's gradient dropped
    return dK.copy()


def _shared_rows_strict(idx_row, ctx, T):
    # token t keeps only the entries before its own position
    row = np.asarray(idx_row, dtype=np.int64)
    out = np.full((T, row.size), -1, dtype=np.int64)
    for t in range(T):
        keep = row[(row >= 0) & (row < ctx - T + t)]
        out[t, : keep.size] = keep
    return out


_real_target = O.indexer_target


def _target_head_sum(q, k_rows, idx, tau, lse):
    # summed over the heads instead of averaged
    return _real_target(q, k_rows, idx, tau, lse) * q.shape[0]


_real_kl = O.indexer_kl


def _kl_grad_sign(target, scores_sel, valid):
    # gradient target - u instead of u - target
    loss, grad = _real_kl(target, scores_sel, valid)
    return loss, -grad


def _block_means_shifted(keys, Bs, n_blocks):
    # the mean of each block taken one row late
    k = np.vstack([keys[1:], keys[-1:]])
    return k[: n_blocks * Bs].reshape(n_blocks, Bs, keys.shape[1]).mean(axis=1)


_real_keys = O.index_keys_f64


def _keys_without_scale(kI, kI_scale):
    # fp8 codes used without their per-token scale
    return _real_keys(kI, None if kI_scale is None else np.ones_like(np.asarray(kI_scale)))


def _bf16_low_half(bits):
    # the bits placed one position too low in the fp32 word
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(15)
    return u.view(np.float32).astype(np.float64)


def _pad_with_zero(sel, K):
    # padding with position 0 instead of -1
    out = np.zeros(K, dtype=np.int64)
    s = np.sort(np.asarray(sel, dtype=np.int64))
    out[: s.size] = s
    return out


MUTANTS = [
    ("indexer_scores", _no_relu),
    ("indexer_scores", _max_heads),
    ("forced_positions", _window_exclusive),
    ("top_fill", _ties_high),
    ("coarse_block_scores", _coarse_sum),
    ("eligible_blocks", _eligible_all),
    ("attend", _attend_no_tau),
    ("attend", _attend_modulo_heads),
    ("decode_e4m3fn", _e4m3_bias8),
    ("index_query_f64", _query_no_scale),
    ("index_query_f64", _query_shared_scale),
    ("attend_backward", _bwd_no_delta),
    ("attend_backward", _bwd_dk_without_tau),
    ("query_positions", _positions_reversed),
    ("mla_kv", _mla_value_last_columns),
    ("select_fine_given_kept", _fine_block_offset),
    ("encode_e4m3fn", _e4m3_encode_truncate),
    ("quantize_key_rows", _quantize_scale_240),
    ("cache_append", _append_one_late),
    ("completed_blocks", _completed_first_row),
    ("keep_blocks", _keep_one_fewer),
    ("hi_candidates", _hi_cand_no_tail),
    ("mla_row_grad", _mla_grad_without_dv),
    ("shared_selection_rows", _shared_rows_strict),
    ("indexer_target", _target_head_sum),
    ("indexer_kl", _kl_grad_sign),
    ("block_means", _block_means_shifted),
    ("index_keys_f64", _keys_without_scale),
    ("decode_bf16", _bf16_low_half),
    ("pad_sorted", _pad_with_zero),
]


@pytest.mark.parametrize("name,fn", MUTANTS, ids=[f"{n}:{f.__name__}" for n, f in MUTANTS])
def test_mutant_is_caught(monkeypatch, name, fn):
    monkeypatch.setattr(O, name, fn)
    assert _run_pins(ALL), f"no pin caught the planted mistake in {name}"


def test_unmutated_oracle_passes_battery():
    assert not _run_pins(ALL)
