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
                        "test_selection_without_forced_is_lexsort_and_partition"):
                for seed in range(4):
                    fn(seed)
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
       "test_attention_backward_finite_differences", "test_attention_backward_closed_forms"]


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
]


@pytest.mark.parametrize("name,fn", MUTANTS, ids=[f"{n}:{f.__name__}" for n, f in MUTANTS])
def test_mutant_is_caught(monkeypatch, name, fn):
    monkeypatch.setattr(O, name, fn)
    assert _run_pins(ALL), f"no pin caught the planted mistake in {name}"


def test_unmutated_oracle_passes_battery():
    assert not _run_pins(ALL)
