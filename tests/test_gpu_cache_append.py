"""lsa_cache_append on the GPU against the oracle's cache append (reading R12 quantisation,
reading R25 positions and block summaries).

Bit-exact: the fp8 key bytes and per-token scales (both sides quantise in fp32 with
correctly rounded divisions and round-to-nearest-even), the copied bf16 rows, and the
positions left untouched. The block summaries of completed blocks equal lsa_block_means
over the same cache byte for byte, and the oracle's float64 block means within fp32
summation error. Cases: fp8 and bf16 key caches, D = 64 and 128, an MLA row set and a
K/V pair, positions past the cache end (skipped), pos0 = NULL (the last T rows),
appends that complete several blocks, and a token-by-token decode loop against one bulk
append.
"""
import numpy as np
import pytest
import torch

import long_context_sparse_07_amd as L
from oracle import lsa_oracle as O

pytestmark = pytest.mark.gpu


def _bf16_keys(rng, shape, tiny_rows=()):
    k = (rng.standard_normal(shape) / np.sqrt(shape[-1])).astype(np.float32)
    k.reshape(-1, shape[-1])[list(tiny_rows)] *= 1e-3  # rows whose codes are mostly subnormal
    kt = torch.from_numpy(k).to(torch.bfloat16)
    return kt, kt.to(torch.float32).numpy()


def _rows(rng, shape):
    return torch.from_numpy(rng.integers(0, 1 << 16, shape, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)


def _append_both(rng, B, N, D, T, pos0, fp8, row_shapes, kbar_blocks=0, Bs=64, prefill=None):
    """GPU append into caches (optionally prefilled) and the oracle on host copies."""
    k_new, k32 = _bf16_keys(rng, (B, T, D), tiny_rows=(0,))
    rows_new = [_rows(rng, (B, T) + rs) for rs in row_shapes]
    if prefill is None:
        kc = np.zeros((B, N, D), np.uint8 if fp8 else np.uint16)
        sc = np.zeros((B, N), np.float32)
        rcs = [np.zeros((B, N) + rs, np.uint16) for rs in row_shapes]
    else:
        kc, sc, rcs = prefill
    g_k = torch.from_numpy(kc.copy()).cuda()
    g_k = g_k.view(torch.float8_e4m3fn) if fp8 else g_k.view(torch.int16).view(torch.bfloat16)
    g_s = torch.from_numpy(sc.copy()).cuda()
    g_rows = [torch.from_numpy(r.copy().view(np.int16)).cuda().view(torch.bfloat16) for r in rcs]
    g_kbar = torch.full((B, max(kbar_blocks, 1), D), -7.0, dtype=torch.float32, device="cuda") if kbar_blocks else None
    g_pos0 = torch.tensor(pos0, dtype=torch.int32, device="cuda") if pos0 is not None else None
    L.lsa_cache_append(k_new.cuda(), g_k, k_scale=g_s if fp8 else None,
                       rows=[(rn.cuda(), gr) for rn, gr in zip(rows_new, g_rows)], pos0=g_pos0, kbar=g_kbar,
                       block_size=Bs)
    torch.cuda.synchronize()
    caches = {"k": kc.copy(), "scale": sc.copy(), "rows": [r.copy() for r in rcs]}
    p0 = np.array(pos0) if pos0 is not None else np.full(B, N - T)
    written = O.cache_append(caches, k32, [r.view(torch.int16).numpy().view(np.uint16) for r in rows_new], p0, fp8)
    gk = g_k.view(torch.uint8).cpu().numpy() if fp8 else g_k.view(torch.int16).cpu().numpy().view(np.uint16)
    got = {"k": gk, "scale": g_s.cpu().numpy(),
           "rows": [r.view(torch.int16).cpu().numpy().view(np.uint16) for r in g_rows]}
    return got, caches, written, (g_k, g_s, g_kbar)


def _assert_same(got, want, fp8):
    assert np.array_equal(got["k"], want["k"]), f"{np.count_nonzero(got['k'] != want['k'])} key bytes differ"
    if fp8:
        assert np.array_equal(got["scale"], want["scale"])
    for g, w in zip(got["rows"], want["rows"]):
        assert np.array_equal(g, w)


@pytest.mark.parametrize("fp8,D", [(True, 128), (True, 64), (False, 128), (False, 64)])
def test_append_matches_oracle(fp8, D):
    rng = np.random.default_rng(40 + D + fp8)
    B, N, T = 3, 300, 5
    pos0 = [0, 37, 298]  # sequence 2: its last three tokens fall past the end and are skipped
    got, want, written, _ = _append_both(rng, B, N, D, T, pos0, fp8, [(576,), (4, 128)])
    assert len(written) == 5 + 5 + 2
    _assert_same(got, want, fp8)


def test_pos0_null_appends_the_last_rows():
    rng = np.random.default_rng(41)
    got, want, written, _ = _append_both(rng, 2, 128, 128, 3, None, True, [(576,)])
    assert [s for _, s in written] == [125, 126, 127] * 2
    _assert_same(got, want, True)


def test_quantisation_extremes():
    # a zero key row (scale from the 1e-12 floor), a row with one large value (most codes
    # subnormal or zero) and a row of equal magnitudes (every code +-448)
    B, T, D, N = 1, 3, 128, 16
    k = np.zeros((B, T, D), np.float32)
    k[0, 1, 5] = 3.0
    k[0, 1, 6:] = 1e-4
    k[0, 2] = np.where(np.arange(D) % 2 == 0, 0.5, -0.5)
    k_new = torch.from_numpy(k).to(torch.bfloat16)
    k32 = k_new.to(torch.float32).numpy()
    g_k = torch.zeros((B, N, D), dtype=torch.uint8, device="cuda").view(torch.float8_e4m3fn)
    g_s = torch.zeros((B, N), dtype=torch.float32, device="cuda")
    L.lsa_cache_append(k_new.cuda(), g_k, k_scale=g_s, pos0=torch.zeros(B, dtype=torch.int32, device="cuda"))
    codes, scale = O.quantize_key_rows(k32[0])
    assert np.array_equal(g_k.view(torch.uint8).cpu().numpy()[0, :T], codes)
    assert np.array_equal(g_s.cpu().numpy()[0, :T], scale)
    assert np.all((codes[2] & 0x7F) == 0x7E)


def test_block_summaries_of_completed_blocks():
    rng = np.random.default_rng(42)
    B, N, D, Bs, nb = 2, 512, 128, 64, 8
    # a prefilled cache (rows 0..199 of sequence 0, 0..127 of sequence 1)
    k_all, k32_all = _bf16_keys(rng, (B, N, D))
    kc = np.zeros((B, N, D), np.uint8)
    sc = np.zeros((B, N), np.float32)
    for b, n in ((0, 200), (1, 128)):
        kc[b, :n], sc[b, :n] = O.quantize_key_rows(k32_all[b, :n])
    # 150 new tokens: sequence 0 fills rows 200..349 (completes blocks 3 and 4), sequence 1
    # rows 128..277 (completes blocks 2 and 3)
    got, want, written, (g_k, g_s, g_kbar) = _append_both(rng, B, N, D, 150, [200, 128], True, [], kbar_blocks=nb,
                                                          Bs=Bs, prefill=(kc, sc, []))
    _assert_same(got, want, True)
    done = O.completed_blocks(written, Bs, nb)
    assert done == [(0, 3), (0, 4), (1, 2), (1, 3)]
    ref = L.lsa_block_means(g_k, Bs, k_scale=g_s, n_blocks=nb).cpu().numpy()
    kbar = g_kbar.cpu().numpy()
    keys = O.index_keys_f64(want["k"], want["scale"])
    for b in range(B):
        for j in range(nb):
            if (b, j) in done:
                assert np.array_equal(kbar[b, j], ref[b, j])  # same bytes as the summary kernel
                exact = O.block_means(keys[b], Bs, nb)[j]
                assert np.allclose(kbar[b, j], exact, rtol=1e-5, atol=1e-6)
            else:
                assert np.all(kbar[b, j] == -7.0)  # untouched


def test_token_by_token_equals_bulk():
    rng = np.random.default_rng(43)
    B, N, D, T, Bs, nb = 2, 256, 128, 70, 32, 8
    k_new, _ = _bf16_keys(rng, (B, T, D))
    rows_new = _rows(rng, (B, T, 576))
    pos0 = torch.tensor([10, 100], dtype=torch.int32, device="cuda")

    def fresh():
        return (torch.zeros((B, N, D), dtype=torch.uint8, device="cuda").view(torch.float8_e4m3fn),
                torch.zeros((B, N), dtype=torch.float32, device="cuda"),
                torch.zeros((B, N, 576), dtype=torch.bfloat16, device="cuda"),
                torch.zeros((B, nb, D), dtype=torch.float32, device="cuda"))
    bulk = fresh()
    L.lsa_cache_append(k_new.cuda(), bulk[0], k_scale=bulk[1], rows=[(rows_new.cuda(), bulk[2])], pos0=pos0,
                       kbar=bulk[3], block_size=Bs)
    step = fresh()
    for t in range(T):
        L.lsa_cache_append(k_new[:, t:t + 1].contiguous().cuda(), step[0], k_scale=step[1],
                           rows=[(rows_new[:, t:t + 1].contiguous().cuda(), step[2])], pos0=pos0 + t,
                           kbar=step[3], block_size=Bs)
    torch.cuda.synchronize()
    assert torch.equal(bulk[0].view(torch.uint8), step[0].view(torch.uint8))
    assert torch.equal(bulk[1], step[1])
    assert torch.equal(bulk[2].view(torch.int16), step[2].view(torch.int16))
    assert torch.equal(bulk[3], step[3])


def test_append_full_size_cache_shapes():
    # the two cache shapes the benchmark times: 8 sequences of 131072 rows (fp8 key of 128
    # plus a 576-wide MLA row, one token each) and one sequence of 1M rows (bf16 key of 64,
    # a 128-wide row, four tokens completing a block of 64 with its summary)
    rng = np.random.default_rng(45)
    # 128K fp8
    B, N, D = 8, 131072, 128
    k_new, k32 = _bf16_keys(rng, (B, 1, D))
    row_new = _rows(rng, (B, 1, 576))
    pos0 = rng.integers(0, N, B).astype(np.int32)
    g_k = torch.zeros((B, N, D), dtype=torch.uint8, device="cuda").view(torch.float8_e4m3fn)
    g_s = torch.zeros((B, N), dtype=torch.float32, device="cuda")
    g_r = torch.zeros((B, N, 576), dtype=torch.bfloat16, device="cuda")
    L.lsa_cache_append(k_new.cuda(), g_k, k_scale=g_s, rows=[(row_new.cuda(), g_r)],
                       pos0=torch.from_numpy(pos0).cuda())
    torch.cuda.synchronize()
    codes, scale = O.quantize_key_rows(k32[:, 0])
    kb = g_k.view(torch.uint8)
    for b in range(B):
        s = int(pos0[b])
        assert np.array_equal(kb[b, s].cpu().numpy(), codes[b]) and g_s[b, s].item() == scale[b]
        assert torch.equal(g_r[b, s].view(torch.int16).cpu(), row_new[b, 0].view(torch.int16))
    assert int((kb != 0).any(dim=-1).sum()) <= B and int((g_s != 0).sum()) == B
    del g_k, g_s, g_r
    # 1M bf16 with a block summary
    N, D, T, Bs = 1 << 20, 64, 4, 64
    k_new, _ = _bf16_keys(rng, (1, T, D))
    row_new = _rows(rng, (1, T, 128))
    g_k = torch.from_numpy(rng.standard_normal((1, N, D)).astype(np.float32)).to(torch.bfloat16).cuda()
    g_r = torch.zeros((1, N, 128), dtype=torch.bfloat16, device="cuda")
    kbar = torch.full((1, N // Bs, D), -7.0, dtype=torch.float32, device="cuda")
    p0 = (N // 2 // Bs) * Bs + Bs - T  # the four tokens complete one block
    L.lsa_cache_append(k_new.cuda(), g_k, rows=[(row_new.cuda(), g_r)],
                       pos0=torch.tensor([p0], dtype=torch.int32, device="cuda"), kbar=kbar, block_size=Bs)
    torch.cuda.synchronize()
    assert torch.equal(g_k[0, p0:p0 + T].view(torch.int16).cpu(), k_new[0].view(torch.int16))
    j = (p0 + T - 1) // Bs
    bits = g_k[0, j * Bs:(j + 1) * Bs].view(torch.int16).cpu().numpy().view(np.uint16)
    want = O.block_means(O.index_keys_f64(bits, None), Bs, 1)[0]
    assert np.allclose(kbar[0, j].cpu().numpy(), want, rtol=1e-5, atol=1e-6)
    assert int((kbar != -7.0).any(dim=-1).sum()) == 1  # only the completed block
