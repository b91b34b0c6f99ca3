"""C ABI checks that need no GPU: the library loads and exports every function the
header declares; the Python descriptors have the C layout; every argument error is
reported with its status code before any HIP call."""
import ctypes
import os
import re
import subprocess

import pytest

import long_context_sparse_07_amd as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lsa.h")

FAKE = 0x7F0000000000  # 256-byte aligned, never dereferenced (validation fails first)


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(lsa_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_function():
    lib = L.lib()
    names = declared_functions()
    assert {"lsa_index", "lsa_block_means", "lsa_select", "lsa_attend", "lsa_select_workspace_bytes",
            "lsa_attend_workspace_bytes", "lsa_workspace_clear", "lsa_status_str", "lsa_last_error",
            "lsa_version", "lsa_select_attend", "lsa_cache_append"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in lsa.h but not exported"
    assert lib.lsa_version() == 1


def test_descriptor_layout_matches_c(tmp_path):
    structs = {"lsa_index_desc": L.IndexDesc, "lsa_block_means_desc": L.BlockMeansDesc,
               "lsa_select_desc": L.SelectDesc, "lsa_attend_desc": L.AttendDesc,
               "lsa_attend_bwd_desc": L.AttendBwdDesc, "lsa_index_target_desc": L.IndexTargetDesc,
               "lsa_cache_append_desc": L.CacheAppendDesc}
    lines = ['#include <stdio.h>', '#include <stddef.h>', f'#include "{HEADER}"', "int main(void){"]
    for cname, py in structs.items():
        lines.append(f'printf("{cname} size %zu\\n", sizeof({cname}));')
        for fname, _ in py._fields_:
            lines.append(f'printf("{cname} {fname} %zu\\n", offsetof({cname}, {fname}));')
    lines.append("return 0;}")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", "/opt/rocm/include", str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    got = {}
    for line in out:
        if line:
            c, f, v = line.split()
            got[(c, f)] = int(v)
    for cname, py in structs.items():
        assert got[(cname, "size")] == ctypes.sizeof(py), cname
        for fname, _ in py._fields_:
            assert got[(cname, fname)] == getattr(py, fname).offset, (cname, fname)


def _index_desc(**kw):
    base = dict(mode=L.LSA_INDEX_TOKENS, B=2, T=1, N=1024, H=64, D=128, q=FAKE, w=FAKE, k=FAKE,
                k_dtype=L.LSA_FP8_E4M3FN, k_scale=FAKE, scores=FAKE)
    base.update(kw)
    return L.IndexDesc(**base)


def _select_desc(**kw):
    base = dict(B=2, T=1, N=1024, scores=FAKE, n_cols=1024, K=256, sink=16, window=64, causal=1, idx=FAKE)
    base.update(kw)
    return L.SelectDesc(**base)


def _attend_desc(**kw):
    base = dict(B=2, T=1, N=1024, Hq=64, Hkv=1, d_qk=576, d_v=512, q=FAKE, k=FAKE, k_stride_b=1024 * 576,
                k_stride_n=576, k_stride_h=576, v=FAKE, v_stride_b=1024 * 576, v_stride_n=576, v_stride_h=576,
                idx=FAKE, K=256, softmax_scale=0.04, out=FAKE, out_dtype=L.LSA_BF16, n_layers=1)
    base.update(kw)
    return L.AttendDesc(**base)


def _idx(d):
    return L.lib().lsa_index(ctypes.byref(d), None)


def _sel(d, ws=FAKE, nbytes=1 << 40):
    return L.lib().lsa_select(ctypes.byref(d), ws, nbytes, None)


def _att(d, ws=FAKE, nbytes=1 << 40):
    return L.lib().lsa_attend(ctypes.byref(d), ws, nbytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(scores=None), -1), (dict(k_scale=None), -1),
    (dict(B=0), -2), (dict(T=2000), -2), (dict(mode=7), -2),
    (dict(k_dtype=9), -3), (dict(k_dtype=L.LSA_F32), -3),
    (dict(q=FAKE + 2), -5), (dict(scores=FAKE + 4), -5),
    (dict(H=12), -6), (dict(D=96), -6),
    (dict(mode=L.LSA_INDEX_BLOCKS, k_dtype=L.LSA_BF16), -3),
    (dict(mode=L.LSA_INDEX_BLOCKS, k_dtype=L.LSA_F32, block_size=64, n_blocks=17), -2),
    (dict(mode=L.LSA_INDEX_BLOCKS, k_dtype=L.LSA_F32, block_size=64, n_blocks=16, window=64, H=65), -6),
    (dict(mode=L.LSA_INDEX_BLOCKS, k_dtype=L.LSA_F32, block_size=64, n_blocks=16, window=62), -6),
    (dict(kept=FAKE, n_keep=0, block_size=64), -2),
    # fp8 queries: a known dtype, fp8 keys and D = 128 only
    (dict(q_dtype=9), -3), (dict(q_dtype=L.LSA_F32), -3),
    (dict(q_dtype=L.LSA_FP8_E4M3FN, k_dtype=L.LSA_BF16, k_scale=None), -6),
    (dict(q_dtype=L.LSA_FP8_E4M3FN, D=64), -6),
])
def test_index_argument_errors(kw, code):
    assert _idx(_index_desc(**kw)) == code
    assert L.lib().lsa_last_error()


@pytest.mark.parametrize("kw,code", [
    (dict(select_ws=FAKE + 16, select_ws_bytes=1 << 30), -5),
    (dict(select_ws=FAKE, select_ws_bytes=100), -7),
    (dict(select_ws=FAKE, select_ws_bytes=1 << 30, select_ws_state=2), -2),
    (dict(select_ws=FAKE, select_ws_bytes=1 << 30, sink=-1), -2),
    (dict(select_ws=FAKE, select_ws_bytes=1 << 30, kept=FAKE, n_keep=16, block_size=64, window=32), -6),
])
def test_index_priming_errors(kw, code):
    assert _idx(_index_desc(**kw)) == code


def test_index_null_desc():
    assert L.lib().lsa_index(None, None) == -1


@pytest.mark.parametrize("kw,code", [
    (dict(K=0, sink=0, window=0), -4), (dict(sink=200, window=100), -4), (dict(sink=-1), -4),
    (dict(causal=0), -4), (dict(K=5000, sink=0, window=0), -6), (dict(n_cols=0), -2),
    (dict(kept=FAKE, n_keep=4, block_size=64), -2), (dict(B=70000), -6),
    (dict(kept=FAKE, n_keep=16, block_size=128, window=64), -6),
])
def test_select_argument_errors(kw, code):
    assert _sel(_select_desc(**kw)) == code


def test_select_workspace_state_errors():
    assert _sel(_select_desc(workspace_state=3)) == -2
    # causal = 0 with a primed workspace is the BLOCKS indexer's block selection: no kept map
    assert _sel(_select_desc(workspace_state=L.LSA_WS_PRIMED, causal=0, sink=0, window=0, kept=FAKE, n_keep=16,
                             block_size=64)) == -2


def test_select_workspace_and_pointer_errors():
    d = _select_desc()
    need = L.lib().lsa_select_workspace_bytes(ctypes.byref(d))
    assert need > 0
    assert _sel(d, FAKE, need - 1) == -7
    assert _sel(d, None, need) == -7
    assert _sel(d, FAKE + 16, need) == -5
    assert _sel(_select_desc(idx=None)) == -1
    assert _sel(_select_desc(scores=FAKE + 1)) == -5
    # larger problems need more workspace
    assert L.lib().lsa_select_workspace_bytes(ctypes.byref(_select_desc(B=8))) > need
    assert L.lib().lsa_select_workspace_bytes(ctypes.byref(_select_desc(K=0, sink=0, window=0))) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(out=None), -1), (dict(K=0), -4), (dict(Hq=63, Hkv=2), -2),
    (dict(d_qk=64, d_v=64), -6), (dict(Hq=48), -6), (dict(out_dtype=5), -3),
    (dict(k_stride_n=577, v_stride_n=577), -5), (dict(v=FAKE + 256), -6),
    (dict(q=FAKE + 8), -5), (dict(n_layers=0), -2), (dict(n_splits=-1), -2),
    (dict(K=2048 * 128 + 1), -6),
    # paged caches: sizes must be >= 1 and the pool's rows must fit int32
    (dict(block_table=FAKE, page_size=0, max_pages=16, num_pages=32), -2),
    (dict(block_table=FAKE, page_size=64, max_pages=0, num_pages=32), -2),
    (dict(block_table=FAKE, page_size=64, max_pages=16, num_pages=0), -2),
    (dict(block_table=FAKE, page_size=1 << 16, max_pages=16, num_pages=1 << 15), -2),
])
def test_attend_argument_errors(kw, code):
    assert _att(_attend_desc(**kw)) == code


def test_attend_workspace_rules():
    d = _attend_desc(n_splits=4)
    need = L.lib().lsa_attend_workspace_bytes(ctypes.byref(d))
    # bf16 partial rows (256-byte aligned), then fp32 (m, l) per head and split
    assert need == 2 * 4 * 64 * 512 * 2 + 2 * 4 * 64 * 2 * 4
    assert _att(d, FAKE, need - 4) == -7
    assert _att(d, None, 0) == -7
    one = _attend_desc(n_splits=1)
    assert L.lib().lsa_attend_workspace_bytes(ctypes.byref(one)) == 0


def _sel_att(ds, da, ws=FAKE, nbytes=1 << 40, wa=FAKE, na=1 << 40):
    return L.lib().lsa_select_attend(ctypes.byref(ds), ctypes.byref(da), ws, nbytes, wa, na, None)


@pytest.mark.parametrize("skw,akw,code", [
    (dict(), dict(B=3), -2), (dict(), dict(K=512), -2), (dict(), dict(N=2048), -2),
    (dict(), dict(idx=FAKE + 4096), -2),
    (dict(kept=FAKE, n_keep=16, block_size=64), dict(), -6),
    (dict(scores=None), dict(), -1), (dict(), dict(q=None), -1), (dict(), dict(out=None), -1),
    (dict(K=0, sink=0, window=0), dict(), -4), (dict(), dict(Hq=48), -6),
    (dict(), dict(q=FAKE + 8), -5), (dict(idx=FAKE + 2), dict(idx=None), -5),
    (dict(), dict(idx_shared=1), -6),   # a shared index row: the separate calls only
])
def test_select_attend_argument_errors(skw, akw, code):
    assert _sel_att(_select_desc(**skw), _attend_desc(**akw)) == code
    assert L.lib().lsa_last_error()


def test_select_attend_workspace_errors():
    ds, da = _select_desc(), _attend_desc(n_splits=4)
    sneed = L.lib().lsa_select_workspace_bytes(ctypes.byref(ds))
    aneed = L.lib().lsa_attend_workspace_bytes(ctypes.byref(da))
    assert _sel_att(ds, da, FAKE, sneed - 1) == -7
    assert _sel_att(ds, da, None, sneed) == -7
    assert _sel_att(ds, da, FAKE, sneed, FAKE, aneed - 4) == -7
    assert _sel_att(ds, da, FAKE, sneed, None, aneed) == -7
    assert _sel_att(ds, da, FAKE + 16, sneed) == -5
    assert _sel_att(ds, da, FAKE, sneed, FAKE + 16, aneed) == -5
    assert L.lib().lsa_select_attend(None, ctypes.byref(da), FAKE, sneed, FAKE, aneed, None) == -1
    assert L.lib().lsa_select_attend(ctypes.byref(ds), None, FAKE, sneed, FAKE, aneed, None) == -1


def _append_desc(rows=1, **kw):
    d = L.CacheAppendDesc(B=2, T=1, N=1024, D=128, k_new=FAKE, k_cache=FAKE, k_dtype=L.LSA_FP8_E4M3FN,
                          k_scale=FAKE, n_rows=rows)
    for i in range(rows):
        d.rows_new[i] = FAKE
        d.rows_cache[i] = FAKE
        d.row_elems[i] = 576
        d.rows_stride_b[i] = 1024 * 576
        d.rows_stride_n[i] = 576
    for k, v in kw.items():
        setattr(d, k, v)
    return d


@pytest.mark.parametrize("kw,code", [
    (dict(k_new=None), -1), (dict(k_cache=None), -1), (dict(k_scale=None), -1),
    (dict(B=0), -2), (dict(T=0), -2), (dict(n_rows=3), -2),
    (dict(k_dtype=L.LSA_F32), -3), (dict(D=96), -6), (dict(B=70000), -6),
    (dict(k_new=FAKE + 8), -5), (dict(k_cache=FAKE + 4), -5),
    (dict(kbar=FAKE, block_size=64, n_blocks=17), -2), (dict(kbar=FAKE, block_size=0, n_blocks=1), -2),
    (dict(kbar=FAKE + 2, block_size=64, n_blocks=16), -5),
])
def test_cache_append_argument_errors(kw, code):
    assert L.lib().lsa_cache_append(ctypes.byref(_append_desc(**kw)), None) == code
    assert L.lib().lsa_last_error()


def test_cache_append_row_set_errors():
    lib = L.lib()
    d = _append_desc()
    d.row_elems[0] = 570
    assert lib.lsa_cache_append(ctypes.byref(d), None) == -2
    d = _append_desc()
    d.rows_stride_n[0] = 500
    assert lib.lsa_cache_append(ctypes.byref(d), None) == -2
    d = _append_desc()
    d.rows_cache[0] = FAKE + 8
    assert lib.lsa_cache_append(ctypes.byref(d), None) == -5
    d = _append_desc()
    d.rows_new[0] = None
    assert lib.lsa_cache_append(ctypes.byref(d), None) == -1
    assert lib.lsa_cache_append(None, None) == -1


def test_status_strings():
    lib = L.lib()
    for code in range(-8, 1):
        assert lib.lsa_status_str(code).decode().startswith(L.STATUS[code])
    assert lib.lsa_workspace_clear(None, 16, None) == -1
    assert lib.lsa_workspace_clear(FAKE + 4, 16, None) == -5
    assert lib.lsa_workspace_clear(None, 0, None) == 0
    assert lib.lsa_index_launch_events(None, None) == 0  # the measurement hooks, cleared
    assert lib.lsa_attend_launch_events(None, None) == 0


def _bwd_desc(**kw):
    base = dict(B=2, T=1, N=1024, Hq=64, Hkv=1, d_qk=576, d_v=512, q=FAKE, k=FAKE, k_stride_b=1024 * 576,
                k_stride_n=576, k_stride_h=576, v=FAKE, v_stride_b=1024 * 576, v_stride_n=576, v_stride_h=576,
                idx=FAKE, K=256, softmax_scale=0.04, out=FAKE, lse=FAKE, dout=FAKE, dq=FAKE, dk=FAKE)
    base.update(kw)
    return L.AttendBwdDesc(**base)


def _bwd(d, ws=FAKE, nbytes=1 << 40):
    return L.lib().lsa_attend_backward(ctypes.byref(d), ws, nbytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(dout=None), -1), (dict(lse=None), -1), (dict(dk=None), -1),
    (dict(d_qk=128, d_v=128, Hkv=8, k_stride_h=128, v_stride_h=128, k_stride_n=1024, v_stride_n=1024,
          k_stride_b=1 << 20, v_stride_b=1 << 20, v=FAKE + 4096), -1),   # GQA needs dv
    (dict(K=0), -4), (dict(Hq=63, Hkv=2), -2), (dict(B=0), -2),
    (dict(d_qk=64, d_v=64), -6), (dict(Hq=128), -6), (dict(v=FAKE + 256), -6),
    (dict(k_stride_n=577, v_stride_n=577), -5), (dict(out=FAKE + 8), -5), (dict(dq=FAKE + 2), -5),
    (dict(T=40000), -6),
])
def test_attend_backward_argument_errors(kw, code):
    assert _bwd(_bwd_desc(**kw)) == code


def test_attend_backward_workspace_rules():
    d = _bwd_desc()
    need = L.lib().lsa_attend_backward_workspace_bytes(ctypes.byref(d))
    # one query token per sequence: only the per-32-row-tile dq parts (the row gradients go
    # straight to dk); with more query tokens, per (query, KV head, selected row) one MLA
    # row of fp32 before them
    assert need == 2 * 64 * 8 * 576 * 4
    need3 = L.lib().lsa_attend_backward_workspace_bytes(ctypes.byref(_bwd_desc(T=3)))
    assert need3 == 2 * 3 * 256 * 576 * 4 + 2 * 3 * 64 * 8 * 576 * 4
    assert _bwd(d, FAKE, need - 1) == -7
    assert _bwd(d, None, need) == -7
    assert _bwd(d, FAKE + 16, need) == -5
    assert L.lib().lsa_attend_backward_workspace_bytes(ctypes.byref(_bwd_desc(K=0))) == 0


def _tgt_desc(**kw):
    base = dict(B=2, T=1, N=1024, Hq=64, Hkv=1, d_qk=576, q=FAKE, k=FAKE, k_stride_b=1024 * 576, k_stride_n=576,
                k_stride_h=576, idx=FAKE, K=256, softmax_scale=0.04, lse=FAKE, scores=FAKE, n_cols=1024,
                target=FAKE, grad=FAKE, loss=FAKE)
    base.update(kw)
    return L.IndexTargetDesc(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(scores=None), -1), (dict(loss=None), -1), (dict(K=0), -4), (dict(B=0), -2),
    (dict(Hq=63, Hkv=2), -2), (dict(n_cols=1000), -2), (dict(d_qk=64), -6), (dict(Hq=128), -6),
    (dict(T=40000), -6), (dict(k_stride_n=577), -5), (dict(q=FAKE + 8), -5), (dict(grad=FAKE + 2), -5),
])
def test_index_target_argument_errors(kw, code):
    assert L.lib().lsa_index_target(ctypes.byref(_tgt_desc(**kw)), None) == code


def test_index_select_workspace_by_path():
    # decode rows (one query token per sequence): the selection workspace, plus the scores
    # when the caller does not take them; prefill rows (thousands of query tokens per
    # sequence): the candidate lists, 4 bytes per row then 8 per row and position
    lib = L.lib()
    dec = _index_desc(B=2, T=1, N=8192, sink=64, window=512)
    with_sc = lib.lsa_index_select_workspace_bytes(ctypes.byref(dec), 2048)
    dec.scores = None
    assert lib.lsa_index_select_workspace_bytes(ctypes.byref(dec), 2048) >= with_sc + 2 * 8192 * 4
    pre = _index_desc(B=1, T=2048, N=8192, sink=64, window=512)
    want = 2048 * 4 + 2048 * 8192 * 8
    assert lib.lsa_index_select_workspace_bytes(ctypes.byref(pre), 2048) == want
    pre.scores = None
    assert lib.lsa_index_select_workspace_bytes(ctypes.byref(pre), 2048) == want
    # H = 16 has no whole-row prefill kernel: the selection workspace again
    pre16 = _index_desc(B=1, T=2048, N=8192, H=16, sink=64, window=512)
    assert lib.lsa_index_select_workspace_bytes(ctypes.byref(pre16), 2048) != 2048 * 4 + 2048 * 8192 * 8
