// C ABI of liblsa.so: argument validation (host only, before any HIP call) and
// dispatch to the gfx950 kernels. See include/lsa.h for the contract.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "../../include/lsa.h"
#include "kernels.h"

namespace {

thread_local char g_err[512] = "";

int32_t fail(int32_t code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

int32_t hip_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return LSA_OK;
    return fail(LSA_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

constexpr int64_t kMaxGridY = 65535;

}  // namespace

extern "C" {

int32_t lsa_version(void) { return LSA_VERSION; }

const char *lsa_status_str(int32_t s) {
    switch (s) {
        case LSA_OK: return "LSA_OK";
        case LSA_E_NULL: return "LSA_E_NULL: a required pointer is NULL";
        case LSA_E_SHAPE: return "LSA_E_SHAPE: a size is out of range or inconsistent";
        case LSA_E_DTYPE: return "LSA_E_DTYPE: unknown or unsupported dtype";
        case LSA_E_BUDGET: return "LSA_E_BUDGET: K < 1 or sink + window > K";
        case LSA_E_ALIGN: return "LSA_E_ALIGN: pointer or stride not 16-byte aligned";
        case LSA_E_UNSUPPORTED: return "LSA_E_UNSUPPORTED: no kernel for this shape";
        case LSA_E_WORKSPACE: return "LSA_E_WORKSPACE: workspace missing or too small";
        case LSA_E_HIP: return "LSA_E_HIP: a HIP launch failed";
        default: return "unknown lsa status";
    }
}

const char *lsa_last_error(void) { return g_err; }

// ----------------------------------------------------------------------------- index

// lsa_index with a selection workspace: the scores, and the selection histogram from the
// indexer epilogue when the kernel has one query per workgroup, else from the
// selection's own histogram pass.
static int32_t index_primed(const lsa_index_desc *d, lsa::IndexTokensArgs a, void *select_ws, bool ws_clean,
                            hipStream_t s, const char *fn) {
    const bool hi = d->kept != nullptr;
    lsa::SelectArgs sa{};
    sa.B = d->B;
    sa.T = d->T;
    sa.N = d->N;
    sa.ctx_len = d->ctx_len;
    sa.scores = a.scores;
    sa.n_cols = a.n_out;
    sa.kept = d->kept;
    sa.n_keep = a.n_keep;
    sa.block_size = hi ? d->block_size : 1;
    sa.K = 0x3FFFFFFF;  // the histogram counts every candidate
    sa.sink = d->sink;
    sa.window = d->window;
    sa.causal = true;
    sa.ws_clean = ws_clean;
    sa.vec = (a.n_out & 3) == 0;  // scores are 16-byte aligned
    hipError_t e;
    // rows the one-launch selection takes need no histogram (it leaves the workspace clean)
    if (lsa::select_small(a.n_out)) return hip_status(lsa::launch_index_tokens(a, s), fn);
    if (lsa::index_tokens_fused_hist(d->H, d->T, hi)) {
        if (!sa.ws_clean) {
            e = lsa::launch_clear(select_ws, lsa::select_zero_bytes(d->B * d->T), s);
            if (e != hipSuccess) return hip_status(e, fn);
        }
        a.sel_hist = reinterpret_cast<uint32_t *>(select_ws);
        a.sink = d->sink;
        a.window = d->window;
        return hip_status(lsa::launch_index_tokens(a, s), fn);
    }
    e = lsa::launch_index_tokens(a, s);
    if (e != hipSuccess) return hip_status(e, fn);
    return hip_status(lsa::launch_select_hist(sa, select_ws, s), fn);
}

// Checks of a TOKENS index descriptor shared by lsa_index and lsa_index_select (pointers
// q, w, k; sizes; key and query types); fills the kernel arguments.
static int32_t index_tokens_check(const lsa_index_desc *d, lsa::IndexTokensArgs &a, const char *fn) {
    if (!d->q || !d->w || !d->k) return fail(LSA_E_NULL, "%s: q, w and k are required", fn);
    if (d->B < 1 || d->T < 1 || d->N < 1 || d->H < 1 || d->D < 1)
        return fail(LSA_E_SHAPE, "%s: B, T, N, H, D must be >= 1 (got %d %d %d %d %d)", fn, d->B, d->T, d->N, d->H, d->D);
    if (d->T > d->N) return fail(LSA_E_SHAPE, "%s: T=%d exceeds N=%d", fn, d->T, d->N);
    if (!aligned16(d->q) || !aligned16(d->k) || !aligned4(d->w) || (d->scores && !aligned16(d->scores)))
        return fail(LSA_E_ALIGN, "%s: q, k, scores must be 16-byte aligned", fn);
    if (d->B > kMaxGridY) return fail(LSA_E_UNSUPPORTED, "%s: B=%d too large", fn, d->B);
    if (d->k_dtype != LSA_BF16 && d->k_dtype != LSA_FP8_E4M3FN)
        return fail(LSA_E_DTYPE, "%s: TOKENS keys must be bf16 or fp8-e4m3fn (got %d)", fn, d->k_dtype);
    const bool fp8 = d->k_dtype == LSA_FP8_E4M3FN;
    if (fp8 && !d->k_scale) return fail(LSA_E_NULL, "%s: fp8 keys need k_scale", fn);
    const bool hi = d->kept != nullptr;
    if (hi) {
        if (d->n_keep < 1 || d->block_size < 1)
            return fail(LSA_E_SHAPE, "%s: HI fine stage needs n_keep >= 1 and block_size >= 1", fn);
        if ((int64_t)d->n_keep * d->block_size > INT32_MAX / 2)
            return fail(LSA_E_SHAPE, "%s: n_keep * block_size too large", fn);
        if (d->T > kMaxGridY) return fail(LSA_E_UNSUPPORTED, "%s: T=%d too large", fn, d->T);
    }
    if (!lsa::index_tokens_supported(d->H, d->D, hi))
        return fail(LSA_E_UNSUPPORTED, "%s: no token kernel for H=%d D=%d%s", fn, d->H, d->D, hi ? " (HI)" : "");
    if (d->q_dtype != 0 && d->q_dtype != LSA_BF16 && d->q_dtype != LSA_FP8_E4M3FN)
        return fail(LSA_E_DTYPE, "%s: q_dtype must be 0, LSA_BF16 or LSA_FP8_E4M3FN (got %d)", fn, d->q_dtype);
    const bool qf8 = d->q_dtype == LSA_FP8_E4M3FN;
    if (qf8 && (!fp8 || d->D != 128)) return fail(LSA_E_UNSUPPORTED, "%s: fp8 queries need fp8 keys and D=128", fn);
    a = lsa::IndexTokensArgs{};
    a.B = d->B;
    a.T = d->T;
    a.N = d->N;
    a.H = d->H;
    a.D = d->D;
    a.ctx_len = d->ctx_len;
    a.q = reinterpret_cast<const uint16_t *>(d->q);
    a.w = d->w;
    a.k = d->k;
    a.fp8 = fp8;
    a.qf8 = qf8;
    a.k_scale = fp8 ? d->k_scale : nullptr;
    a.kept = d->kept;
    a.n_keep = hi ? d->n_keep : 0;
    a.block_size = hi ? d->block_size : 0;
    a.scores = d->scores;
    a.n_out = hi ? d->n_keep * d->block_size : d->N;
    return LSA_OK;
}

int32_t lsa_index_launch_events(void *start_event, void *stop_event) {
    lsa::set_index_launch_events(reinterpret_cast<hipEvent_t>(start_event), reinterpret_cast<hipEvent_t>(stop_event));
    return LSA_OK;
}

int32_t lsa_attend_launch_events(void *start_event, void *stop_event) {
    lsa::set_attend_launch_events(reinterpret_cast<hipEvent_t>(start_event), reinterpret_cast<hipEvent_t>(stop_event));
    return LSA_OK;
}

int32_t lsa_index(const lsa_index_desc *d, void *stream) {
    if (!d) return fail(LSA_E_NULL, "lsa_index: desc is NULL");
    if (!d->q || !d->w || !d->k || !d->scores) return fail(LSA_E_NULL, "lsa_index: q, w, k and scores are required");
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (d->mode == LSA_INDEX_TOKENS) {
        lsa::IndexTokensArgs a;
        int32_t rc = index_tokens_check(d, a, "lsa_index");
        if (rc != LSA_OK) return rc;
        const bool hi = d->kept != nullptr;
        if (d->select_ws) {
            if (d->sink < 0 || d->window < 0) return fail(LSA_E_SHAPE, "lsa_index: sink and window must be >= 0");
            if (d->select_ws_state != LSA_WS_UNKNOWN && d->select_ws_state != LSA_WS_CLEAN)
                return fail(LSA_E_SHAPE, "lsa_index: select_ws_state must be LSA_WS_UNKNOWN or LSA_WS_CLEAN");
            if ((int64_t)d->B * d->T > kMaxGridY) return fail(LSA_E_UNSUPPORTED, "lsa_index: B*T too large to prime");
            if (hi && d->window < d->block_size - 1)
                return fail(LSA_E_UNSUPPORTED, "lsa_index: priming with a kept map needs window >= block_size - 1");
            const size_t need = lsa::select_workspace_bytes(d->B * d->T, hi ? d->n_keep * d->block_size : d->N, hi);
            if (d->select_ws_bytes < need)
                return fail(LSA_E_WORKSPACE, "lsa_index: select_ws of %zu bytes needed, %zu given", need, d->select_ws_bytes);
            if ((reinterpret_cast<uintptr_t>(d->select_ws) & 255u) != 0)
                return fail(LSA_E_ALIGN, "lsa_index: select_ws not 256-byte aligned");
        }
        if (!d->select_ws) return hip_status(lsa::launch_index_tokens(a, s), "lsa_index");
        return index_primed(d, a, d->select_ws, d->select_ws_state == LSA_WS_CLEAN, s, "lsa_index");
    }
    if (d->mode == LSA_INDEX_BLOCKS) {
        if (d->B < 1 || d->T < 1 || d->N < 1 || d->H < 1 || d->D < 1)
            return fail(LSA_E_SHAPE, "lsa_index: B, T, N, H, D must be >= 1 (got %d %d %d %d %d)", d->B, d->T, d->N, d->H,
                        d->D);
        if (d->T > d->N) return fail(LSA_E_SHAPE, "lsa_index: T=%d exceeds N=%d", d->T, d->N);
        if (!aligned16(d->q) || !aligned16(d->k) || !aligned4(d->w) || !aligned16(d->scores))
            return fail(LSA_E_ALIGN, "lsa_index: q, k, scores must be 16-byte aligned");
        if (d->B > kMaxGridY) return fail(LSA_E_UNSUPPORTED, "lsa_index: B=%d too large", d->B);
        if (d->k_dtype != LSA_F32) return fail(LSA_E_DTYPE, "lsa_index: BLOCKS mode reads fp32 block means");
        if (d->block_size < 1 || d->n_blocks < 1 || (int64_t)d->n_blocks * d->block_size > d->N)
            return fail(LSA_E_SHAPE, "lsa_index: BLOCKS needs block_size >= 1, 1 <= n_blocks <= N / block_size");
        if (d->sink < 0 || d->window < 0) return fail(LSA_E_SHAPE, "lsa_index: sink and window must be >= 0");
        if (d->window < d->block_size - 1)
            return fail(LSA_E_UNSUPPORTED, "lsa_index: BLOCKS needs window >= block_size - 1 (window=%d block_size=%d)",
                        d->window, d->block_size);
        if (d->D != 64 && d->D != 128) return fail(LSA_E_UNSUPPORTED, "lsa_index: BLOCKS needs D in {64,128}");
        if (d->H > 64) return fail(LSA_E_UNSUPPORTED, "lsa_index: BLOCKS needs H <= 64");
        if (d->T > kMaxGridY) return fail(LSA_E_UNSUPPORTED, "lsa_index: T=%d too large", d->T);
        lsa::IndexBlocksArgs a{};
        a.B = d->B;
        a.T = d->T;
        a.N = d->N;
        a.H = d->H;
        a.D = d->D;
        a.ctx_len = d->ctx_len;
        a.q = reinterpret_cast<const uint16_t *>(d->q);
        a.w = d->w;
        a.kbar = reinterpret_cast<const float *>(d->k);
        a.n_blocks = d->n_blocks;
        a.block_size = d->block_size;
        a.sink = d->sink;
        a.window = d->window;
        a.scores = d->scores;
        if (d->select_ws) {  // priming the block selection (no causal mask, no forced set)
            if (d->select_ws_state != LSA_WS_UNKNOWN && d->select_ws_state != LSA_WS_CLEAN)
                return fail(LSA_E_SHAPE, "lsa_index: select_ws_state must be LSA_WS_UNKNOWN or LSA_WS_CLEAN");
            if ((int64_t)d->B * d->T > kMaxGridY) return fail(LSA_E_UNSUPPORTED, "lsa_index: B*T too large to prime");
            const size_t need = lsa::select_workspace_bytes(d->B * d->T, d->n_blocks, false);
            if (d->select_ws_bytes < need)
                return fail(LSA_E_WORKSPACE, "lsa_index: select_ws of %zu bytes needed, %zu given", need, d->select_ws_bytes);
            if ((reinterpret_cast<uintptr_t>(d->select_ws) & 255u) != 0)
                return fail(LSA_E_ALIGN, "lsa_index: select_ws not 256-byte aligned");
            // rows the one-launch selection takes need no histogram (it leaves the workspace clean)
            if (!lsa::select_small(d->n_blocks)) {
                if (d->select_ws_state != LSA_WS_CLEAN) {
                    const hipError_t e = lsa::launch_clear(d->select_ws, lsa::select_zero_bytes(d->B * d->T), s);
                    if (e != hipSuccess) return hip_status(e, "lsa_index");
                }
                a.sel_hist = reinterpret_cast<uint32_t *>(d->select_ws);
            }
        }
        return hip_status(lsa::launch_index_blocks(a, s), "lsa_index");
    }
    return fail(LSA_E_SHAPE, "lsa_index: unknown mode %d", d->mode);
}

int32_t lsa_block_means(const lsa_block_means_desc *d, void *stream) {
    if (!d) return fail(LSA_E_NULL, "lsa_block_means: desc is NULL");
    if (!d->k || !d->kbar) return fail(LSA_E_NULL, "lsa_block_means: k and kbar are required");
    if (d->k_dtype != LSA_BF16 && d->k_dtype != LSA_FP8_E4M3FN)
        return fail(LSA_E_DTYPE, "lsa_block_means: keys must be bf16 or fp8-e4m3fn");
    const bool fp8 = d->k_dtype == LSA_FP8_E4M3FN;
    if (fp8 && !d->k_scale) return fail(LSA_E_NULL, "lsa_block_means: fp8 keys need k_scale");
    if (d->B < 1 || d->N < 1 || d->block_size < 1 || d->n_blocks < 1 ||
        (int64_t)d->n_blocks * d->block_size > d->N)
        return fail(LSA_E_SHAPE, "lsa_block_means: need B, N, block_size, n_blocks >= 1 and n_blocks*block_size <= N");
    if (d->D != 64 && d->D != 128) return fail(LSA_E_UNSUPPORTED, "lsa_block_means: D must be 64 or 128");
    if (d->B > kMaxGridY) return fail(LSA_E_UNSUPPORTED, "lsa_block_means: B too large");
    lsa::BlockMeansArgs a{};
    a.B = d->B;
    a.N = d->N;
    a.D = d->D;
    a.k = d->k;
    a.fp8 = fp8;
    a.k_scale = fp8 ? d->k_scale : nullptr;
    a.block_size = d->block_size;
    a.n_blocks = d->n_blocks;
    a.kbar = d->kbar;
    return hip_status(lsa::launch_block_means(a, reinterpret_cast<hipStream_t>(stream)), "lsa_block_means");
}

// ----------------------------------------------------------------------------- select

static int32_t select_check(const lsa_select_desc *d, lsa::SelectArgs &a) {
    if (!d) return fail(LSA_E_NULL, "lsa_select: desc is NULL");
    if (d->B < 1 || d->T < 1 || d->N < 1 || d->n_cols < 1)
        return fail(LSA_E_SHAPE, "lsa_select: B, T, N, n_cols must be >= 1");
    if (d->K < 1 || d->sink < 0 || d->window < 0 || (int64_t)d->sink + d->window > d->K)
        return fail(LSA_E_BUDGET, "lsa_select: need K >= 1 and 0 <= sink + window <= K (K=%d sink=%d window=%d)", d->K,
                    d->sink, d->window);
    if (d->K > 4096) return fail(LSA_E_UNSUPPORTED, "lsa_select: K=%d above 4096", d->K);
    if (d->workspace_state != LSA_WS_UNKNOWN && d->workspace_state != LSA_WS_CLEAN &&
        d->workspace_state != LSA_WS_PRIMED)
        return fail(LSA_E_SHAPE, "lsa_select: unknown workspace_state %d", d->workspace_state);
    // causal = 0 reads a workspace primed by the BLOCKS indexer (every finite score counted)
    if (d->workspace_state == LSA_WS_PRIMED && !d->causal && d->kept)
        return fail(LSA_E_SHAPE, "lsa_select: a primed workspace with causal = 0 takes no kept map");
    if (!d->causal && (d->sink || d->window))
        return fail(LSA_E_BUDGET, "lsa_select: sink and window need causal = 1");
    if (d->kept && (d->n_keep < 1 || d->block_size < 1 || (int64_t)d->n_keep * d->block_size < d->n_cols))
        return fail(LSA_E_SHAPE, "lsa_select: a kept map needs n_keep * block_size >= n_cols");
    if (d->kept && d->causal && d->window < d->block_size - 1)
        return fail(LSA_E_UNSUPPORTED, "lsa_select: a kept map needs window >= block_size - 1 (window=%d block_size=%d)",
                    d->window, d->block_size);
    if ((int64_t)d->B * d->T > kMaxGridY) return fail(LSA_E_UNSUPPORTED, "lsa_select: B*T too large");
    a = lsa::SelectArgs{};
    a.B = d->B;
    a.T = d->T;
    a.N = d->N;
    a.ctx_len = d->ctx_len;
    a.scores = d->scores;
    a.n_cols = d->n_cols;
    a.kept = d->kept;
    a.n_keep = d->kept ? d->n_keep : 0;
    a.block_size = d->kept ? d->block_size : 1;
    a.K = d->K;
    a.sink = d->sink;
    a.window = d->window;
    a.causal = d->causal != 0;
    a.ws_clean = d->workspace_state == LSA_WS_CLEAN;
    a.primed = d->workspace_state == LSA_WS_PRIMED;
    a.vec = (d->n_cols & 3) == 0 && aligned16(d->scores);
    a.idx = d->idx;
    return LSA_OK;
}

size_t lsa_select_workspace_bytes(const lsa_select_desc *d) {
    lsa::SelectArgs a;
    if (select_check(d, a) != LSA_OK) return 0;
    return lsa::select_workspace_bytes(a.B * a.T, a.n_cols, a.kept != nullptr);
}

int32_t lsa_select(const lsa_select_desc *d, void *ws, size_t ws_bytes, void *stream) {
    lsa::SelectArgs a;
    int32_t rc = select_check(d, a);
    if (rc != LSA_OK) return rc;
    if (!d->scores || !d->idx) return fail(LSA_E_NULL, "lsa_select: scores and idx are required");
    if (!aligned4(d->scores) || !aligned4(d->idx)) return fail(LSA_E_ALIGN, "lsa_select: misaligned scores or idx");
    const size_t need = lsa::select_workspace_bytes(a.B * a.T, a.n_cols, a.kept != nullptr);
    if (!ws || ws_bytes < need)
        return fail(LSA_E_WORKSPACE, "lsa_select: workspace of %zu bytes needed, %zu given", need, ws_bytes);
    if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return fail(LSA_E_ALIGN, "lsa_select: workspace not 256-byte aligned");
    return hip_status(lsa::launch_select(a, ws, reinterpret_cast<hipStream_t>(stream)), "lsa_select");
}

// ----------------------------------------------------------------------------- index + select

// lsa_index_select's candidate-list layout: the per-row list lengths, then [rows][N]
// composites (emission path only).
static size_t cand_offset(int rows) { return ((size_t)rows * 4 + 255) & ~(size_t)255; }

// Checks of lsa_index_select's arguments; fills the indexer arguments, the path (emit:
// the indexer writes candidate lists that the selection reads instead of the scores) and
// the workspace size.
static int32_t index_select_check(const lsa_index_desc *d, int32_t K, lsa::IndexTokensArgs &a, size_t &ws_need,
                                  bool &emit) {
    if (!d) return fail(LSA_E_NULL, "lsa_index_select: desc is NULL");
    if (d->mode != LSA_INDEX_TOKENS) return fail(LSA_E_UNSUPPORTED, "lsa_index_select: TOKENS mode only");
    if (d->kept) return fail(LSA_E_UNSUPPORTED, "lsa_index_select: no kept map (call lsa_index, then lsa_select)");
    int32_t rc = index_tokens_check(d, a, "lsa_index_select");
    if (rc != LSA_OK) return rc;
    if (K < 1 || d->sink < 0 || d->window < 0 || (int64_t)d->sink + d->window > K)
        return fail(LSA_E_BUDGET, "lsa_index_select: need K >= 1 and 0 <= sink + window <= K (K=%d sink=%d window=%d)",
                    K, d->sink, d->window);
    if (K > 4096) return fail(LSA_E_UNSUPPORTED, "lsa_index_select: K=%d above 4096", K);
    if ((int64_t)d->B * d->T > kMaxGridY) return fail(LSA_E_UNSUPPORTED, "lsa_index_select: B*T too large");
    const int rows = d->B * d->T;
    emit = lsa::index_tokens_emits(d->B, d->T, d->N, d->H, d->D, false) && lsa::select_cand_fits(d->N);
    if (emit) {
        // the list lengths and one list of up to N composites per row
        ws_need = cand_offset(rows) + (size_t)rows * d->N * 8;
        return LSA_OK;
    }
    // the selection's workspace, then the scores when the caller does not ask for them
    ws_need = lsa::select_workspace_bytes(rows, d->N, false);
    if (!d->scores) ws_need += (size_t)rows * d->N * 4 + 256;
    return LSA_OK;
}

size_t lsa_index_select_workspace_bytes(const lsa_index_desc *d, int32_t K) {
    lsa::IndexTokensArgs a;
    size_t need = 0;
    bool emit = false;
    if (index_select_check(d, K, a, need, emit) != LSA_OK) return 0;
    return need;
}

int32_t lsa_index_select(const lsa_index_desc *d, int32_t K, int32_t *idx, void *ws, size_t ws_bytes,
                         int32_t ws_state, void *stream) {
    lsa::IndexTokensArgs a;
    size_t need = 0;
    bool emit = false;
    int32_t rc = index_select_check(d, K, a, need, emit);
    if (rc != LSA_OK) return rc;
    if (!idx) return fail(LSA_E_NULL, "lsa_index_select: idx is required");
    if (!aligned4(idx)) return fail(LSA_E_ALIGN, "lsa_index_select: misaligned idx");
    if (ws_state != LSA_WS_UNKNOWN && ws_state != LSA_WS_CLEAN)
        return fail(LSA_E_SHAPE, "lsa_index_select: workspace_state must be LSA_WS_UNKNOWN or LSA_WS_CLEAN");
    if (!ws || ws_bytes < need)
        return fail(LSA_E_WORKSPACE, "lsa_index_select: workspace of %zu bytes needed, %zu given", need, ws_bytes);
    if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
        return fail(LSA_E_ALIGN, "lsa_index_select: workspace not 256-byte aligned");
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const int rows = d->B * d->T;
    lsa::SelectArgs sa{};
    sa.B = d->B;
    sa.T = d->T;
    sa.N = d->N;
    sa.ctx_len = d->ctx_len;
    sa.n_cols = d->N;
    sa.block_size = 1;
    sa.K = K;
    sa.sink = d->sink;
    sa.window = d->window;
    sa.causal = true;
    sa.idx = idx;
    if (emit) {
        // the indexer lists each row's candidates that can still reach its fill (scores
        // written only when asked for), the selection ranks the lists
        a.cand_cnt = reinterpret_cast<uint32_t *>(ws);
        a.cand = reinterpret_cast<uint64_t *>(reinterpret_cast<char *>(ws) + cand_offset(rows));
        a.K = K;
        a.sink = d->sink;
        a.window = d->window;
        hipError_t e = lsa::launch_index_tokens(a, s);
        if (e != hipSuccess) return hip_status(e, "lsa_index_select");
        return hip_status(lsa::launch_select_cand(sa, a.cand, a.cand_cnt, s), "lsa_index_select");
    }
    if (!a.scores) {
        const size_t sel_bytes = lsa::select_workspace_bytes(rows, d->N, false);
        a.scores = reinterpret_cast<float *>((reinterpret_cast<uintptr_t>(ws) + sel_bytes + 255) & ~(uintptr_t)255);
    }
    // the indexer priming the selection workspace, then the selection on its scores
    rc = index_primed(d, a, ws, ws_state == LSA_WS_CLEAN, s, "lsa_index_select");
    if (rc != LSA_OK) return rc;
    sa.scores = a.scores;
    sa.primed = true;
    sa.vec = (d->N & 3) == 0;
    return hip_status(lsa::launch_select(sa, ws, s), "lsa_index_select");
}

// ----------------------------------------------------------------------------- attend

static int32_t attend_check(const lsa_attend_desc *d, lsa::AttendArgs &a) {
    if (!d) return fail(LSA_E_NULL, "lsa_attend: desc is NULL");
    if (d->B < 1 || d->T < 1 || d->N < 1 || d->Hq < 1 || d->Hkv < 1 || d->n_layers < 1)
        return fail(LSA_E_SHAPE, "lsa_attend: B, T, N, Hq, Hkv, n_layers must be >= 1");
    if (d->K < 1) return fail(LSA_E_BUDGET, "lsa_attend: K must be >= 1");
    if (d->Hq % d->Hkv) return fail(LSA_E_SHAPE, "lsa_attend: Hq=%d not a multiple of Hkv=%d", d->Hq, d->Hkv);
    const int g = d->Hq / d->Hkv;
    if (!lsa::attend_supported(d->d_qk, d->d_v, g))
        return fail(LSA_E_UNSUPPORTED, "lsa_attend: no kernel for d_qk=%d d_v=%d group=%d", d->d_qk, d->d_v, g);
    if (d->out_dtype != LSA_BF16 && d->out_dtype != LSA_F32) return fail(LSA_E_DTYPE, "lsa_attend: out must be bf16 or f32");
    const int64_t strides[] = {d->k_stride_b, d->k_stride_n, d->k_stride_h, d->v_stride_b, d->v_stride_n, d->v_stride_h,
                               d->layer_stride_k, d->layer_stride_v, d->layer_stride_q};
    for (int64_t st : strides)
        if (st < 0 || st % 8) return fail(LSA_E_ALIGN, "lsa_attend: strides must be non-negative multiples of 8 elements");
    if (d->n_layers > 1 && (d->layer_stride_out % 8 || d->layer_stride_lse < 0 || d->layer_stride_out < 0))
        return fail(LSA_E_ALIGN, "lsa_attend: output layer stride must be a multiple of 8 elements");
    if (d->d_qk == 576 && (d->v != d->k || d->v_stride_b != d->k_stride_b || d->v_stride_n != d->k_stride_n ||
                           d->v_stride_h != d->k_stride_h || d->layer_stride_v != d->layer_stride_k))
        return fail(LSA_E_UNSUPPORTED, "lsa_attend: d_qk=576 is the MLA latent layout: v must alias k with equal strides");
    if ((int64_t)d->T * d->Hkv > kMaxGridY || (int64_t)d->B * d->n_layers > kMaxGridY)
        return fail(LSA_E_UNSUPPORTED, "lsa_attend: grid too large");
    if (d->n_splits < 0) return fail(LSA_E_SHAPE, "lsa_attend: n_splits must be >= 0");
    if (d->block_table) {
        if (d->page_size < 1 || d->max_pages < 1 || d->num_pages < 1)
            return fail(LSA_E_SHAPE, "lsa_attend: paged caches need page_size, max_pages, num_pages >= 1");
        if ((int64_t)d->num_pages * d->page_size > INT32_MAX)
            return fail(LSA_E_SHAPE, "lsa_attend: page pool of %lld rows above 2^31 - 1",
                        (long long)d->num_pages * d->page_size);
    }
    a = lsa::AttendArgs{};
    a.B = d->B;
    a.T = d->T;
    a.N = d->N;
    a.Hq = d->Hq;
    a.Hkv = d->Hkv;
    a.d_qk = d->d_qk;
    a.d_v = d->d_v;
    a.q = reinterpret_cast<const uint16_t *>(d->q);
    a.k = reinterpret_cast<const uint16_t *>(d->k);
    a.ksb = d->k_stride_b;
    a.ksn = d->k_stride_n;
    a.ksh = d->k_stride_h;
    a.v = reinterpret_cast<const uint16_t *>(d->v);
    a.vsb = d->v_stride_b;
    a.vsn = d->v_stride_n;
    a.vsh = d->v_stride_h;
    a.idx = d->idx;
    a.K = d->K;
    a.scale = d->softmax_scale;
    a.out = d->out;
    a.out_f32 = d->out_dtype == LSA_F32;
    a.lse = d->lse;
    a.L = d->n_layers;
    a.lsq = d->layer_stride_q;
    a.lsk = d->layer_stride_k;
    a.lsv = d->layer_stride_v;
    a.lso = d->layer_stride_out;
    a.lsl = d->layer_stride_lse;
    a.idx_shared = d->idx_shared != 0;
    a.ctx_len = d->idx_shared ? d->ctx_len : nullptr;
    a.bt = d->block_table;
    a.page_size = d->block_table ? d->page_size : 1;
    a.max_pages = d->block_table ? d->max_pages : 0;
    a.num_pages = d->block_table ? d->num_pages : 0;
    a.n_splits = 1;
    int sp = d->n_splits > 0 ? d->n_splits : lsa::attend_default_splits(a);
    const int smin = (d->K + 2047) / 2048;
    if (smin > lsa::kAttendMaxSplits)
        return fail(LSA_E_UNSUPPORTED, "lsa_attend: K=%d above %d", d->K, 2048 * lsa::kAttendMaxSplits);
    if (sp < smin) sp = smin;
    if (sp > (d->K + 31) / 32) sp = (d->K + 31) / 32;
    if (sp > lsa::kAttendMaxSplits) sp = lsa::kAttendMaxSplits;
    a.n_splits = sp;
    return LSA_OK;
}

size_t lsa_attend_workspace_bytes(const lsa_attend_desc *d) {
    lsa::AttendArgs a;
    if (attend_check(d, a) != LSA_OK) return 0;
    return lsa::attend_workspace_bytes(a);
}

static int32_t attend_pointers(const lsa_attend_desc *d) {
    if (!d->q || !d->k || !d->v || !d->idx || !d->out) return fail(LSA_E_NULL, "lsa_attend: q, k, v, idx, out are required");
    if (!aligned16(d->q) || !aligned16(d->k) || !aligned16(d->v) || !aligned16(d->out) || !aligned4(d->idx) ||
        (d->lse && !aligned4(d->lse)))
        return fail(LSA_E_ALIGN, "lsa_attend: q, k, v, out must be 16-byte aligned");
    return LSA_OK;
}

int32_t lsa_attend(const lsa_attend_desc *d, void *ws, size_t ws_bytes, void *stream) {
    lsa::AttendArgs a;
    int32_t rc = attend_check(d, a);
    if (rc != LSA_OK) return rc;
    if ((rc = attend_pointers(d)) != LSA_OK) return rc;
    const size_t need = lsa::attend_workspace_bytes(a);
    if (need && (!ws || ws_bytes < need))
        return fail(LSA_E_WORKSPACE, "lsa_attend: workspace of %zu bytes needed, %zu given", need, ws_bytes);
    if (need && (reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
        return fail(LSA_E_ALIGN, "lsa_attend: workspace not 256-byte aligned");
    return hip_status(lsa::launch_attend(a, ws, reinterpret_cast<hipStream_t>(stream)), "lsa_attend");
}

int32_t lsa_attend_noalloc(const lsa_attend_desc *d, void *stream) {
    lsa::AttendArgs a;
    int32_t rc = attend_check(d, a);
    if (rc != LSA_OK) return rc;
    if ((rc = attend_pointers(d)) != LSA_OK) return rc;
    const size_t need = lsa::attend_workspace_bytes(a);
    if (need > lsa::kAttendStaticScratchBytes)
        return fail(LSA_E_WORKSPACE,
                    "lsa_attend_noalloc: %zu bytes of split partials needed, the static buffer holds %zu "
                    "(ask for fewer splits, or call lsa_attend with a workspace)",
                    need, lsa::kAttendStaticScratchBytes);
    void *ws = nullptr;
    if (need) {
        hipStream_t s = reinterpret_cast<hipStream_t>(stream);
        int dev = 0;
        hipError_t e = s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
        if (e == hipSuccess) e = lsa::attend_static_scratch(dev, &ws);
        if (e != hipSuccess) return hip_status(e, "lsa_attend_noalloc: static buffer");
    }
    return hip_status(lsa::launch_attend(a, ws, reinterpret_cast<hipStream_t>(stream)), "lsa_attend_noalloc");
}

int32_t lsa_select_attend(const lsa_select_desc *sd, const lsa_attend_desc *ad, void *sel_ws, size_t sel_ws_bytes,
                          void *att_ws, size_t att_ws_bytes, void *stream) {
    lsa::SelectArgs sa;
    int32_t rc = select_check(sd, sa);
    if (rc != LSA_OK) return rc;
    lsa::AttendArgs a;
    rc = attend_check(ad, a);
    if (rc != LSA_OK) return rc;
    if (sd->kept) return fail(LSA_E_UNSUPPORTED, "lsa_select_attend: no kept map (call lsa_select, then lsa_attend)");
    if (sd->B != ad->B || sd->T != ad->T || sd->N != ad->N || sd->K != ad->K)
        return fail(LSA_E_SHAPE, "lsa_select_attend: selection and attention disagree on B, T, N or K");
    if (ad->idx && ad->idx != sd->idx) return fail(LSA_E_SHAPE, "lsa_select_attend: att->idx must be NULL or sel->idx");
    if (ad->idx_shared) return fail(LSA_E_UNSUPPORTED, "lsa_select_attend: a shared index row (call lsa_select, then lsa_attend)");
    if (!sd->scores || !sd->idx || !ad->q || !ad->k || !ad->v || !ad->out)
        return fail(LSA_E_NULL, "lsa_select_attend: scores, idx, q, k, v, out are required");
    if (!aligned4(sd->scores) || !aligned4(sd->idx) || !aligned16(ad->q) || !aligned16(ad->k) || !aligned16(ad->v) ||
        !aligned16(ad->out) || (ad->lse && !aligned4(ad->lse)))
        return fail(LSA_E_ALIGN, "lsa_select_attend: misaligned scores, idx, q, k, v, out or lse");
    const size_t sneed = lsa::select_workspace_bytes(sa.B * sa.T, sa.n_cols, false);
    if (!sel_ws || sel_ws_bytes < sneed)
        return fail(LSA_E_WORKSPACE, "lsa_select_attend: selection workspace of %zu bytes needed, %zu given", sneed,
                    sel_ws_bytes);
    const size_t aneed = lsa::attend_workspace_bytes(a);
    if (aneed && (!att_ws || att_ws_bytes < aneed))
        return fail(LSA_E_WORKSPACE, "lsa_select_attend: attention workspace of %zu bytes needed, %zu given", aneed,
                    att_ws_bytes);
    if ((reinterpret_cast<uintptr_t>(sel_ws) & 255u) != 0 || (aneed && (reinterpret_cast<uintptr_t>(att_ws) & 255u) != 0))
        return fail(LSA_E_ALIGN, "lsa_select_attend: workspaces must be 256-byte aligned");
    return hip_status(lsa::launch_select_attend(sa, sel_ws, a, att_ws, reinterpret_cast<hipStream_t>(stream)),
                      "lsa_select_attend");
}

// ----------------------------------------------------------------------------- attention backward

static int32_t attend_bwd_check(const lsa_attend_bwd_desc *d, lsa::AttendBwdArgs &a) {
    if (!d) return fail(LSA_E_NULL, "lsa_attend_backward: desc is NULL");
    if (d->B < 1 || d->T < 1 || d->N < 1 || d->Hq < 1 || d->Hkv < 1)
        return fail(LSA_E_SHAPE, "lsa_attend_backward: B, T, N, Hq, Hkv must be >= 1");
    if (d->K < 1) return fail(LSA_E_BUDGET, "lsa_attend_backward: K must be >= 1");
    if (d->Hq % d->Hkv) return fail(LSA_E_SHAPE, "lsa_attend_backward: Hq=%d not a multiple of Hkv=%d", d->Hq, d->Hkv);
    const bool mla = d->d_qk == 576 && d->d_v == 512;
    if (!mla && !(d->d_qk == 128 && d->d_v == 128))
        return fail(LSA_E_UNSUPPORTED, "lsa_attend_backward: no kernel for d_qk=%d d_v=%d", d->d_qk, d->d_v);
    if (d->Hq / d->Hkv > 64) return fail(LSA_E_UNSUPPORTED, "lsa_attend_backward: more than 64 query heads per KV head");
    const int64_t strides[] = {d->k_stride_b, d->k_stride_n, d->k_stride_h, d->v_stride_b, d->v_stride_n, d->v_stride_h};
    for (int64_t st : strides)
        if (st < 0 || st % 8) return fail(LSA_E_ALIGN, "lsa_attend_backward: strides must be non-negative multiples of 8 elements");
    if (mla && (d->v != d->k || d->v_stride_b != d->k_stride_b || d->v_stride_n != d->k_stride_n ||
                d->v_stride_h != d->k_stride_h))
        return fail(LSA_E_UNSUPPORTED, "lsa_attend_backward: d_qk=576 is the MLA latent layout: v must alias k with equal strides");
    if ((int64_t)d->B * d->T > kMaxGridY || d->Hkv > kMaxGridY)
        return fail(LSA_E_UNSUPPORTED, "lsa_attend_backward: grid too large");
    a = lsa::AttendBwdArgs{};
    a.B = d->B;
    a.T = d->T;
    a.N = d->N;
    a.Hq = d->Hq;
    a.Hkv = d->Hkv;
    a.K = d->K;
    a.q = reinterpret_cast<const uint16_t *>(d->q);
    a.k = reinterpret_cast<const uint16_t *>(d->k);
    a.ksb = d->k_stride_b;
    a.ksn = d->k_stride_n;
    a.ksh = d->k_stride_h;
    a.v = reinterpret_cast<const uint16_t *>(d->v);
    a.vsb = d->v_stride_b;
    a.vsn = d->v_stride_n;
    a.vsh = d->v_stride_h;
    a.idx = d->idx;
    a.scale = d->softmax_scale;
    a.out = reinterpret_cast<const uint16_t *>(d->out);
    a.lse = d->lse;
    a.dout = reinterpret_cast<const uint16_t *>(d->dout);
    a.dq = d->dq;
    a.dk = d->dk;
    a.dv = mla ? nullptr : d->dv;
    a.mla = mla;
    return LSA_OK;
}

size_t lsa_attend_backward_workspace_bytes(const lsa_attend_bwd_desc *d) {
    lsa::AttendBwdArgs a;
    if (attend_bwd_check(d, a) != LSA_OK) return 0;
    return lsa::attend_bwd_workspace_bytes(a);
}

int32_t lsa_attend_backward(const lsa_attend_bwd_desc *d, void *ws, size_t ws_bytes, void *stream) {
    lsa::AttendBwdArgs a;
    const int32_t rc = attend_bwd_check(d, a);
    if (rc != LSA_OK) return rc;
    if (!d->q || !d->k || !d->v || !d->idx || !d->out || !d->lse || !d->dout || !d->dq || !d->dk || (!a.mla && !d->dv))
        return fail(LSA_E_NULL, "lsa_attend_backward: q, k, v, idx, out, lse, dout, dq, dk (and dv unless MLA) are required");
    if (!aligned16(d->q) || !aligned16(d->k) || !aligned16(d->v) || !aligned16(d->out) || !aligned16(d->dout) ||
        !aligned4(d->lse) || !aligned4(d->dq) || !aligned16(d->dk) || (!a.mla && !aligned16(d->dv)))
        return fail(LSA_E_ALIGN, "lsa_attend_backward: q, k, v, out, dout, dk, dv must be 16-byte aligned, lse and dq 4-byte");
    const size_t need = lsa::attend_bwd_workspace_bytes(a);
    if (!ws || ws_bytes < need)
        return fail(LSA_E_WORKSPACE, "lsa_attend_backward: workspace of %zu bytes needed, %zu given", need, ws_bytes);
    if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
        return fail(LSA_E_ALIGN, "lsa_attend_backward: workspace not 256-byte aligned");
    return hip_status(lsa::launch_attend_bwd(a, ws, reinterpret_cast<hipStream_t>(stream)), "lsa_attend_backward");
}

// ----------------------------------------------------------------------------- indexer target

int32_t lsa_index_target(const lsa_index_target_desc *d, void *stream) {
    if (!d) return fail(LSA_E_NULL, "lsa_index_target: desc is NULL");
    if (!d->q || !d->k || !d->idx || !d->lse || !d->scores || !d->target || !d->grad || !d->loss)
        return fail(LSA_E_NULL, "lsa_index_target: q, k, idx, lse, scores, target, grad, loss are required");
    if (d->B < 1 || d->T < 1 || d->N < 1 || d->Hq < 1 || d->Hkv < 1)
        return fail(LSA_E_SHAPE, "lsa_index_target: B, T, N, Hq, Hkv must be >= 1");
    if (d->K < 1) return fail(LSA_E_BUDGET, "lsa_index_target: K must be >= 1");
    if (d->Hq % d->Hkv) return fail(LSA_E_SHAPE, "lsa_index_target: Hq=%d not a multiple of Hkv=%d", d->Hq, d->Hkv);
    if (d->n_cols < d->N) return fail(LSA_E_SHAPE, "lsa_index_target: n_cols=%d below N=%d", d->n_cols, d->N);
    if (d->d_qk != 128 && d->d_qk != 576) return fail(LSA_E_UNSUPPORTED, "lsa_index_target: no kernel for d_qk=%d", d->d_qk);
    if (d->Hq / d->Hkv > 64) return fail(LSA_E_UNSUPPORTED, "lsa_index_target: more than 64 query heads per KV head");
    if ((int64_t)d->B * d->T > kMaxGridY) return fail(LSA_E_UNSUPPORTED, "lsa_index_target: grid too large");
    const int64_t strides[] = {d->k_stride_b, d->k_stride_n, d->k_stride_h};
    for (int64_t st : strides)
        if (st < 0 || st % 8) return fail(LSA_E_ALIGN, "lsa_index_target: strides must be non-negative multiples of 8 elements");
    if (!aligned16(d->q) || !aligned16(d->k) || !aligned4(d->lse) || !aligned4(d->scores) || !aligned4(d->target) ||
        !aligned4(d->grad) || !aligned4(d->loss))
        return fail(LSA_E_ALIGN, "lsa_index_target: q, k must be 16-byte aligned, fp32 arrays 4-byte");
    lsa::IndexTargetArgs a{};
    a.B = d->B;
    a.T = d->T;
    a.N = d->N;
    a.Hq = d->Hq;
    a.Hkv = d->Hkv;
    a.K = d->K;
    a.dqk = d->d_qk;
    a.q = reinterpret_cast<const uint16_t *>(d->q);
    a.k = reinterpret_cast<const uint16_t *>(d->k);
    a.ksb = d->k_stride_b;
    a.ksn = d->k_stride_n;
    a.ksh = d->k_stride_h;
    a.idx = d->idx;
    a.scale = d->softmax_scale;
    a.lse = d->lse;
    a.scores = d->scores;
    a.n_cols = d->n_cols;
    a.target = d->target;
    a.grad = d->grad;
    a.loss = d->loss;
    return hip_status(lsa::launch_index_target(a, reinterpret_cast<hipStream_t>(stream)), "lsa_index_target");
}

int32_t lsa_cache_append(const lsa_cache_append_desc *d, void *stream) {
    if (!d) return fail(LSA_E_NULL, "lsa_cache_append: desc is NULL");
    if (!d->k_new || !d->k_cache) return fail(LSA_E_NULL, "lsa_cache_append: k_new and k_cache are required");
    if (d->B < 1 || d->T < 1 || d->N < 1) return fail(LSA_E_SHAPE, "lsa_cache_append: B, T, N must be >= 1");
    if (d->k_dtype != LSA_FP8_E4M3FN && d->k_dtype != LSA_BF16)
        return fail(LSA_E_DTYPE, "lsa_cache_append: the key cache must be fp8-e4m3fn or bf16");
    const bool fp8 = d->k_dtype == LSA_FP8_E4M3FN;
    if (fp8 && !d->k_scale) return fail(LSA_E_NULL, "lsa_cache_append: fp8 keys need k_scale");
    if (d->D != 64 && d->D != 128) return fail(LSA_E_UNSUPPORTED, "lsa_cache_append: D must be 64 or 128");
    if (d->n_rows < 0 || d->n_rows > 2) return fail(LSA_E_SHAPE, "lsa_cache_append: n_rows must be 0, 1 or 2");
    if (d->B > kMaxGridY) return fail(LSA_E_UNSUPPORTED, "lsa_cache_append: B too large");
    if (!aligned16(d->k_new) || !aligned16(d->k_cache) || (fp8 && !aligned4(d->k_scale)))
        return fail(LSA_E_ALIGN, "lsa_cache_append: k_new and k_cache must be 16-byte aligned");
    for (int i = 0; i < d->n_rows; ++i) {
        if (!d->rows_new[i] || !d->rows_cache[i]) return fail(LSA_E_NULL, "lsa_cache_append: row set %d is NULL", i);
        if (d->row_elems[i] < 8 || d->row_elems[i] % 8 || d->rows_stride_b[i] < 0 || d->rows_stride_b[i] % 8 ||
            d->rows_stride_n[i] < d->row_elems[i] || d->rows_stride_n[i] % 8)
            return fail(LSA_E_SHAPE, "lsa_cache_append: row set %d needs row_elems and strides multiples of 8 "
                        "(row stride >= row_elems)", i);
        if (!aligned16(d->rows_new[i]) || !aligned16(d->rows_cache[i]))
            return fail(LSA_E_ALIGN, "lsa_cache_append: row set %d must be 16-byte aligned", i);
    }
    if (d->kbar) {
        if (d->block_size < 1 || d->n_blocks < 1 || (int64_t)d->n_blocks * d->block_size > d->N)
            return fail(LSA_E_SHAPE, "lsa_cache_append: kbar needs block_size >= 1, 1 <= n_blocks <= N / block_size");
        if (!aligned4(d->kbar)) return fail(LSA_E_ALIGN, "lsa_cache_append: misaligned kbar");
        if ((int64_t)d->T / d->block_size + 1 > 0x7FFFFFFF) return fail(LSA_E_UNSUPPORTED, "lsa_cache_append: T too large");
    }
    lsa::CacheAppendArgs a{};
    a.B = d->B;
    a.T = d->T;
    a.N = d->N;
    a.D = d->D;
    a.pos0 = d->pos0;
    a.k_new = reinterpret_cast<const uint16_t *>(d->k_new);
    a.k_cache = d->k_cache;
    a.fp8 = fp8;
    a.k_scale = fp8 ? d->k_scale : nullptr;
    a.n_rows = d->n_rows;
    for (int i = 0; i < d->n_rows; ++i) {
        a.rows_new[i] = reinterpret_cast<const uint16_t *>(d->rows_new[i]);
        a.rows_cache[i] = reinterpret_cast<uint16_t *>(d->rows_cache[i]);
        a.row_elems[i] = d->row_elems[i];
        a.stride_b[i] = d->rows_stride_b[i];
        a.stride_n[i] = d->rows_stride_n[i];
    }
    a.kbar = d->kbar;
    a.block_size = d->kbar ? d->block_size : 1;
    a.n_blocks = d->kbar ? d->n_blocks : 0;
    return hip_status(lsa::launch_cache_append(a, reinterpret_cast<hipStream_t>(stream)), "lsa_cache_append");
}

int32_t lsa_workspace_clear(void *ptr, size_t bytes, void *stream) {
    if (bytes == 0) return LSA_OK;
    if (!ptr) return fail(LSA_E_NULL, "lsa_workspace_clear: ptr is NULL");
    if (!aligned16(ptr)) return fail(LSA_E_ALIGN, "lsa_workspace_clear: ptr must be 16-byte aligned");
    return hip_status(lsa::launch_clear(ptr, bytes, reinterpret_cast<hipStream_t>(stream)), "lsa_workspace_clear");
}

}  // extern "C"
