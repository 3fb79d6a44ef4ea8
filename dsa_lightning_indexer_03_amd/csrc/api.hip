// C ABI of the lightning-indexer library: argument checks (all on the host,
// before any launch), workspace sizing and kernel dispatch.  The entry points
// are documented in include/dsaidx.h.
#include <stdarg.h>
#include <stdio.h>

#include "device_once.h"
#include "dsaidx.h"
#include "kernels.h"

namespace {

thread_local char g_err[320];

dsaidx_status fail(dsaidx_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

dsaidx_status hip_fail(hipError_t e, const char* what) {
    return fail(DSAIDX_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

using dsaidx::kMaxTopk;
constexpr int kMaxL = 131072;
constexpr int kMaxSelectCols = 4194304;

bool prefill_is_fused(int dtype, int H, int D) {
    return (dtype == DSAIDX_BF16 || dtype == DSAIDX_FP8_E4M3) && D == 128 && H % 16 == 0 && H >= 16 && H <= 64;
}

size_t decode_score_stride(int max_ctx) { return (size_t)((max_ctx + 63) / 64) * 64; }

}  // namespace

extern "C" {

int dsaidx_version(void) { return 100; }

const char* dsaidx_status_string(int s) {
    switch (s) {
        case DSAIDX_OK: return "ok";
        case DSAIDX_ERR_NULL: return "required pointer is NULL";
        case DSAIDX_ERR_SHAPE: return "invalid or inconsistent size";
        case DSAIDX_ERR_DTYPE: return "unknown dtype";
        case DSAIDX_ERR_UNSUPPORTED: return "outside the supported ranges";
        case DSAIDX_ERR_WORKSPACE: return "workspace too small";
        case DSAIDX_ERR_HIP: return "HIP launch failed";
        default: return "unknown status";
    }
}

const char* dsaidx_last_error(void) { return g_err; }

dsaidx_status indexer_kcache_append(const void* k, int k_dtype, const int32_t* seq_ids,
                                    const int32_t* positions, const int32_t* block_table, int B,
                                    int max_pages_per_seq, uint8_t* k_cache, float* k_scale, int num_pages,
                                    int T, int D, int page_size, void* stream) {
    g_err[0] = 0;
    if (T < 0 || B < 1 || max_pages_per_seq < 1 || num_pages < 1 || D < 1 || page_size < 1)
        return fail(DSAIDX_ERR_SHAPE, "T=%d B=%d max_pages_per_seq=%d num_pages=%d D=%d page_size=%d", T, B,
                    max_pages_per_seq, num_pages, D, page_size);
    if (k_dtype != DSAIDX_F32 && k_dtype != DSAIDX_BF16 && k_dtype != DSAIDX_FP8_E4M3)
        return fail(DSAIDX_ERR_DTYPE, "k_dtype=%d", k_dtype);
    if (k_dtype == DSAIDX_FP8_E4M3) return fail(DSAIDX_ERR_UNSUPPORTED, "new keys must be bf16 or f32");
    if (D != 128) return fail(DSAIDX_ERR_UNSUPPORTED, "D=%d (128)", D);
    if (page_size != 64) return fail(DSAIDX_ERR_UNSUPPORTED, "page_size=%d (64)", page_size);
    if (T == 0) return DSAIDX_OK;
    if (!k) return fail(DSAIDX_ERR_NULL, "k is NULL");
    if (!seq_ids) return fail(DSAIDX_ERR_NULL, "seq_ids is NULL");
    if (!positions) return fail(DSAIDX_ERR_NULL, "positions is NULL");
    if (!block_table) return fail(DSAIDX_ERR_NULL, "block_table is NULL");
    if (!k_cache) return fail(DSAIDX_ERR_NULL, "k_cache is NULL");
    if (!k_scale) return fail(DSAIDX_ERR_NULL, "k_scale is NULL");
    if (!aligned16(k) || ((uintptr_t)k_cache & 7u) != 0)
        return fail(DSAIDX_ERR_UNSUPPORTED, "k must be 16-byte and k_cache 8-byte aligned");
    dsaidx::KcacheArgs a{};
    a.k = k;
    a.seq_ids = seq_ids;
    a.positions = positions;
    a.block_table = block_table;
    a.k_cache = k_cache;
    a.k_scale = k_scale;
    a.T = T;
    a.B = B;
    a.max_pages = max_pages_per_seq;
    const hipError_t e = dsaidx::launch_kcache_append(a, k_dtype == DSAIDX_BF16 ? 1 : 0, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "indexer_kcache_append");
    return DSAIDX_OK;
}

dsaidx_status indexer_topk_gather(const void* latent_cache, int row_bytes, const int32_t* block_table,
                                  int max_pages_per_seq, int num_pages, int page_size,
                                  const int32_t* topk_idx, int B, int topk, void* out, void* stream) {
    g_err[0] = 0;
    if (!latent_cache) return fail(DSAIDX_ERR_NULL, "latent_cache is NULL");
    if (!block_table) return fail(DSAIDX_ERR_NULL, "block_table is NULL");
    if (!topk_idx) return fail(DSAIDX_ERR_NULL, "topk_idx is NULL");
    if (!out) return fail(DSAIDX_ERR_NULL, "out is NULL");
    if (B < 1 || topk < 1 || max_pages_per_seq < 1 || num_pages < 1 || page_size < 1 || row_bytes < 1)
        return fail(DSAIDX_ERR_SHAPE, "B=%d topk=%d max_pages_per_seq=%d num_pages=%d page_size=%d row_bytes=%d",
                    B, topk, max_pages_per_seq, num_pages, page_size, row_bytes);
    if (page_size != 64) return fail(DSAIDX_ERR_UNSUPPORTED, "page_size=%d (64)", page_size);
    if (row_bytes % 16 != 0 || row_bytes > 65536)
        return fail(DSAIDX_ERR_UNSUPPORTED, "row_bytes=%d (a multiple of 16, at most 65536)", row_bytes);
    if (!aligned16(latent_cache) || !aligned16(out))
        return fail(DSAIDX_ERR_UNSUPPORTED, "latent_cache and out must be 16-byte aligned");
    dsaidx::GatherArgs a{};
    a.cache = reinterpret_cast<const uint8_t*>(latent_cache);
    a.block_table = block_table;
    a.idx = topk_idx;
    a.out = reinterpret_cast<uint8_t*>(out);
    a.B = B;
    a.K = topk;
    a.max_pages = max_pages_per_seq;
    a.row_bytes = row_bytes;
    const hipError_t e = dsaidx::launch_topk_gather(a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "indexer_topk_gather");
    return DSAIDX_OK;
}

dsaidx_status indexer_topk_gather_layers(const void* const* latent_caches, void* const* outs, int n_layers,
                                         int row_bytes, const int32_t* block_table, int max_pages_per_seq,
                                         int num_pages, int page_size, const int32_t* topk_idx, int B, int topk,
                                         void* stream) {
    g_err[0] = 0;
    if (!latent_caches) return fail(DSAIDX_ERR_NULL, "latent_caches is NULL");
    if (!outs) return fail(DSAIDX_ERR_NULL, "outs is NULL");
    if (!block_table) return fail(DSAIDX_ERR_NULL, "block_table is NULL");
    if (!topk_idx) return fail(DSAIDX_ERR_NULL, "topk_idx is NULL");
    if (n_layers < 1 || B < 1 || topk < 1 || max_pages_per_seq < 1 || num_pages < 1 || page_size < 1 ||
        row_bytes < 1)
        return fail(DSAIDX_ERR_SHAPE,
                    "n_layers=%d B=%d topk=%d max_pages_per_seq=%d num_pages=%d page_size=%d row_bytes=%d",
                    n_layers, B, topk, max_pages_per_seq, num_pages, page_size, row_bytes);
    if (n_layers > dsaidx::kMaxGatherLayers)
        return fail(DSAIDX_ERR_UNSUPPORTED, "n_layers=%d (at most %d per call)", n_layers,
                    dsaidx::kMaxGatherLayers);
    if (page_size != 64) return fail(DSAIDX_ERR_UNSUPPORTED, "page_size=%d (64)", page_size);
    if (row_bytes % 16 != 0 || row_bytes > 65536)
        return fail(DSAIDX_ERR_UNSUPPORTED, "row_bytes=%d (a multiple of 16, at most 65536)", row_bytes);
    dsaidx::GatherLayersArgs a{};
    for (int l = 0; l < n_layers; ++l) {
        if (!latent_caches[l]) return fail(DSAIDX_ERR_NULL, "latent_caches[%d] is NULL", l);
        if (!outs[l]) return fail(DSAIDX_ERR_NULL, "outs[%d] is NULL", l);
        if (!aligned16(latent_caches[l]) || !aligned16(outs[l]))
            return fail(DSAIDX_ERR_UNSUPPORTED, "latent_caches[%d] and outs[%d] must be 16-byte aligned", l, l);
        a.cache[l] = reinterpret_cast<const uint8_t*>(latent_caches[l]);
        a.out[l] = reinterpret_cast<uint8_t*>(outs[l]);
    }
    a.block_table = block_table;
    a.idx = topk_idx;
    a.B = B;
    a.K = topk;
    a.max_pages = max_pages_per_seq;
    a.row_bytes = row_bytes;
    a.n_layers = n_layers;
    const hipError_t e = dsaidx::launch_topk_gather_layers(a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "indexer_topk_gather_layers");
    return DSAIDX_OK;
}

dsaidx_status dsaidx_probe_mfma(int kind, int blocks, int iters, float* out, void* stream) {
    g_err[0] = 0;
    if (!out) return fail(DSAIDX_ERR_NULL, "out is NULL");
    if (kind < 0 || kind > 2) return fail(DSAIDX_ERR_UNSUPPORTED, "kind=%d (0, 1 or 2)", kind);
    if (blocks < 1 || blocks > 65536 || iters < 1 || iters > (1 << 20))
        return fail(DSAIDX_ERR_SHAPE, "blocks=%d iters=%d", blocks, iters);
    const hipError_t e = dsaidx::launch_probe_mfma(kind, blocks, iters, out, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "dsaidx_probe_mfma");
    return DSAIDX_OK;
}

dsaidx_status dsaidx_probe_page_read(const uint8_t* k_cache, const float* k_scale, const int32_t* page_ids, int n,
                                     int blocks, float* out, void* stream) {
    g_err[0] = 0;
    if (!k_cache || !k_scale || !page_ids || !out) return fail(DSAIDX_ERR_NULL, "a required pointer is NULL");
    if (n < 1 || blocks < 1 || blocks > 65536) return fail(DSAIDX_ERR_SHAPE, "n=%d blocks=%d", n, blocks);
    if (!aligned16(k_cache)) return fail(DSAIDX_ERR_UNSUPPORTED, "k_cache must be 16-byte aligned");
    const hipError_t e =
        dsaidx::launch_probe_page_read(k_cache, k_scale, page_ids, n, blocks, out, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "dsaidx_probe_page_read");
    return DSAIDX_OK;
}

size_t topk_select_workspace_bytes(int rows, int cols, int topk) {
    (void)rows; (void)cols; (void)topk;
    return 0;
}

dsaidx_status topk_select(const float* scores, int rows, int cols, int64_t row_stride,
                          const int32_t* row_len, int topk, int32_t* idx_out, float* val_out,
                          void* workspace, size_t workspace_bytes, void* stream) {
    (void)workspace; (void)workspace_bytes;
    g_err[0] = 0;
    if (!scores) return fail(DSAIDX_ERR_NULL, "scores is NULL");
    if (!idx_out) return fail(DSAIDX_ERR_NULL, "idx_out is NULL");
    if (rows < 1 || cols < 1 || topk < 1) return fail(DSAIDX_ERR_SHAPE, "rows=%d cols=%d topk=%d must be >= 1", rows, cols, topk);
    if (row_stride < cols) return fail(DSAIDX_ERR_SHAPE, "row_stride=%lld < cols=%d", (long long)row_stride, cols);
    if (topk > kMaxTopk) return fail(DSAIDX_ERR_UNSUPPORTED, "topk=%d > %d", topk, kMaxTopk);
    if (cols > kMaxSelectCols) return fail(DSAIDX_ERR_UNSUPPORTED, "cols=%d > %d", cols, kMaxSelectCols);
    dsaidx::SelectArgs a{};
    a.scores = scores;
    a.row_stride = row_stride;
    a.cols = cols;
    a.row_len = row_len;
    a.causal_L = 0;
    a.hist = nullptr;
    a.topk = topk;
    a.idx_out = idx_out;
    a.val_out = val_out;
    hipError_t e = dsaidx::launch_topk_select(a, rows, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "topk_select");
    return DSAIDX_OK;
}

size_t indexer_prefill_workspace_bytes(int B, int L, int H, int D, int topk, int qk_dtype, int want_scores) {
    (void)topk;
    if (B < 1 || L < 1) return 0;
    if (prefill_is_fused(qk_dtype, H, D)) return dsaidx::prefill_fused_workspace_bytes(B, L, qk_dtype);
    if (want_scores) return 0;
    return (size_t)B * (size_t)L * (size_t)L * sizeof(float);
}

}  // extern "C"

// Scratch of indexer_prefill_noalloc, the entry point that allocates nothing:
// one copy of this array per device, held until the process ends.  Host code
// never uses the array's name as a device address (in host code it is only
// a stand-in); the device address comes from hipGetSymbolAddress, taken once
// per device with that device current.
static constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

dsaidx::PerDevice<void*> g_scratch_ptr;

// Workspace of one prefill call: the caller's (checked against `need`), or,
// for the entry point that allocates nothing, this device's scratch array.
dsaidx_status prefill_workspace(bool noalloc, void* workspace, size_t workspace_bytes, size_t need, void** out) {
    if (noalloc) {
        if (need > kNoAllocScratchBytes)
            return fail(DSAIDX_ERR_UNSUPPORTED,
                        "this call needs %zu bytes of scratch; indexer_prefill_noalloc holds %zu (call "
                        "indexer_prefill with a workspace instead)", need, kNoAllocScratchBytes);
        const hipError_t e =
            g_scratch_ptr.get([](int, void** p) { return hipGetSymbolAddress(p, HIP_SYMBOL(scratch)); }, out);
        if (e != hipSuccess) return hip_fail(e, "indexer_prefill_noalloc (scratch address)");
        return DSAIDX_OK;
    }
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(DSAIDX_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
    if (need > 0 && !aligned16(workspace)) return fail(DSAIDX_ERR_UNSUPPORTED, "workspace must be 16-byte aligned");
    *out = workspace;
    return DSAIDX_OK;
}

dsaidx_status prefill_run(const void* q, const float* q_scale, const void* k, const float* k_scale,
                          int qk_dtype, const float* w, int B, int L, int H, int D, int topk,
                          int32_t* topk_idx, float* topk_score, float* scores,
                          void* workspace, size_t workspace_bytes, void* stream, bool noalloc) {
    if (!q) return fail(DSAIDX_ERR_NULL, "q is NULL");
    if (!k) return fail(DSAIDX_ERR_NULL, "k is NULL");
    if (!w) return fail(DSAIDX_ERR_NULL, "w is NULL");
    if (!topk_idx) return fail(DSAIDX_ERR_NULL, "topk_idx is NULL");
    if (qk_dtype != DSAIDX_F32 && qk_dtype != DSAIDX_BF16 && qk_dtype != DSAIDX_FP8_E4M3)
        return fail(DSAIDX_ERR_DTYPE, "qk_dtype=%d", qk_dtype);
    if (qk_dtype == DSAIDX_FP8_E4M3) {
        if (!q_scale) return fail(DSAIDX_ERR_NULL, "q_scale is NULL for fp8 inputs");
        if (!k_scale) return fail(DSAIDX_ERR_NULL, "k_scale is NULL for fp8 inputs");
    } else if (q_scale || k_scale) {
        return fail(DSAIDX_ERR_SHAPE, "q_scale/k_scale must be NULL unless qk_dtype is FP8");
    }
    if (B < 1 || L < 1 || H < 1 || D < 1 || topk < 1)
        return fail(DSAIDX_ERR_SHAPE, "B=%d L=%d H=%d D=%d topk=%d must be >= 1", B, L, H, D, topk);
    if (L > kMaxL) return fail(DSAIDX_ERR_UNSUPPORTED, "L=%d > %d", L, kMaxL);
    if (H % 4 != 0 || H > 64) return fail(DSAIDX_ERR_UNSUPPORTED, "H=%d (multiple of 4 in [4, 64])", H);
    if (D != 32 && D != 64 && D != 128) return fail(DSAIDX_ERR_UNSUPPORTED, "D=%d (32, 64 or 128)", D);
    if (topk > kMaxTopk) return fail(DSAIDX_ERR_UNSUPPORTED, "topk=%d > %d", topk, kMaxTopk);
    if (!aligned16(q) || !aligned16(k)) return fail(DSAIDX_ERR_UNSUPPORTED, "q and k must be 16-byte aligned");
    if ((size_t)B * (size_t)L > (size_t)0x7FFFFFFF) return fail(DSAIDX_ERR_UNSUPPORTED, "B*L too large");

    dsaidx::PrefillArgs a{};
    a.q = q;
    a.q_scale = q_scale;
    a.k = k;
    a.k_scale = k_scale;
    a.w = w;
    a.B = B;
    a.L = L;
    a.H = H;
    a.D = D;
    a.topk = topk;
    a.inv_sqrt_d = 1.0f / sqrtf((float)D);
    a.idx_out = topk_idx;
    a.val_out = topk_score;
    a.scores = scores;
    hipStream_t st = (hipStream_t)stream;

    const size_t need = indexer_prefill_workspace_bytes(B, L, H, D, topk, qk_dtype, scores ? 1 : 0);
    void* ws = nullptr;
    const dsaidx_status wst = prefill_workspace(noalloc, workspace, workspace_bytes, need, &ws);
    if (wst != DSAIDX_OK) return wst;
    if (prefill_is_fused(qk_dtype, H, D)) {
        a.workspace = ws;
        hipError_t e = dsaidx::launch_prefill_fused(a, qk_dtype, st);
        if (e != hipSuccess) return hip_fail(e, "indexer_prefill (fused)");
        return DSAIDX_OK;
    }
    float* mat = scores ? scores : reinterpret_cast<float*>(ws);
    hipError_t e = dsaidx::launch_prefill_scores_generic(a, qk_dtype, mat, st);
    if (e != hipSuccess) return hip_fail(e, "indexer_prefill (scores)");
    dsaidx::SelectArgs s{};
    s.scores = mat;
    s.row_stride = L;
    s.cols = L;
    s.row_len = nullptr;
    s.causal_L = L;
    s.hist = nullptr;
    s.topk = topk;
    s.idx_out = topk_idx;
    s.val_out = topk_score;
    e = dsaidx::launch_topk_select(s, B * L, st);
    if (e != hipSuccess) return hip_fail(e, "indexer_prefill (select)");
    return DSAIDX_OK;
}

}  // namespace

extern "C" {

dsaidx_status indexer_prefill(const void* q, const float* q_scale, const void* k, const float* k_scale,
                              int qk_dtype, const float* w, int B, int L, int H, int D, int topk,
                              int32_t* topk_idx, float* topk_score, float* scores,
                              void* workspace, size_t workspace_bytes, void* stream) {
    g_err[0] = 0;
    return prefill_run(q, q_scale, k, k_scale, qk_dtype, w, B, L, H, D, topk, topk_idx, topk_score, scores,
                       workspace, workspace_bytes, stream, false);
}

size_t indexer_prefill_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

dsaidx_status indexer_prefill_noalloc(const void* q, const float* q_scale, const void* k, const float* k_scale,
                                      int qk_dtype, const float* w, int B, int L, int H, int D, int topk,
                                      int32_t* topk_idx, float* topk_score, float* scores, void* stream) {
    g_err[0] = 0;
    return prefill_run(q, q_scale, k, k_scale, qk_dtype, w, B, L, H, D, topk, topk_idx, topk_score, scores,
                       nullptr, 0, stream, true);
}

size_t indexer_prefill_chunk_paged_workspace_bytes(int B, int T, int max_kv_len, int q_dtype) {
    if (B < 1 || T < 1 || max_kv_len < 1) return 0;
    if (q_dtype == DSAIDX_BF16) return dsaidx::prefill_bf16_varlen_workspace_bytes(B, T, max_kv_len);
    return dsaidx::prefill_ws_workspace_bytes(B, max_kv_len, (T + 7) / 8 + B);
}

dsaidx_status indexer_prefill_chunk_paged(const void* q, const float* q_scale, int q_dtype, const float* w,
                                          const int32_t* cu_seqlens_q, const int32_t* q_start,
                                          const uint8_t* k_cache, const float* k_scale,
                                          const int32_t* block_table, int max_pages_per_seq, int num_pages,
                                          int B, int T, int max_kv_len, int H, int D, int page_size, int topk,
                                          int32_t* topk_idx, float* topk_score,
                                          void* workspace, size_t workspace_bytes, void* stream) {
    g_err[0] = 0;
    if (!q) return fail(DSAIDX_ERR_NULL, "q is NULL");
    if (!w) return fail(DSAIDX_ERR_NULL, "w is NULL");
    if (!cu_seqlens_q) return fail(DSAIDX_ERR_NULL, "cu_seqlens_q is NULL");
    if (!q_start) return fail(DSAIDX_ERR_NULL, "q_start is NULL");
    if (!k_cache) return fail(DSAIDX_ERR_NULL, "k_cache is NULL");
    if (!k_scale) return fail(DSAIDX_ERR_NULL, "k_scale is NULL");
    if (!block_table) return fail(DSAIDX_ERR_NULL, "block_table is NULL");
    if (!topk_idx) return fail(DSAIDX_ERR_NULL, "topk_idx is NULL");
    if (q_dtype != DSAIDX_F32 && q_dtype != DSAIDX_BF16 && q_dtype != DSAIDX_FP8_E4M3)
        return fail(DSAIDX_ERR_DTYPE, "q_dtype=%d", q_dtype);
    if (B < 1 || T < 1 || max_kv_len < 1 || H < 1 || D < 1 || page_size < 1 || topk < 1 || max_pages_per_seq < 1 ||
        num_pages < 1)
        return fail(DSAIDX_ERR_SHAPE, "B=%d T=%d max_kv_len=%d H=%d D=%d page_size=%d topk=%d max_pages_per_seq=%d "
                    "num_pages=%d", B, T, max_kv_len, H, D, page_size, topk, max_pages_per_seq, num_pages);
    if ((int64_t)max_kv_len > (int64_t)max_pages_per_seq * page_size)
        return fail(DSAIDX_ERR_SHAPE, "max_kv_len = %d > max_pages_per_seq * page_size = %lld", max_kv_len,
                    (long long)max_pages_per_seq * page_size);
    if (q_dtype == DSAIDX_F32) return fail(DSAIDX_ERR_UNSUPPORTED, "chunk queries must be fp8 or bf16");
    if (q_dtype == DSAIDX_FP8_E4M3 && !q_scale) return fail(DSAIDX_ERR_NULL, "q_scale is NULL (fp8 queries)");
    if (q_dtype == DSAIDX_BF16 && q_scale)
        return fail(DSAIDX_ERR_UNSUPPORTED, "q_scale must be NULL for bf16 queries");
    if (H % 16 != 0 || H > 64) return fail(DSAIDX_ERR_UNSUPPORTED, "H=%d (16, 32, 48 or 64)", H);
    if (D != 128) return fail(DSAIDX_ERR_UNSUPPORTED, "D=%d (128)", D);
    if (page_size != 64) return fail(DSAIDX_ERR_UNSUPPORTED, "page_size=%d (64)", page_size);
    if (topk > kMaxTopk) return fail(DSAIDX_ERR_UNSUPPORTED, "topk=%d > %d", topk, kMaxTopk);
    if (max_kv_len > kMaxL) return fail(DSAIDX_ERR_UNSUPPORTED, "max_kv_len=%d > %d", max_kv_len, kMaxL);
    if ((int64_t)T + 8 * (int64_t)B > (int64_t)0x7FFFFFFF) return fail(DSAIDX_ERR_UNSUPPORTED, "T too large");
    if (!aligned16(q) || !aligned16(k_cache)) return fail(DSAIDX_ERR_UNSUPPORTED, "q and k_cache must be 16-byte aligned");
    if (!aligned16(workspace)) return fail(DSAIDX_ERR_UNSUPPORTED, "workspace must be 16-byte aligned");
    const size_t need = indexer_prefill_chunk_paged_workspace_bytes(B, T, max_kv_len, q_dtype);
    if (!workspace || workspace_bytes < need)
        return fail(DSAIDX_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
    dsaidx::PrefillArgs a{};
    a.q = q;
    a.q_scale = q_scale;
    a.k = k_cache;
    a.k_scale = k_scale;
    a.w = w;
    a.B = B;
    a.L = 0;
    a.H = H;
    a.D = D;
    a.topk = topk;
    a.inv_sqrt_d = 1.0f / sqrtf((float)D);
    a.idx_out = topk_idx;
    a.val_out = topk_score;
    a.scores = nullptr;
    a.workspace = workspace;
    a.block_table = block_table;
    a.max_pages = max_pages_per_seq;
    a.cu_q = cu_seqlens_q;
    a.q_start = q_start;
    a.T = T;
    a.max_kv = max_kv_len;
    const hipError_t e = q_dtype == DSAIDX_BF16 ? dsaidx::launch_prefill_bf16_varlen(a, (hipStream_t)stream)
                                                : dsaidx::launch_prefill_ws_varlen(a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "indexer_prefill_chunk_paged");
    return DSAIDX_OK;
}

size_t indexer_decode_paged_workspace_bytes(int B, int max_context_len, int H, int D, int topk) {
    (void)H; (void)D; (void)topk;
    if (B < 1 || max_context_len < 0) return 0;
    // candidate scores and positions: [B][stride] each; per-query counters
    // [B][kCtrlStride]; page prefix over queries [B+1].
    return (size_t)B * decode_score_stride(max_context_len) * 8u +
           (size_t)B * dsaidx::kCtrlStride * sizeof(uint32_t) +
           (size_t)(B + 1) * sizeof(int32_t);
}

dsaidx_status indexer_decode_paged(const void* q, int q_dtype, const float* w,
                                   const uint8_t* k_cache, const float* k_scale,
                                   const int32_t* block_table, int max_pages_per_seq,
                                   const int32_t* context_lens, int max_context_len,
                                   int B, int H, int D, int page_size, int num_pages, int topk,
                                   int32_t* topk_idx, float* topk_score,
                                   void* workspace, size_t workspace_bytes, void* stream) {
    g_err[0] = 0;
    if (!q) return fail(DSAIDX_ERR_NULL, "q is NULL");
    if (!w) return fail(DSAIDX_ERR_NULL, "w is NULL");
    if (!k_cache) return fail(DSAIDX_ERR_NULL, "k_cache is NULL");
    if (!k_scale) return fail(DSAIDX_ERR_NULL, "k_scale is NULL");
    if (!block_table) return fail(DSAIDX_ERR_NULL, "block_table is NULL");
    if (!context_lens) return fail(DSAIDX_ERR_NULL, "context_lens is NULL");
    if (!topk_idx) return fail(DSAIDX_ERR_NULL, "topk_idx is NULL");
    if (q_dtype != DSAIDX_F32 && q_dtype != DSAIDX_BF16 && q_dtype != DSAIDX_FP8_E4M3)
        return fail(DSAIDX_ERR_DTYPE, "q_dtype=%d", q_dtype);
    if (B < 1 || H < 1 || D < 1 || page_size < 1 || num_pages < 1 || max_pages_per_seq < 1 || topk < 1 ||
        max_context_len < 0)
        return fail(DSAIDX_ERR_SHAPE, "B=%d H=%d D=%d page_size=%d num_pages=%d max_pages_per_seq=%d topk=%d "
                    "max_context_len=%d", B, H, D, page_size, num_pages, max_pages_per_seq, topk, max_context_len);
    if ((int64_t)max_context_len > (int64_t)max_pages_per_seq * page_size)
        return fail(DSAIDX_ERR_SHAPE, "max_context_len=%d > max_pages_per_seq*page_size=%lld", max_context_len,
                    (long long)max_pages_per_seq * page_size);
    if (q_dtype != DSAIDX_BF16) return fail(DSAIDX_ERR_UNSUPPORTED, "decode queries must be bf16");
    if (H % 16 != 0 || H > 64) return fail(DSAIDX_ERR_UNSUPPORTED, "H=%d (16, 32, 48 or 64)", H);
    if (D != 128) return fail(DSAIDX_ERR_UNSUPPORTED, "D=%d (128)", D);
    if (page_size != 64) return fail(DSAIDX_ERR_UNSUPPORTED, "page_size=%d (64)", page_size);
    if (topk > kMaxTopk) return fail(DSAIDX_ERR_UNSUPPORTED, "topk=%d > %d", topk, kMaxTopk);
    if (max_context_len > kMaxSelectCols) return fail(DSAIDX_ERR_UNSUPPORTED, "max_context_len too large");
    if (!aligned16(q) || !aligned16(k_cache)) return fail(DSAIDX_ERR_UNSUPPORTED, "q and k_cache must be 16-byte aligned");
    if (!aligned16(workspace)) return fail(DSAIDX_ERR_UNSUPPORTED, "workspace must be 16-byte aligned");
    const size_t need = indexer_decode_paged_workspace_bytes(B, max_context_len, H, D, topk);
    if (!workspace || workspace_bytes < need)
        return fail(DSAIDX_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);

    hipStream_t st = (hipStream_t)stream;
    const size_t stride = decode_score_stride(max_context_len);
    char* wp = reinterpret_cast<char*>(workspace);
    float* cand_score = reinterpret_cast<float*>(wp);
    int32_t* cand_pos = reinterpret_cast<int32_t*>(wp + (size_t)B * stride * 4);
    uint32_t* ctrl = reinterpret_cast<uint32_t*>(wp + (size_t)B * stride * 8);  // [B][kCtrlStride]
    int32_t* prefix = reinterpret_cast<int32_t*>(ctrl + (size_t)B * dsaidx::kCtrlStride);
    hipError_t e;
    // Exact selection over each query's candidates (every score that can
    // be selected is among them), run by the scan's final kernel.
    dsaidx::SelectArgs s{};
    s.scores = cand_score;
    s.row_stride = (int64_t)stride;
    s.cols = (int)(stride > 0 ? stride : 1);
    s.row_len = reinterpret_cast<const int32_t*>(ctrl + 1);
    s.counter_stride = dsaidx::kCtrlStride;
    s.level0_bin = nullptr;
    s.causal_L = 0;
    s.pos = cand_pos;
    s.hist = nullptr;
    s.pre_count = nullptr;
    s.total = context_lens;
    s.total_max = max_context_len;
    s.topk = topk;
    s.idx_out = topk_idx;
    s.val_out = topk_score;
    if (max_context_len > 0) {
        dsaidx::DecodeArgs d{};
        d.q = reinterpret_cast<const uint16_t*>(q);
        d.w = w;
        d.k_cache = k_cache;
        d.k_scale = k_scale;
        d.block_table = block_table;
        d.max_pages = max_pages_per_seq;
        d.context_lens = context_lens;
        d.max_ctx = max_context_len;
        d.B = B;
        d.topk = topk;
        d.inv_sqrt_d = 1.0f / sqrtf((float)D);
        d.ctrl = ctrl;
        d.prefix = prefix;
        d.cand_score = cand_score;
        d.cand_pos = cand_pos;
        d.cand_stride = (int64_t)stride;
        e = dsaidx::launch_decode_scan(d, s, H, st);
        if (e != hipSuccess) return hip_fail(e, "indexer_decode_paged (scan)");
    } else {
        e = dsaidx::launch_zero_u32(ctrl, (size_t)B * dsaidx::kCtrlStride, st);
        if (e != hipSuccess) return hip_fail(e, "indexer_decode_paged (clear)");
        e = dsaidx::launch_topk_select(s, B, st);
        if (e != hipSuccess) return hip_fail(e, "indexer_decode_paged (select)");
    }
    return DSAIDX_OK;
}

}  // extern "C"
