// Internal interface between the C-ABI layer (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsaidx {

constexpr int kHistBins = 2048;        // first radix digit: score key bits [31:21]
constexpr int kCtrlStride = 64;        // u32 words between per-query counters (own cache lines)
constexpr int kMaxTopk = 2048;          // largest k any entry point accepts

struct SelectArgs {
    const float* scores;
    int64_t row_stride;
    int cols;
    const int32_t* row_len;   // nullable: entries of row r = row_len[r * counter_stride] (else cols)
    int causal_L;             // > 0: row r has (r % causal_L) + 1 entries
    const int32_t* pos;       // nullable [rows][row_stride]: position of each entry (else its column)
    const uint32_t* hist;     // nullable [rows][kHistBins] first-digit histogram of the entries
    const uint32_t* level0_bin;  // nullable [rows * counter_stride]: every entry of row r has first
                                 // digit level0_bin[r * counter_stride] (the histogram is then skipped)
    int counter_stride;       // element stride of row_len and pre_count (0 means 1)
    const uint32_t* pre_count;  // nullable: output slots [0, pre_count[r * counter_stride]) already hold selected
                                // positions that outrank every entry of the row
    const int32_t* total;     // nullable [rows]: valid positions of the row, clamped to [0, total_max];
    int total_max;            //   the row returns min(topk, total) positions (default: its entry count)
    int topk;
    int32_t* idx_out;
    float* val_out;           // nullable
};

struct DecodeArgs {
    const uint16_t* q;        // [B][H][D] bf16
    const float* w;           // [B][H]
    const uint8_t* k_cache;   // [pages][page_size][D]
    const float* k_scale;     // [pages][page_size]
    const int32_t* block_table;
    int max_pages;
    const int32_t* context_lens;
    int max_ctx;              // context lengths are clamped to [0, max_ctx]
    int B;
    int topk;
    float inv_sqrt_d;
    uint32_t* ctrl;           // [B][kCtrlStride] per-query words: 1 = candidate count, 2 = floor key
    int32_t* prefix;          // [B+1] exclusive prefix of per-query page counts (large batches only)
    float* cand_score;        // [B][cand_stride] candidate scores
    int32_t* cand_pos;        // [B][cand_stride] candidate positions
    int64_t cand_stride;      // >= max_ctx
};

struct PrefillArgs {
    const void* q;
    const float* q_scale;
    const void* k;
    const float* k_scale;
    const float* w;
    int B, L, H, D;
    int topk;
    float inv_sqrt_d;
    int32_t* idx_out;
    float* val_out;           // nullable
    float* scores;            // nullable [B][L][L]
    void* workspace;          // prefill_fused_workspace_bytes(B, L, dtype) bytes (fused path)
    // set by the fused launcher from the workspace:
    float* ks_adj;            // [B][Lpad] key scales times 2^Pk
    uint8_t* kexp;            // [B][Lpad] E8M0 bytes 127 - Pk, lane-major within each 64-key chunk
    int Lpad;                 // keys rounded up to a multiple of 64
    // A chunk of L queries at positions q0 .. q0+L-1 against a paged fp8 key
    // cache (k = the page pool [pages][64][D], k_scale = [pages][64]); key s
    // of sequence b sits in page block_table[b][s / 64], slot s % 64.
    int q0;
    int Lk;                   // keys the chunk sees: q0 + L
    const int32_t* block_table;
    int max_pages;
    // Variable-length chunks against the paged cache: the query rows of
    // sequence b are cu_q[b] .. cu_q[b+1]-1 (T rows in all), at positions
    // q_start[b] ..; its cache holds keys 0 .. q_start[b] + (cu_q[b+1] -
    // cu_q[b]) - 1, at most max_kv keys.  `plan` (set by the launcher, in the
    // workspace) lists the 8-row blocks, heaviest first.
    const int32_t* cu_q;
    const int32_t* q_start;
    int T;
    int max_kv;
    int2* plan;
    int n_plan;
};

// Indexer K-cache write path: T new keys quantised to FP8 and appended.
struct KcacheArgs {
    const void* k;               // [T][128] bf16 bit patterns or f32
    const int32_t* seq_ids;      // [T] sequence of each key (outside [0, B): not written)
    const int32_t* positions;    // [T] its position (outside [0, max_pages * 64): not written)
    const int32_t* block_table;  // [B][max_pages] page ids
    uint8_t* k_cache;            // [num_pages][64][128] E4M3FN codes
    float* k_scale;              // [num_pages][64] one scale per cached token
    int64_t T;
    int B, max_pages;
};

// The selection's consumer: rows of a paged latent cache at selected positions.
struct GatherArgs {
    const uint8_t* cache;        // [num_pages][64][row_bytes]
    const int32_t* block_table;  // [B][max_pages] page ids
    const int32_t* idx;          // [B][K] positions (-1 or outside the table: zero row)
    uint8_t* out;                // [B][K][row_bytes]
    int B, K, max_pages, row_bytes;
};

// Index Share: the same selection gathered from several layers' latent caches.
constexpr int kMaxGatherLayers = 64;
struct GatherLayersArgs {
    const uint8_t* cache[kMaxGatherLayers];  // per layer [num_pages][64][row_bytes]
    uint8_t* out[kMaxGatherLayers];          // per layer [B][K][row_bytes]
    const int32_t* block_table;              // [B][max_pages] page ids, shared by the layers
    const int32_t* idx;                      // [B][K] positions, shared by the layers
    int B, K, max_pages, row_bytes, n_layers;
};

size_t topk_select_smem_bytes();
hipError_t launch_topk_select(const SelectArgs& a, int rows, hipStream_t stream);
hipError_t launch_zero_u32(uint32_t* p, size_t n, hipStream_t stream);
// sample and floor, main scan, then verification + repair + selection (s)
hipError_t launch_decode_scan(const DecodeArgs& a, const SelectArgs& s, int H, hipStream_t stream);
hipError_t launch_prefill_scores_generic(const PrefillArgs& a, int dtype, float* out, hipStream_t stream);
hipError_t launch_prefill_fused(const PrefillArgs& a, int dtype, hipStream_t stream);
size_t prefill_fused_workspace_bytes(int B, int L, int dtype);
// bf16 queries of variable-length chunks against the paged fp8 cache.
size_t prefill_bf16_varlen_workspace_bytes(int B, int T, int max_kv);
hipError_t launch_prefill_bf16_varlen(const PrefillArgs& a, hipStream_t stream);
// Warp-specialised fp8 prefill (csrc/prefill_ws.hip): whole sequences
// (L <= 131072) and variable-length chunks against the paged cache.
size_t prefill_ws_workspace_bytes(int B, int max_keys, int n_plan);
hipError_t launch_prefill_ws(const PrefillArgs& a, hipStream_t stream);
hipError_t launch_prefill_ws_varlen(const PrefillArgs& a, hipStream_t stream);
hipError_t launch_kcache_append(const KcacheArgs& a, int dtype, hipStream_t stream);
hipError_t launch_topk_gather(const GatherArgs& a, hipStream_t stream);
hipError_t launch_topk_gather_layers(const GatherLayersArgs& a, hipStream_t stream);
// Measurement probes (csrc/probes.hip).
hipError_t launch_probe_mfma(int kind, int blocks, int iters, float* out, hipStream_t stream);
hipError_t launch_probe_page_read(const uint8_t* k_cache, const float* k_scale, const int32_t* page_ids, int n,
                                  int blocks, float* out, hipStream_t stream);

}  // namespace dsaidx
