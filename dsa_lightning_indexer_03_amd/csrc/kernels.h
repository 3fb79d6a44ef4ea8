// Internal interface between the C-ABI layer (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsaidx {

constexpr int kHistBins = 2048;        // first radix digit: score key bits [31:21]
constexpr int kDecodeSplit = 4096;     // tokens per decode workgroup
constexpr int kFusedTokensPerBlock = 4;
constexpr int kFusedCap = 4096;        // per-row candidate buffer (entries)

struct SelectArgs {
    const float* scores;
    int64_t row_stride;
    int cols;
    const int32_t* row_len;   // nullable
    int causal_L;             // > 0: row r has (r % causal_L) + 1 valid entries
    const uint32_t* hist;     // nullable [rows][kHistBins] first-digit histogram
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
    float inv_sqrt_d;
    float* scores;            // [B][score_stride]
    int64_t score_stride;
    uint32_t* hist;           // [B][kHistBins]
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
};

size_t topk_select_smem_bytes();
hipError_t launch_topk_select(const SelectArgs& a, int rows, hipStream_t stream);
hipError_t launch_zero_u32(uint32_t* p, size_t n, hipStream_t stream);
hipError_t launch_decode_scan(const DecodeArgs& a, int H, int max_ctx, hipStream_t stream);
hipError_t launch_prefill_scores_generic(const PrefillArgs& a, int dtype, float* out, hipStream_t stream);
hipError_t launch_prefill_fused(const PrefillArgs& a, int dtype, hipStream_t stream);

}  // namespace dsaidx
