// Decode-step scan of a paged FP8 indexer key cache.
//
// One query per decode step scores every position of its cached context
// (the decode walkthrough of "Lightning Indexer explained", section 2: one
// dot of the current query against the whole indexer cache).  The scan is
// bound by the cache bytes it streams (128 fp8 bytes + a 4-byte scale per
// position), so the kernel is laid out for HBM:
//
// * grid = (ceil(max_ctx / 4096), B): each workgroup scans a 4096-position
//   split of one query's context; each of its 4 waves takes whole 64-token
//   pages, page by page.
// * A page's 16-key subtile is 16 rows x 128 B = 2 KB contiguous; lane
//   (n = lane % 16, g = lane / 16) loads the 32 bytes [32g, 32g+32) of row n
//   with two 16-byte loads, so a wave's loads are fully coalesced.
// * fp8 keys are widened to bf16 in registers (exact: every E4M3 value is a
//   bf16 value) and the query's heads go through bf16 MFMA 16x16x32 with the
//   head index on M and the key on N.  The query stays bf16, as stored.
// * The contraction dimension is split consistently on both operands: in
//   k-step j lane group g covers the dims [32g + 8j, 32g + 8j + 8), so each
//   lane widens exactly the 32 bytes it loaded.
// * Epilogue in registers: sum over the lane's 4 head rows of
//   c[h] * max(S, 0) with c = w / sqrt(D), then a 4-way cross-lane
//   reduce-scatter (permlane32/permlane16 swaps) that leaves lane l holding
//   the score of key s0 + l of the 64-key page; times the key's fp32 scale.
// * Scores go to a [B][stride] fp32 workspace (4 bytes written per 132
//   bytes read) and into a per-workgroup LDS histogram of the first radix
//   digit, flushed to a per-query global histogram that the selector uses
//   to skip its first pass.
#include "common.h"
#include "kernels.h"

namespace dsaidx {

namespace {

constexpr int kD = 128;
constexpr int kPage = 64;
constexpr int kThreadsDec = 256;

__device__ __forceinline__ v8bf widen8(int d0, int d1) {
    uint32_t u[4] = {fp8x2_to_bf16x2<false>(d0), fp8x2_to_bf16x2<true>(d0),
                     fp8x2_to_bf16x2<false>(d1), fp8x2_to_bf16x2<true>(d1)};
    return __builtin_bit_cast(v8bf, u);
}

// Lane l (group g = l/16, column n = l%16) holds v[st] = its partial sum for
// key 16*st + n.  Returns the full sum over the 4 lane groups for key l.
__device__ __forceinline__ float reduce_scatter4(const float v[4]) {
    auto s02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[0]), __float_as_uint(v[2]), false, false);
    auto s13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[1]), __float_as_uint(v[3]), false, false);
    const float a0 = __uint_as_float(s02[0]) + __uint_as_float(s02[1]);
    const float a1 = __uint_as_float(s13[0]) + __uint_as_float(s13[1]);
    auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(a0), __float_as_uint(a1), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

template <int HB>
__global__ void __launch_bounds__(kThreadsDec)
decode_scan_kernel(DecodeArgs a) {
    __shared__ uint32_t hist[kHistBins];
    const int b = blockIdx.y;
    int ctx = a.context_lens[b];
    ctx = ctx < 0 ? 0 : (ctx > a.max_ctx ? a.max_ctx : ctx);
    const int s_begin = blockIdx.x * kDecodeSplit;
    if (s_begin >= ctx) return;
    const int s_end = min(ctx, s_begin + kDecodeSplit);
    for (int i = threadIdx.x; i < kHistBins; i += kThreadsDec) hist[i] = 0;
    __syncthreads();

    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    const int n = lane & 15, g = lane >> 4;
    constexpr int H = HB * 16;

    v8bf A[HB][4];
    const uint16_t* qb = a.q + (size_t)b * H * kD;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            A[hb][j] = *reinterpret_cast<const v8bf*>(qb + (16 * hb + n) * kD + 32 * g + 8 * j);
    float c[HB][4];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
        for (int i = 0; i < 4; ++i) c[hb][i] = a.w[(size_t)b * H + 16 * hb + 4 * g + i] * a.inv_sqrt_d;

    const int32_t* bt = a.block_table + (size_t)b * a.max_pages;
    float* out = a.scores + (size_t)b * a.score_stride;

    for (int s0 = s_begin + kPage * wave; s0 < s_end; s0 += kPage * (kThreadsDec / kWave)) {
        const int page = bt[s0 / kPage];
        const uint8_t* pbase = a.k_cache + (size_t)page * kPage * kD;
        v4i kr[4][2];
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const uint8_t* rp = pbase + (16 * st + n) * kD + 32 * g;
            kr[st][0] = *reinterpret_cast<const v4i*>(rp);
            kr[st][1] = *reinterpret_cast<const v4i*>(rp + 16);
        }
        const float kscale = a.k_scale[(size_t)page * kPage + lane];
        float part[4];
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            v4f acc[HB];
#pragma unroll
            for (int hb = 0; hb < HB; ++hb) acc[hb] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const v4i& h = kr[st][j >> 1];
                const v8bf B = widen8(h[(j & 1) * 2], h[(j & 1) * 2 + 1]);
#pragma unroll
                for (int hb = 0; hb < HB; ++hb)
                    acc[hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[hb][j], B, acc[hb], 0, 0, 0);
            }
            float p = 0.f;
#pragma unroll
            for (int hb = 0; hb < HB; ++hb)
#pragma unroll
                for (int i = 0; i < 4; ++i) p = fmaf(c[hb][i], fmaxf(acc[hb][i], 0.f), p);
            part[st] = p;
        }
        const float score = reduce_scatter4(part) * kscale;
        const int s = s0 + lane;
        if (s < s_end) {
            out[s] = score;
            atomicAdd(&hist[score_key(score) >> 21], 1u);
        }
    }
    __syncthreads();
    uint32_t* gh = a.hist + (size_t)b * kHistBins;
    for (int i = threadIdx.x; i < kHistBins; i += kThreadsDec)
        if (hist[i]) atomicAdd(&gh[i], hist[i]);
}

__global__ void zero_u32_kernel(uint32_t* p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

}  // namespace

hipError_t launch_zero_u32(uint32_t* p, size_t n, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    size_t blocks = (n + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    hipLaunchKernelGGL(zero_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n);
    return hipGetLastError();
}

hipError_t launch_decode_scan(const DecodeArgs& a, int H, int max_ctx, hipStream_t stream) {
    const dim3 grid((unsigned)((max_ctx + kDecodeSplit - 1) / kDecodeSplit), (unsigned)a.B);
    switch (H / 16) {
        case 1: hipLaunchKernelGGL(decode_scan_kernel<1>, grid, dim3(kThreadsDec), 0, stream, a); break;
        case 2: hipLaunchKernelGGL(decode_scan_kernel<2>, grid, dim3(kThreadsDec), 0, stream, a); break;
        case 3: hipLaunchKernelGGL(decode_scan_kernel<3>, grid, dim3(kThreadsDec), 0, stream, a); break;
        case 4: hipLaunchKernelGGL(decode_scan_kernel<4>, grid, dim3(kThreadsDec), 0, stream, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace dsaidx
