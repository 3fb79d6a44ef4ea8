// Measurement probes: what the chip delivers, on this machine, for the three
// resources the indexer's kernels are bound by.  They compute nothing of the
// method; the benchmark reports each kernel's fraction of these measured
// peaks beside its fraction of the published ones.
//
// * Matrix cores: every wave of a full grid runs long chains of the MFMA
//   shapes the kernels use -- v_mfma_scale_f32_16x16x128_f8f6f4 (fp8 x fp8,
//   E8M0 scales, the prefill's score contraction), v_mfma_f32_16x16x32_bf16
//   (the bf16 prefill and the decode scan) and v_mfma_f32_16x16x32_f16 (the
//   head sums) -- with eight independent accumulators per wave, so issue,
//   not latency, sets the rate.
// * HBM: whole 64-token pages of the fp8 key cache (8 KB of codes + 256 B of
//   scales each) read through a page list, the decode scan's access pattern
//   without its arithmetic: each wave streams its pages with four pages of
//   loads in flight, lane (n, g) loading the 32 bytes [32g, 32g+32) of row n
//   of each 16-row subtile (the scan's own layout), and folds the bytes into
//   one word so no load is dead.
#include "common.h"
#include "kernels.h"

namespace dsaidx {
namespace {

typedef _Float16 v8h_p __attribute__((ext_vector_type(8)));

constexpr int kProbeThreads = 256;
constexpr int kChains = 8;

template <int KIND>  // 0: fp8 16x16x128 scaled, 1: bf16 16x16x32, 2: f16 16x16x32
__global__ void __launch_bounds__(kProbeThreads)
probe_mfma_kernel(int iters, float* out) {
    v4f acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = v4f{0.f, 0.f, 0.f, 0.f};
    // operands of 2^-6 each (E4M3 0x08, bf16 0x3C80, f16 0x2400): every
    // accumulator stays finite over any iteration count used here
    const int a8 = 0x08080808;
    const v8i A8 = v8i{a8, a8, a8, a8, a8, a8, a8, a8};
    const uint32_t abf = 0x3C803C80u, ah = 0x24002400u;
    const v4i Abf = v4i{(int)abf, (int)abf, (int)abf, (int)abf};
    const v4i Ah = v4i{(int)ah, (int)ah, (int)ah, (int)ah};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int c = 0; c < kChains; ++c) {
            if constexpr (KIND == 0)
                acc[c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A8, A8, acc[c], 0, 0, 0, 127, 0, 127);
            else if constexpr (KIND == 1)
                acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, Abf),
                                                                 __builtin_bit_cast(v8bf, Abf), acc[c], 0, 0, 0);
            else
                acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h_p, Ah),
                                                                __builtin_bit_cast(v8h_p, Ah), acc[c], 0, 0, 0);
        }
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < kChains; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
    out[(size_t)blockIdx.x * kProbeThreads + threadIdx.x] = s;
}

constexpr int kPageBytes = 64 * 128;
constexpr int kInFlight = 4;  // pages of loads in flight per wave

__global__ void __launch_bounds__(kProbeThreads)
probe_page_read_kernel(const uint8_t* k_cache, const float* k_scale, const int32_t* page_ids, int n, float* out) {
    const int lane = lane_id();
    const int n_ = lane & 15, g = lane >> 4;
    const uint32_t lane_off = (uint32_t)(n_ * 128 + 32 * g);
    const int waves = (int)(gridDim.x * (kProbeThreads / kWave));
    const int wave = (int)(blockIdx.x * (kProbeThreads / kWave) + threadIdx.x / kWave);
    uint32_t fold = 0u;
    for (int p0 = wave * kInFlight; p0 < n; p0 += waves * kInFlight) {
        v4i v[kInFlight][4][2];
        float sc[kInFlight];
#pragma unroll
        for (int u = 0; u < kInFlight; ++u) {
            const int p = min(p0 + u, n - 1);  // past the end: the last page again
            const int page = page_ids[p];
            const uint8_t* base = k_cache + (size_t)page * kPageBytes + lane_off;
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                v[u][st][0] = *reinterpret_cast<const v4i*>(base + st * 16 * 128);
                v[u][st][1] = *reinterpret_cast<const v4i*>(base + st * 16 * 128 + 16);
            }
            sc[u] = k_scale[(size_t)page * 64 + lane];
        }
#pragma unroll
        for (int u = 0; u < kInFlight; ++u) {
#pragma unroll
            for (int st = 0; st < 4; ++st)
#pragma unroll
                for (int h = 0; h < 2; ++h) fold ^= (uint32_t)(v[u][st][h][0] ^ v[u][st][h][1] ^ v[u][st][h][2] ^ v[u][st][h][3]);
            fold ^= __float_as_uint(sc[u]);
        }
    }
    out[(size_t)blockIdx.x * kProbeThreads + threadIdx.x] = __uint_as_float(fold & 0x007FFFFFu);
}

}  // namespace

hipError_t launch_probe_mfma(int kind, int blocks, int iters, float* out, hipStream_t stream) {
    switch (kind) {
        case 0: hipLaunchKernelGGL(probe_mfma_kernel<0>, dim3(blocks), dim3(kProbeThreads), 0, stream, iters, out); break;
        case 1: hipLaunchKernelGGL(probe_mfma_kernel<1>, dim3(blocks), dim3(kProbeThreads), 0, stream, iters, out); break;
        case 2: hipLaunchKernelGGL(probe_mfma_kernel<2>, dim3(blocks), dim3(kProbeThreads), 0, stream, iters, out); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_probe_page_read(const uint8_t* k_cache, const float* k_scale, const int32_t* page_ids, int n,
                                  int blocks, float* out, hipStream_t stream) {
    hipLaunchKernelGGL(probe_page_read_kernel, dim3(blocks), dim3(kProbeThreads), 0, stream, k_cache, k_scale,
                       page_ids, n, out);
    return hipGetLastError();
}

}  // namespace dsaidx
