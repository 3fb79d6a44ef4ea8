// Materialising prefill scorer for the shapes the fused MFMA path does not
// cover (fp32 inputs, small H or D).  Writes the full causal score matrix
// I[b][t][s] (-inf for s > t, the masking of the tutorial listing in "From
// principle to code", section 3); the selector then runs over its rows.
//
// Workgroup = 4 waves = 4 query tokens x 64 keys: wave w owns token t, lane l
// owns key s = s_base + l.  The 64 keys of the tile are decoded once into LDS
// (padded rows, no bank conflicts on the per-lane column walk); the query
// values are wave-uniform broadcasts.  Plain fp32 FMA, fp8 scales applied
// once per (t, i, s) after the dot of the raw codes.
#include "common.h"
#include "kernels.h"

namespace dsaidx {

namespace {

constexpr int kMaxD = 128;

template <int DT>
__device__ __forceinline__ float load_val(const void* base, size_t i) {
    if constexpr (DT == 0) {
        return reinterpret_cast<const float*>(base)[i];
    } else if constexpr (DT == 1) {
        return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(base)[i] << 16);
    } else {
        return __builtin_amdgcn_cvt_f32_fp8((int)reinterpret_cast<const uint8_t*>(base)[i], 0);
    }
}

template <int DT>
__global__ void __launch_bounds__(256)
prefill_scores_generic_kernel(PrefillArgs a, float* out) {
    __shared__ float kt[64][kMaxD + 1];
    const int b = blockIdx.z;
    const int s_base = blockIdx.x * 64;
    const int t0 = blockIdx.y * 4;
    const int L = a.L, H = a.H, D = a.D;
    const bool live = s_base <= t0 + 3;  // some (t, s) of the tile is causal
    if (live) {
        for (int e = threadIdx.x; e < 64 * D; e += 256) {
            const int r = e / D, cc = e % D;
            const int sr = s_base + r;
            kt[r][cc] = sr < L ? load_val<DT>(a.k, ((size_t)b * L + sr) * D + cc) : 0.f;
        }
    }
    __syncthreads();
    const int t = t0 + (int)(threadIdx.x / kWave);
    const int s = s_base + lane_id();
    if (t >= L || s >= L) return;
    float I = -INFINITY;
    if (s <= t) {
        I = 0.f;
        const size_t qrow = ((size_t)b * L + t) * H;
        const float ks = DT == 2 ? a.k_scale[(size_t)b * L + s] : 1.f;
        for (int i = 0; i < H; ++i) {
            float dot = 0.f;
            for (int cc = 0; cc < D; ++cc) dot = fmaf(load_val<DT>(a.q, (qrow + i) * D + cc), kt[lane_id()][cc], dot);
            const float qs = DT == 2 ? a.q_scale[qrow + i] : 1.f;
            I = fmaf(a.w[qrow + i], fmaxf(dot * qs * ks * a.inv_sqrt_d, 0.f), I);
        }
    }
    out[((size_t)b * L + t) * L + s] = I;
}

}  // namespace

hipError_t launch_prefill_scores_generic(const PrefillArgs& a, int dtype, float* out, hipStream_t stream) {
    const dim3 grid((unsigned)((a.L + 63) / 64), (unsigned)((a.L + 3) / 4), (unsigned)a.B);
    switch (dtype) {
        case 0: hipLaunchKernelGGL(prefill_scores_generic_kernel<0>, grid, dim3(256), 0, stream, a, out); break;
        case 1: hipLaunchKernelGGL(prefill_scores_generic_kernel<1>, grid, dim3(256), 0, stream, a, out); break;
        case 2: hipLaunchKernelGGL(prefill_scores_generic_kernel<2>, grid, dim3(256), 0, stream, a, out); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace dsaidx
