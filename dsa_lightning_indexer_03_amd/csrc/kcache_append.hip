// Indexer K-cache write path: per-token FP8 (E4M3FN) quantisation of new
// keys and their append into the paged cache that the decode scan reads.
//
// The pages keep the indexer's keys in an FP8 cache of its own, written once
// per token and read by every later step ("Lightning Indexer explained",
// sections 2.1 and 2.4 of the decode walkthrough and section 5; "Study MLA
// Indexer", data-flow diagram and the notes on its two caches).  This
// library's reading of what they leave open:
//   scale  = absmax(key) / 448 in fp32 (1 for an all-zero key);
//   code_d = the E4M3FN value nearest to key_d / scale (a binary32
//            quotient), ties to even, magnitudes above 448 saturated;
//   the key of sequence b at position p goes to page block_table[b][p / 64],
//   slot p % 64.
//
// Layout: 16 lanes per key, so a wave quantises four 128-wide keys at once.
// Each lane holds 8 elements (16 bytes of bf16 or 32 of f32), the absmax is
// a 16-lane xor reduction, and each lane stores 8 codes (8 bytes) of the
// 128-byte row; the first lane of the 16 stores the scale.  Every lane group
// takes two keys, with all their loads issued before either is used, and
// the grid covers all keys in one pass (measured on 8.4M keys: two keys per
// group beat one, four and eight -- registers against loads in flight --
// and a grid-stride loop over fewer workgroups was slower).
// The hardware conversion rounds to nearest even; values are clamped to
// +-448 first, so none overflows.  The quotient must be the correctly
// rounded one (a plain reciprocal multiply can land on the other side of a
// code midpoint): one correctly rounded reciprocal per key and two fma
// corrections per element give it (see the kernel).  HBM bound: per key 256 bytes
// (bf16) or 512 (f32) of key and 8 of placement read, 132 written.
#include "common.h"
#include "kernels.h"

namespace dsaidx {
namespace {

constexpr int kD = 128;
constexpr int kPage = 64;
constexpr int kThreads = 256;
constexpr int kUnroll = 2;  // keys per lane group

template <int DT>  // 0 = f32, 1 = bf16
__device__ __forceinline__ void load_key(const KcacheArgs& a, int64_t i, int l16, float (&x)[8]) {
    if constexpr (DT == 1) {
        const v4i u = *reinterpret_cast<const v4i*>(reinterpret_cast<const uint16_t*>(a.k) + i * kD + 8 * l16);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[2 * j] = __uint_as_float((uint32_t)u[j] << 16);
            x[2 * j + 1] = __uint_as_float((uint32_t)u[j] & 0xFFFF0000u);
        }
    } else {
        const float* p = reinterpret_cast<const float*>(a.k) + i * kD + 8 * l16;
        const v4f lo = *reinterpret_cast<const v4f*>(p);
        const v4f hi = *reinterpret_cast<const v4f*>(p + 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[j] = lo[j];
            x[4 + j] = hi[j];
        }
    }
}

template <int DT>
__global__ void __launch_bounds__(kThreads)
kcache_append_kernel(KcacheArgs a) {
    const int l16 = threadIdx.x & 15;
    const int64_t g0 = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 4;  // this lane group
    const int64_t G = ((int64_t)gridDim.x * kThreads) >> 4;                   // lane groups in the grid
    const int64_t limit = (int64_t)a.max_pages * kPage;
    for (int64_t i0 = g0; i0 < a.T; i0 += kUnroll * G) {
        // the keys i0 + u*G: placement words first, then the rows, then the page ids
        int b[kUnroll], p[kUnroll];
        bool ok[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t i = i0 + u * G;
            b[u] = i < a.T ? a.seq_ids[i] : -1;
            p[u] = i < a.T ? a.positions[i] : -1;
        }
        float x[kUnroll][8];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t i = i0 + u * G;
            if (i < a.T) load_key<DT>(a, i, l16, x[u]);
            else
#pragma unroll
                for (int j = 0; j < 8; ++j) x[u][j] = 0.f;
        }
        int64_t row[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            ok[u] = b[u] >= 0 && b[u] < a.B && p[u] >= 0 && (int64_t)p[u] < limit;
            row[u] = ok[u] ? (int64_t)a.block_table[(int64_t)b[u] * a.max_pages + p[u] / kPage] * kPage + p[u] % kPage
                           : 0;
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            float m = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(x[u][j]));
#pragma unroll
            for (int d = 8; d >= 1; d >>= 1) m = fmaxf(m, __shfl_xor(m, d, 16));
            const float scale = m > 0.f ? m / 448.f : 1.f;
            float q[8];
            if (scale >= 0x1p-80f && scale <= 0x1p+80f) {
                // RN(x / scale) from y = RN(1 / scale) (one correctly rounded
                // division per key): q0 = RN(x y) lies within 1.5 ulp of
                // x / scale; one correction q1 = RN(q0 + r0 y) with the
                // remainder r0 = x - scale q0 taken in an fma is within half an
                // ulp plus a few 2^-24 ulp, so faithful; the remainder of a
                // faithful quotient is exact, and one more correction from it
                // gives the correctly rounded quotient (Markstein's theorem for
                // a correctly rounded reciprocal).  No step overflows (|x y| <=
                // 448.1) and the remainders stay off the subnormal grid for
                // |x| >= 2^-100; below that the quotient is under 2^-19, whose
                // E4M3 code is a signed zero on any path.  The sign is put back
                // for x = -0, which the corrections turn into +0.
                const float y = 1.f / scale;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float xv = x[u][j];
                    const float q0 = xv * y;
                    const float q1 = fmaf(fmaf(-scale, q0, xv), y, q0);
                    const float q2 = fmaf(fmaf(-scale, q1, xv), y, q1);
                    q[j] = fminf(fmaxf(__builtin_copysignf(q2, xv), -448.f), 448.f);
                }
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) q[j] = fminf(fmaxf(x[u][j] / scale, -448.f), 448.f);
            }
            int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
            w0 = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], w0, true);
            int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(q[4], q[5], 0, false);
            w1 = __builtin_amdgcn_cvt_pk_fp8_f32(q[6], q[7], w1, true);
            if (ok[u]) {
                *reinterpret_cast<uint2*>(a.k_cache + row[u] * kD + 8 * l16) = uint2{(uint32_t)w0, (uint32_t)w1};
                if (l16 == 0) a.k_scale[row[u]] = scale;
            }
        }
    }
}

}  // namespace

hipError_t launch_kcache_append(const KcacheArgs& a, int dtype, hipStream_t stream) {
    if (a.T <= 0) return hipSuccess;
    // 16 lanes per key, kUnroll keys per lane group: every key in one pass
    // (at most 2^26 workgroups for T < 2^31)
    const int64_t blocks = (a.T * 16 + kThreads * kUnroll - 1) / (kThreads * kUnroll);
    if (dtype == 1)
        hipLaunchKernelGGL(kcache_append_kernel<1>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(kcache_append_kernel<0>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace dsaidx
