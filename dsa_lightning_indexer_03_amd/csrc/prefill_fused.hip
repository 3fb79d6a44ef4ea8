// Fused prefill: MFMA scoring + ReLU + weighted head reduction + causal mask
// + streaming top-k, with the [L, L] score matrix kept out of HBM.
//
// What is computed: for every token t and history position s <= t,
// I[t,s] = sum_i w[t,i] * ReLU(q[t,i] . k[s] / sqrt(D))  ("From principle to
// code", section 2.1; one shared key per token, "Lightning Indexer
// explained", section 4), then the top-k positions of row t by (I desc,
// s asc).  As a contraction this is Q[L*H, D] x K[L, D]^T restricted to the
// causal half; D = 128 and H is a multiple of 16.
//
// fp8 inputs, at every supported length, run in the kernel with specialised
// waves (prefill_ws.hip).  This file holds the bf16 kernel: every supported
// length (L <= 131072; positions past 65536 in the 17-bit candidate
// encoding), and chunks of bf16 queries against the paged fp8 cache.  Key
// chunks are staged through LDS once per workgroup of eight tokens, and the
// weighted head sum runs on the matrix cores (details at the kernel).
// Each wave keeps a streaming top-k for its row: a candidate buffer of
// (key, position) pairs in LDS.  A score enters the buffer only if its
// order-preserving key beats the row threshold.  When the buffer nears
// capacity it is compacted: one radix digit below the buffer's common key
// prefix locates the bin of the k-th largest key, the bin's lower edge
// becomes the new threshold and everything below it is dropped.  The buffer
// always holds every entry that can still be in the row's top k; its order
// carries no meaning (ties are broken by the stored positions).  At the end
// an exact radix select over the buffer finds the k-th largest key and ties
// at that key go to the lowest positions.
#include <type_traits>

#include "common.h"
#include "device_once.h"
#include "kernels.h"
#include "rowbuf.h"
#include "varlen.h"

namespace dsaidx {

namespace {

constexpr int kD = 128;
constexpr int pad64(int n) { return (n + 63) / 64 * 64; }

// Rank r of the speculative floor in a row's sample, from the expected
// number ec of sampled keys at or above the row's k-th largest: 3.5 standard
// deviations (plus 8) above it.  The floor fails only if the sample holds r
// keys above the k-th largest (about 1e-5 per row for the sampling model at
// ec ~ 128), and a failed floor is caught and rescanned.  A wider margin
// leaves long rows near their buffer's capacity, so they compact more.
__device__ __forceinline__ uint32_t spec_rank(float ec) {
    return (uint32_t)ceilf(ec + 3.5f * sqrtf(ec) + 8.f);
}


// ---------------------------------------------------------------------------
// bf16 queries, keys staged through LDS, head sums on the matrix cores: whole
// sequences of bf16 keys (L <= 131072), and chunks of bf16 queries against
// the paged fp8 key cache (variable length, positions up to 131072).
//
// The 8 waves of a workgroup (8 consecutive query rows of one sequence, all
// with the same last 64-key chunk) walk the key chunks in lockstep: every
// chunk is fetched from L2 once per workgroup with direct global->LDS loads
// (no VGPRs in flight), rows stored with their 16-byte pieces XOR-swizzled
// so the MFMA operand reads spread over the LDS banks.
//
// Epilogue.  The score of key s is sum_h c_h max(S_h, 0) times the key's
// scale (1 for bf16 keys), with c_h = w_h / sqrt(D) and S_h the dot product
// of the stored values.  |S_h| <= |q_h|_1 * max_d |k_d| <= 2^Pq_h * 2^Pk,
// with Pq_h taken per head of the token and Pk per key.  A key pre-pass
// writes every key times 2^-Pk to the workspace as bf16 (exact: a power of
// two), with the key's scale times 2^Pk as its adjusted scale; fp8 keys of
// the paged cache are widened to bf16 there (exact: every E4M3 value is a
// bf16 value).  Each query head's A rows are scaled by its own 2^-Pq_h in
// registers.  So the score MFMAs (bf16 x bf16 16x16x32 into fp32, four
// k-steps per 16 heads x 16 keys) leave every value in [-1, 1] at its own
// head's scale.  There the conversion to f16 with its [0, 1] clamp is
// max(S, 0) itself, rounded to nearest (relative error <= 2^-11 down to
// 2^-14 of the head's bound, however far the heads' magnitudes spread), and
// the weighted sum over heads is one more MFMA (f16, 16x16x32) with the
// weights c_h * 2^Pq_h * 2^E as its A operand.  Its weights for subtile st
// sit in the rows 4st..4st+3 only, so the four subtiles of a chunk
// accumulate into one tile whose element 0 in lane l is the score of key
// 64*chunk + l: no cross-lane reduction.  The factor 2^-E and the adjusted
// key scale finish the score.
//
// Pipeline:
// * A 64-key chunk is 16 KB.  Two stages fit the LDS beside the eight rows'
//   2560-entry candidate buffers.  One barrier per chunk, at its end: it
//   certifies that the next chunk has landed and that every wave is done
//   with this one, whose slot then receives the chunk after next.
// * A chunk runs as four regions, one 16-key subtile each: its 16 score
//   MFMAs (4 k-steps of 16x16x32 bf16 per head block), the head sums of the
//   previous subtile and a share of the previous chunk's appends, while the
//   next subtile's B operands are read from LDS.
// * A compaction request made before the barrier is read right after it and
//   acted on in the same iteration, so the buffer needs one chunk of slack.
// ---------------------------------------------------------------------------
constexpr int kBfWaves = 8;
constexpr int kBfCap = 2560;
// a row asking for compaction (count above kBfCap - 64) always takes part (count above its cut rank + 128)
static_assert(kMaxTopk + 128 < kBfCap - kWave, "the requesting row joins its compaction");
constexpr int kBfStages = 2;
constexpr size_t kBfWaveBytes = (size_t)(kBfCap + kWave) * 6 + 128 * 4;
constexpr size_t kBfStageKeyBytes = 64 * kD * 2;
constexpr size_t kBfStageScaleOff = kBfStageKeyBytes;
constexpr size_t kBfStageBytes = kBfStageKeyBytes + 64 * 4;
static_assert(kBfStages * kBfStageBytes + kBfWaves * kBfWaveBytes + 16 <= 160 * 1024, "LDS budget");

// bf16 key pre-pass: for key s of sequence b (positions up to the 64-padded
// length; rows past the end repeat row L-1): 2^Pk > max_d |k_d| (Pk = 0 for
// a zero row), the key times 2^-Pk to kscaled and 2^Pk to ks_adj.
__global__ void __launch_bounds__(256)
prefill_key_prep_bf16_kernel(PrefillArgs a, uint16_t* kscaled) {
    static_assert(kBfWaves == kBlockRows, "one query row per wave");
    const int64_t gi = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int Lp = a.Lpad;
    if (gi >= (int64_t)a.B * Lp) return;
    const int b = (int)(gi / Lp), s = (int)(gi % Lp);
    const int sr = s < a.L ? s : a.L - 1;
    const v4i* row = reinterpret_cast<const v4i*>(reinterpret_cast<const uint16_t*>(a.k) + ((size_t)b * a.L + sr) * kD);
    v4i v[kD / 8];
    uint32_t mx = 0;  // largest magnitude bit pattern: bf16 magnitudes order like their bits
#pragma unroll
    for (int c = 0; c < kD / 8; ++c) {
        v[c] = row[c];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint32_t x = (uint32_t)v[c][d] & 0x7FFF7FFFu;
            mx = max(mx, max(x & 0xFFFFu, x >> 16));
        }
    }
    const float vmax = __uint_as_float(mx << 16);
    const int pk = vmax > 0.f ? __builtin_amdgcn_frexp_expf(vmax) : 0;  // 2^pk > vmax
    a.ks_adj[gi] = ldexpf(1.0f, pk);
    v4i* dst = reinterpret_cast<v4i*>(kscaled + (size_t)gi * kD);
#pragma unroll
    for (int c = 0; c < kD / 8; ++c) {
        v4i o;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint32_t x = (uint32_t)v[c][d];
            const uint32_t lo = __float_as_uint(ldexpf(__uint_as_float(x << 16), -pk)) >> 16;
            const uint32_t hi = __float_as_uint(ldexpf(__uint_as_float(x & 0xFFFF0000u), -pk)) >> 16;
            o[d] = (int)(lo | (hi << 16));
        }
        dst[c] = o;
    }
}

// The same pre-pass for chunks against the paged fp8 cache: key s < pad64(Lk)
// of sequence b (rows past the end repeat key Lk-1) is read from its cache
// slot, widened to bf16 and scaled by 2^-Pk (both exact), and its adjusted
// scale is k_scale * 2^Pk.
__global__ void __launch_bounds__(256)
prefill_key_prep_paged_fp8_kernel(PrefillArgs a, uint16_t* kscaled) {
    const int64_t gi = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int Lp = a.Lpad;
    if (gi >= (int64_t)a.B * Lp) return;
    const int b = (int)(gi / Lp), s = (int)(gi % Lp);
    const int Lq = a.cu_q[b + 1] - a.cu_q[b];
    const int Lk = min(max(a.q_start[b], 0) + Lq, a.max_kv);
    if (Lq <= 0 || Lk <= 0 || s >= pad64(Lk)) return;
    const size_t slot = key_slot<true>(a, b, s < Lk ? s : Lk - 1);
    const v4i* row = reinterpret_cast<const v4i*>(reinterpret_cast<const uint8_t*>(a.k) + slot * kD);
    v4i v[kD / 16];
    uint32_t mx = 0;
#pragma unroll
    for (int c = 0; c < kD / 16; ++c) {
        v[c] = row[c];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint32_t x = (uint32_t)v[c][d] & 0x7F7F7F7Fu;  // magnitudes: e4m3 orders like its bits
            mx = max(mx, max(max(x & 0xFFu, (x >> 8) & 0xFFu), max((x >> 16) & 0xFFu, x >> 24)));
        }
    }
    const float vmax = __builtin_amdgcn_cvt_f32_fp8((int)mx, 0);
    const int pk = vmax > 0.f ? __builtin_amdgcn_frexp_expf(vmax) : 0;  // 2^pk > vmax
    a.ks_adj[gi] = ldexpf(a.k_scale[slot], pk);
    v4i* dst = reinterpret_cast<v4i*>(kscaled + (size_t)gi * kD);
#pragma unroll
    for (int c = 0; c < kD / 16; ++c) {
        v4i o[2];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(v[c][d], false);
            const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(v[c][d], true);
            // at most 4 significant bits, scaled by a power of two: the top
            // 16 bits of the fp32 pattern are the exact bf16 value
            const uint32_t b0 = __float_as_uint(ldexpf(lo[0], -pk)) >> 16;
            const uint32_t b1 = __float_as_uint(ldexpf(lo[1], -pk)) >> 16;
            const uint32_t b2 = __float_as_uint(ldexpf(hi[0], -pk)) >> 16;
            const uint32_t b3 = __float_as_uint(ldexpf(hi[1], -pk)) >> 16;
            o[d >> 1][2 * (d & 1)] = (int)(b0 | (b1 << 16));
            o[d >> 1][2 * (d & 1) + 1] = (int)(b2 | (b3 << 16));
        }
        dst[2 * c] = o[0];
        dst[2 * c + 1] = o[1];
    }
}

template <int HB, bool VARLEN, bool P17>
__global__ void __launch_bounds__(kBfWaves * kWave)
prefill_fused_bf16_staged_kernel(PrefillArgs a, const uint16_t* kscaled) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    __shared__ uint32_t flags[4];  // [0..2] compaction requests, [3] rescan request
    using Pos = uint16_t;
    constexpr int W = kBfWaves;
    constexpr int CAP = kBfCap;
    constexpr int H = 16 * HB;
    constexpr int NX = (HB + 1) / 2;
    Seg sg;
    if (!block_seg<VARLEN>(a, sg)) return;
    const int b = sg.b, blk = sg.blk;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
    const int tl_raw = blk * W + wave;  // the wave's row within the sequence's rows
    const bool live = tl_raw < sg.Lq;   // waves past the end only help stage keys
    const int tl = live ? tl_raw : sg.Lq - 1;
    const int t = sg.q0 + tl;           // its position
    const int tv = min(t, sg.Lk - 1);   // its last valid key
    const int last_row = min(blk * W + W - 1, sg.Lq - 1);
    // Short rows, no scores asked for: a row with at most k valid positions
    // selects all of them, so a block whose rows all qualify writes
    // positions 0 .. t, then -1, without scoring.
    if (!a.val_out && !a.scores && sg.q0 + last_row + 1 <= a.topk) {
        if (live) {
            int32_t* out = a.idx_out + (size_t)(sg.row0 + tl_raw) * a.topk;
            for (int j = lane_id(); j < a.topk; j += kWave) out[j] = j <= tv ? j : -1;
        }
        return;
    }
    const int lane = lane_id();
    const int n = lane & 15, g = lane >> 4;

    RowBuf<Pos> rb;
    unsigned char* wbase = smem_raw + kBfStages * kBfStageBytes + wave * kBfWaveBytes;
    rb.key = reinterpret_cast<uint32_t*>(wbase);
    rb.hist = reinterpret_cast<uint32_t*>(wbase + (size_t)(CAP + kWave) * 4);
    rb.pos = reinterpret_cast<Pos*>(wbase + (size_t)(CAP + kWave) * 4 + 128 * 4);

    const size_t row_t = (size_t)sg.row0 + tl;
    // Query: lane (m, g) holds, for k-step j, q[t][16hb+m][32g+8j .. +8].
    // Each head h gets its own exponent, 2^Pq_h >= |q_h|_1, its operand rows
    // are scaled by 2^-Pq_h (exact) and 2^Pq_h moves into its weight: every
    // S_h then lies in [-1, 1] at its own scale, so the f16 conversion keeps
    // its relative precision however far the heads' magnitudes spread (the
    // weights, f16 normals over 29 binades, carry the spread instead).
    v4i Aw[HB][4];
    {
        const uint16_t* qrow = reinterpret_cast<const uint16_t*>(a.q) + row_t * H * kD;
#pragma unroll
        for (int hb = 0; hb < HB; ++hb)
#pragma unroll
            for (int j = 0; j < 4; ++j) Aw[hb][j] = *reinterpret_cast<const v4i*>(qrow + (16 * hb + n) * kD + 32 * g + 8 * j);
    }
    v8h Wh[4][NX];
    float Fscale;  // 2^-E
    {
        int Pqh[HB];  // exponent of this lane's head 16hb + n
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
            float sabs = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const uint32_t x = (uint32_t)Aw[hb][j][d] & 0x7FFF7FFFu;
                    sabs += __uint_as_float(x << 16) + __uint_as_float(x & 0xFFFF0000u);
                }
            sabs += __shfl_xor(sabs, 16, kWave);
            sabs += __shfl_xor(sabs, 32, kWave);
            Pqh[hb] = sabs > 0.f ? __builtin_amdgcn_frexp_expf(sabs) : 0;  // 2^Pq_h > |q_h|_1
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const uint32_t x = (uint32_t)Aw[hb][j][d];
                    const uint32_t lo = __float_as_uint(ldexpf(__uint_as_float(x << 16), -Pqh[hb])) >> 16;
                    const uint32_t hi = __float_as_uint(ldexpf(__uint_as_float(x & 0xFFFF0000u), -Pqh[hb])) >> 16;
                    Aw[hb][j][d] = (int)(lo | (hi << 16));
                }
        }
        // head weights c_h 2^Pq_h (no query scales here); lane (m, g) of the
        // weight operand needs heads 16hb + 4g + i, whose exponents sit in
        // lane 4g + i
        float cf[HB][4];
        float mx = 0.f;
#pragma unroll
        for (int hb = 0; hb < HB; ++hb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ph = __shfl(Pqh[hb], 4 * g + i, kWave);
                cf[hb][i] = ldexpf(a.w[row_t * H + 16 * hb + 4 * g + i] * a.inv_sqrt_d, ph);
                mx = fmaxf(mx, fabsf(cf[hb][i]));
            }
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) mx = fmaxf(mx, __shfl_xor(mx, d, kWave));
        int E = mx > 0.f ? 15 - __builtin_amdgcn_frexp_expf(mx) : 0;
        E = E < -100 ? -100 : (E > 100 ? 100 : E);
        Fscale = ldexpf(1.0f, -E);
        const int own_st = n >> 2;
#pragma unroll
        for (int x = 0; x < NX; ++x) {
            v8h wv;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int hb = 2 * x + (j >> 2);
                wv[j] = hb < HB ? (_Float16)ldexpf(cf[hb < HB ? hb : 0][j & 3], E) : (_Float16)0.f;
            }
#pragma unroll
            for (int st = 0; st < 4; ++st) Wh[st][x] = st == own_st ? wv : v8h{0, 0, 0, 0, 0, 0, 0, 0};
        }
    }

    const uint16_t* kbase = kscaled + (size_t)b * a.Lpad * kD;
    const float* ksadj = a.ks_adj + (size_t)b * a.Lpad;
    const int Lk = sg.Lk;
    float* srow = (!VARLEN && a.scores && live) ? a.scores + row_t * Lk : nullptr;
    // the block's last chunk, the same for every wave of it
    const int last = min((sg.q0 + last_row) / 64, (Lk - 1) / 64);

    // Chunk order, sample and speculative floor: as in the fp8 kernel.
    const int S = last + 1 >= 32 ? (last + 1) / 16 : 0;
    auto chunk_next = [&](int i, int prev) -> int {
        if (i > last) return prev;
        if (i < S) return 16 * i + 15;
        if (i == S) return 0;
        int c = prev + 1;
        if ((c & 15) == 15 && c < 16 * S) ++c;
        return c;
    };
    const int chunk0 = S > 0 ? 15 : 0;

    // Stage slot i % 2 receives the i-th chunk of the order: thread x of the
    // block copies two 16-byte pieces (LDS piece p = x + 512c holds, in row
    // p/16, the global piece (p%16) ^ (row & 15)); wave 0 also copies the
    // chunk's 64 adjusted key scales.  The padded rows exist in the scaled
    // copy, so no clamping is needed.
    auto stage_chunk = [&](int slot, int chunk) {
        unsigned char* dst = smem_raw + slot * kBfStageBytes;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int p = (int)threadIdx.x + 512 * c;
            const int r = p >> 4;
            const uint16_t* src = kbase + (size_t)(chunk * 64 + r) * kD + 8 * ((p & 15) ^ (r & 15));
            __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(dst + 1024 * wave + 8192 * c),
                                             16, 0, 0);
        }
        if (wave == 0)
            __builtin_amdgcn_global_load_lds(ksadj + chunk * 64 + lane,
                                             (__attribute__((address_space(3))) void*)(dst + kBfStageScaleOff), 4, 0, 0);
    };
    // B operands of subtile st: k-step j = the 8 dims [32g + 8j, +8) of key
    // row 16st + n, stored at piece (4g + j) ^ n of that row.
    auto load_bsub = [&](int slot, int st, v8bf (&B_)[4]) {
        const unsigned char* cur = smem_raw + slot * kBfStageBytes + (16 * st + n) * (kD * 2);
#pragma unroll
        for (int j = 0; j < 4; ++j) B_[j] = *reinterpret_cast<const v8bf*>(cur + 16 * ((4 * g + j) ^ n));
    };
    auto load_ks = [&](int slot) {
        return *reinterpret_cast<const float*>(smem_raw + slot * kBfStageBytes + kBfStageScaleOff + 4 * lane);
    };
    auto cvt_pair = [&](const v4f (&acc)[HB], int x, int j2) -> v2h {
        const int hb = 2 * x + (j2 >> 1);
        if (hb >= HB) return v2h{0, 0};
        const v2f f = v2f{acc[hb][2 * (j2 & 1)], acc[hb][2 * (j2 & 1) + 1]};
        const v2h r = __builtin_convertvector(f, v2h);
        return __builtin_elementwise_min(__builtin_elementwise_max(r, v2h{0, 0}), v2h{1, 1});
    };
    // One region: the 4*HB score MFMAs of a subtile (operands B_, results
    // mm) and the head sums of the previous subtile ep (weights of subtile
    // EST, added to P), interleaved step by step; extra(k) after step k.
    auto region = [&](auto est, const v8bf (&B_)[4], v4f (&mm)[HB], const v4f (&ep)[HB], v4f& P, auto&& extra) {
        constexpr int NM = 4 * HB;
        constexpr int NI = NX * 5;
        constexpr int es = decltype(est)::value;
        v8h X = v8h{0, 0, 0, 0, 0, 0, 0, 0};
        // a wave inside a region issues ahead of its SIMD partner outside one
        // (measured: 2% faster here; the eight-wave fp8 kernel ran 4% slower)
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int k = 0; k < NM; ++k) {
            const int j = k / HB, hb = k % HB;
            mm[hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, Aw[hb][j]), B_[j],
                                                             j == 0 ? v4f{0.f, 0.f, 0.f, 0.f} : mm[hb], 0, 0, 0);
#pragma unroll
            for (int e = (k * NI) / NM; e < ((k + 1) * NI) / NM; ++e) {
                const int x = e / 5, it = e % 5;
                if (it < 4) {
                    const v2h r = cvt_pair(ep, x, it);
                    X[2 * it] = r[0];
                    X[2 * it + 1] = r[1];
                } else {
                    P = __builtin_amdgcn_mfma_f32_16x16x32_f16(Wh[es][x], X, P, 0, 0, 0);
                }
            }
            extra(k);
            __builtin_amdgcn_sched_barrier(0x0094);  // SALU, VMEM and LDS may cross
        }
        __builtin_amdgcn_s_setprio(0);
    };
    auto pin = [&](v4f (&acc)[HB]) {
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) asm volatile("" : "+v"(acc[hb]));
    };

    struct FinState { float score; uint32_t key; int s; bool app; uint64_t m; int below; };
    const int K = a.topk;
    int nb = 0;
    uint32_t thr = 0u;
    uint32_t thr_eff = 0u;  // thr while the wave appends, else 0xFFFFFFFF
    bool active = live;
    bool floored = false;
    uint32_t r_spec = 0;
    bool spec_ok = live && tv + 1 > 2 * K;  // speculative compaction cuts (first pass only)
    if (live && S >= 2 && tv + 1 > 2 * K) {
        const float ec = 64.f * (float)S * (float)K / (float)(tv + 1);
        r_spec = spec_rank(ec);
    }
    auto finish_piece = [&](int piece, FinState& f, int chunk, const v4f& P, float ks) {
        if (piece == 0) f.score = P[0] * (ks * Fscale);
        if (piece == 1) {
            f.s = chunk * 64 + lane;
            f.key = entry_word<P17>(f.score, (uint32_t)f.s);
        }
        if (piece == 2) f.app = (f.s <= tv) & (f.key > thr_eff);
        if (piece == 3) {
            f.m = wave_ballot(f.app);
            f.below = lanes_below(f.m);
            asm volatile("" : "+v"(f.below));  // computed by every lane: keeps the select branch-free
        }
        if (piece == 4) {
            const int o = f.app ? nb + f.below : CAP + lane;
            rb.key[o] = f.key;
            rb.pos[o] = (Pos)f.s;
            nb += __builtin_popcountll(f.m);
        }
    };
    auto finish_tail = [&](int fslot, int chunk, float score) {
        if (srow && active) {
            const int s = chunk * 64 + lane;
            if (s < Lk) srow[s] = s <= t ? score : -INFINITY;
        }
        if (active && nb > CAP - kWave && lane == 0) flags[fslot] = 1u;
    };

    if (threadIdx.x == 0) flags[3] = 0u;
    for (int pass = 0;; ++pass) {
        v4f acc0[HB], acc1[HB];
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) acc1[hb] = v4f{0.f, 0.f, 0.f, 0.f};
        v8bf Bc[4], Bn[4];
        v4f Pcur = v4f{0.f, 0.f, 0.f, 0.f};  // head sums of the chunk in progress
        float ks_prev = 0.f;
        int chunk_prev = 0;
        if (threadIdx.x < 3) flags[threadIdx.x] = 0u;
        int c_stage = chunk0;
        stage_chunk(0, c_stage);
        c_stage = chunk_next(1, c_stage);
        stage_chunk(1, c_stage);
        // chunk 0 landed: at most this wave's copies of chunk 1 in flight
        if (wave == 0) __builtin_amdgcn_s_waitcnt(0x0F73);  // vmcnt(3)
        else __builtin_amdgcn_s_waitcnt(0x0F72);            // vmcnt(2)
        __syncthreads();
        load_bsub(0, 0, Bc);
        float ks_cur = load_ks(0);
        int chunk_cur = chunk0;
        for (int i = 0; i <= last; ++i) {
            const int sl = i & 1;
            const v4f Pprev = Pcur;  // chunk i-1 still lacks its last subtile
            v4f Pfin = Pprev;
            // Region 0: subtile 0 of chunk i; head sums of subtile 3 of chunk i-1.
            __builtin_amdgcn_sched_barrier(0);
            load_bsub(sl, 1, Bn);
            region(std::integral_constant<int, 3>{}, Bc, acc0, acc1, Pfin, [](int) {});
            asm volatile("" : "+v"(Pfin));
            pin(acc0);
            __builtin_amdgcn_sched_barrier(0);
            // Region 1: subtile 1; head sums of subtile 0 (a new chunk sum);
            // appends of chunk i-1 start (discarded before the first chunk).
            const bool fin_on = i >= 1;
            const bool was_active = active;
            active = active && fin_on;
            thr_eff = active ? thr : 0xFFFFFFFFu;
            FinState fs;
            const int nb0 = nb;
            Pcur = v4f{0.f, 0.f, 0.f, 0.f};
            load_bsub(sl, 2, Bc);
            region(std::integral_constant<int, 0>{}, Bn, acc1, acc0, Pcur, [&](int k) {
                if (k == 1) finish_piece(0, fs, chunk_prev, Pfin, ks_prev);
                if (k == 2 * HB + 1) finish_piece(1, fs, chunk_prev, Pfin, ks_prev);
            });
            pin(acc1);
            __builtin_amdgcn_sched_barrier(0);
            // Region 2: subtile 2; head sums of subtile 1; the appends end.
            load_bsub(sl, 3, Bn);
            region(std::integral_constant<int, 1>{}, Bc, acc0, acc1, Pcur, [&](int k) {
                if (k == 0) finish_piece(2, fs, chunk_prev, Pfin, ks_prev);
                if (k == HB) finish_piece(3, fs, chunk_prev, Pfin, ks_prev);
                if (k == 2 * HB + 1) finish_piece(4, fs, chunk_prev, Pfin, ks_prev);
            });
            asm volatile("" : "+v"(fs.score));
            pin(acc0);
            __builtin_amdgcn_sched_barrier(0);
            active = was_active;
            if (!fin_on) nb = nb0;
            if (fin_on) finish_tail(i % 3, chunk_prev, fs.score);
            // The next chunk's copies (issued after the previous barrier) and
            // any score-matrix stores complete; the barrier then makes every
            // wave's copies visible and certifies that every wave is done
            // with this chunk's slot (subtile 3's operands are in registers).
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
            __syncthreads();
            // Compaction requests of this iteration's appends (slot i % 3,
            // set before the barrier); slot (i-1) % 3 was read by every wave
            // before it and is cleared for reuse two iterations on.
            const uint32_t flag_word = flags[i % 3];
            if (threadIdx.x == 0 && i >= 1) flags[(i + 2) % 3] = 0u;
            // Chunk i+2 goes to chunk i's slot (a clamped dummy past the end),
            // and the next chunk's first operands are read while region 3
            // multiplies.
            c_stage = chunk_next(i + 2, c_stage);
            stage_chunk(sl, c_stage);
            ks_prev = ks_cur;
            chunk_prev = chunk_cur;
            chunk_cur = chunk_next(i + 1, chunk_cur);
            if (i < last) {
                load_bsub(sl ^ 1, 0, Bc);
                ks_cur = load_ks(sl ^ 1);
            }
            // Region 3: subtile 3; head sums of subtile 2.
            __builtin_amdgcn_sched_barrier(0);
            region(std::integral_constant<int, 2>{}, Bn, acc1, acc0, Pcur, [](int) {});
            asm volatile("" : "+v"(Pcur));
            pin(acc1);
            __builtin_amdgcn_sched_barrier(0);
            // The sample's appends (order indices 0..S-1) end in iteration S:
            // the speculative floor is set before any other append.  Then the
            // cooperative compaction.
            if (i == S && r_spec != 0u && active && (uint32_t)nb > r_spec) {
                uint32_t fl;
                nb = wave_floor(rb, nb, r_spec, &fl);
                thr = fl == 0u ? 0u : fl - 1u;
                floored = true;
            }
            // A long row cuts speculatively: of the 64 i keys scanned so far
            // (order indices 0 .. i-1), about k 64 i / (t+1) belong to its
            // final top k; the cut rank is that count plus three and a half
            // standard deviations and 8 (capped at k), verified with the floor.
            if (flag_word != 0u && active) {
                uint32_t r = (uint32_t)K;
                if (spec_ok) {
                    const float row_keys = (float)(tv + 1);
                    r = min(r, spec_rank((float)K * fminf(64.f * (float)i, row_keys) / row_keys));
                }
                if (nb > (int)r + 128) {
                    bool sp;
                    nb = wave_compact(rb, nb, (uint32_t)K, &thr, CAP + 128, r, &sp);
                    floored |= sp;
                }
            }
        }
        // Head sums of the last chunk's subtile 3, then its appends.
        {
            v4f Pl = Pcur;
#pragma unroll
            for (int x = 0; x < NX; ++x) {
                v8h X;
#pragma unroll
                for (int it = 0; it < 4; ++it) {
                    const v2h r = cvt_pair(acc1, x, it);
                    X[2 * it] = r[0];
                    X[2 * it + 1] = r[1];
                }
                Pl = __builtin_amdgcn_mfma_f32_16x16x32_f16(Wh[3][x], X, Pl, 0, 0, 0);
            }
            FinState fs;
            thr_eff = active ? thr : 0xFFFFFFFFu;
#pragma unroll
            for (int p = 0; p < 5; ++p) finish_piece(p, fs, chunk_prev, Pl, ks_prev);
            // no compaction follows: the slot is not read again in this pass
            finish_tail((last + 1) % 3, chunk_prev, fs.score);
        }
        __builtin_amdgcn_s_waitcnt(0x0000);  // no stage copy or LDS read may still be in flight
        if (pass == 1) break;
        // Verification of the floor; any failing row makes the whole block
        // scan again, with only the failing waves appending.
        const bool redo = active && floored && nb < K;
        if (redo && lane == 0) flags[3] = 1u;
        __syncthreads();
        if (flags[3] == 0u) break;
        active = redo;
        if (redo) {
            nb = 0;
            thr = 0u;
            floored = false;
        }
        r_spec = 0u;
        spec_ok = false;
    }
    if (!live) return;
    if (srow) {
        for (int s = (last + 1) * 64 + lane; s < Lk; s += kWave) srow[s] = -INFINITY;
    }
    __builtin_amdgcn_wave_barrier();
    wave_emit<Pos, P17>(rb, nb, K, a.idx_out + row_t * K, a.val_out ? a.val_out + row_t * K : nullptr);
}

constexpr bool staged_bf16_path(int dtype, int L) { return dtype == 1 && L <= 131072; }

template <int HB, bool P17>
hipError_t launch_bf16_staged(const PrefillArgs& a_in, hipStream_t stream) {
    PrefillArgs a = a_in;
    a.Lpad = pad64(a.L);
    a.ks_adj = reinterpret_cast<float*>(a.workspace);
    uint16_t* kscaled = reinterpret_cast<uint16_t*>(a.ks_adj + (size_t)a.B * a.Lpad);
    {
        const int64_t n = (int64_t)a.B * a.Lpad;
        hipLaunchKernelGGL(prefill_key_prep_bf16_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a,
                           kscaled);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const size_t smem = kBfStages * kBfStageBytes + (size_t)kBfWaves * kBfWaveBytes;
    static PerDevice<int> lds_once;
    {
        hipError_t e = set_lds_limit(lds_once, (const void*)prefill_fused_bf16_staged_kernel<HB, false, P17>,
                                     (int)smem);
        if (e != hipSuccess) return e;
    }
    const int nblk = (a.L + kBfWaves - 1) / kBfWaves;
    hipLaunchKernelGGL((prefill_fused_bf16_staged_kernel<HB, false, P17>), dim3((unsigned)(nblk * a.B)),
                       dim3(kBfWaves * kWave), smem, stream, a, (const uint16_t*)kscaled);
    return hipGetLastError();
}

// Workspace of a bf16 chunk call: adjusted scales [B][pad64(max_kv)] fp32,
// scaled bf16 keys [B][pad64(max_kv)][128], the block plan.
size_t bf16_varlen_scaled_off(int B, int max_kv) { return (size_t)B * pad64(max_kv) * 4; }
size_t bf16_varlen_plan_off(int B, int max_kv) { return (size_t)B * pad64(max_kv) * (4 + 2 * kD); }

template <int HB, bool P17>
hipError_t launch_bf16_varlen(const PrefillArgs& a_in, hipStream_t stream) {
    PrefillArgs a = a_in;
    a.Lpad = pad64(a.max_kv);
    a.ks_adj = reinterpret_cast<float*>(a.workspace);
    uint16_t* kscaled = reinterpret_cast<uint16_t*>(static_cast<char*>(a.workspace) +
                                                    bf16_varlen_scaled_off(a.B, a.max_kv));
    a.n_plan = (a.T + kBlockRows - 1) / kBlockRows + a.B;
    a.plan = reinterpret_cast<int2*>(static_cast<char*>(a.workspace) + bf16_varlen_plan_off(a.B, a.max_kv));
    hipLaunchKernelGGL(varlen_plan_kernel, dim3(1), dim3(1024), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n = (int64_t)a.B * a.Lpad;
    hipLaunchKernelGGL(prefill_key_prep_paged_fp8_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a,
                       kscaled);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const size_t smem = kBfStages * kBfStageBytes + (size_t)kBfWaves * kBfWaveBytes;
    static PerDevice<int> lds_once;
    if ((e = set_lds_limit(lds_once, (const void*)prefill_fused_bf16_staged_kernel<HB, true, P17>, (int)smem)) !=
        hipSuccess)
        return e;
    hipLaunchKernelGGL((prefill_fused_bf16_staged_kernel<HB, true, P17>), dim3((unsigned)a.n_plan),
                       dim3(kBfWaves * kWave), smem, stream, a, (const uint16_t*)kscaled);
    return hipGetLastError();
}

template <int HB>
hipError_t launch_bf16(const PrefillArgs& a, hipStream_t stream) {
    if (!staged_bf16_path(1, a.L)) return hipErrorInvalidValue;
    // positions past 65536 take the 17-bit candidate encoding
    return a.L > 65536 ? launch_bf16_staged<HB, true>(a, stream) : launch_bf16_staged<HB, false>(a, stream);
}

}  // namespace

size_t prefill_fused_workspace_bytes(int B, int L, int dtype) {
    const size_t n = (size_t)B * pad64(L);
    if (dtype == 2) return prefill_ws_workspace_bytes(B, L, 0);
    if (staged_bf16_path(dtype, L)) return n * (4 + 2 * kD);      // fp32 adjusted scales, then the scaled keys
    return 0;
}

size_t prefill_bf16_varlen_workspace_bytes(int B, int T, int max_kv) {
    const size_t n_plan = (size_t)(T + kBlockRows - 1) / kBlockRows + B;
    return bf16_varlen_plan_off(B, max_kv) + n_plan * sizeof(int2);
}

hipError_t launch_prefill_bf16_varlen(const PrefillArgs& a, hipStream_t stream) {
    const bool p17 = a.max_kv > 65536;
    switch (a.H / 16) {
        case 1: return p17 ? launch_bf16_varlen<1, true>(a, stream) : launch_bf16_varlen<1, false>(a, stream);
        case 2: return p17 ? launch_bf16_varlen<2, true>(a, stream) : launch_bf16_varlen<2, false>(a, stream);
        case 3: return p17 ? launch_bf16_varlen<3, true>(a, stream) : launch_bf16_varlen<3, false>(a, stream);
        case 4: return p17 ? launch_bf16_varlen<4, true>(a, stream) : launch_bf16_varlen<4, false>(a, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_prefill_fused(const PrefillArgs& a, int dtype, hipStream_t stream) {
    if (dtype == 2) return launch_prefill_ws(a, stream);  // fp8: the kernel with specialised waves
    if (dtype == 1) {
        switch (a.H / 16) {
            case 1: return launch_bf16<1>(a, stream);
            case 2: return launch_bf16<2>(a, stream);
            case 3: return launch_bf16<3>(a, stream);
            case 4: return launch_bf16<4>(a, stream);
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace dsaidx
