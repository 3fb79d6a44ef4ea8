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
// Three kernels, by dtype and length:
// * fp8, L <= 65536 (the headline path) and bf16, L <= 65536: key chunks are
//   staged through LDS once per workgroup of eight tokens, and the weighted
//   head sum runs on the matrix cores (sections further down).
// * bf16 and fp8 beyond L = 65536 (positions need 32 bits, buffers grow): the
//   unstaged kernel below, whose layout is:
// * workgroup = W independent waves; wave w owns query token t = W*blk + w and
//   all 16*HB of its heads.  Blocks are issued heaviest (largest t) first.
//   W = 4 with 4096-entry buffers and 32-bit positions (W = 8 with
//   3072-entry buffers and 16-bit positions for L <= 65536, reached only
//   when the staged kernels are switched off at build time).
// * the token's queries sit in registers as MFMA A operands for the whole
//   scan (head on M);  keys stream through registers as B operands (key on
//   N), 16 keys per subtile, 64 keys per step.  No LDS is used for keys and
//   waves never wait for each other; the four waves of a workgroup read the
//   same key rows close together in time, so the vector L1 serves most of it.
// * fp8: one v_mfma_scale_f32_16x16x128_f8f6f4 (E4M3 x E4M3, scales off) per
//   16 heads x 16 keys; bf16: four v_mfma_f32_16x16x32_bf16.  The contraction
//   dimension is split the same way on both operands: lane group g owns the
//   dims [32g, 32g+32).
// * epilogue in registers: c[t,h] * max(S, 0) summed over the lane's heads,
//   with c = w * q_scale / sqrt(D) (exact refactoring: ReLU commutes with a
//   positive scale, and the key's fp8 scale is applied once per key after
//   the head sum), then a cross-lane reduce-scatter leaves lane l with the
//   score of key s0 + l.
// All three keep a streaming top-k per wave: a per-row candidate buffer of
// (key, position) pairs in LDS, filled in position order.  A score enters the
// buffer only if its order-preserving key beats the row threshold.  When the
// buffer nears capacity it is compacted: one radix digit below the buffer's
// common key prefix locates the bin of the k-th largest key, the bin's lower
// edge becomes the new threshold and everything below it is dropped (stable,
// so the buffer stays in position order).  The buffer always holds every
// entry that can still be in the row's top k.  At the end an exact radix
// select over the buffer finds the k-th largest key and ties at that key go
// to the lowest positions.
#include <type_traits>

#include "common.h"
#include "device_once.h"
#include "kernels.h"
#include "rowbuf.h"

namespace dsaidx {

namespace {

constexpr int kD = 128;

#ifndef DSAIDX_PREFILL_DEPTH
#define DSAIDX_PREFILL_DEPTH 1   // key chunks in flight ahead of the one multiplied (1 or 2)
#endif
#ifndef DSAIDX_PREFILL_STAGED
#define DSAIDX_PREFILL_STAGED 1  // fp8 with L <= 65536: stage keys through LDS
#endif
#ifndef DSAIDX_PREFILL_WS
#define DSAIDX_PREFILL_WS 1  // fp8: the kernel with specialised waves (prefill_ws.hip), all L
#endif
#ifndef DSAIDX_PREFILL_STAGED_BF16
#define DSAIDX_PREFILL_STAGED_BF16 1  // bf16 with L <= 65536: stage keys through LDS
#endif
constexpr int kPrefetch = DSAIDX_PREFILL_DEPTH >= 2 ? 2 : 1;

template <bool POS16>
struct BufCfg {
    using Pos = typename std::conditional<POS16, uint16_t, uint32_t>::type;
    static constexpr int kWaves = POS16 ? 8 : 4;      // waves (= tokens) per workgroup
    static constexpr int kCap = POS16 ? 3072 : 4096;  // candidates per row
    static constexpr size_t kWaveBytes = (size_t)kCap * (4 + sizeof(Pos)) + 256 * 4;
};

__device__ __forceinline__ float reduce_scatter4(const float v[4]) {
    auto s02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[0]), __float_as_uint(v[2]), false, false);
    auto s13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[1]), __float_as_uint(v[3]), false, false);
    const float a0 = __uint_as_float(s02[0]) + __uint_as_float(s02[1]);
    const float a1 = __uint_as_float(s13[0]) + __uint_as_float(s13[1]);
    auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(a0), __float_as_uint(a1), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// Short-row bypass: a row with at most K valid positions selects all of
// them (positions 0 .. tp, then -1), so when no score is asked for, a block
// whose rows all qualify writes that directly and scores nothing.  Returns
// true when the block took the bypass (uniform over the block).
__device__ __forceinline__ bool short_rows_bypass(const PrefillArgs& a, int b, int blk, int W, int L, int q0,
                                                  int t_raw, bool live) {
    if (a.val_out || a.scores) return false;
    const int last_row = min(blk * W + W - 1, L - 1);
    if (q0 + last_row + 1 > a.topk) return false;
    if (live) {
        const int tp = q0 + t_raw;
        int32_t* out = a.idx_out + ((size_t)b * L + t_raw) * a.topk;
        for (int j = lane_id(); j < a.topk; j += kWave) out[j] = j <= tp ? j : -1;
    }
    return true;
}

template <int DT>  // 1 = bf16, 2 = fp8 e4m3
struct Operands;

template <>
struct Operands<2> {
    // A: lane (m, g) holds q[t][16hb+m][32g .. 32g+32) as 32 fp8 bytes.
    template <int HB>
    struct A { v8i a[HB]; };
    template <int HB>
    __device__ static void load_a(A<HB>& A_, const uint8_t* qrow0, int m, int g) {
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
            const uint8_t* p = qrow0 + (size_t)(16 * hb + m) * kD + 32 * g;
            const v4i lo = *reinterpret_cast<const v4i*>(p);
            const v4i hi = *reinterpret_cast<const v4i*>(p + 16);
            A_.a[hb] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
    }
    struct Bt { v4i lo, hi; };
    __device__ static void load_b(Bt& b, const uint8_t* krow, int g) {
        const uint8_t* p = krow + 32 * g;
        b.lo = *reinterpret_cast<const v4i*>(p);
        b.hi = *reinterpret_cast<const v4i*>(p + 16);
    }
    template <int HB>
    __device__ static void mma(v4f (&acc)[HB], const A<HB>& A_, const Bt& b) {
        const v8i bb = v8i{b.lo[0], b.lo[1], b.lo[2], b.lo[3], b.hi[0], b.hi[1], b.hi[2], b.hi[3]};
#pragma unroll
        for (int hb = 0; hb < HB; ++hb)
            acc[hb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A_.a[hb], bb, v4f{0.f, 0.f, 0.f, 0.f},
                                                                        0, 0, 0, 0, 0, 0);
    }
    static constexpr int kRowBytes = kD;
};

template <>
struct Operands<1> {
    // A: lane (m, g) holds, for k-step j, q[t][16hb+m][32g+8j .. +8] (bf16).
    template <int HB>
    struct A { v8bf a[HB][4]; };
    template <int HB>
    __device__ static void load_a(A<HB>& A_, const uint8_t* qrow0, int m, int g) {
#pragma unroll
        for (int hb = 0; hb < HB; ++hb)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                A_.a[hb][j] = *reinterpret_cast<const v8bf*>(qrow0 + ((size_t)(16 * hb + m) * kD + 32 * g + 8 * j) * 2);
    }
    struct Bt { v8bf b[4]; };
    __device__ static void load_b(Bt& b, const uint8_t* krow, int g) {
#pragma unroll
        for (int j = 0; j < 4; ++j) b.b[j] = *reinterpret_cast<const v8bf*>(krow + (32 * g + 8 * j) * 2);
    }
    template <int HB>
    __device__ static void mma(v4f (&acc)[HB], const A<HB>& A_, const Bt& b) {
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
            v4f c = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A_.a[hb][j], b.b[j], c, 0, 0, 0);
            acc[hb] = c;
        }
    }
    static constexpr int kRowBytes = kD * 2;
};

template <int DT, int HB, bool POS16>
__global__ void __launch_bounds__(BufCfg<POS16>::kWaves * kWave)
prefill_fused_kernel(PrefillArgs a) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    using Op = Operands<DT>;
    using Cfg = BufCfg<POS16>;
    using Pos = typename Cfg::Pos;
    constexpr int W = Cfg::kWaves;
    constexpr int CAP = Cfg::kCap;
    constexpr int H = 16 * HB;
    const int L = a.L;
    const int nblk = (L + W - 1) / W;
    const int b = blockIdx.x % a.B;
    const int blk = nblk - 1 - (int)(blockIdx.x / a.B);  // heaviest first
    const int wave = threadIdx.x / kWave;
    const int t = blk * W + wave;
    if (t >= L) return;
    const int lane = lane_id();
    const int n = lane & 15, g = lane >> 4;

    RowBuf<Pos> rb;
    unsigned char* wbase = smem_raw + wave * Cfg::kWaveBytes;
    rb.key = reinterpret_cast<uint32_t*>(wbase);
    rb.hist = reinterpret_cast<uint32_t*>(wbase + (size_t)CAP * 4);
    rb.pos = reinterpret_cast<Pos*>(wbase + (size_t)CAP * 4 + 256 * 4);

    const size_t row_t = (size_t)b * L + t;
    const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.k) + (size_t)b * L * Op::kRowBytes;
    typename Op::template A<HB> Aq;
    Op::template load_a<HB>(Aq, reinterpret_cast<const uint8_t*>(a.q) + row_t * H * Op::kRowBytes, n, g);

    // Head coefficients of the lane's accumulator rows: c = w * q_scale / sqrt(D)
    // (fp8) or w / sqrt(D) (bf16).  The fp8 epilogue uses the identity
    //   sum_i c_i max(S_i, 0) = 1/2 sum_i c_i |S_i| + 1/2 sum_i c_i S_i,
    // so its coefficients carry the 1/2.
    constexpr float kHalf = DT == 2 ? 0.5f : 1.0f;
    float c[HB][4];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int h = 16 * hb + 4 * g + i;
            float cf = a.w[row_t * H + h] * (a.inv_sqrt_d * kHalf);
            if constexpr (DT == 2) cf *= a.q_scale[row_t * H + h];
            c[hb][i] = cf;
        }

    // fp8: the linear half 1/2 sum_i c_i S_i = u . k with u = sum_i c_i q_i (in
    // code units) is one more MFMA block.  u (fp32) is split into six fp8
    // pieces with power-of-two scales, piece p = e4m3(r_p / 2^e_p), r_{p+1} =
    // r_p - piece_p * 2^e_p; each piece shrinks the largest residual by 2^4,
    // so the dropped remainder is below 2^-24 of max|u|.  Pieces 0..3 sit in
    // rows 0, 4, 8, 12 of the extra A block and pieces 4, 5 in rows 1, 5, so
    // every lane group folds at most two of them into its partial sum.
    v8i Alin = v8i{0, 0, 0, 0, 0, 0, 0, 0};
    float lin0 = 0.f, lin1 = 0.f;
    if constexpr (DT == 2) {
        const uint8_t* qrow = reinterpret_cast<const uint8_t*>(a.q) + row_t * H * kD;
        const int tu = __builtin_amdgcn_readfirstlane((int)row_t);
        float u0 = 0.f, u1 = 0.f;  // dims 2*lane, 2*lane+1
        for (int h = 0; h < H; ++h) {
            const float ch = a.w[(size_t)tu * H + h] * a.q_scale[(size_t)tu * H + h] * (a.inv_sqrt_d * 0.5f);
            const int two = (int)*reinterpret_cast<const uint16_t*>(qrow + (size_t)h * kD + 2 * lane);
            const auto f = __builtin_amdgcn_cvt_pk_f32_fp8(two, false);
            u0 = fmaf(ch, f[0], u0);
            u1 = fmaf(ch, f[1], u1);
        }
        uint8_t* pieces = reinterpret_cast<uint8_t*>(rb.hist);  // 6 x 128 bytes of scratch
        float sc[6];
#pragma unroll
        for (int pc = 0; pc < 6; ++pc) {
            float m = fmaxf(fabsf(u0), fabsf(u1));
#pragma unroll
            for (int d = 32; d >= 1; d >>= 1) m = fmaxf(m, __shfl_xor(m, d, kWave));
            // smallest power of two >= m / 448, so every |r / scale| <= 448
            const bool live = m > 1e-30f;  // a vanishing residual ends the pieces
            const float scale = live ? ldexpf(1.0f, __builtin_amdgcn_frexp_expf(m * (1.0f / 448.0f))) : 0.f;
            const float inv = live ? 1.0f / scale : 0.f;
            const int code = __builtin_amdgcn_cvt_pk_fp8_f32(u0 * inv, u1 * inv, 0, false);
            const auto dec = __builtin_amdgcn_cvt_pk_f32_fp8(code, false);
            u0 -= dec[0] * scale;
            u1 -= dec[1] * scale;
            *reinterpret_cast<uint16_t*>(pieces + pc * kD + 2 * lane) = (uint16_t)(code & 0xFFFF);
            sc[pc] = scale;
        }
        __builtin_amdgcn_wave_barrier();
        // lane (row n, group g) of the extra A block
        int pc_of_row = -1;
        if ((n & 3) == 0) pc_of_row = n >> 2;               // rows 0, 4, 8, 12 -> pieces 0..3
        else if (n == 1 || n == 5) pc_of_row = 4 + (n >> 2);  // rows 1, 5 -> pieces 4, 5
        if (pc_of_row >= 0) {
            const v4i lo = *reinterpret_cast<const v4i*>(pieces + pc_of_row * kD + 32 * g);
            const v4i hi = *reinterpret_cast<const v4i*>(pieces + pc_of_row * kD + 32 * g + 16);
            Alin = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
        // output rows 4g (piece g) and 4g+1 (piece 4+g for g < 2)
        lin0 = g == 0 ? sc[0] : g == 1 ? sc[1] : g == 2 ? sc[2] : sc[3];
        lin1 = g == 0 ? sc[4] : g == 1 ? sc[5] : 0.f;
        __builtin_amdgcn_wave_barrier();
    }
    (void)Alin; (void)lin0; (void)lin1;

    const float* kscale = DT == 2 ? a.k_scale + (size_t)b * L : nullptr;
    float* srow = a.scores ? a.scores + row_t * L : nullptr;

    auto load_chunk = [&](int s0, typename Op::Bt (&Bk)[4], float& ksc) {
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const int s = min(s0 + 16 * st + n, L - 1);
            Op::load_b(Bk[st], kbase + (size_t)s * Op::kRowBytes, g);
        }
        if constexpr (DT == 2) {
            ksc = kscale[min(s0 + lane, L - 1)];
        }
    };

    int nb = 0;           // candidates in the buffer (wave-uniform)
    uint32_t thr = 0u;    // append iff key > thr
    const int last = t / 64;

    // One step over the 64 keys of `chunk`, held in `cur`; the next chunk's
    // keys are loaded into `nxt` first.  Called with alternating buffers.
    auto step = [&](int chunk, typename Op::Bt (&cur)[4], float ksc, typename Op::Bt (&nxt)[4], float& ksn) {
        const int s0 = chunk * 64;
        if (chunk + kPrefetch <= last) load_chunk(s0 + 64 * kPrefetch, nxt, ksn);
        float part[4];
        if constexpr (DT == 2) {
            v4f acc[4][HB], accl[4];
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                Op::template mma<HB>(acc[st], Aq, cur[st]);
                const v8i bb = v8i{cur[st].lo[0], cur[st].lo[1], cur[st].lo[2], cur[st].lo[3],
                                   cur[st].hi[0], cur[st].hi[1], cur[st].hi[2], cur[st].hi[3]};
                accl[st] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(Alin, bb, v4f{0.f, 0.f, 0.f, 0.f},
                                                                              0, 0, 0, 0, 0, 0);
            }
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                float pp = fmaf(lin0, accl[st][0], lin1 * accl[st][1]);
#pragma unroll
                for (int hb = 0; hb < HB; ++hb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) pp = fmaf(c[hb][i], fabsf(acc[st][hb][i]), pp);
                part[st] = pp;
            }
        } else {
            v4f acc[4][HB];
#pragma unroll
            for (int st = 0; st < 4; ++st) Op::template mma<HB>(acc[st], Aq, cur[st]);
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                float pp = 0.f;
#pragma unroll
                for (int hb = 0; hb < HB; ++hb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) pp = fmaf(c[hb][i], relu(acc[st][hb][i]), pp);
                part[st] = pp;
            }
        }
        const float score = reduce_scatter4(part) * ksc;
        const int s = s0 + lane;
        const bool valid = s <= t;
        if (srow && s < L) srow[s] = valid ? score : -INFINITY;
        const uint32_t key = score_key(score);
        const bool app = valid && key > thr;
        const uint64_t m = wave_ballot(app);
        if (app) {
            const int o = nb + lanes_below(m);
            rb.key[o] = key;
            rb.pos[o] = (Pos)s;
        }
        nb += __builtin_popcountll(m);
        if (nb > CAP - kWave) {
            __builtin_amdgcn_wave_barrier();
            nb = wave_compact(rb, nb, (uint32_t)a.topk, &thr, CAP);
        }
    };

#if DSAIDX_PREFILL_DEPTH >= 2
    // keys two chunks ahead are in flight: three buffers in rotation
    typename Op::Bt bx[4], by[4], bz[4];
    float kx = 1.f, ky = 1.f, kz = 1.f;
    load_chunk(0, bx, kx);
    if (last >= 1) load_chunk(64, by, ky);
    for (int chunk = 0; chunk <= last; chunk += 3) {
        step(chunk, bx, kx, bz, kz);
        if (chunk + 1 <= last) step(chunk + 1, by, ky, bx, kx);
        if (chunk + 2 <= last) step(chunk + 2, bz, kz, by, ky);
    }
#else
    typename Op::Bt bx[4], by[4];
    float kx = 1.f, ky = 1.f;
    load_chunk(0, bx, kx);
    for (int chunk = 0; chunk <= last; chunk += 2) {
        step(chunk, bx, kx, by, ky);
        if (chunk + 1 <= last) step(chunk + 1, by, ky, bx, kx);
    }
#endif
    if (srow) {
        for (int s = (last + 1) * 64 + lane; s < L; s += kWave) srow[s] = -INFINITY;
    }
    __builtin_amdgcn_wave_barrier();
    wave_emit(rb, nb, a.topk, a.idx_out + row_t * a.topk, a.val_out ? a.val_out + row_t * a.topk : nullptr);
}

template <int DT, int HB, bool POS16>
hipError_t launch_one(const PrefillArgs& a, hipStream_t stream) {
    using Cfg = BufCfg<POS16>;
    const size_t smem = (size_t)Cfg::kWaves * Cfg::kWaveBytes;
    static PerDevice<int> lds_once;
    hipError_t e = set_lds_limit(lds_once, (const void*)prefill_fused_kernel<DT, HB, POS16>, (int)smem);
    if (e != hipSuccess) return e;
    const int nblk = (a.L + Cfg::kWaves - 1) / Cfg::kWaves;
    hipLaunchKernelGGL((prefill_fused_kernel<DT, HB, POS16>), dim3((unsigned)(nblk * a.B)),
                       dim3(Cfg::kWaves * kWave), smem, stream, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// fp8, L <= 65536: keys staged through LDS, head sums on the matrix cores.
//
// The 8 waves of a workgroup (8 consecutive tokens, all with the same last
// 64-key chunk) walk the chunks in lockstep: every 64-key chunk (8 KB of fp8
// rows) is fetched from L2 once per workgroup with direct global->LDS loads
// (no VGPRs in flight), triple-buffered, one barrier per chunk.  Rows are
// stored with their 16-byte segments XOR-swizzled by ((row >> 1) & 7) so the
// MFMA operand reads (16 rows at a 128-byte stride) spread over the LDS banks.
//
// Epilogue.  The score of key s is sum_h c_h max(S_h, 0) times the key's
// scale, with c_h = w_h * q_scale_h / sqrt(D) and S_h the dot product of the
// fp8 values.  |S_h| <= |q_h|_1 * max_d |k_d| <= 2^Pq_h * 2^Pk, with Pq_h
// taken per head of the token and Pk per key (a pre-pass over the keys), so
// the score MFMAs, run with the E8M0 operand scales 2^-Pq_h (A, one per row,
// i.e. per head) and 2^-Pk (B, one per key column), leave every value in
// [-1, 1] at its own head's scale.  There the conversion to f16 with its
// [0, 1] clamp is max(S, 0) itself, rounded to nearest (relative error
// <= 2^-11 down to 2^-14 of the head's bound, however far the heads'
// magnitudes spread), and the weighted sum over heads is one more MFMA
// (f16, 16x16x32) with the weights c_h * 2^Pq_h * 2^E as its A operand.  Its
// weights for subtile st sit in the rows 4st..4st+3 only, so the four
// subtiles of a chunk accumulate into one tile whose element 0 in lane l is
// the score of key 64*chunk + l: no cross-lane reduction.  The factor 2^-E
// and the key's scale times 2^Pk finish the score.
// ---------------------------------------------------------------------------
constexpr int kStagedWaves = 8;
// Candidates per row: the most that fit beside three key chunks.  Every
// compaction request makes all waves compact, so the buffer's slack above k
// sets how often the whole block stalls.
constexpr int kStagedCap = 2712;
constexpr int kStages = 3;
// per wave: keys [CAP + 64] u32, histogram [256] u16, positions [CAP + 64] u16; the
// 64 slots past CAP take the writes of lanes that do not append
constexpr size_t kStagedWaveBytes = (size_t)(kStagedCap + kWave) * 6 + 128 * 4;
// Buffer walks read whole 256-entry steps, masking entries past the count,
// so the last step reads up to entry kWalkEnd - 1.  Its keys stay within the
// wave's keys and histogram; its positions can run past the wave's region
// (into the next wave's, or into this padding after the last one).
constexpr int kWalkEnd = (kStagedCap - 1) / 256 * 256 + 256;
constexpr size_t kStagedTailPad = 128;
static_assert((size_t)kWalkEnd * 4 <= (size_t)(kStagedCap + kWave) * 4 + 128 * 4, "key walk stays in the region");
static_assert((size_t)kWalkEnd * 2 <= (size_t)(kStagedCap + kWave) * 2 + kStagedTailPad, "position walk padding");
static_assert(kStagedWaveBytes % 16 == 0, "wave regions stay 16-byte aligned");
constexpr size_t kStageKeyBytes = 64 * kD;                 // one chunk of fp8 keys,
constexpr size_t kStageScaleOff = kStageKeyBytes;          // their fp32 scales times 2^Pk,
constexpr size_t kStageExpOff = kStageKeyBytes + 64 * 4;   // their E8M0 bytes (64 used of 256)
constexpr size_t kStageBytes = kStageExpOff + 256;
constexpr size_t kStagedLds = kStages * kStageBytes + (size_t)kStagedWaves * kStagedWaveBytes + kStagedTailPad;
static_assert(kStagedLds + 16 <= 160 * 1024, "LDS budget");

// Key pre-pass: for key s of sequence b (positions up to the 64-padded
// length; rows past the end repeat row L-1, as the staged copies do):
// 2^Pk >= max_d |k_d| (Pk = 0 for a zero row), ks_adj = k_scale * 2^Pk and
// the E8M0 byte 127 - Pk, stored at 64*chunk + 4*(s % 16) + (s % 64) / 16 so
// that lane n of a chunk finds the bytes of its four subtiles in one word.
template <bool PAGED>
__global__ void __launch_bounds__(256)
prefill_key_exp_kernel(PrefillArgs a) {
    const int64_t gi = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int Lp = a.Lpad;
    if (gi >= (int64_t)a.B * Lp) return;
    const int b = (int)(gi / Lp), s = (int)(gi % Lp);
    const int Lk = PAGED ? a.Lk : a.L;
    const int sr = s < Lk ? s : Lk - 1;
    // the key's slot: row sr of sequence b, or its page-pool slot
    const size_t slot = PAGED ? (size_t)a.block_table[(size_t)b * a.max_pages + sr / 64] * 64 + sr % 64
                              : (size_t)b * a.L + sr;
    const uint8_t* row = reinterpret_cast<const uint8_t*>(a.k) + slot * kD;
    uint32_t mx = 0;
#pragma unroll
    for (int c = 0; c < kD / 16; ++c) {
        const v4i v = *reinterpret_cast<const v4i*>(row + 16 * c);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint32_t x = (uint32_t)v[d] & 0x7F7F7F7Fu;  // magnitudes: e4m3 orders like its bits
            mx = max(mx, max(max(x & 0xFFu, (x >> 8) & 0xFFu), max((x >> 16) & 0xFFu, x >> 24)));
        }
    }
    const float vmax = __builtin_amdgcn_cvt_f32_fp8((int)mx, 0);
    const int pk = vmax > 0.f ? __builtin_amdgcn_frexp_expf(vmax) : 0;  // 2^pk > vmax
    a.ks_adj[gi] = ldexpf(a.k_scale[slot], pk);
    const int c = s / 64, n = s % 16, q = (s % 64) / 16;
    a.kexp[(size_t)b * Lp + 64 * c + 4 * n + q] = (uint8_t)(127 - pk);
}

// Rank r of the speculative floor in a row's sample, from the expected
// number ec of sampled keys at or above the row's k-th largest: 3.5 standard
// deviations (plus 8) above it.  The floor fails only if the sample holds r
// keys above the k-th largest (about 1e-5 per row for the sampling model at
// ec ~ 128), and a failed floor is caught and rescanned.  A wider margin
// leaves long rows near their buffer's capacity, so they compact more.
__device__ __forceinline__ uint32_t spec_rank(float ec) {
    return (uint32_t)ceilf(ec + 3.5f * sqrtf(ec) + 8.f);
}

template <int HB, bool PAGED>
__global__ void __launch_bounds__(kStagedWaves * kWave)
prefill_fused_fp8_staged_kernel(PrefillArgs a) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    __shared__ uint32_t flags[4];  // [0..2] compaction requests, [3] rescan request
    using Op = Operands<2>;
    using Pos = uint16_t;
    constexpr int W = kStagedWaves;
    constexpr int CAP = kStagedCap;
    constexpr int H = 16 * HB;
    const int L = a.L;
    const int nblk = (L + W - 1) / W;
    const int b = blockIdx.x % a.B;
    const int blk = nblk - 1 - (int)(blockIdx.x / a.B);  // heaviest first
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
    const int t_raw = blk * W + wave;
    const bool live = t_raw < L;        // waves past the end only help stage keys
    const int t = live ? t_raw : L - 1;
    // A chunk of queries against the paged cache starts at position q0 and
    // sees Lk keys; a whole sequence has q0 = 0 and Lk = L.
    const int q0 = PAGED ? a.q0 : 0;
    const int Lk = PAGED ? a.Lk : L;
    const int tp = q0 + t;              // the token's position: its row sees keys 0 .. tp
    if (short_rows_bypass(a, b, blk, W, L, q0, t_raw, live)) return;
    const int lane = lane_id();
    const int n = lane & 15, g = lane >> 4;

    RowBuf<Pos> rb;
    unsigned char* wbase = smem_raw + kStages * kStageBytes + wave * kStagedWaveBytes;
    rb.key = reinterpret_cast<uint32_t*>(wbase);
    rb.hist = reinterpret_cast<uint32_t*>(wbase + (size_t)(CAP + kWave) * 4);
    rb.pos = reinterpret_cast<Pos*>(wbase + (size_t)(CAP + kWave) * 4 + 128 * 4);

    const size_t row_t = (size_t)b * L + t;
    const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.k) + (size_t)b * L * kD;
    typename Op::template A<HB> Aq;
    Op::template load_a<HB>(Aq, reinterpret_cast<const uint8_t*>(a.q) + row_t * H * kD, n, g);

    // Head weights as the A operand of the f16 head-sum MFMA x (x < NX), in
    // the contraction order k = 8g + j: head 32x + 4g + j for j < 4, head
    // 32x + 16 + 4g + (j - 4) for j >= 4; subtile st uses rows 4st..4st+3.
    constexpr int NX = (HB + 1) / 2;
    v8h Wh[4][NX];
    float Fscale;  // 2^-E
    int sa[HB];    // E8M0 A scale of the score MFMAs, per lane: 127 - Pq of head 16hb + n (the lane's A row)
    {
        // Each head h gets its own exponent: 2^Pq_h >= |q_h|_1 (fp8 values).
        // Lane (m, g) sums its 32 bytes of head 16hb + m; the four lane
        // groups of a row add up, so every lane of row m holds |q_h|_1.
        int pq[HB];
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
            float sabs = 0.f;
#pragma unroll
            for (int d = 0; d < 8; ++d) {
                const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(Aq.a[hb][d], false);
                const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(Aq.a[hb][d], true);
                sabs += (fabsf(lo[0]) + fabsf(lo[1])) + (fabsf(hi[0]) + fabsf(hi[1]));
            }
            sabs += __shfl_xor(sabs, 16, kWave);
            sabs += __shfl_xor(sabs, 32, kWave);
            pq[hb] = sabs > 0.f ? __builtin_amdgcn_frexp_expf(sabs) : 0;  // 2^Pq > |q_h|_1
            sa[hb] = 127 - pq[hb];
        }
        // Head weights c_h = w q_scale / sqrt(D) for the lane's accumulator
        // rows h = 16hb + 4g + i, times 2^Pq_h (the scale the score MFMA took
        // out of head h), then all of them by one 2^E that puts the largest
        // in f16's top binade.
        float cf[HB][4];
        float mx = 0.f;
#pragma unroll
        for (int hb = 0; hb < HB; ++hb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int h = 16 * hb + 4 * g + i;
                const int pqh = __shfl(pq[hb], 4 * g + i, kWave);
                cf[hb][i] = ldexpf(a.w[row_t * H + h] * a.q_scale[row_t * H + h] * a.inv_sqrt_d, pqh);
                mx = fmaxf(mx, fabsf(cf[hb][i]));
            }
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) mx = fmaxf(mx, __shfl_xor(mx, d, kWave));
        int E = mx > 0.f ? 15 - __builtin_amdgcn_frexp_expf(mx) : 0;
        E = E < -60 ? -60 : (E > 100 ? 100 : E);
        Fscale = ldexpf(1.0f, -E);
        // lane (m, g) of the weight operand: row m = n, contraction group g
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

    const float* ksadj = a.ks_adj + (size_t)b * a.Lpad;
    const uint8_t* kexp = a.kexp + (size_t)b * a.Lpad;
    float* srow = (a.scores && live) ? a.scores + row_t * L : nullptr;
    const int last = (q0 + min(blk * W + W - 1, L - 1)) / 64;   // same for every wave of the block

    // Chunk order.  When the block spans at least 32 chunks, a strided sample
    // (chunks 16i+15, i < S) is scored first; the rest follow in increasing
    // order.  After the sample each long row sets a speculative floor: the
    // lower edge of the radix bin holding the r-th largest sampled key, with
    // r three and a half standard deviations above the expected number of
    // sampled keys at or above the row's k-th largest.  Keys below the floor
    // are never appended.  The floor is verified at the end: if fewer than k
    // keys of the row cleared it, some of the top k may have been dropped and
    // the row is scanned again without a floor.  Otherwise every dropped key
    // lies below the k-th largest and the selection is exact.
    const int S = last + 1 >= 32 ? (last + 1) / 16 : 0;
    // Chunk of order index i from the chunk of index i-1 (scalar, no
    // division): the sample 16i+15 for i < S, then 0, 1, ... skipping the
    // sampled chunks; past the last index the last chunk again (the stage
    // copies issued past the end re-read it).
    auto chunk_next = [&](int i, int prev) -> int {
        if (i > last) return prev;
        if (i < S) return 16 * i + 15;
        if (i == S) return 0;
        int c = prev + 1;
        if ((c & 15) == 15 && c < 16 * S) ++c;
        return c;
    };
    const int chunk0 = S > 0 ? 15 : 0;

    // Stage slot i % 3 receives the i-th chunk of the order: thread x of the
    // block copies 16 key bytes (LDS slot x = row x/8, segment x%8 holds
    // global segment (x%8) ^ ((row >> 1) & 7) of that row), wave 0 also copies
    // the chunk's 64 adjusted key scales and wave 1 its 64 E8M0 bytes (lanes
    // 16..63 repeat them into the unused tail).  Rows past the end are
    // clamped to L-1; they only ever feed masked scores.
    const int srow_i = threadIdx.x >> 3;
    const int sseg = (threadIdx.x & 7) ^ ((srow_i >> 1) & 7);
    auto stage_chunk = [&](int slot, int chunk) {
        unsigned char* dst = smem_raw + slot * kStageBytes;
        const int r = min(chunk * 64 + srow_i, Lk - 1);
        // a 64-key chunk is one page of the paged cache
        const uint8_t* src =
            PAGED ? reinterpret_cast<const uint8_t*>(a.k) +
                        ((size_t)a.block_table[(size_t)b * a.max_pages + (r >> 6)] * 64 + (r & 63)) * kD + 16 * sseg
                  : kbase + (size_t)r * kD + 16 * sseg;
        __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(dst + 1024 * wave),
                                         16, 0, 0);
        if (wave == 0)
            __builtin_amdgcn_global_load_lds(ksadj + chunk * 64 + lane,
                                             (__attribute__((address_space(3))) void*)(dst + kStageScaleOff),
                                             4, 0, 0);
        if (wave == 1)
            __builtin_amdgcn_global_load_lds(kexp + chunk * 64 + 4 * (lane & 15),
                                             (__attribute__((address_space(3))) void*)(dst + kStageExpOff),
                                             4, 0, 0);
    };
    // Swizzled byte offset of (row r, 16-byte segment j) inside a stage.
    // Rows r and r+1 share a swizzle value and lie in opposite bank halves,
    // so the 16 rows one operand read touches use all 64 banks once.
    auto soff = [](int r, int j) { return r * kD + 16 * (j ^ ((r >> 1) & 7)); };

    const int K = a.topk;
    int nb = 0;
    uint32_t thr = 0u;
    bool active = live;   // this wave scores and appends in the current pass
    bool floored = false; // a speculative floor is in force
    uint32_t r_spec = 0;  // rank of the floor in the sample (0: no floor)
    if (live && S >= 2 && tp + 1 > 2 * K) {
        const float ec = 64.f * (float)S * (float)K / (float)(tp + 1);
        r_spec = spec_rank(ec);
    }

    // Pipeline.  The i-th chunk is copied three chunks ahead into the slot
    // of chunk i-3 (free once every wave has read that chunk into registers)
    // and waited for at the barrier in the middle of iteration i-1, so a copy
    // has about two chunk-times to arrive.  Within a chunk the work runs at
    // half-chunk (32-key) granularity: while the matrix cores multiply one
    // half, the head sums of the previous one are formed.  Issue is in order
    // within a wave and the waves of a SIMD run in step (one barrier per
    // chunk), so the overlap has to come from within each wave: each region
    // below is branch-free and interleaves its instructions step by step.
    struct HalfAcc { v4f s[2][HB]; };
    struct HalfB { v8i b[2]; };
    auto load_b = [&](int slot, int half, HalfB& B_) {
        const unsigned char* cur = smem_raw + slot * kStageBytes;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int r = 16 * (2 * half + q) + n;
            const v4i lo = *reinterpret_cast<const v4i*>(cur + soff(r, 2 * g));
            const v4i hi = *reinterpret_cast<const v4i*>(cur + soff(r, 2 * g + 1));
            B_.b[q] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
    };
    // Adjusted scale of key (i-th chunk)*64 + lane, and the E8M0 bytes of
    // the lane's four subtile keys; read while the chunk's slot is still
    // owned (before the barrier that lets chunk i+3 overwrite it).
    auto load_ks = [&](int slot) {
        return *reinterpret_cast<const float*>(smem_raw + slot * kStageBytes + kStageScaleOff + 4 * lane);
    };
    auto load_sb = [&](int slot) {
        return *reinterpret_cast<const int*>(smem_raw + slot * kStageBytes + kStageExpOff + 4 * n);
    };
    // Score MFMA of subtile 2*MH + q (q in {0, 1}) and head block hb.
    auto score_mma = [&](auto mh, int q, int hb, const HalfB& B_, int sb) -> v4f {
        constexpr int s0 = 2 * decltype(mh)::value;
        if (q == 0)
            return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(Aq.a[hb], B_.b[0], v4f{0.f, 0.f, 0.f, 0.f},
                                                                      0, 0, 0, sa[hb], s0, sb);
        return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(Aq.a[hb], B_.b[1], v4f{0.f, 0.f, 0.f, 0.f},
                                                                  0, 0, 0, sa[hb], s0 + 1, sb);
    };
    // Conversion j2 (of 4) of the B operand of head MFMA x for subtile q of
    // half A_: the pair of heads (hb = 2x + j2/2, i = 2(j2%2), +1) as f16,
    // clamped to [0, 1].
    auto cvt_pair = [&](const HalfAcc& A_, int q, int x, int j2) -> v2h {
        const int hb = 2 * x + (j2 >> 1);
        if (hb >= HB) return v2h{0, 0};
        const v2f f = v2f{A_.s[q][hb][2 * (j2 & 1)], A_.s[q][hb][2 * (j2 & 1) + 1]};
        const v2h r = __builtin_convertvector(f, v2h);
        return __builtin_elementwise_min(__builtin_elementwise_max(r, v2h{0, 0}), v2h{1, 1});
    };
    // One region: the 2*HB score MFMAs of half MH (operands B_, results mm)
    // and the head sums of half EH of the previous results ep (added to P),
    // interleaved step by step.  Step k issues score MFMA k, then its share
    // of the head-sum work (items: four conversions, then the head MFMA they
    // feed), then extra(k).  The scheduling barrier after each step keeps
    // the VALU and MFMA order as written; LDS, SALU and memory instructions
    // may still move across.
    auto region = [&](auto mh, auto eh, const HalfB& B_, int sb, HalfAcc& mm, const HalfAcc& ep, v4f& P,
                      auto&& extra) {
        constexpr int NM = 2 * HB;
        constexpr int NI = 2 * NX * 5;
        constexpr int st0 = 2 * decltype(eh)::value;
        v8h X = v8h{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int k = 0; k < NM; ++k) {
            mm.s[k / HB][k % HB] = score_mma(mh, k / HB, k % HB, B_, sb);
#pragma unroll
            for (int e = (k * NI) / NM; e < ((k + 1) * NI) / NM; ++e) {
                const int qx = e / 5, it = e % 5;
                const int qq = qx / NX, x = qx % NX;
                if (it < 4) {
                    const v2h r = cvt_pair(ep, qq, x, it);
                    X[2 * it] = r[0];
                    X[2 * it + 1] = r[1];
                } else {
                    P = __builtin_amdgcn_mfma_f32_16x16x32_f16(Wh[st0 + qq][x], X, P, 0, 0, 0);
                }
            }
            extra(k);
            __builtin_amdgcn_sched_barrier(0x0094);  // SALU, VMEM and LDS may cross
        }
    };
    // Head sums of half EH of A_ added to P, not interleaved (after the last chunk).
    auto epi_half = [&](auto eh, const HalfAcc& A_, v4f P) {
        constexpr int st0 = 2 * decltype(eh)::value;
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int x = 0; x < NX; ++x) {
                v8h X;
#pragma unroll
                for (int it = 0; it < 4; ++it) {
                    const v2h r = cvt_pair(A_, q, x, it);
                    X[2 * it] = r[0];
                    X[2 * it + 1] = r[1];
                }
                P = __builtin_amdgcn_mfma_f32_16x16x32_f16(Wh[st0 + q][x], X, P, 0, 0, 0);
            }
        return P;
    };
    // Keeps a half's MFMAs in the region that issues them (they would
    // otherwise sink to the region that reads their results).
    auto pin_half = [&](HalfAcc& A_) {
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int hb = 0; hb < HB; ++hb) asm volatile("" : "+v"(A_.s[q][hb]));
    };
    // Appending the scores of the chunk whose head sums are complete, above
    // the floor and in lane order, in five pieces spread over the steps of a
    // region.  Branch free: lanes that do not append write a slot of their
    // own past CAP.
    struct FinState { float score; uint32_t key; int s; bool app; uint64_t m; int below; };
    uint32_t thr_eff = 0u;  // thr while the wave appends, else 0xFFFFFFFF
    auto finish_piece = [&](int piece, FinState& f, int chunk, const v4f& P, float ks) {
        if (piece == 0) f.score = P[0] * (ks * Fscale);
        if (piece == 1) f.key = score_key(f.score);
        if (piece == 2) {
            f.s = chunk * 64 + lane;
            // bitwise, not short-circuit (a branch here would split the
            // region); an inactive wave's threshold admits nothing
            f.app = (f.s <= tp) & (f.key > thr_eff);
        }
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
    // The rest of an append step: the optional score-matrix row and the
    // compaction request (flag slot `fslot`) when the buffer nears capacity.
    auto finish_tail = [&](int fslot, int chunk, float score) {
        if (srow && active) {
            const int s = chunk * 64 + lane;
            if (s < Lk) srow[s] = s <= tp ? score : -INFINITY;
        }
        if (active && nb > CAP - 2 * kWave && lane == 0) flags[fslot] = 1u;
    };

    if (threadIdx.x == 0) flags[3] = 0u;
    for (int pass = 0;; ++pass) {
        HalfAcc hA, hB;
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int hb = 0; hb < HB; ++hb) hB.s[q][hb] = v4f{0.f, 0.f, 0.f, 0.f};
        HalfB bA, bB;
        v4f Pacc = v4f{0.f, 0.f, 0.f, 0.f};  // head sums of the chunk in progress
        float ks_prev = 0.f;
        int chunk_prev = 0;  // chunk id of the previous iteration
        if (threadIdx.x < 3) flags[threadIdx.x] = 0u;
        // order indices 0..2 into slots 0..2; c_stage tracks index i+3
        int c_stage = chunk0;
        stage_chunk(0, c_stage);
        c_stage = chunk_next(1, c_stage);
        stage_chunk(1, c_stage);
        c_stage = chunk_next(2, c_stage);
        stage_chunk(2, c_stage);
        // chunk 0 landed: at most this wave's copies of chunks 1 and 2 in
        // flight (waves 0 and 1 issue two copies per chunk, the others one)
        if (wave <= 1) __builtin_amdgcn_s_waitcnt(0x0F74);                // vmcnt(4)
        else __builtin_amdgcn_s_waitcnt(0x0F72);                          // vmcnt(2)
        __syncthreads();
        load_b(0, 0, bA);
        int sb_next = load_sb(0);
        int chunk_cur = chunk0;  // chunk of order index i
        // slots of order indices i, i+1, i+2 (mod 3)
        int s0 = 0, s1 = 1, s2 = 2;
        for (int i = 0; i <= last; ++i) {
            const int sb_cur = sb_next;
            // Region 1: first half of chunk i on the MFMA (operands read during
            // the previous region 2), head sums of the second half of chunk
            // i-1 (zeros before the first chunk); the second half's operands
            // and the chunk's key scales are read here, before the barrier
            // that releases the chunk's stage slot.
            __builtin_amdgcn_sched_barrier(0);
            load_b(s0, 1, bB);
            const float ks_cur = load_ks(s0);
            region(std::integral_constant<int, 0>{}, std::integral_constant<int, 1>{}, bA, sb_cur, hA, hB, Pacc,
                   [](int) {});
            // keep this epilogue here (it would otherwise sink into a branch below)
            asm volatile("" : "+v"(Pacc));
            pin_half(hA);
            __builtin_amdgcn_sched_barrier(0);
            // This wave's copies of chunk i+1 have landed once at most its
            // copies of chunk i+2 are in flight (loads complete in issue
            // order); the barrier then makes every wave's copies visible and
            // certifies that every wave is done reading chunk i's slot.  With
            // the score matrix requested, the row's stores share the counter:
            // wait for all.
            if (a.scores) __builtin_amdgcn_s_waitcnt(0x0F70);             // vmcnt(0)
            else if (wave <= 1) __builtin_amdgcn_s_waitcnt(0x0F72);       // vmcnt(2)
            else __builtin_amdgcn_s_waitcnt(0x0F71);                      // vmcnt(1)
            __syncthreads();
            // Compaction request of the appends of chunk i-2 (made at the end
            // of iteration i-1; slot (i-2) % 3 = s1), read now and acted on
            // after region 2, so the read's latency hides under the MFMAs.
            // Slot j % 3 belongs to the appends of the j-th chunk: set at the
            // end of iteration j+1, read in j+2, cleared in j+3 (each step
            // separated by a barrier).
            const uint32_t flag_word = flags[s1];
            if (threadIdx.x == 0 && i >= 3) flags[s0] = 0u;
            // Chunk i+3 goes to chunk i's slot.  Past the last chunk the copy
            // is a clamped dummy, so every chunk issues the same loads.
            c_stage = chunk_next(i + 3, c_stage);
            stage_chunk(s0, c_stage);
            // Region 2: second half of chunk i on the MFMA, head sums of its
            // first half, the appends of chunk i-1 (discarded before the first
            // chunk: nothing is valid yet) and the first-half operands of
            // chunk i+1 (landed, per the barrier above).
            const v4f Pfin = Pacc;
            const bool fin_on = i >= 1;
            const bool was_active = active;
            active = active && fin_on;
            thr_eff = active ? thr : 0xFFFFFFFFu;
            FinState fs;
            const int nb0 = nb;
            __builtin_amdgcn_sched_barrier(0);
            load_b(s1, 0, bA);
            sb_next = load_sb(s1);
            Pacc = v4f{0.f, 0.f, 0.f, 0.f};
            region(std::integral_constant<int, 1>{}, std::integral_constant<int, 0>{}, bB, sb_cur, hB, hA, Pacc,
                   [&](int k) {
#pragma unroll
                       for (int p = 0; p < 5; ++p)
                           if ((p < 2 * HB - 1 ? p : 2 * HB - 1) == k) finish_piece(p, fs, chunk_prev, Pfin, ks_prev);
                   });
            asm volatile("" : "+v"(Pacc), "+v"(fs.score));
            pin_half(hB);
            __builtin_amdgcn_sched_barrier(0);
            active = was_active;
            if (!fin_on) nb = nb0;
            // Buffer maintenance after the appends of chunk i-1.  The sample's
            // appends (chunks 0..S-1 of the order) end in iteration S: the
            // speculative floor is set before any other append.  Then the
            // cooperative compaction: a request from any wave makes every
            // wave compact, so the block pays one stall per event.
            if (i == S && r_spec != 0u && active && (uint32_t)nb > r_spec) {
                uint32_t fl;
                nb = wave_floor(rb, nb, r_spec, &fl);
                thr = fl == 0u ? 0u : fl - 1u;
                floored = true;
            }
            if (i >= 2 && flag_word != 0u && active && nb > K) nb = wave_compact(rb, nb, (uint32_t)K, &thr, CAP);
            if (fin_on) finish_tail(s2, chunk_prev, fs.score);
            ks_prev = ks_cur;
            chunk_prev = chunk_cur;
            chunk_cur = chunk_next(i + 1, chunk_cur);
            const int sx = s0;
            s0 = s1; s1 = s2; s2 = sx;
        }
        Pacc = epi_half(std::integral_constant<int, 1>{}, hB, Pacc);
        {
            FinState fs;
            thr_eff = active ? thr : 0xFFFFFFFFu;
#pragma unroll
            for (int p = 0; p < 5; ++p) finish_piece(p, fs, chunk_prev, Pacc, ks_prev);
            finish_tail(s2, chunk_prev, fs.score);  // no compaction follows: the flag is cleared at the next pass
        }
        __builtin_amdgcn_s_waitcnt(0x0000);  // no stage copy or LDS read may still be in flight
        if (pass == 1) break;
        // Verification of the floor (see above); any failing row makes the
        // whole block scan again, with only the failing waves appending.
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
    }
    if (!live) return;
    if (srow) {
        for (int s = (last + 1) * 64 + lane; s < Lk; s += kWave) srow[s] = -INFINITY;
    }
    __builtin_amdgcn_wave_barrier();
    wave_emit(rb, nb, K, a.idx_out + row_t * K, a.val_out ? a.val_out + row_t * K : nullptr);
}

// ---------------------------------------------------------------------------
// bf16, L <= 65536: keys staged through LDS, head sums on the matrix cores.
//
// The scheme of the fp8 kernel above, with what bf16 changes:
// * A key pre-pass writes every key times 2^-Pk (exact: a power of two) to
//   the workspace, with 2^Pk as its adjusted scale, and each query head's A
//   rows are scaled by its own 2^-Pq_h in registers (2^Pq_h goes into the
//   head's weight).  So again every S_h lies in [-1, 1], the clamped f16
//   conversion is the ReLU and the head sum is an f16 MFMA.
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

template <int HB>
__global__ void __launch_bounds__(kBfWaves * kWave)
prefill_fused_bf16_staged_kernel(PrefillArgs a, const uint16_t* kscaled) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    __shared__ uint32_t flags[4];  // [0..2] compaction requests, [3] rescan request
    using Pos = uint16_t;
    constexpr int W = kBfWaves;
    constexpr int CAP = kBfCap;
    constexpr int H = 16 * HB;
    constexpr int NX = (HB + 1) / 2;
    const int L = a.L;
    const int nblk = (L + W - 1) / W;
    const int b = blockIdx.x % a.B;
    const int blk = nblk - 1 - (int)(blockIdx.x / a.B);  // heaviest first
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
    const int t_raw = blk * W + wave;
    const bool live = t_raw < L;        // waves past the end only help stage keys
    const int t = live ? t_raw : L - 1;
    if (short_rows_bypass(a, b, blk, W, L, 0, t_raw, live)) return;
    const int lane = lane_id();
    const int n = lane & 15, g = lane >> 4;

    RowBuf<Pos> rb;
    unsigned char* wbase = smem_raw + kBfStages * kBfStageBytes + wave * kBfWaveBytes;
    rb.key = reinterpret_cast<uint32_t*>(wbase);
    rb.hist = reinterpret_cast<uint32_t*>(wbase + (size_t)(CAP + kWave) * 4);
    rb.pos = reinterpret_cast<Pos*>(wbase + (size_t)(CAP + kWave) * 4 + 128 * 4);

    const size_t row_t = (size_t)b * L + t;
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
    float* srow = (a.scores && live) ? a.scores + row_t * L : nullptr;
    const int last = (min(blk * W + W - 1, L - 1)) / 64;   // same for every wave of the block

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
    if (live && S >= 2 && t + 1 > 2 * K) {
        const float ec = 64.f * (float)S * (float)K / (float)(t + 1);
        r_spec = spec_rank(ec);
    }
    auto finish_piece = [&](int piece, FinState& f, int chunk, const v4f& P, float ks) {
        if (piece == 0) f.score = P[0] * (ks * Fscale);
        if (piece == 1) f.key = score_key(f.score);
        if (piece == 2) {
            f.s = chunk * 64 + lane;
            f.app = (f.s <= t) & (f.key > thr_eff);
        }
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
            if (s < L) srow[s] = s <= t ? score : -INFINITY;
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
            if (flag_word != 0u && active && nb > K) nb = wave_compact(rb, nb, (uint32_t)K, &thr, CAP + 128);
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
    }
    if (!live) return;
    if (srow) {
        for (int s = (last + 1) * 64 + lane; s < L; s += kWave) srow[s] = -INFINITY;
    }
    __builtin_amdgcn_wave_barrier();
    wave_emit(rb, nb, K, a.idx_out + row_t * K, a.val_out ? a.val_out + row_t * K : nullptr);
}

constexpr bool staged_path(int dtype, int L) { return DSAIDX_PREFILL_STAGED && dtype == 2 && L <= 65536; }
constexpr bool staged_bf16_path(int dtype, int L) { return DSAIDX_PREFILL_STAGED_BF16 && dtype == 1 && L <= 65536; }
constexpr int pad64(int L) { return (L + 63) / 64 * 64; }

template <int HB, bool PAGED = false>
hipError_t launch_fp8_staged(const PrefillArgs& a_in, hipStream_t stream) {
    PrefillArgs a = a_in;
    if (!PAGED) {
        a.q0 = 0;
        a.Lk = a.L;
    }
    a.Lpad = pad64(a.Lk);
    a.ks_adj = reinterpret_cast<float*>(a.workspace);
    a.kexp = reinterpret_cast<uint8_t*>(a.ks_adj + (size_t)a.B * a.Lpad);
    {
        const int64_t n = (int64_t)a.B * a.Lpad;
        hipLaunchKernelGGL(prefill_key_exp_kernel<PAGED>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                           a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const size_t smem = kStagedLds;
    static PerDevice<int> lds_once;
    {
        hipError_t e = set_lds_limit(lds_once, (const void*)prefill_fused_fp8_staged_kernel<HB, PAGED>, (int)smem);
        if (e != hipSuccess) return e;
    }
    const int nblk = (a.L + kStagedWaves - 1) / kStagedWaves;
    hipLaunchKernelGGL((prefill_fused_fp8_staged_kernel<HB, PAGED>), dim3((unsigned)(nblk * a.B)),
                       dim3(kStagedWaves * kWave), smem, stream, a);
    return hipGetLastError();
}

template <int HB>
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
        hipError_t e = set_lds_limit(lds_once, (const void*)prefill_fused_bf16_staged_kernel<HB>, (int)smem);
        if (e != hipSuccess) return e;
    }
    const int nblk = (a.L + kBfWaves - 1) / kBfWaves;
    hipLaunchKernelGGL((prefill_fused_bf16_staged_kernel<HB>), dim3((unsigned)(nblk * a.B)), dim3(kBfWaves * kWave),
                       smem, stream, a, (const uint16_t*)kscaled);
    return hipGetLastError();
}

template <int DT, int HB>
hipError_t launch_pos(const PrefillArgs& a, hipStream_t stream) {
    if (staged_path(DT, a.L)) return launch_fp8_staged<HB>(a, stream);
    if (staged_bf16_path(DT, a.L)) return launch_bf16_staged<HB>(a, stream);
    return a.L <= 65536 ? launch_one<DT, HB, true>(a, stream) : launch_one<DT, HB, false>(a, stream);
}

}  // namespace

size_t prefill_fused_workspace_bytes(int B, int L, int dtype) {
    const size_t n = (size_t)B * pad64(L);
    if (DSAIDX_PREFILL_WS && dtype == 2) return prefill_ws_workspace_bytes(B, L, 0);
    if (staged_path(dtype, L)) return (n * 5 + 255) / 256 * 256;  // fp32 adjusted scales, then the E8M0 bytes
    if (staged_bf16_path(dtype, L)) return n * (4 + 2 * kD);      // fp32 adjusted scales, then the scaled keys
    return 0;
}

hipError_t launch_prefill_chunk_paged(const PrefillArgs& a, hipStream_t stream) {
    switch (a.H / 16) {
        case 1: return launch_fp8_staged<1, true>(a, stream);
        case 2: return launch_fp8_staged<2, true>(a, stream);
        case 3: return launch_fp8_staged<3, true>(a, stream);
        case 4: return launch_fp8_staged<4, true>(a, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_prefill_fused(const PrefillArgs& a, int dtype, hipStream_t stream) {
    const int hb = a.H / 16;
    if (DSAIDX_PREFILL_WS && dtype == 2) return launch_prefill_ws(a, stream);
    if (dtype == 2) {
        switch (hb) {
            case 1: return launch_pos<2, 1>(a, stream);
            case 2: return launch_pos<2, 2>(a, stream);
            case 3: return launch_pos<2, 3>(a, stream);
            case 4: return launch_pos<2, 4>(a, stream);
        }
    } else if (dtype == 1) {
        switch (hb) {
            case 1: return launch_pos<1, 1>(a, stream);
            case 2: return launch_pos<1, 2>(a, stream);
            case 3: return launch_pos<1, 3>(a, stream);
            case 4: return launch_pos<1, 4>(a, stream);
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace dsaidx
