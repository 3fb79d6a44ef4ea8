// Fused fp8 prefill with specialised waves: the score contraction, ReLU,
// weighted head sum and causal mask of the lightning indexer ("From
// principle to code", section 2.1; one shared key per token, "Lightning
// Indexer explained", section 4) and the per-row top-k (section 1 of the
// same page: k positions per query, ties to the lower position), with the
// [L, L] score matrix kept out of HBM.
//
// Layout.  A workgroup owns 8 consecutive query rows of one sequence and
// has 8 waves in two roles, one of each per SIMD (waves w and w + 4 share a
// SIMD):
// * matrix waves 0..3: wave m holds the fp8 queries of rows 2m and 2m+1 in
//   registers (MFMA A operands, head on M) and does nothing but multiply:
//   per 16-key subtile, 2 x H/16 scaled fp8 MFMAs (16x16x128, per-head E8M0
//   A scales, per-key B scales) and the head sums of the previous subtile
//   (clamped f16 conversion = ReLU, then an f16 MFMA against the head
//   weights).  Every 64-key chunk it writes each row's 64 scores to a small
//   LDS ring;
// * selection waves 4..7: wave 4+m owns the candidate buffers of rows 2m and
//   2m+1 (streaming top-k, speculative floor, compaction, final selection)
//   and issues the direct global->LDS copies of the key chunks.
// So the matrix cores see one instruction stream per SIMD with no
// bookkeeping in it, and the selection work runs beside it on the other
// wave.
//
// Pipeline (one workgroup barrier per chunk).  Iteration i ends with barrier
// i.  The matrix waves run, in iteration i, the last subtile of chunk i-1 and
// the first three of chunk i, then write chunk i-1's scores to ring slot
// (i-1) % 2.  The selection waves, in iteration i, append the scores of chunk
// i-2 (ring slot i % 2) and copy chunk i+2 into the stage slot chunk i-1 has
// just freed, then wait for their copies of chunk i+1: barrier i certifies
// that chunk i+1 has landed, that chunk i's last subtile has been read and
// that the ring holds chunk i-1.  Three stage slots, two ring slots.
//
// Scaling.  |S_h| = |q_h . k| <= |q_h|_1 max_d |k_d| < 2^Pq_h 2^Pk with Pq_h
// per head (from the query registers) and Pk per key (a pre-pass), so the
// scaled MFMA with A scale 2^-Pq_h and B scale 2^-Pk leaves every value in
// [-1, 1] at its own head's scale; there the f16 conversion with its [0, 1]
// clamp is max(S, 0) rounded to nearest.  The head weights
// c_h = w_h q_scale_h / sqrt(D) times 2^Pq_h, times one 2^E that puts the
// largest in f16's top binade, are the A operand of the head sum in all 16
// rows; the four subtiles of a chunk accumulate into four tiles, and lane l
// takes element 0 of tile l / 16: the score of key 64 chunk + l.  2^-E and
// the key's scale times 2^Pk finish it.
//
// Rows and keys.  Whole sequences (keys contiguous, row t sees keys 0..t) or
// variable-length chunks of rows against the paged key cache (row i of
// sequence b is position q_start[b] + i and sees keys 0 .. that position; a
// 64-key chunk is one 64-token page).  Positions up to 131072: beyond 65536
// the candidate buffers keep 17-bit positions in their 16-bit layout by
// giving up the key's lowest bit (rowbuf.h).
#include "common.h"
#include "device_once.h"
#include "kernels.h"
#include "rowbuf.h"
#include "varlen.h"

namespace dsaidx {

namespace {

constexpr int kD = 128;
constexpr int kWsWaves = 8;    // 4 matrix waves + 4 selection waves
constexpr int kWsRows = kBlockRows;  // query rows per workgroup
// Candidates per row: the most that fit beside three key stages and the
// score ring.
constexpr int kWsCap = 2624;
// a row asking for compaction (count above kWsCap - 128) always takes part (count above its cut rank + 128)
static_assert(kMaxTopk + 128 < kWsCap - 2 * kWave, "the requesting row joins its compaction");
constexpr int kWsStages = 3;
constexpr size_t kWsStageKeyBytes = 64 * kD;               // one chunk of fp8 keys,
constexpr size_t kWsStageScaleOff = kWsStageKeyBytes;      // their fp32 scales times 2^Pk,
constexpr size_t kWsStageExpOff = kWsStageKeyBytes + 256;  // their E8M0 bytes (64 used of 256)
constexpr size_t kWsStageBytes = kWsStageExpOff + 256;
constexpr size_t kWsRingOff = kWsStages * kWsStageBytes;
constexpr size_t kWsRingBytes = 2 * kWsRows * 64 * 4;      // two slots of 8 rows x 64 scores
constexpr size_t kWsRowsOff = kWsRingOff + kWsRingBytes;
// per row: keys [CAP + 64] u32, histogram [256] u16, positions [CAP + 64] u16
constexpr size_t kWsRowBytes = (size_t)(kWsCap + kWave) * 6 + 128 * 4;
// buffer walks read whole 256-entry steps: the last one reads up to entry
// kWsWalkEnd - 1, whose positions run past the row's region by up to this much
constexpr int kWsWalkEnd = (kWsCap - 1) / 256 * 256 + 256;
constexpr size_t kWsTailPad = 256;
constexpr size_t kWsLds = kWsRowsOff + kWsRows * kWsRowBytes + kWsTailPad;
static_assert((size_t)kWsWalkEnd * 4 <= (size_t)(kWsCap + kWave) * 4 + 128 * 4, "key walk stays in the row");
static_assert((size_t)kWsWalkEnd * 2 <= (size_t)(kWsCap + kWave) * 2 + kWsTailPad, "position walk padding");
static_assert(kWsRowBytes % 16 == 0 && kWsStageBytes % 16 == 0, "16-byte aligned regions");
static_assert(kWsLds + 16 <= 160 * 1024, "LDS budget");

constexpr int pad64(int n) { return (n + 63) / 64 * 64; }

// Workgroup barrier of the selection waves.  A fence-based barrier treats
// the key-chunk copies in flight (global -> LDS, counted by vmcnt) as
// pending LDS writes and drains them all, including the one just issued for
// two chunks ahead; these waves instead wait for their copies explicitly,
// only as far as the pipeline needs, so the barrier itself waits for this
// wave's LDS accesses only.  The memory clobbers keep the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Rank of the speculative floor in a row's sample (ec = expected number of
// sampled keys at or above the row's k-th largest): three and a half
// standard deviations above it, plus 8.
__device__ __forceinline__ uint32_t spec_rank(float ec) {
    return (uint32_t)ceilf(ec + 3.5f * sqrtf(ec) + 8.f);
}

// Key pre-pass, one thread per key s < pad64(Lk) of sequence b (rows past
// the end repeat key Lk-1, as the stage copies do): 2^Pk > max_d |k_d| (Pk = 0
// for a zero row), ks_adj = k_scale * 2^Pk and the E8M0 byte 127 - Pk at
// 64 chunk + 4 (s % 16) + (s % 64) / 16, so lane n of a chunk finds the
// bytes of its four subtiles in one word.
template <bool VARLEN>
__global__ void __launch_bounds__(256)
ws_key_prep_kernel(PrefillArgs a) {
    const int64_t gi = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int Lp = a.Lpad;
    if (gi >= (int64_t)a.B * Lp) return;
    const int b = (int)(gi / Lp), s = (int)(gi % Lp);
    int Lk;
    if constexpr (VARLEN) {
        const int Lq = a.cu_q[b + 1] - a.cu_q[b];
        Lk = min(max(a.q_start[b], 0) + Lq, a.max_kv);
        if (Lq <= 0 || Lk <= 0 || s >= pad64(Lk)) return;
    } else {
        Lk = a.L;
    }
    const int sr = s < Lk ? s : Lk - 1;
    const size_t slot = key_slot<VARLEN>(a, b, sr);
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

template <int HB, bool VARLEN, bool P17, bool ROWS>
__global__ void __launch_bounds__(kWsWaves * kWave)
prefill_ws_fp8_kernel(PrefillArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ uint32_t flags[4];  // [i % 3]: compaction requested in iteration i; [3]: rescan requested
    __shared__ int emit_n[4];      // candidates of row 2m+1 (-1: no row), handed to matrix wave m
    using Pos = uint16_t;
    constexpr int H = 16 * HB;
    constexpr int NX = (HB + 1) / 2;   // head-sum MFMAs per row and subtile (32 heads each)
    constexpr int CAP = kWsCap;
    const v4f zero4 = v4f{0.f, 0.f, 0.f, 0.f};

    Seg sg;
    if (!block_seg<VARLEN>(a, sg)) return;
    const int wave = uniform((int)threadIdx.x / kWave);
    const int lane = lane_id();
    const int n = lane & 15, g = lane >> 4;
    const int K = a.topk;
    const int last_row = min(sg.blk * kWsRows + kWsRows - 1, sg.Lq - 1);
    // the block's last chunk, the same for its 8 rows (keys past a row's
    // position are masked)
    const int last = min((sg.q0 + last_row) / 64, (sg.Lk - 1) / 64);
    const int n_ch = last + 1;

    // Short rows, no scores asked for: a row with at most k valid positions
    // selects all of them, so a block whose rows all qualify writes
    // positions 0 .. p, then -1, without scoring.
    if (!a.val_out && !a.scores && sg.q0 + last_row + 1 <= K) {
        const int t = sg.blk * kWsRows + wave;
        if (t < sg.Lq) {
            const int tp = sg.q0 + t;
            int32_t* out = a.idx_out + (size_t)(sg.row0 + t) * K;
            for (int j = lane; j < K; j += kWave) out[j] = j <= tp ? j : -1;
        }
        return;
    }

    // Chunk order: when the block spans at least 32 chunks, a strided sample
    // (chunks 16i+15, i < S) first, then 0, 1, ... skipping the sampled
    // ones; past the last order index, the last chunk again.
    const int S = n_ch >= 32 ? n_ch / 16 : 0;
    auto chunk_next = [&](int i, int prev) -> int {
        if (i > last) return prev;
        if (i < S) return 16 * i + 15;
        if (i == S) return 0;
        int c = prev + 1;
        if ((c & 15) == 15 && c < 16 * S) ++c;
        return c;
    };
    const int chunk0 = S > 0 ? 15 : 0;

    const bool mma = wave < 4;
    const int m = mma ? wave : wave - 4;
    const int t0 = sg.blk * kWsRows + 2 * m;  // this wave's rows: t0, t0 + 1
    float* ring = reinterpret_cast<float*>(smem + kWsRingOff);
    const float* ksadj = a.ks_adj + (size_t)sg.b * a.Lpad;
    const uint8_t* kexp = a.kexp + (size_t)sg.b * a.Lpad;

    // ---------------- matrix waves: operands and weights ----------------
    v8i Aq[2][HB];
    int sa[2][HB];   // E8M0 A scale per lane: 127 - Pq of head 16hb + n (the lane's A row)
    v8h Wv[2][NX];   // head weights, the same in all 16 rows
    float Fs[2];     // 2^-E
    if (mma) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int t = min(t0 + j, sg.Lq - 1);
            const size_t row = (size_t)(sg.row0 + t);
            const uint8_t* qrow = reinterpret_cast<const uint8_t*>(a.q) + row * H * kD;
            int pq[HB];
#pragma unroll
            for (int hb = 0; hb < HB; ++hb) {
                const uint8_t* p = qrow + (size_t)(16 * hb + n) * kD + 32 * g;
                const v4i lo = *reinterpret_cast<const v4i*>(p);
                const v4i hi = *reinterpret_cast<const v4i*>(p + 16);
                Aq[j][hb] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                // |q_h|_1 of head 16hb + n: the lane's 32 bytes, then the four lane groups
                float sabs = 0.f;
#pragma unroll
                for (int d = 0; d < 8; ++d) {
                    const auto f0 = __builtin_amdgcn_cvt_pk_f32_fp8(Aq[j][hb][d], false);
                    const auto f1 = __builtin_amdgcn_cvt_pk_f32_fp8(Aq[j][hb][d], true);
                    sabs += (fabsf(f0[0]) + fabsf(f0[1])) + (fabsf(f1[0]) + fabsf(f1[1]));
                }
                sabs += __shfl_xor(sabs, 16, kWave);
                sabs += __shfl_xor(sabs, 32, kWave);
                pq[hb] = sabs > 0.f ? __builtin_amdgcn_frexp_expf(sabs) : 0;  // 2^Pq > |q_h|_1
                sa[j][hb] = 127 - pq[hb];
            }
            // weights of the lane's contraction slots: heads 16hb + 4g + i
            float cf[HB][4];
            float mx = 0.f;
#pragma unroll
            for (int hb = 0; hb < HB; ++hb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int h = 16 * hb + 4 * g + i;
                    const int pqh = __shfl(pq[hb], 4 * g + i, kWave);
                    cf[hb][i] = ldexpf(a.w[row * H + h] * a.q_scale[row * H + h] * a.inv_sqrt_d, pqh);
                    mx = fmaxf(mx, fabsf(cf[hb][i]));
                }
#pragma unroll
            for (int d = 32; d >= 1; d >>= 1) mx = fmaxf(mx, __shfl_xor(mx, d, kWave));
            int E = mx > 0.f ? 15 - __builtin_amdgcn_frexp_expf(mx) : 0;
            E = E < -60 ? -60 : (E > 100 ? 100 : E);
            Fs[j] = ldexpf(1.0f, -E);
            // contraction slot 8g + jj of head MFMA x: head 32x + 4g + jj (jj < 4),
            // 32x + 16 + 4g + (jj - 4) (jj >= 4)
#pragma unroll
            for (int x = 0; x < NX; ++x) {
                v8h wv;
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) {
                    const int hb = 2 * x + (jj >> 2);
                    wv[jj] = hb < HB ? (_Float16)ldexpf(cf[hb < HB ? hb : 0][jj & 3], E) : (_Float16)0.f;
                }
                Wv[j][x] = wv;
            }
        }
    }

    // ---------------- selection waves: candidate buffers ----------------
    RowBuf<Pos> rb[2];
    int nb[2];
    uint32_t thr[2], rspec[2];
    bool live[2], act[2], floored[2], spec_ok[2];
    int tp[2];
    // score-matrix rows as global (not generic) pointers: a generic store
    // could address LDS, and the barrier's release would then have to wait
    // for every vector-memory operation in flight, stage copies included
    typedef __attribute__((address_space(1))) float gfloat;
    gfloat* srow[2];
    if (!mma) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            unsigned char* base = smem + kWsRowsOff + (size_t)(2 * m + j) * kWsRowBytes;
            rb[j].key = reinterpret_cast<uint32_t*>(base);
            rb[j].hist = reinterpret_cast<uint32_t*>(base + (size_t)(CAP + kWave) * 4);
            rb[j].pos = reinterpret_cast<Pos*>(base + (size_t)(CAP + kWave) * 4 + 128 * 4);
            const int t = t0 + j;
            live[j] = t < sg.Lq;
            tp[j] = sg.q0 + min(t, sg.Lq - 1);
            act[j] = live[j];
            nb[j] = 0;
            thr[j] = 0u;
            floored[j] = false;
            rspec[j] = 0u;
            spec_ok[j] = live[j] && tp[j] + 1 > 2 * K;
            if (live[j] && S >= 2 && tp[j] + 1 > 2 * K)
                rspec[j] = spec_rank(64.f * (float)S * (float)K / (float)(tp[j] + 1));
            srow[j] = (ROWS && live[j]) ? (gfloat*)(a.scores + (size_t)(sg.row0 + t) * a.L) : nullptr;
        }
    }

    // Stage copies (selection waves): slot x = 64 * piece + lane of a stage
    // holds row x / 8, 16-byte segment x % 8, which is global segment
    // (x % 8) ^ ((row >> 1) & 7) of that row; rows past the keys repeat key
    // Lk-1.  Wave 4 also copies the chunk's 64 adjusted scales, wave 5 its
    // E8M0 bytes (lanes 16..63 repeat them into the unused tail).
    // Selection wave m copies pieces P and P + 2 (P = m % 2 + 4 (m / 2)):
    // 16 rows apart, they share the swizzle, so the second piece sits 2048
    // bytes after the first both in the chunk and in the stage, and one LDS
    // base (M0) with an instruction offset serves both copies.
    const uint8_t* kbytes = reinterpret_cast<const uint8_t*>(a.k);
    // this lane's two pieces: byte offset inside a 64-key chunk, and row
    uint32_t poff[2];
    int prow[2];
    const int piece0 = (m & 1) + 4 * (m >> 1);
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int x = 64 * (piece0 + 2 * r) + lane;
        const int row = x >> 3;
        prow[r] = row;
        poff[r] = (uint32_t)(row * kD + 16 * ((x & 7) ^ ((row >> 1) & 7)));
    }
    auto stage_chunk = [&](int slot, int chunk) {
        unsigned char* dst = smem + slot * kWsStageBytes;
        if (chunk * 64 + 64 <= sg.Lk) {
            // every row of the chunk is a key: one chunk base (a page of the
            // paged cache) plus the lane's fixed offsets
            const uint8_t* base = VARLEN ? kbytes + (size_t)a.block_table[(size_t)sg.b * a.max_pages + chunk] * (64 * kD)
                                         : kbytes + ((size_t)sg.b * a.L + (size_t)chunk * 64) * kD;
            auto* ldst = (__attribute__((address_space(3))) void*)(dst + 1024 * piece0);
            __builtin_amdgcn_global_load_lds(base + poff[0], ldst, 16, 0, 0);
            __builtin_amdgcn_global_load_lds(base + poff[0], ldst, 16, 2048, 0);  // piece P + 2
        } else {
            // the last chunk: rows past the keys repeat key Lk-1
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int rg = min(chunk * 64 + prow[r], sg.Lk - 1);
                const uint8_t* src = kbytes + key_slot<VARLEN>(a, sg.b, rg) * kD + (poff[r] & (kD - 1));
                __builtin_amdgcn_global_load_lds(src,
                                                 (__attribute__((address_space(3))) void*)(dst + 1024 * (piece0 + 2 * r)),
                                                 16, 0, 0);
            }
        }
        if (m == 0)
            __builtin_amdgcn_global_load_lds(ksadj + chunk * 64 + lane,
                                             (__attribute__((address_space(3))) void*)(dst + kWsStageScaleOff), 4, 0,
                                             0);
        if (m == 1)
            __builtin_amdgcn_global_load_lds(kexp + chunk * 64 + 4 * (lane & 15),
                                             (__attribute__((address_space(3))) void*)(dst + kWsStageExpOff), 4, 0,
                                             0);
    };
    // vmcnt waits: this wave's copies of one chunk (3 for waves 4 and 5, else 2)
    auto wait_copies_but_one_chunk = [&]() {
        if (ROWS) __builtin_amdgcn_s_waitcnt(0x0F70);            // score-row stores share the counter
        else if (m < 2) __builtin_amdgcn_s_waitcnt(0x0F73);      // vmcnt(3)
        else __builtin_amdgcn_s_waitcnt(0x0F72);                 // vmcnt(2)
    };

    // Matrix-wave pieces.  Swizzled byte offset of (row r, segment j) in a
    // stage: rows r and r+1 share a swizzle and sit in opposite bank halves,
    // so the 16 rows an operand read touches use all 64 banks once.
    auto soff = [](int r, int j) { return r * kD + 16 * (j ^ ((r >> 1) & 7)); };
    auto read_B = [&](int slot, int st, v8i& Bo) {
        const unsigned char* cur = smem + slot * kWsStageBytes;
        const int r = 16 * st + n;
        const v4i lo = *reinterpret_cast<const v4i*>(cur + soff(r, 2 * g));
        const v4i hi = *reinterpret_cast<const v4i*>(cur + soff(r, 2 * g + 1));
        Bo = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    auto read_ks = [&](int slot) {
        return *reinterpret_cast<const float*>(smem + slot * kWsStageBytes + kWsStageScaleOff + 4 * lane);
    };
    auto read_sb = [&](int slot) {
        return *reinterpret_cast<const int*>(smem + slot * kWsStageBytes + kWsStageExpOff + 4 * n);
    };
    // Conversion j2 (of 4) of head MFMA x's B operand from score tiles acc:
    // heads (hb = 2x + j2/2, rows 2(j2%2), +1) as f16 clamped to [0, 1].
    auto cvt_pair = [&](const v4f (&acc)[HB], int x, int j2) -> v2h {
        const int hb = 2 * x + (j2 >> 1);
        if (hb >= HB) return v2h{0, 0};
        const v2f f = v2f{acc[hb][2 * (j2 & 1)], acc[hb][2 * (j2 & 1) + 1]};
        const v2h r = __builtin_convertvector(f, v2h);
        return __builtin_elementwise_min(__builtin_elementwise_max(r, v2h{0, 0}), v2h{1, 1});
    };
    // Head-sum tiles: subtiles 0 and 2 of a chunk accumulate into Pa, 1 and 3
    // into Pb; a tile is read (element 0, lanes of its subtile) one region
    // after its MFMAs were issued, before the tile is reused.
    v4f Pa[2] = {}, Pb[2] = {};
    // One region: the 2*HB score MFMAs of subtile ST (operand Bo, scale word
    // sb), interleaved step by step with the head sums of the previous
    // subtile into Pt.  The score tiles `acc` are updated in place: step k
    // first converts the previous subtile's values it needs -- only tiles k
    // and later, which this region has not yet overwritten (the conversion
    // order follows the tile order) -- then issues score MFMA k into tile k,
    // so one set of tiles serves both subtiles.  `next` (the B operand of
    // the following region, from stage slot nslot) is read right after the
    // first MFMA and held there: the LDS wait before a region's first MFMA
    // (which the compiler makes a full drain) then finds every read it
    // covers long arrived, and the new read's latency hides under this
    // region's remaining MFMAs.
    auto no_extra = [] {};
    auto region = [&](auto st, auto has_next, const v8i& Bo, int sb, v4f (&acc)[2][HB], v4f (&Pt)[2], v8i& next,
                      int nslot, int nst, bool pin, auto&& after_first) {
        constexpr int ST = decltype(st)::value;
        constexpr int NM = 2 * HB;
        constexpr int NI = 2 * NX * 5;
        __builtin_amdgcn_sched_barrier(0);
        v8h X[2];
#pragma unroll
        for (int k = 0; k < NM; ++k) {
            const int j = k / HB, hb = k % HB;
#pragma unroll
            for (int e = (k * NI) / NM; e < ((k + 1) * NI) / NM; ++e) {
                const int jj = e / (NX * 5), x = (e / 5) % NX, it = e % 5;
                if (it < 4) {
                    const v2h r = cvt_pair(acc[jj], x, it);
                    X[jj][2 * it] = r[0];
                    X[jj][2 * it + 1] = r[1];
                } else {
                    Pt[jj] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Wv[jj][x], X[jj], x == 0 ? zero4 : Pt[jj], 0, 0, 0);
                }
            }
            acc[j][hb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(Aq[j][hb], Bo, zero4, 0, 0, 0, sa[j][hb],
                                                                           ST, sb);
            if (k == 0) {
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (decltype(has_next)::value) read_B(nslot, nst, next);
                after_first();
                __builtin_amdgcn_sched_barrier(0);
            } else {
                __builtin_amdgcn_sched_barrier(0x0094);  // SALU, VMEM and LDS may cross
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        // Outside the branch-free steady state, keep the MFMAs in the block
        // that issues them (they would otherwise sink into the conditional
        // block that reads their results).  This waits for their results.
        if (pin) {
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int hb = 0; hb < HB; ++hb) asm volatile("" : "+v"(acc[j][hb]));
        }
    };
    // Head sums of tiles `in` into Pt, not interleaved (after the last chunk).
    auto heads_only = [&](const v4f (&in)[2][HB], v4f (&Pt)[2]) {
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int x = 0; x < NX; ++x) {
                v8h X;
#pragma unroll
                for (int it = 0; it < 4; ++it) {
                    const v2h r = cvt_pair(in[jj], x, it);
                    X[2 * it] = r[0];
                    X[2 * it + 1] = r[1];
                }
                Pt[jj] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Wv[jj][x], X, x == 0 ? zero4 : Pt[jj], 0, 0, 0);
            }
    };
    // lane l's score comes from subtile l / 16: take it from tile Pt when it holds subtile st
    float sc_acc[2] = {0.f, 0.f};
    auto take = [&](const v4f (&Pt)[2], int st) {
#pragma unroll
        for (int j = 0; j < 2; ++j) sc_acc[j] = g == st ? Pt[j][0] : sc_acc[j];
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    using T0 = std::integral_constant<bool, false>;
    using T1 = std::integral_constant<bool, true>;

    // Both roles run the same number of barriers per pass: one after the
    // prologue, one per iteration (n_ch + 2), one after the verification.
    if (mma) {
        for (int pass = 0;; ++pass) {
            __syncthreads();  // chunk 0 has landed
            v8i Bo0, Bo1;
            v4f acc[2][HB];
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int hb = 0; hb < HB; ++hb) acc[j][hb] = zero4;
            read_B(0, 0, Bo0);
            int sb_cur = read_sb(0), sb_prev = 0;
            float ks_cur = read_ks(0), ks_prev = 0.f;
            int s_cur = 0;  // stage slot of order index i
            // Iteration i (ending with barrier i): the last subtile of chunk
            // i-1 (region 3), the first three of chunk i (regions 0..2),
            // chunk i-1's scores to the ring.  The first iteration has no
            // chunk i-1, the drain (i = n_ch) no chunk i, the last (n_ch + 1)
            // neither; every other iteration is the branch-free body below.
            // Region r uses B operand Bo[r % 2] and reads the next region's
            // into the other one (subtile 0 of chunk i comes from its slot,
            // readable after barrier i-1).
            // chunk i-1's scores (lane l: key 64 (i-1) + l), written to the
            // ring inside the next region, after its first MFMA
            float outv[2];
            auto finish_scores = [&]() {
#pragma unroll
                for (int j = 0; j < 2; ++j) outv[j] = sc_acc[j] * (ks_prev * Fs[j]);
            };
            auto write_scores = [&](int i) {
                float* slot = ring + (size_t)(((i - 1) & 1) * kWsRows + 2 * m) * 64 + lane;
#pragma unroll
                for (int j = 0; j < 2; ++j) slot[64 * j] = outv[j];
            };
            // The steady-state iteration with its stage slot (i % 3) and ring
            // slot ((i-1) % 2) known at compile time: every LDS address is a
            // register base plus an immediate offset.
            auto body_c = [&](int i, auto sc, auto rp) {
                constexpr int SC = decltype(sc)::value;
                constexpr int RP = decltype(rp)::value;
                sb_prev = sb_cur;
                ks_prev = ks_cur;
                sb_cur = read_sb(SC);
                ks_cur = read_ks(SC);
                region(I3{}, T1{}, Bo1, sb_prev, acc, Pa, Bo0, SC, 0, false, no_extra);  // heads: chunk i-1, subtile 2
                take(Pb, 1);
                region(I0{}, T1{}, Bo0, sb_cur, acc, Pb, Bo1, SC, 1, false, no_extra);   // heads: chunk i-1, subtile 3
                take(Pa, 2);
                region(I1{}, T1{}, Bo1, sb_cur, acc, Pa, Bo0, SC, 2, false, no_extra);   // heads: chunk i, subtile 0
                take(Pb, 3);
                finish_scores();
                region(I2{}, T1{}, Bo0, sb_cur, acc, Pb, Bo1, SC, 3, false,              // heads: chunk i, subtile 1
                       [&] {
                           float* slot = ring + (size_t)(RP * kWsRows + 2 * m) * 64 + lane;
#pragma unroll
                           for (int j = 0; j < 2; ++j) slot[64 * j] = outv[j];
                       });
                take(Pa, 0);
                (void)i;
            };
            auto body = [&](int i, bool pin) {
                sb_prev = sb_cur;
                ks_prev = ks_cur;
                sb_cur = read_sb(s_cur);
                ks_cur = read_ks(s_cur);
                region(I3{}, T1{}, Bo1, sb_prev, acc, Pa, Bo0, s_cur, 0, pin, no_extra);  // heads: chunk i-1, subtile 2
                take(Pb, 1);
                region(I0{}, T1{}, Bo0, sb_cur, acc, Pb, Bo1, s_cur, 1, pin, no_extra);   // heads: chunk i-1, subtile 3
                take(Pa, 2);
                region(I1{}, T1{}, Bo1, sb_cur, acc, Pa, Bo0, s_cur, 2, pin, no_extra);   // heads: chunk i, subtile 0
                take(Pb, 3);
                finish_scores();
                region(I2{}, T1{}, Bo0, sb_cur, acc, Pb, Bo1, s_cur, 3, pin,              // heads: chunk i, subtile 1
                       [&] { write_scores(i); });
                take(Pa, 0);
            };
            // i = 0: chunk 0's first three subtiles (the head sums of region 0
            // read the zero tiles into Pb, unused)
            region(I0{}, T1{}, Bo0, sb_cur, acc, Pb, Bo1, 0, 1, true, no_extra);
            region(I1{}, T1{}, Bo1, sb_cur, acc, Pa, Bo0, 0, 2, true, no_extra);
            region(I2{}, T1{}, Bo0, sb_cur, acc, Pb, Bo1, 0, 3, true, no_extra);
            take(Pa, 0);
            __syncthreads();
            // iterations 1 .. n_ch-1: six at a time (stage slots 1 2 0 1 2 0, ring
            // slots 0 1 0 1 0 1), then the rest
            int i = 1;
            for (; i + 6 <= n_ch; i += 6) {
                body_c(i, I1{}, I0{});
                __syncthreads();
                body_c(i + 1, I2{}, I1{});
                __syncthreads();
                body_c(i + 2, I0{}, I0{});
                __syncthreads();
                body_c(i + 3, I1{}, I1{});
                __syncthreads();
                body_c(i + 4, I2{}, I0{});
                __syncthreads();
                body_c(i + 5, I0{}, I1{});
                __syncthreads();
            }
            s_cur = i % 3;
            for (; i < n_ch; ++i) {
                body(i, false);
                __syncthreads();
                s_cur = s_cur == 2 ? 0 : s_cur + 1;
            }
            // i = n_ch: the last chunk's last subtile and its scores
            ks_prev = ks_cur;
            region(I3{}, T0{}, Bo1, sb_cur, acc, Pa, Bo0, 0, 0, true, no_extra);
            take(Pb, 1);
            heads_only(acc, Pb);
            take(Pa, 2);
            take(Pb, 3);
            finish_scores();
            write_scores(n_ch);
            __syncthreads();
            // i = n_ch + 1: the selection waves append the last chunk
            __syncthreads();
            __syncthreads();  // the selection waves' verification
            if (pass == 1 || flags[3] == 0u) break;
        }
        // The final selection of row 2m+1 (its candidates are in LDS); the
        // selection wave takes row 2m meanwhile.
        __syncthreads();
        const int n1 = emit_n[m];
        if (n1 >= 0) {
            RowBuf<Pos> r1;
            unsigned char* base = smem + kWsRowsOff + (size_t)(2 * m + 1) * kWsRowBytes;
            r1.key = reinterpret_cast<uint32_t*>(base);
            r1.hist = reinterpret_cast<uint32_t*>(base + (size_t)(CAP + kWave) * 4);
            r1.pos = reinterpret_cast<Pos*>(base + (size_t)(CAP + kWave) * 4 + 128 * 4);
            const size_t row = (size_t)(sg.row0 + t0 + 1);
            wave_emit<Pos, P17>(r1, n1, K, a.idx_out + row * K, a.val_out ? a.val_out + row * K : nullptr);
        }
        return;
    }

    // ---------------- selection waves ----------------
    // They are the longer side of the pipeline: where both waves of a SIMD
    // can issue, this one goes first (the matrix wave's MFMAs still fill the
    // matrix core between its own instructions).
    __builtin_amdgcn_s_setprio(1);
    if (m == 0 && lane == 3) flags[3] = 0u;
    for (int pass = 0;; ++pass) {
        if (m == 0 && lane < 3) flags[lane] = 0u;
        int c_stage = chunk0;   // chunk of the latest staged order index
        int c_sel = chunk0;     // chunk of order index i - 2
        stage_chunk(0, c_stage);
        c_stage = chunk_next(1, c_stage);
        stage_chunk(1, c_stage);
        c_stage = chunk_next(2, c_stage);
        stage_chunk(2, c_stage);
        // chunk 0 has landed once at most this wave's copies of chunks 1 and 2 are in flight
        if (ROWS) __builtin_amdgcn_s_waitcnt(0x0F70);
        else if (m < 2) __builtin_amdgcn_s_waitcnt(0x0F76);   // vmcnt(6)
        else __builtin_amdgcn_s_waitcnt(0x0F74);              // vmcnt(4)
        lds_barrier();
        int s_cur = 0;
        for (int i = 0; i <= n_ch + 1; ++i) {
            // Chunk of order index i+2 into the slot chunk i-1 freed at barrier
            // i-1, first, so the copy has the whole iteration to land.
            if (i >= 1) {
                c_stage = chunk_next(i + 2, c_stage);
                stage_chunk(s_cur == 0 ? 2 : s_cur - 1, c_stage);
            }
            const int s_prev = s_cur == 0 ? 2 : s_cur - 1;   // (i - 1) % 3
            const int s_next = s_cur == 2 ? 0 : s_cur + 1;   // (i + 1) % 3
            // The compaction request of iteration i-1 is read right behind the
            // ring, so that one LDS wait covers both reads.
            uint32_t fw_raw;
            if (i >= 2) {
                // Appends of chunk i-2 (ring slot i % 2).  Branch free: lanes
                // that do not append write a slot of their own past CAP.
                const int c = c_sel;
                const float* slot = ring + (size_t)((i & 1) * kWsRows + 2 * m) * 64 + lane;
                float sc[2];
#pragma unroll
                for (int j = 0; j < 2; ++j) sc[j] = slot[64 * j];
                fw_raw = flags[s_prev];
                const int s = c * 64 + lane;
                // both rows step by step, so that their dependency chains interleave
                uint32_t wd[2];
                bool app[2];
                uint64_t msk[2];
                int o[2];
#pragma unroll
                for (int j = 0; j < 2; ++j) wd[j] = entry_word<P17>(sc[j], (uint32_t)s);
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    // last position the row appends (-1 while it is idle)
                    const int lastp = act[j] ? min(tp[j], sg.Lk - 1) : -1;
                    const bool above = wd[j] > thr[j], inrow = s <= lastp;
                    app[j] = above & inrow;
                    msk[j] = wave_ballot(above) & wave_ballot(inrow);
                }
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    int ob = nb[j] + lanes_below(msk[j]);
                    asm volatile("" : "+v"(ob));  // computed by every lane: the select stays branch free
                    o[j] = app[j] ? ob : CAP + lane;
                }
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    rb[j].key[o[j]] = wd[j];
                    rb[j].pos[o[j]] = (Pos)s;
                    nb[j] += __builtin_popcountll(msk[j]);
                    if (ROWS && act[j] && s < sg.Lk) srow[j][s] = s <= tp[j] ? sc[j] : -INFINITY;
                }
                c_sel = chunk_next(i - 1, c_sel);
            } else {
                fw_raw = flags[s_prev];
            }
            const uint32_t fw = i >= 1 ? fw_raw : 0u;
            // Compaction requested after the appends of iteration i-1 (read
            // only now, behind this iteration's appends): every row of the
            // block well above its cut rank compacts at once, so the block
            // stalls once per event.  A request leaves two chunks of slack.
            // A long row cuts speculatively: of the n_seen keys scanned so
            // far, about k n_seen / (t+1) belong to its final top k, so the
            // cut rank is that count plus three and a half standard
            // deviations and 8 (capped at k), verified with the floors.
            if (i >= 1) {
                if (m == 0 && lane == 0) flags[s_next] = 0u;
                if (fw != 0u) {
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        uint32_t r = (uint32_t)K;
                        if (spec_ok[j]) {
                            const float rows_keys = (float)(tp[j] + 1);
                            const float seen = fminf(64.f * (float)(i - 1), rows_keys);
                            r = min(r, spec_rank((float)K * seen / rows_keys));
                        }
                        if (act[j] && nb[j] > (int)r + 128) {
                            bool sp;
                            nb[j] = wave_compact(rb[j], nb[j], (uint32_t)K, &thr[j], CAP, r, &sp);
                            floored[j] |= sp;
                        }
                    }
                }
            }
            if (i >= 2 && i - 2 == S - 1) {
                // the sample is in: set each long row's speculative floor
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    if (rspec[j] != 0u && act[j] && (uint32_t)nb[j] > rspec[j]) {
                        uint32_t fl;
                        nb[j] = wave_floor(rb[j], nb[j], rspec[j], &fl);
                        thr[j] = fl == 0u ? 0u : fl - 1u;
                        floored[j] = true;
                    }
            }
            bool req = false;
#pragma unroll
            for (int j = 0; j < 2; ++j) req |= act[j] && nb[j] > CAP - 2 * kWave;
            if (req && lane == 0) flags[s_cur] = 1u;
            wait_copies_but_one_chunk();  // chunk i+1 has landed
            lds_barrier();
            s_cur = s_next;
        }
        __builtin_amdgcn_s_waitcnt(0x0000);  // no stage copy may still be in flight
        // Verification of the floors: a floored row with fewer than k keys at
        // or above its floor may have dropped some of its top k, and makes
        // the whole block scan again, with only such rows appending.
        bool redo[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) redo[j] = act[j] && floored[j] && nb[j] < K;
        if ((redo[0] || redo[1]) && lane == 0) flags[3] = 1u;
        __syncthreads();
        if (pass == 1 || flags[3] == 0u) break;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            act[j] = redo[j];
            rspec[j] = 0u;
            spec_ok[j] = false;
            if (redo[j]) {
                nb[j] = 0;
                thr[j] = 0u;
                floored[j] = false;
            }
        }
    }
    if (ROWS) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
            if (live[j])
                for (int s = n_ch * 64 + lane; s < a.L; s += kWave) srow[j][s] = -INFINITY;
    }
    if (lane == 0) emit_n[m] = live[1] ? nb[1] : -1;
    lds_barrier();
    if (live[0]) {
        const size_t row = (size_t)(sg.row0 + t0);
        wave_emit<Pos, P17>(rb[0], nb[0], K, a.idx_out + row * K, a.val_out ? a.val_out + row * K : nullptr);
    }
}

template <int HB, bool VARLEN, bool P17, bool ROWS>
hipError_t launch_ws(const PrefillArgs& a, unsigned grid, hipStream_t stream) {
    static PerDevice<int> lds_once;
    hipError_t e = set_lds_limit(lds_once, (const void*)prefill_ws_fp8_kernel<HB, VARLEN, P17, ROWS>, (int)kWsLds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((prefill_ws_fp8_kernel<HB, VARLEN, P17, ROWS>), dim3(grid), dim3(kWsWaves * kWave), kWsLds,
                       stream, a);
    return hipGetLastError();
}

// The score matrix is a separate instantiation (ROWS): without it the chunk
// loop issues no global stores, so its barriers need not wait for them.
template <int HB, bool VARLEN>
hipError_t launch_ws_mode(const PrefillArgs& a, unsigned grid, bool p17, hipStream_t stream) {
    if constexpr (VARLEN) {
        return p17 ? launch_ws<HB, true, true, false>(a, grid, stream) : launch_ws<HB, true, false, false>(a, grid, stream);
    } else {
        if (a.scores)
            return p17 ? launch_ws<HB, false, true, true>(a, grid, stream)
                       : launch_ws<HB, false, false, true>(a, grid, stream);
        return p17 ? launch_ws<HB, false, true, false>(a, grid, stream) : launch_ws<HB, false, false, false>(a, grid, stream);
    }
}

template <bool VARLEN>
hipError_t launch_ws_hb(const PrefillArgs& a, unsigned grid, bool p17, hipStream_t stream) {
    switch (a.H / 16) {
        case 1: return launch_ws_mode<1, VARLEN>(a, grid, p17, stream);
        case 2: return launch_ws_mode<2, VARLEN>(a, grid, p17, stream);
        case 3: return launch_ws_mode<3, VARLEN>(a, grid, p17, stream);
        case 4: return launch_ws_mode<4, VARLEN>(a, grid, p17, stream);
    }
    return hipErrorInvalidValue;
}

size_t scales_bytes(int B, int max_keys) { return ((size_t)B * pad64(max_keys) * 5 + 255) / 256 * 256; }

}  // namespace

size_t prefill_ws_workspace_bytes(int B, int max_keys, int n_plan) {
    return scales_bytes(B, max_keys) + (size_t)n_plan * sizeof(int2);
}

hipError_t launch_prefill_ws(const PrefillArgs& a_in, hipStream_t stream) {
    PrefillArgs a = a_in;
    a.q0 = 0;
    a.Lk = a.L;
    a.Lpad = pad64(a.L);
    a.max_kv = a.L;
    a.ks_adj = reinterpret_cast<float*>(a.workspace);
    a.kexp = reinterpret_cast<uint8_t*>(a.ks_adj + (size_t)a.B * a.Lpad);
    const int64_t nk = (int64_t)a.B * a.Lpad;
    hipLaunchKernelGGL(ws_key_prep_kernel<false>, dim3((unsigned)((nk + 255) / 256)), dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned grid = (unsigned)((a.L + kWsRows - 1) / kWsRows * a.B);
    return launch_ws_hb<false>(a, grid, a.L > 65536, stream);
}

hipError_t launch_prefill_ws_varlen(const PrefillArgs& a_in, hipStream_t stream) {
    PrefillArgs a = a_in;
    a.Lpad = pad64(a.max_kv);
    a.ks_adj = reinterpret_cast<float*>(a.workspace);
    a.kexp = reinterpret_cast<uint8_t*>(a.ks_adj + (size_t)a.B * a.Lpad);
    a.n_plan = (a.T + kWsRows - 1) / kWsRows + a.B;
    a.plan = reinterpret_cast<int2*>(reinterpret_cast<char*>(a.workspace) + scales_bytes(a.B, a.max_kv));
    hipLaunchKernelGGL(varlen_plan_kernel, dim3(1), dim3(1024), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t nk = (int64_t)a.B * a.Lpad;
    hipLaunchKernelGGL(ws_key_prep_kernel<true>, dim3((unsigned)((nk + 255) / 256)), dim3(256), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return launch_ws_hb<true>(a, (unsigned)a.n_plan, a.max_kv > 65536, stream);
}

}  // namespace dsaidx
