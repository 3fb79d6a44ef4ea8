// Fused prefill: MFMA scoring + ReLU + weighted head reduction + causal mask
// + streaming top-k, with the [L, L] score matrix kept out of HBM.
//
// What is computed: for every token t and history position s <= t,
// I[t,s] = sum_i w[t,i] * ReLU(q[t,i] . k[s] / sqrt(D))  ("From formula to
// code", section 2.1; one shared key per token, "Lightning Indexer
// explained", section 4), then the top-k positions of row t by (I desc,
// s asc).  As a contraction this is Q[L*H, D] x K[L, D]^T restricted to the
// causal half; D = 128 and H is a multiple of 16.
//
// Layout of the work:
// * workgroup = W independent waves; wave w owns query token t = W*blk + w and
//   all 16*HB of its heads.  Blocks are issued heaviest (largest t) first.
//   For L <= 65536 positions fit 16 bits: W = 8 waves (two per SIMD, so one
//   wave's MFMAs overlap the other's VALU epilogue) with 3072-entry buffers;
//   longer sequences use W = 4 with 4096-entry buffers and 32-bit positions.
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
// * streaming top-k per wave: a per-row candidate buffer of (key, position)
//   pairs in LDS, filled in position order.  A score enters the
//   buffer only if its order-preserving key beats the row threshold.  When
//   the buffer nears capacity it is compacted: one radix digit below the
//   buffer's common key prefix locates the bin of the k-th largest key, the
//   bin's lower edge becomes the new threshold and everything below it is
//   dropped (stable, so the buffer stays in position order).  The buffer
//   always holds every entry that can still be in the row's top k.  At the
//   end an exact radix select over the buffer finds the k-th largest key and
//   ties at that key go to the lowest positions.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace dsaidx {

namespace {

constexpr int kD = 128;

template <bool POS16>
struct BufCfg {
    using Pos = typename std::conditional<POS16, uint16_t, uint32_t>::type;
    static constexpr int kWaves = POS16 ? 8 : 4;      // waves (= tokens) per workgroup
    static constexpr int kCap = POS16 ? 3072 : 4096;  // candidates per row
    static constexpr size_t kWaveBytes = (size_t)kCap * (4 + sizeof(Pos)) + 256 * 4;
};

__device__ __forceinline__ uint32_t wave_or(uint32_t v) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v |= __shfl_xor(v, d, kWave);
    return v;
}
__device__ __forceinline__ uint32_t wave_and(uint32_t v) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v &= __shfl_xor(v, d, kWave);
    return v;
}

__device__ __forceinline__ float reduce_scatter4(const float v[4]) {
    auto s02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[0]), __float_as_uint(v[2]), false, false);
    auto s13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[1]), __float_as_uint(v[3]), false, false);
    const float a0 = __uint_as_float(s02[0]) + __uint_as_float(s02[1]);
    const float a1 = __uint_as_float(s13[0]) + __uint_as_float(s13[1]);
    auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(a0), __float_as_uint(a1), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// Per-wave candidate buffer in LDS.
template <typename Pos>
struct RowBuf {
    uint32_t* key;
    Pos* pos;
    uint32_t* hist;  // 256 bins
};

// Histogram of the 8-bit (or narrower) digit (key >> shift) & mask over the
// buffer entries whose key matches (key & pm) == pv.
template <typename Pos>
__device__ __forceinline__ void wave_hist(const RowBuf<Pos>& rb, int n, uint32_t pm, uint32_t pv,
                                          int shift, uint32_t dmask) {
    const int l = lane_id();
#pragma unroll
    for (int i = 0; i < 4; ++i) rb.hist[l + 64 * i] = 0u;
    __builtin_amdgcn_wave_barrier();
    for (int j = l; j < n; j += kWave) {
        const uint32_t k = rb.key[j];
        if ((k & pm) == pv) atomicAdd(&rb.hist[(k >> shift) & dmask], 1u);
    }
    __builtin_amdgcn_wave_barrier();
}

// Bin (counting down from the top) where the running count reaches `need`.
// Returns the bin; *above = count in bins above it.
template <typename Pos>
__device__ __forceinline__ uint32_t wave_find_bin(const RowBuf<Pos>& rb, uint32_t need, uint32_t* above,
                                                  uint32_t* in_bin) {
    const int l = lane_id();
    uint32_t c[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = rb.hist[255 - 4 * l - i];
    const uint32_t loc = c[0] + c[1] + c[2] + c[3];
    const uint32_t incl = wave_incl_scan(loc);
    uint32_t run = incl - loc;
    int hit = -1;
    uint32_t ab = 0, cnt = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (hit < 0 && run < need && need <= run + c[i]) { hit = i; ab = run; cnt = c[i]; }
        run += c[i];
    }
    const uint64_t m = wave_ballot(hit >= 0);
    const int src = __builtin_ctzll(m);
    const int bin = 255 - 4 * l - (hit < 0 ? 0 : hit);
    *above = __shfl(ab, src, kWave);
    *in_bin = __shfl(cnt, src, kWave);
    return (uint32_t)__shfl(bin, src, kWave);
}

// Common leading bits of all buffer keys: returns their count; *pv = value.
template <typename Pos>
__device__ __forceinline__ int wave_common_prefix(const RowBuf<Pos>& rb, int n, uint32_t* pv) {
    uint32_t o = 0u, a = 0xFFFFFFFFu;
    for (int j = lane_id(); j < n; j += kWave) {
        const uint32_t k = rb.key[j];
        o |= k;
        a &= k;
    }
    o = wave_or(o);
    a = wave_and(a);
    const uint32_t diff = o ^ a;
    const int cp = diff == 0u ? 32 : __clz(diff);
    *pv = cp == 0 ? 0u : (a & (0xFFFFFFFFu << (32 - cp)));
    return cp;
}

// Exact k-th largest key of the buffer: returns kappa, *ties = how many
// entries equal to kappa belong to the top `need` (the rest of the top are
// strictly greater).
template <typename Pos>
__device__ uint32_t wave_kth_key(const RowBuf<Pos>& rb, int n, uint32_t need, uint32_t* ties) {
    uint32_t pv;
    const int cp = wave_common_prefix(rb, n, &pv);
    uint32_t pm = cp == 0 ? 0u : (0xFFFFFFFFu << (32 - cp));
    int hi = 32 - cp;
    while (hi > 0) {
        const int width = hi < 8 ? hi : 8;
        const int shift = hi - width;
        const uint32_t dmask = (1u << width) - 1u;
        wave_hist(rb, n, pm, pv, shift, dmask);
        uint32_t above, inb;
        const uint32_t b = wave_find_bin(rb, need, &above, &inb);
        need -= above;
        pv |= b << shift;
        pm |= dmask << shift;
        hi = shift;
    }
    *ties = need;
    return pv;
}

// Drops buffer entries that cannot be in the top k.  Returns the new count
// and the new append threshold (append iff key > *thr).
template <typename Pos>
__device__ int wave_compact(const RowBuf<Pos>& rb, int n, uint32_t K, uint32_t* thr, int cap) {
    const int l = lane_id();
    uint32_t pv;
    const int cp = wave_common_prefix(rb, n, &pv);
    uint32_t lo_edge;  // keep keys >= lo_edge
    bool exact = false;
    uint32_t kappa = 0, ties = 0;
    if (cp < 32) {
        const int hi = 32 - cp;
        const int width = hi < 8 ? hi : 8;
        const int shift = hi - width;
        const uint32_t dmask = (1u << width) - 1u;
        const uint32_t pm = cp == 0 ? 0u : (0xFFFFFFFFu << (32 - cp));
        wave_hist(rb, n, pm, pv, shift, dmask);
        uint32_t above, inb;
        const uint32_t b = wave_find_bin(rb, K, &above, &inb);
        lo_edge = pv | (b << shift);
        // Too many entries would survive (a crowded bin): fall back to exact.
        if (above + inb > (uint32_t)(cap - 512)) exact = true;
    } else {
        exact = true;  // all keys equal
    }
    if (exact) kappa = wave_kth_key(rb, n, K, &ties);

    int wpos = 0;
    uint32_t tie_seen = 0;
    for (int j0 = 0; j0 < n; j0 += kWave) {
        const int j = j0 + l;
        const bool ok = j < n;
        const uint32_t k = ok ? rb.key[j] : 0u;
        const Pos p = ok ? rb.pos[j] : (Pos)0;
        bool keep;
        if (exact) {
            const bool eq = ok && k == kappa;
            const uint64_t me = wave_ballot(eq);
            const uint32_t rank = tie_seen + (uint32_t)lanes_below(me);
            keep = ok && (k > kappa || (eq && rank < ties));
            tie_seen += (uint32_t)__builtin_popcountll(me);
        } else {
            keep = ok && k >= lo_edge;
        }
        const uint64_t m = wave_ballot(keep);
        if (keep) {
            const int o = wpos + lanes_below(m);
            rb.key[o] = k;
            rb.pos[o] = p;
        }
        wpos += __builtin_popcountll(m);
    }
    __builtin_amdgcn_wave_barrier();
    *thr = exact ? kappa : (lo_edge == 0u ? 0u : lo_edge - 1u);
    return wpos;
}

// Writes the exact top K of the buffer (or all of it when n <= K) to the
// output row, then the -1 / -inf padding.
template <typename Pos>
__device__ void wave_emit(const RowBuf<Pos>& rb, int n, int K, int32_t* idx, float* val) {
    const int l = lane_id();
    if (n <= K) {
        for (int j = l; j < K; j += kWave) {
            if (j < n) {
                idx[j] = (int32_t)rb.pos[j];
                if (val) val[j] = key_score(rb.key[j]);
            } else {
                idx[j] = -1;
                if (val) val[j] = -INFINITY;
            }
        }
        return;
    }
    uint32_t ties;
    const uint32_t kappa = wave_kth_key(rb, n, (uint32_t)K, &ties);
    int wpos = 0;
    uint32_t tie_seen = 0;
    for (int j0 = 0; j0 < n; j0 += kWave) {
        const int j = j0 + l;
        const bool ok = j < n;
        const uint32_t k = ok ? rb.key[j] : 0u;
        const bool eq = ok && k == kappa;
        const uint64_t me = wave_ballot(eq);
        const uint32_t rank = tie_seen + (uint32_t)lanes_below(me);
        const bool keep = ok && (k > kappa || (eq && rank < ties));
        tie_seen += (uint32_t)__builtin_popcountll(me);
        const uint64_t m = wave_ballot(keep);
        const int o = wpos + lanes_below(m);
        if (keep && o < K) {  // exactly K entries are kept
            idx[o] = (int32_t)rb.pos[j];
            if (val) val[o] = key_score(k);
        }
        wpos += __builtin_popcountll(m);
    }
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

    float c[HB][4];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int h = 16 * hb + 4 * g + i;
            float cf = a.w[row_t * H + h] * a.inv_sqrt_d;
            if constexpr (DT == 2) cf *= a.q_scale[row_t * H + h];
            c[hb][i] = cf;
        }
    const float* kscale = DT == 2 ? a.k_scale + (size_t)b * L : nullptr;
    float* srow = a.scores ? a.scores + row_t * L : nullptr;

    auto load_chunk = [&](int s0, typename Op::Bt (&Bk)[4], float& ksc) {
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            int s = s0 + 16 * st + n;
            s = s < L ? s : L - 1;
            Op::load_b(Bk[st], kbase + (size_t)s * Op::kRowBytes, g);
        }
        if constexpr (DT == 2) {
            const int s = s0 + lane;
            ksc = kscale[s < L ? s : L - 1];
        }
    };

    int nb = 0;           // candidates in the buffer (wave-uniform)
    uint32_t thr = 0u;    // append iff key > thr
    const int last = t / 64;
    typename Op::Bt Bn[4];
    float ksn = 1.f;
    load_chunk(0, Bn, ksn);
    for (int chunk = 0; chunk <= last; ++chunk) {
        const int s0 = chunk * 64;
        typename Op::Bt Bk[4];
#pragma unroll
        for (int st = 0; st < 4; ++st) Bk[st] = Bn[st];
        const float ksc = ksn;
        if constexpr (DT == 2) {
            if (chunk < last) load_chunk(s0 + 64, Bn, ksn);   // prefetch the next chunk's keys
        }
        v4f acc[4][HB];
#pragma unroll
        for (int st = 0; st < 4; ++st) Op::template mma<HB>(acc[st], Aq, Bk[st]);
        if constexpr (DT != 2) {
            if (chunk < last) load_chunk(s0 + 64, Bn, ksn);
        }
        float part[4];
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            float p = 0.f;
#pragma unroll
            for (int hb = 0; hb < HB; ++hb)
#pragma unroll
                for (int i = 0; i < 4; ++i) p = fmaf(c[hb][i], relu(acc[st][hb][i]), p);
            part[st] = p;
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
    }
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
    static bool attr = false;
    if (!attr) {
        hipError_t e = hipFuncSetAttribute((const void*)prefill_fused_kernel<DT, HB, POS16>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        if (e != hipSuccess) return e;
        attr = true;
    }
    const int nblk = (a.L + Cfg::kWaves - 1) / Cfg::kWaves;
    hipLaunchKernelGGL((prefill_fused_kernel<DT, HB, POS16>), dim3((unsigned)(nblk * a.B)),
                       dim3(Cfg::kWaves * kWave), smem, stream, a);
    return hipGetLastError();
}

template <int DT, int HB>
hipError_t launch_pos(const PrefillArgs& a, hipStream_t stream) {
    return a.L <= 65536 ? launch_one<DT, HB, true>(a, stream) : launch_one<DT, HB, false>(a, stream);
}

}  // namespace

hipError_t launch_prefill_fused(const PrefillArgs& a, int dtype, hipStream_t stream) {
    const int hb = a.H / 16;
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
