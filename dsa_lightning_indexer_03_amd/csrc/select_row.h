// Exact top-k of one row, the body of the token selector: shared by the
// standalone selector kernel and the decode step's final kernel.
//
// One 1024-thread workgroup owns one row.  Selection is a radix select over
// a 54-bit composite  (score key, ~position):  the order-preserving 32-bit
// key of the score (larger = better) followed by the bit-inverted position
// (so among equal scores the lower position is better).  All composites of a
// row are distinct, so the k-th largest composite C* splits the row exactly:
// the selected set is every entry with composite >= C*.
//
// Digits, most significant first:  key[31:21], key[20:10], key[9:0],
// ~pos[21:11], ~pos[10:0].  A row that fits in LDS is read once, into LDS,
// and every digit is resolved there.  Otherwise the first digit's histogram
// is supplied by the producer of the scores or built by one pass over the
// row, and as soon as the entries that still tie with the chosen prefix fit
// in LDS, one pass over the row writes every entry above the prefix straight
// to the output and copies the tied ones to LDS; the remaining digits are
// then resolved in LDS.  The descent stops at the first digit where the
// entries tied with the prefix exactly fill the remaining slots.
#pragma once
#include "common.h"
#include "kernels.h"

namespace dsaidx {
namespace sel {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kBins = 2048;
constexpr int kCap = 12288;  // LDS candidate capacity (entries)

struct Level {
    int on_idx;   // 0: digit taken from the key, 1: from ~position
    int shift;
    int bits;
};
// Digit i of the composite, most significant first.
__device__ __forceinline__ Level level_at(int i) {
    switch (i) {
        case 0: return {0, 21, 11};
        case 1: return {0, 10, 11};
        case 2: return {0, 0, 10};
        case 3: return {1, 11, 11};
        default: return {1, 0, 11};
    }
}

struct SelShared {
    uint32_t hist[kBins];
    uint32_t cand_key[kCap];
    uint32_t cand_pos[kCap];
    uint32_t wave_tot[kWaves];
    uint32_t out_n;
    uint32_t cand_n;
    uint32_t bin;
    uint32_t above;
};

__device__ __forceinline__ uint32_t level_digit(const Level& lv, uint32_t key, uint32_t npos) {
    uint32_t src = lv.on_idx ? npos : key;
    return (src >> lv.shift) & ((1u << lv.bits) - 1u);
}

// Exclusive block-wide prefix sum of one value per thread.
__device__ inline uint32_t block_excl_scan(uint32_t v, SelShared& sh) {
    const int w = threadIdx.x / kWave;
    uint32_t inc = wave_incl_scan(v);
    if (lane_id() == kWave - 1) sh.wave_tot[w] = inc;
    __syncthreads();
    if (w == 0) {
        uint32_t t = lane_id() < kWaves ? sh.wave_tot[lane_id()] : 0u;
        uint32_t ti = wave_incl_scan(t);
        if (lane_id() < kWaves) sh.wave_tot[lane_id()] = ti - t;
    }
    __syncthreads();
    uint32_t r = inc - v + sh.wave_tot[w];
    __syncthreads();
    return r;
}

// Finds the bin b (counting from the top) where the running count reaches
// `need`; stores b and the count of entries in bins above b.
__device__ inline void find_bin(SelShared& sh, int nbins, uint32_t need) {
    const int t = threadIdx.x;
    const int per = nbins / kThreads;  // 1 or 2 (10- or 11-bit digit)
    uint32_t c0 = 0, c1 = 0;
    int b0 = -1, b1 = -1;
    if (per == 2) {
        b0 = nbins - 1 - 2 * t;
        b1 = b0 - 1;
        c0 = sh.hist[b0];
        c1 = sh.hist[b1];
    } else {
        b0 = nbins - 1 - t;
        c0 = sh.hist[b0];
    }
    uint32_t excl = block_excl_scan(c0 + c1, sh);
    if (excl < need && need <= excl + c0) {
        sh.bin = (uint32_t)b0;
        sh.above = excl;
    } else if (per == 2 && excl + c0 < need && need <= excl + c0 + c1) {
        sh.bin = (uint32_t)b1;
        sh.above = excl + c0;
    }
    __syncthreads();
}

__device__ __forceinline__ void emit(SelShared& sh, bool take, uint32_t pos, float v,
                                     int32_t* idx_out, float* val_out, uint32_t limit) {
    uint64_t m = wave_ballot(take);
    if (m == 0) return;
    uint32_t base = 0;
    const int leader = __builtin_ctzll(m);
    if (lane_id() == leader) base = atomicAdd(&sh.out_n, (uint32_t)__builtin_popcountll(m));
    base = __shfl(base, leader, kWave);
    if (take) {
        uint32_t o = base + (uint32_t)lanes_below(m);
        if (o >= limit) return;  // cannot happen: exactly `limit` entries are emitted
        idx_out[o] = (int32_t)pos;
        if (val_out) val_out[o] = v;
    }
}

// The row's first 4 * kThreads entries, loaded by the caller before it knew
// the row's length (lane t holds entries t + u * kThreads, inside the row's
// stride); used only where they are below the length.
struct Preload {
    float v[4];
    uint32_t p[4];
};

// Selects row `row` of `a` with the whole workgroup (kThreads threads) and
// the LDS block `sh`.  n_known >= 0 overrides the row's entry count; with
// use_pre, `pre` holds the row's first entries already loaded.
__device__ __forceinline__ void select_row(const SelectArgs& a, const int row, SelShared& sh, const int n_known,
                                          const Preload& pre, const bool use_pre) {
    const int t = threadIdx.x;
    const float* src = a.scores + (int64_t)row * a.row_stride;
    const int32_t* psrc = a.pos ? a.pos + (int64_t)row * a.row_stride : nullptr;
    int n = a.cols;
    if (a.causal_L > 0) n = (row % a.causal_L) + 1;
    const int64_t cstride = a.counter_stride > 0 ? a.counter_stride : 1;
    if (a.causal_L <= 0 && a.row_len) n = a.row_len[row * cstride];
    if (n_known >= 0) n = n_known;
    n = n < 0 ? 0 : (n > a.cols ? a.cols : n);
    const int K = a.topk;
    // Output slots [0, G) were filled by the producer; this row returns
    // min(K, total) positions in all, R of them chosen here among n entries.
    const int G = a.pre_count ? (int)min(a.pre_count[row * cstride], (uint32_t)K) : 0;
    int total = n;
    if (a.total) {
        total = a.total[row];
        total = total < 0 ? 0 : (total > a.total_max ? a.total_max : total);
    }
    const int Rtot = total < K ? total : K;
    int R = Rtot - G;
    R = R < 0 ? 0 : (R > n ? n : R);
    int32_t* idx_out = a.idx_out + (int64_t)row * K + G;
    float* val_out = a.val_out ? a.val_out + (int64_t)row * K + G : nullptr;

    if (R == n || R == 0) {  // every entry, or none, is selected
        for (int j = t; j < R; j += kThreads) {
            idx_out[j] = psrc ? psrc[j] : j;
            if (val_out) val_out[j] = src[j];
        }
        for (int j = G + R + t; j < K; j += kThreads) {
            a.idx_out[(int64_t)row * K + j] = -1;
            if (a.val_out) a.val_out[(int64_t)row * K + j] = -INFINITY;
        }
        return;
    }

    uint32_t need = (uint32_t)R;
    uint32_t pk = 0, mk = 0, pi = 0, mi = 0;  // fixed prefix (value, mask) of key and ~pos
    bool in_lds = false;
    int level = 0;
    const bool known0 = a.level0_bin != nullptr;
    if (t == 0) {
        sh.out_n = 0;
        sh.cand_n = 0;
    }
    // ---- level-0 histogram (unless every entry's first digit is known) ----
    if (!known0 && n <= kCap) {
        // The whole row goes to LDS, read once (U loads per thread in flight).
        constexpr int U = 4;
        for (int b = t; b < kBins; b += kThreads) sh.hist[b] = 0;
        if (t == 0) sh.cand_n = (uint32_t)n;
        __syncthreads();
        for (int j0 = 0; j0 < n; j0 += U * kThreads) {
            float v[U];
            uint32_t p[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int j = j0 + u * kThreads + t;
                if (use_pre && j0 == 0) {
                    v[u] = pre.v[u];
                    p[u] = pre.p[u];
                } else {
                    v[u] = j < n ? src[j] : 0.f;
                    p[u] = j < n ? (psrc ? (uint32_t)psrc[j] : (uint32_t)j) : 0u;
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int j = j0 + u * kThreads + t;
                const bool ok = j < n;
                const uint32_t key = score_key(v[u]);
                if (ok) {
                    sh.cand_key[j] = key;
                    sh.cand_pos[j] = p[u];
                }
                // The keys of a row's candidates often share their top digit
                // (a decode query's all lie above its floor): the lanes with the
                // first valid lane's digit add their count in one atomic, the
                // others one each.
                const uint64_t mv = wave_ballot(ok);
                if (mv != 0) {
                    const int first = __builtin_ctzll(mv);
                    const uint32_t d = key >> 21;
                    const uint32_t d0 = (uint32_t)__builtin_amdgcn_readlane((int)d, first);
                    const uint64_t ms = wave_ballot(ok && d == d0);
                    if (lane_id() == first) atomicAdd(&sh.hist[d0], (uint32_t)__builtin_popcountll(ms));
                    if (ok && d != d0) atomicAdd(&sh.hist[d], 1u);
                }
            }
        }
        in_lds = true;
    } else if (a.hist) {
        const uint32_t* h = a.hist + (int64_t)row * kBins;
        for (int b = t; b < kBins; b += kThreads) sh.hist[b] = h[b];
    } else if (!known0) {
        for (int b = t; b < kBins; b += kThreads) sh.hist[b] = 0;
        __syncthreads();
        for (int j = t; j < n; j += kThreads) atomicAdd(&sh.hist[score_key(src[j]) >> 21], 1u);
    }
    __syncthreads();

    for (;;) {
        const Level lv = level_at(level);
        uint32_t b, cnt;
        if (known0 && level == 0) {
            b = a.level0_bin[row * cstride];
            cnt = (uint32_t)n;
        } else {
            find_bin(sh, 1 << lv.bits, need);
            b = sh.bin;
            need -= sh.above;
            cnt = sh.hist[b];
        }
        const uint32_t fm = ((1u << lv.bits) - 1u) << lv.shift;
        if (lv.on_idx) { pi |= b << lv.shift; mi |= fm; }
        else           { pk |= b << lv.shift; mk |= fm; }
        __syncthreads();

        if (!in_lds && cnt <= (uint32_t)kCap) {
            // One pass over the row: above the prefix -> output, equal -> LDS.
            for (int j0 = 0; j0 < n; j0 += kThreads) {
                const int j = j0 + t;
                const bool ok = j < n;
                const float v = ok ? src[j] : 0.f;
                const uint32_t p = ok ? (psrc ? (uint32_t)psrc[j] : (uint32_t)j) : 0u;
                const uint32_t key = score_key(v), np = ~p;
                const uint32_t kt = key & mk, it = np & mi;
                const bool above = ok && (kt > pk || (kt == pk && it > pi));
                const bool tie = ok && kt == pk && it == pi;
                emit(sh, above, p, v, idx_out, val_out, (uint32_t)R);
                uint64_t m = wave_ballot(tie);
                if (m) {
                    uint32_t base = 0;
                    const int leader = __builtin_ctzll(m);
                    if (lane_id() == leader) base = atomicAdd(&sh.cand_n, (uint32_t)__builtin_popcountll(m));
                    base = __shfl(base, leader, kWave);
                    const uint32_t o = base + (uint32_t)lanes_below(m);
                    if (tie && o < (uint32_t)kCap) {
                        sh.cand_key[o] = key;
                        sh.cand_pos[o] = p;
                    }
                }
            }
            in_lds = true;
            __syncthreads();
        }
        // Every entry tied with the prefix is selected: no finer digit matters.
        if (level == 4 || (in_lds && cnt == need)) break;
        ++level;

        // Histogram of the next digit over the entries matching the prefix.
        const Level nx = level_at(level);
        for (int x = t; x < kBins; x += kThreads) sh.hist[x] = 0;
        __syncthreads();
        if (in_lds) {
            const int cn = min((int)sh.cand_n, kCap);
            for (int j = t; j < cn; j += kThreads) {
                const uint32_t key = sh.cand_key[j], np = ~sh.cand_pos[j];
                if ((key & mk) == pk && (np & mi) == pi) atomicAdd(&sh.hist[level_digit(nx, key, np)], 1u);
            }
        } else {
            for (int j = t; j < n; j += kThreads) {
                const uint32_t key = score_key(src[j]);
                const uint32_t np = ~(psrc ? (uint32_t)psrc[j] : (uint32_t)j);
                if ((key & mk) == pk && (np & mi) == pi) atomicAdd(&sh.hist[level_digit(nx, key, np)], 1u);
            }
        }
        __syncthreads();
    }

    // Prefix (pk under mk, pi under mi) fixed far enough: every LDS entry at
    // or above it is selected.
    {
        const int cn = min((int)sh.cand_n, kCap);
        for (int j0 = 0; j0 < cn; j0 += kThreads) {
            const int j = j0 + t;
            bool take = false;
            uint32_t pos = 0, key = 0;
            if (j < cn) {
                key = sh.cand_key[j];
                pos = sh.cand_pos[j];
                const uint32_t kt = key & mk, it = ~pos & mi;
                take = kt > pk || (kt == pk && it >= pi);
            }
            emit(sh, take, pos, key_score(key), idx_out, val_out, (uint32_t)R);
        }
    }
    __syncthreads();
    for (int j = Rtot + t; j < K; j += kThreads) {
        a.idx_out[(int64_t)row * K + j] = -1;
        if (a.val_out) a.val_out[(int64_t)row * K + j] = -INFINITY;
    }
}


__device__ __forceinline__ void select_row(const SelectArgs& a, const int row, SelShared& sh, const int n_known) {
    const Preload none{};
    select_row(a, row, sh, n_known, none, false);
}

}  // namespace sel
}  // namespace dsaidx
