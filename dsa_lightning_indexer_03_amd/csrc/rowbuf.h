// Per-wave streaming top-k candidate buffer in LDS, shared by the fused
// prefill kernels: a row's (key, position) pairs, where key is the
// order-preserving 32-bit image of the score (score_key) and a larger key is
// a better entry; among equal keys the lower position wins.  One wave owns a
// buffer and walks it 256 entries per step (lane l holds entries
// 256*step + 4*l .. +3), so every routine below is wave-uniform.
//
// Positions are 16 bits wide (rows up to 65536 positions) or 32 bits.  A
// 17-bit position (rows up to 131072 positions) fits the 16-bit layout when
// the key gives up its lowest bit: the stored word is
//     (score_key & ~1) | (1 - bit 16 of the position)
// and the 16-bit slot holds the position's low 16 bits.  Ordering by (word
// desc, low bits asc) is then exactly ordering by (truncated key desc,
// position asc), so the selection routines need no change; only the final
// decode (entry_pos, entry_score with P17 = true) differs.  The dropped bit
// is below fp32's last mantissa place of the score: a relative change of at
// most 2^-23.
#pragma once

#include "common.h"

namespace dsaidx {
namespace {

// Position and score of a buffer entry (word k, stored position p).
template <bool P17>
__device__ __forceinline__ int32_t entry_pos(uint32_t k, uint32_t p) {
    return P17 ? (int32_t)((((~k) & 1u) << 16) | (p & 0xFFFFu)) : (int32_t)p;
}
template <bool P17>
__device__ __forceinline__ float entry_score(uint32_t k) {
    return key_score(P17 ? (k & ~1u) : k);
}
// The stored word of a score at position s.
template <bool P17>
__device__ __forceinline__ uint32_t entry_word(float score, uint32_t s) {
    const uint32_t k = score_key(score);
    return P17 ? ((k & ~1u) | (((s >> 16) & 1u) ^ 1u)) : k;
}

// Per-wave candidate buffer in LDS.
template <typename Pos>
struct RowBuf {
    uint32_t* key;
    Pos* pos;
    uint32_t* hist;  // 256 16-bit bins, two per word (bin b: word b/2, half b%2)
};

// The buffer routines below walk the buffer 256 entries per step, lane l
// holding entries 256*step + 4*l .. +3 (one 16-byte key read, one 8- or
// 16-byte position read), so each step keeps four independent LDS reads in
// flight instead of one.  Buffer capacities are multiples of 256.
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));

template <typename Pos>
struct Pos4 { Pos v[4]; };

template <typename Pos>
__device__ __forceinline__ Pos4<Pos> read_pos4(const Pos* p) {
    Pos4<Pos> r;
    if constexpr (sizeof(Pos) == 2) {
        const uint2 u = *reinterpret_cast<const uint2*>(p);
        r.v[0] = (Pos)(u.x & 0xFFFF); r.v[1] = (Pos)(u.x >> 16);
        r.v[2] = (Pos)(u.y & 0xFFFF); r.v[3] = (Pos)(u.y >> 16);
    } else {
        const v4u u = *reinterpret_cast<const v4u*>(p);
        r.v[0] = (Pos)u[0]; r.v[1] = (Pos)u[1]; r.v[2] = (Pos)u[2]; r.v[3] = (Pos)u[3];
    }
    return r;
}

// Position as an unsigned value of the buffer's position width, inverted so
// that a lower position compares larger.
template <typename Pos>
__device__ __forceinline__ uint32_t inv_pos(Pos p) {
    return (uint32_t)(Pos)~p;
}

// Histogram of an 8-bit (or narrower) digit over matching buffer entries.
// BY_POS = false: digit (key >> shift) & dmask of the entries whose key has
//   (key & pm) == pv.
// BY_POS = true: digit of the inverted position of the entries whose key
//   equals kappa and whose inverted position has (ipos & pm) == pv.
template <bool BY_POS, typename Pos>
__device__ __forceinline__ void wave_hist(const RowBuf<Pos>& rb, int n, uint32_t kappa, uint32_t pm, uint32_t pv,
                                          int shift, uint32_t dmask) {
    const int l = lane_id();
#pragma unroll
    for (int i = 0; i < 2; ++i) rb.hist[l + 64 * i] = 0u;
    __builtin_amdgcn_wave_barrier();
    for (int j0 = 0; j0 < n; j0 += 256) {
        const int j = j0 + 4 * l;
        const v4u k = *reinterpret_cast<const v4u*>(rb.key + j);
        if constexpr (BY_POS) {
            const Pos4<Pos> p = read_pos4(rb.pos + j);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t ip = inv_pos(p.v[e]);
                if (j + e < n && k[e] == kappa && (ip & pm) == pv) {
                    const uint32_t bin = (ip >> shift) & dmask;
                    atomicAdd(&rb.hist[bin >> 1], 1u << ((bin & 1u) << 4));
                }
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (j + e < n && (k[e] & pm) == pv) {
                    const uint32_t bin = (k[e] >> shift) & dmask;
                    atomicAdd(&rb.hist[bin >> 1], 1u << ((bin & 1u) << 4));
                }
        }
    }
    __builtin_amdgcn_wave_barrier();
}

// Histogram of digit (key >> shift) & (2^width - 1) over all n entries,
// for a digit right below the keys' common prefix (every entry takes part).
// Branch free: a lane past the end adds zero.
template <typename Pos>
__device__ __forceinline__ void wave_hist_top(const RowBuf<Pos>& rb, int n, int shift, int width) {
    const int l = lane_id();
#pragma unroll
    for (int i = 0; i < 2; ++i) rb.hist[l + 64 * i] = 0u;
    __builtin_amdgcn_wave_barrier();
    for (int j0 = 0; j0 < n; j0 += 256) {
        const int j = j0 + 4 * l;
        const v4u k = *reinterpret_cast<const v4u*>(rb.key + j);
        const bool full = j0 + 256 <= n;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            // bin b: word b / 2, half b % 2
            const uint32_t word = __builtin_amdgcn_ubfe(k[e], (uint32_t)shift + 1u, (uint32_t)width - 1u);
            const uint32_t half = __builtin_amdgcn_ubfe(k[e], (uint32_t)shift, 1u);
            const uint32_t inc = (full | (j + e < n)) ? 1u << (half << 4) : 0u;
            atomicAdd(&rb.hist[word], inc);
        }
    }
    __builtin_amdgcn_wave_barrier();
}

// Bin (counting down from the top) where the running count reaches `need`.
// Returns the bin; *above = count in bins above it.
template <typename Pos>
__device__ __forceinline__ uint32_t wave_find_bin(const RowBuf<Pos>& rb, uint32_t need, uint32_t* above,
                                                  uint32_t* in_bin) {
    const int l = lane_id();
    // bins 255-4l .. 252-4l: the high and low halves of words 127-2l, 126-2l
    const uint32_t w_hi = rb.hist[127 - 2 * l], w_lo = rb.hist[126 - 2 * l];
    const uint32_t c[4] = {w_hi >> 16, w_hi & 0xFFFFu, w_lo >> 16, w_lo & 0xFFFFu};
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
    *above = (uint32_t)__builtin_amdgcn_readlane((int)ab, src);
    *in_bin = (uint32_t)__builtin_amdgcn_readlane((int)cnt, src);
    return (uint32_t)__builtin_amdgcn_readlane(bin, src);
}

// Common leading bits of all buffer keys: returns their count; *pv = value.
template <typename Pos>
__device__ __forceinline__ int wave_common_prefix(const RowBuf<Pos>& rb, int n, uint32_t* pv) {
    uint32_t o = 0u, a = 0xFFFFFFFFu;
    const int l = lane_id();
    for (int j0 = 0; j0 < n; j0 += 256) {
        const int j = j0 + 4 * l;
        const v4u k = *reinterpret_cast<const v4u*>(rb.key + j);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (j + e < n) { o |= k[e]; a &= k[e]; }
    }
    o = wave_or(o);
    a = wave_and(a);
    const uint32_t diff = o ^ a;
    const int cp = diff == 0u ? 32 : __clz(diff);
    *pv = cp == 0 ? 0u : (a & (0xFFFFFFFFu << (32 - cp)));
    return cp;
}

// Exact `need`-th largest key of the buffer (1 <= need <= n): returns kappa;
// *ties = how many entries equal to kappa belong to the top `need` (the rest
// of the top are strictly greater); *eq = how many entries equal kappa.
// Early end: when the entries of a digit's bin exactly fill the rest of the
// top, kappa is that bin's lower edge and *ties = *eq = their count, so
// "key > kappa, or key == kappa at any position" is again exactly the top
// `need` (every key of the bin is >= its edge, every key below it is less).
template <typename Pos>
__device__ uint32_t wave_kth_key(const RowBuf<Pos>& rb, int n, uint32_t need, uint32_t* ties, uint32_t* eq) {
    uint32_t pv;
    const int cp = wave_common_prefix(rb, n, &pv);
    uint32_t pm = cp == 0 ? 0u : (0xFFFFFFFFu << (32 - cp));
    int hi = 32 - cp;
    uint32_t inb = (uint32_t)n;  // all keys equal when no digit is left
    bool first = true;
    while (hi > 0) {
        const int width = hi < 8 ? hi : 8;
        const int shift = hi - width;
        const uint32_t dmask = (1u << width) - 1u;
        if (first) wave_hist_top(rb, n, shift, width);  // every entry shares the prefix
        else wave_hist<false>(rb, n, 0u, pm, pv, shift, dmask);
        first = false;
        uint32_t above;
        const uint32_t b = wave_find_bin(rb, need, &above, &inb);
        need -= above;
        pv |= b << shift;
        pm |= dmask << shift;
        hi = shift;
        if (need == inb) break;
    }
    *ties = need;
    *eq = inb;
    return pv;
}

// Tie break at the k-th key: among the entries whose key equals kappa, the
// `ties` lowest positions win (1 <= ties <= count of such entries).  Returns
// the largest winning position; an entry with key kappa wins iff its
// position is <= the result.  Radix select on inverted positions.
template <typename Pos>
__device__ uint32_t wave_tie_cut(const RowBuf<Pos>& rb, int n, uint32_t kappa, uint32_t ties) {
    uint32_t pm = 0u, pv = 0u, need = ties;
    for (int hi = 8 * (int)sizeof(Pos); hi > 0; hi -= 8) {
        const int shift = hi - 8;
        wave_hist<true>(rb, n, kappa, pm, pv, shift, 0xFFu);
        uint32_t above, inb;
        const uint32_t b = wave_find_bin(rb, need, &above, &inb);
        need -= above;
        pv |= b << shift;
        pm |= 0xFFu << shift;
    }
    return inv_pos((Pos)pv);
}

// One pass over the buffer keeping every entry with key > kappa or (key ==
// kappa and position <= pos_cut) when EXACT, else every entry with key >=
// lo_edge, to the buffer front, in place.  Within a step the kept entries
// are written slot by slot (slot e of every lane, then slot e+1), so the
// lanes of one store write consecutive words; this stays below the step's
// own entries (at most 256 kept, starting at or below the step's first
// index), which are already in registers.  Branch free: a lane that drops
// its entry writes it to a slot of its own in the histogram words (not
// needed once the cut is known).
template <bool EXACT, typename Pos>
__device__ int wave_keep_inplace(const RowBuf<Pos>& rb, int n, uint32_t kappa, uint32_t pos_cut, uint32_t lo_edge) {
    const int l = lane_id();
    uint32_t* const dk = rb.hist + l;
    Pos* const dp = reinterpret_cast<Pos*>(rb.hist + kWave) + l;
    int wpos = 0;
    for (int j0 = 0; j0 < n; j0 += 256) {
        const int j = j0 + 4 * l;
        const v4u k = *reinterpret_cast<const v4u*>(rb.key + j);
        const Pos4<Pos> p = read_pos4(rb.pos + j);
        const bool full = j0 + 256 <= n;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            // bitwise, not short-circuit, operators: no branches
            bool keep = EXACT ? ((k[e] > kappa) | ((k[e] == kappa) & ((uint32_t)p.v[e] <= pos_cut))) : k[e] >= lo_edge;
            keep &= full | (j + e < n);
            const uint64_t m = wave_ballot(keep);
            const int o = wpos + lanes_below(m);
            *(keep ? rb.key + o : dk) = k[e];
            *(keep ? rb.pos + o : dp) = p.v[e];
            wpos += __builtin_popcountll(m);
        }
    }
    __builtin_amdgcn_wave_barrier();
    return wpos;
}

// The exact top K (key > kappa, or key == kappa and position <= pos_cut) of
// the buffer to the output row, in buffer order of a step's slots.
template <typename Pos, bool P17 = false>
__device__ int wave_keep_out(const RowBuf<Pos>& rb, int n, uint32_t kappa, uint32_t pos_cut, int32_t* idx,
                             float* val, int limit) {
    const int l = lane_id();
    int wpos = 0;
    for (int j0 = 0; j0 < n; j0 += 256) {
        const int j = j0 + 4 * l;
        const v4u k = *reinterpret_cast<const v4u*>(rb.key + j);
        const Pos4<Pos> p = read_pos4(rb.pos + j);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bool keep = j + e < n && (k[e] > kappa || (k[e] == kappa && (uint32_t)p.v[e] <= pos_cut));
            const uint64_t m = wave_ballot(keep);
            const int o = wpos + lanes_below(m);
            if (keep && o < limit) {
                idx[o] = entry_pos<P17>(k[e], (uint32_t)p.v[e]);
                if (val) val[o] = entry_score<P17>(k[e]);
            }
            wpos += __builtin_popcountll(m);
        }
    }
    return wpos;
}

// Exact cut of the buffer to its top K by (key desc, position asc): returns
// kappa and the position cut for the keep passes.
template <typename Pos>
__device__ __forceinline__ uint32_t wave_exact_cut(const RowBuf<Pos>& rb, int n, uint32_t K, uint32_t* pos_cut) {
    uint32_t ties, eq;
    const uint32_t kappa = wave_kth_key(rb, n, K, &ties, &eq);
    *pos_cut = eq > ties ? wave_tie_cut(rb, n, kappa, ties) : 0xFFFFFFFFu;
    return kappa;
}

// Drops buffer entries that cannot be in the top K (n > K).  Returns the new
// count and the new append floor (append iff key > *thr).  Entries equal to
// the cut key stay admissible: in an out-of-order scan a later one may have
// a lower position.
//
// Speculative cut (1 <= r < K): the cut is the lower edge of the radix bin
// that holds the r-th largest key instead of the K-th, so fewer entries
// survive and the buffer refills later.  Every entry at or above the edge
// stays, so the buffer still holds every scanned key above the new floor;
// *spec reports whether this cut was taken (the caller must then verify at
// the end that at least K keys lie above its floor).  A crowded bin falls
// back to the exact cut at K, which is never speculative.
template <typename Pos>
__device__ int wave_compact(const RowBuf<Pos>& rb, int n, uint32_t K, uint32_t* thr, int cap, uint32_t r = 0u,
                            bool* spec = nullptr) {
    const uint32_t want = (r != 0u && r < K) ? r : K;
    uint32_t pv;
    const int cp = wave_common_prefix(rb, n, &pv);
    uint32_t lo_edge = 0;  // keep keys >= lo_edge
    bool exact = false;
    if (cp < 32) {
        const int hi = 32 - cp;
        const int width = hi < 8 ? hi : 8;
        const int shift = hi - width;
        wave_hist_top(rb, n, shift, width);
        uint32_t above, inb;
        const uint32_t b = wave_find_bin(rb, want, &above, &inb);
        lo_edge = pv | (b << shift);
        // Too many entries would survive (a crowded bin): fall back to exact.
        if (above + inb > (uint32_t)(cap - 256)) exact = true;
    } else {
        exact = true;  // all keys equal
    }
    uint32_t kappa = 0, pos_cut = 0;
    if (exact) kappa = wave_exact_cut(rb, n, K, &pos_cut);
    const int kept = exact ? wave_keep_inplace<true>(rb, n, kappa, pos_cut, 0u)
                           : wave_keep_inplace<false>(rb, n, 0u, 0u, lo_edge);
    const uint32_t fl = exact ? kappa : lo_edge;
    *thr = fl == 0u ? 0u : fl - 1u;
    if (spec) *spec = !exact && want < K;
    return kept;
}

// Speculative floor: keeps the entries whose key is at least the lower edge
// of the radix bin (one digit below the common prefix) that holds the r-th
// largest key, and returns that edge (<= the r-th largest key).  1 <= r <= n.
template <typename Pos>
__device__ int wave_floor(const RowBuf<Pos>& rb, int n, uint32_t r, uint32_t* floor_key) {
    uint32_t pv;
    const int cp = wave_common_prefix(rb, n, &pv);
    uint32_t lo_edge = pv;
    if (cp < 32) {
        const int hi = 32 - cp;
        const int width = hi < 8 ? hi : 8;
        const int shift = hi - width;
        wave_hist_top(rb, n, shift, width);
        uint32_t above, inb;
        const uint32_t b = wave_find_bin(rb, r, &above, &inb);
        lo_edge = pv | (b << shift);
    }
    *floor_key = lo_edge;
    return wave_keep_inplace<false>(rb, n, 0u, 0u, lo_edge);
}

// One pass that splits the buffer at the radix bin `bdig` (the value of
// key >> shift, prefix and digit): entries above the bin -- and, with
// `fill`, those in it -- go to the output row (idx/val from slot 0, in
// buffer order of a step's slots); without `fill`, the bin's entries move to
// the buffer front in place (as in wave_keep_inplace, dropped lanes writing
// a slot of their own in the histogram words).  Returns how many moved.
template <typename Pos, bool P17>
__device__ int wave_split_out(const RowBuf<Pos>& rb, int n, int shift, uint32_t bdig, bool fill, int32_t* idx,
                              float* val) {
    const int l = lane_id();
    uint32_t* const dk = rb.hist + l;
    Pos* const dp = reinterpret_cast<Pos*>(rb.hist + kWave) + l;
    int wpos = 0, opos = 0;
    for (int j0 = 0; j0 < n; j0 += 256) {
        const int j = j0 + 4 * l;
        const v4u k = *reinterpret_cast<const v4u*>(rb.key + j);
        const Pos4<Pos> p = read_pos4(rb.pos + j);
        const bool full = j0 + 256 <= n;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bool in = full | (j + e < n);
            const uint32_t d = k[e] >> shift;
            const bool out = in & ((d > bdig) | (fill & (d == bdig)));
            const bool keep = in & (!fill) & (d == bdig);
            const uint64_t mo = wave_ballot(out);
            if (out) {
                const int o = opos + lanes_below(mo);
                idx[o] = entry_pos<P17>(k[e], (uint32_t)p.v[e]);
                if (val) val[o] = entry_score<P17>(k[e]);
            }
            opos += __builtin_popcountll(mo);
            const uint64_t mk = wave_ballot(keep);
            const int w = wpos + lanes_below(mk);
            *(keep ? rb.key + w : dk) = k[e];
            *(keep ? rb.pos + w : dp) = p.v[e];
            wpos += __builtin_popcountll(mk);
        }
    }
    __builtin_amdgcn_wave_barrier();
    return wpos;
}

// Writes the exact top K of the buffer by (key desc, position asc) -- or all
// of it when n <= K -- to the output row, then the -1 / -inf padding.
//
// Three passes over the buffer: the keys' common prefix, the histogram of
// the digit below it, then one pass that writes every entry above the bin
// holding the K-th key and gathers that bin's entries at the buffer front.
// The rest of the row is the exact top (K - above) of the bin, selected
// over those few entries alone.
template <typename Pos, bool P17 = false>
__device__ void wave_emit(const RowBuf<Pos>& rb, int n, int K, int32_t* idx, float* val) {
    const int l = lane_id();
    if (n <= K) {
        for (int j = l; j < K; j += kWave) {
            if (j < n) {
                idx[j] = entry_pos<P17>(rb.key[j], (uint32_t)rb.pos[j]);
                if (val) val[j] = entry_score<P17>(rb.key[j]);
            } else {
                idx[j] = -1;
                if (val) val[j] = -INFINITY;
            }
        }
        return;
    }
    uint32_t pv;
    const int cp = wave_common_prefix(rb, n, &pv);
    int n2 = n;
    uint32_t above = 0u;
    if (cp < 32) {
        const int hi = 32 - cp;
        const int width = hi < 8 ? hi : 8;
        const int shift = hi - width;
        wave_hist_top(rb, n, shift, width);
        uint32_t inb;
        const uint32_t b = wave_find_bin(rb, (uint32_t)K, &above, &inb);
        const bool fill = above + inb == (uint32_t)K;
        n2 = wave_split_out<Pos, P17>(rb, n, shift, (pv >> shift) | b, fill, idx, val);
        if (fill) return;
    }
    // all keys equal (cp == 32): the K lowest positions, over the whole buffer
    const uint32_t need = (uint32_t)K - above;
    uint32_t pos_cut;
    const uint32_t kappa = wave_exact_cut(rb, n2, need, &pos_cut);
    wave_keep_out<Pos, P17>(rb, n2, kappa, pos_cut, idx + above, val ? val + above : nullptr, (int)need);
}

}  // namespace
}  // namespace dsaidx
