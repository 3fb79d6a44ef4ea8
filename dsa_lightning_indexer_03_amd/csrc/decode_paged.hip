// Decode-step scan of a paged FP8 indexer key cache.
//
// One query per decode step scores every position of its cached context
// (the decode walkthrough of "Lightning Indexer explained", section 2: one
// dot of the current query against the whole indexer cache).  The scan is
// bound by the cache bytes it streams (128 fp8 bytes + a 4-byte scale per
// position), so the kernels are laid out for HBM:
//
// * persistent grid: the (query, page) pairs of all queries form one list
//   that is cut into equal shares, one per resident workgroup; each of a
//   workgroup's 4 waves takes whole 64-token pages (details at the kernel).
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
//
// Writes, not reads, set the price of keeping scores: a score stream of 4 B
// per 132 B read, interleaved with the cache reads, costs about a fifth of
// the scan.  So the scan writes only candidates:
//
// 1. The sample: a strided sample of every long query's pages (one page in
//    kSampleStride or sparser, at most kMaxSamplePages, from a per-query
//    offset) is scored, its keys kept in LDS, and the r-th largest sampled
//    key to 22 bits (two radix digits) becomes the query's floor, with r
//    five standard deviations above the expected number of sampled scores at
//    or above the query's k-th largest.  Workgroup floor(b G / B) of the
//    scan's G does this for query b before it scans (batches up to half the
//    scan's grid; a kernel of its own, one workgroup per query, for larger
//    batches).
// 2. The main scan scores every position and writes only the scores whose
//    key reaches the query's floor, to the query's candidate list (while a
//    floor is still being sampled, a wave keeps the query's scores back, see
//    the scan kernel).
// 3. Verification: if at least min(k, context) candidates reach the floor,
//    the k-th largest score is among them (and so is every score tied with
//    it, since the floor is a key threshold), so the selection over the
//    candidates is exact.  Otherwise a repair pass rescores the query in
//    full.
#include "common.h"
#include "device_once.h"
#include "kernels.h"
#include "select_row.h"

namespace dsaidx {

namespace {

constexpr int kD = 128;
constexpr int kPage = 64;
constexpr int kThreadsDec = 256;
constexpr int kPrefixLds = 2048;   // queries whose page prefix is searched in LDS
#ifndef DSAIDX_SAMPLE_PAGES
#define DSAIDX_SAMPLE_PAGES 32
#endif
constexpr int kSampleStride = 32;                       // at most one sampled page in this many
constexpr int kMaxSamplePages = DSAIDX_SAMPLE_PAGES;    // sampled pages of one query, at most
constexpr int kCandBuf = 1024;     // per-wave LDS candidate buffer (score, position) pairs
#ifndef DSAIDX_PRODUCER_PAGES
#define DSAIDX_PRODUCER_PAGES 24
#endif
constexpr int kProducerPages = DSAIDX_PRODUCER_PAGES;  // fused scan: pages' worth of time spent sampling a query

#ifndef DSAIDX_DECODE_NT
#define DSAIDX_DECODE_NT 0  // 1: non-temporal (streaming) loads of the key cache
#endif

template <typename T>
__device__ __forceinline__ T stream_load(const T* p) {
#if DSAIDX_DECODE_NT
    return __builtin_nontemporal_load(p);
#else
    return *p;
#endif
}

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

__device__ __forceinline__ int clamp_ctx(int ctx, int max_ctx) {
    return ctx < 0 ? 0 : (ctx > max_ctx ? max_ctx : ctx);
}

// Sampling of query b: pages off + stride * i for i < ns, with stride at
// least kSampleStride and large enough that ns <= kMaxSamplePages, and a
// hashed per-query offset off in [0, stride).  Only queries with context
// >= 4k and at least two strides of pages are sampled; the count is the same
// for every offset (pages o + stride i < np for all o < stride when
// i < (np - stride) / stride + 1, and that count is <= np / stride).
struct SamplePlan {
    int stride, off, ns;
};
__device__ __forceinline__ SamplePlan sample_plan(int b, int ctx, int topk) {
    const int np = (ctx + kPage - 1) / kPage;
    SamplePlan p;
    p.stride = (np + kMaxSamplePages - 1) / kMaxSamplePages;
    if (p.stride < kSampleStride) p.stride = kSampleStride;
    p.off = (int)(((uint64_t)((uint32_t)b * 0x9E3779B1u) * (uint32_t)p.stride) >> 32);
    p.ns = (ctx < 4 * topk || np < 2 * p.stride) ? 0 : (np - p.stride) / p.stride + 1;
    return p;
}

// Per-query operands of the scan, lane (n, g): A[hb][j] = the 8 bf16 query
// values of head 16hb + n, dims [32g + 8j, +8); c[hb][i] = w / sqrt(D) of
// head 16hb + 4g + i (the lane's accumulator rows).
template <int HB>
__device__ __forceinline__ void load_query(const DecodeArgs& a, int b, int n, int g, v8bf (&A)[HB][4],
                                           float (&c)[HB][4]) {
    constexpr int H = HB * 16;
    const uint16_t* qb = a.q + (size_t)b * H * kD;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            A[hb][j] = *reinterpret_cast<const v8bf*>(qb + (16 * hb + n) * kD + 32 * g + 8 * j);
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
        for (int i = 0; i < 4; ++i) c[hb][i] = a.w[(size_t)b * H + 16 * hb + 4 * g + i] * a.inv_sqrt_d;
}

// Keys of one page into registers: dst[st][0..1] = the lane's 32 bytes of
// row 16*st + n; ksc = the scale of the lane's key (row lane).
__device__ __forceinline__ void load_page(const DecodeArgs& a, int page, uint32_t lane_off, int lane,
                                          v4i (&dst)[4][2], float& ksc) {
    const uint8_t* pbase = a.k_cache + (size_t)page * kPage * kD;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
        const uint8_t* rp = pbase + lane_off + st * 16 * kD;
        dst[st][0] = stream_load(reinterpret_cast<const v4i*>(rp));
        dst[st][1] = stream_load(reinterpret_cast<const v4i*>(rp + 16));
    }
    ksc = stream_load(a.k_scale + (size_t)page * kPage + lane);
}

// Scores of one page: lane l gets the score of the page's key l.
template <int HB>
__device__ __forceinline__ float page_scores(const v8bf (&A)[HB][4], const float (&c)[HB][4],
                                             const v4i (&cur)[4][2], float ks) {
    float part[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
        v4f acc[HB];
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) acc[hb] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const v4i& h = cur[st][j >> 1];
            const v8bf B = widen8(h[(j & 1) * 2], h[(j & 1) * 2 + 1]);
#pragma unroll
            for (int hb = 0; hb < HB; ++hb)
                acc[hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[hb][j], B, acc[hb], 0, 0, 0);
        }
        float pp = 0.f;
#pragma unroll
        for (int hb = 0; hb < HB; ++hb)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) pp = fmaf(c[hb][ii], relu(acc[hb][ii]), pp);
        part[st] = pp;
    }
    return reduce_scatter4(part) * ks;
}

// Prologue (only for batches too large for the scan's LDS prefix): per-query
// page counts -> exclusive prefix over queries, one workgroup.
__global__ void __launch_bounds__(1024)
decode_prologue_kernel(DecodeArgs a) {
    __shared__ uint32_t wtot[16];
    __shared__ uint32_t carry;
    const int t = threadIdx.x;
    if (t == 0) carry = 0;
    __syncthreads();
    for (int b0 = 0; b0 < a.B; b0 += 1024) {
        const int b = b0 + t;
        uint32_t np = 0;
        if (b < a.B) np = (uint32_t)((clamp_ctx(a.context_lens[b], a.max_ctx) + kPage - 1) / kPage);
        const uint32_t ip = wave_incl_scan(np);
        if (lane_id() == kWave - 1) wtot[t / kWave] = ip;
        __syncthreads();
        uint32_t rp = carry + ip - np;
        for (int w = 0; w < t / kWave; ++w) rp += wtot[w];
        if (b < a.B) a.prefix[b] = (int32_t)rp;
        __syncthreads();
        if (t == 1023) carry = rp + np;
        __syncthreads();
    }
    if (t == 0) a.prefix[a.B] = (int32_t)carry;
}

constexpr int kSfThreads = 512;  // sample-and-floor workgroup

// Bin of the 2048-bin LDS histogram h (NT threads) where the count from the
// top reaches r; also the count in the bins above it.  With r == 0 it
// returns the total count in *above and bin -1.
template <int NT>
__device__ __forceinline__ int bin_from_top(const uint32_t* h, uint32_t r, uint32_t* above, uint32_t* red) {
    const int t = threadIdx.x;
    constexpr int kSfWaves = NT / kWave;
    constexpr int kPer = kHistBins / NT;
    const uint32_t* hl = h + kHistBins - kPer * (t + 1);  // thread t: bins from the top, ascending
    uint32_t loc = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) loc += hl[i];
    const uint32_t incl = wave_incl_scan(loc);
    if (lane_id() == kWave - 1) red[t / kWave] = incl;
    __syncthreads();
    uint32_t run = incl - loc, total = 0;
#pragma unroll
    for (int w = 0; w < kSfWaves; ++w) {
        const uint32_t v = red[w];
        total += v;
        if (w < t / kWave) run += v;
    }
    if (r == 0) {
        __syncthreads();
        *above = total;
        return -1;
    }
    if (t == 0) red[kSfWaves] = 0xFFFFFFFFu;
    __syncthreads();
#pragma unroll
    for (int i = kPer - 1; i >= 0; --i) {
        const uint32_t cnt = hl[i];
        if (run < r && r <= run + cnt) {
            red[kSfWaves] = (uint32_t)(kHistBins - kPer * (t + 1) + i);
            red[kSfWaves + 1] = run;
        }
        run += cnt;
    }
    __syncthreads();
    const int bin = (int)red[kSfWaves];
    *above = red[kSfWaves + 1];
    __syncthreads();
    return bin;
}

// Sample and floor of query b, by the calling workgroup of NT threads.
// 1. The query is staged in LDS; wave w scores the sampled pages w, w + NW,
//    ... (two pages of loads in flight, page ids preloaded one per lane) and
//    keeps their score keys in LDS.
// 2. The floor: the r-th largest valid sampled key cut to its top 22 bits
//    (first digit by histogram, then the next 11 bits inside that bin), with
//    r five standard deviations above the expected number of sampled scores
//    at or above the query's k-th largest.
// Returns the floor key: 0 when the query is not sampled or r exceeds its
// sample (every score is then a candidate); otherwise its low 10 bits are 0.
// LDS: skey [kMaxSamplePages * kPage], h [kHistBins], qsh [64 * kD] bf16,
// csh [64], red [NT / kWave + 2].
template <int HB, int NT>
__device__ __forceinline__ uint32_t sample_floor(const DecodeArgs& a, const int b, uint32_t* skey, uint32_t* h,
                                                 uint16_t* qsh, float* csh, uint32_t* red) {
    constexpr int NW = NT / kWave;
    const int t = threadIdx.x;
    const int lane = lane_id(), wave = t / kWave;
    const int ctx = clamp_ctx(a.context_lens[b], a.max_ctx);
    // The query goes to LDS once per workgroup, with coalesced 16-byte
    // loads issued before anything that depends on the context.  Row r's
    // 16-byte pieces are stored XOR-swizzled by r & 15, so the operand reads
    // below (16 rows, one piece column) touch distinct banks.
    constexpr int H = 16 * HB;
    constexpr int kQPieces = H * kD * 2 / 16;
    constexpr int kQPer = (kQPieces + NT - 1) / NT;
    v4i qv[kQPer];
#pragma unroll
    for (int i = 0; i < kQPer; ++i)
        if (t + i * NT < kQPieces)
            qv[i] = reinterpret_cast<const v4i*>(a.q + (size_t)b * H * kD)[t + i * NT];
    const float wv = t < H ? a.w[(size_t)b * H + t] * a.inv_sqrt_d : 0.f;
    const SamplePlan sp = sample_plan(b, ctx, a.topk);
    if (sp.ns == 0) return 0u;
    // wave w scores the sampled pages w + NW j, j < npw; their page ids sit
    // one per lane (lane j), so no page load waits on a table read
    constexpr int kPerWave = (kMaxSamplePages + NW - 1) / NW;
    static_assert(kPerWave <= kWave, "page ids must fit one per lane");
    const int npw = wave < sp.ns ? (sp.ns - wave + NW - 1) / NW : 0;
    const int mine = wave + NW * lane;
    const int pid = (lane < kPerWave && mine < sp.ns)
                        ? a.block_table[(size_t)b * a.max_pages + sp.off + (size_t)sp.stride * mine] : 0;
    const int n = lane & 15, g = lane >> 4;
    const uint32_t lane_off = (uint32_t)(n * kD + 32 * g);
    v4i p0[4][2], p1[4][2];
    float k0 = 0.f, k1 = 0.f;
    auto page_at = [&](int j) { return __builtin_amdgcn_readlane(pid, j < npw - 1 ? j : npw - 1); };
    if (npw > 0) {  // the first two pages' loads go out before the barrier
        load_page(a, page_at(0), lane_off, lane, p0, k0);
        load_page(a, page_at(1), lane_off, lane, p1, k1);
    }
#pragma unroll
    for (int i = 0; i < kQPer; ++i) {
        const int pc = t + i * NT;
        if (pc < kQPieces) reinterpret_cast<v4i*>(qsh)[(pc & ~15) | ((pc ^ (pc >> 4)) & 15)] = qv[i];
    }
    if (t < H) csh[t] = wv;
    // LDS-only fences: the barrier does not wait for the page loads in flight
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    if (npw > 0) {
        v8bf A[HB][4];
        float c[HB][4];
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
            const int r = 16 * hb + n;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                A[hb][j] = reinterpret_cast<const v8bf*>(qsh)[r * 16 + ((4 * g + j) ^ (r & 15))];
#pragma unroll
            for (int i = 0; i < 4; ++i) c[hb][i] = csh[16 * hb + 4 * g + i];
        }
        for (int j = 0;; j += 2) {
            skey[(wave + NW * j) * kPage + lane] = score_key(page_scores<HB>(A, c, p0, k0));
            if (j + 1 >= npw) break;
            load_page(a, page_at(j + 2), lane_off, lane, p0, k0);  // (again the last page past the end)
            skey[(wave + NW * (j + 1)) * kPage + lane] = score_key(page_scores<HB>(A, c, p1, k1));
            if (j + 2 >= npw) break;
            load_page(a, page_at(j + 3), lane_off, lane, p1, k1);
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the unused prefetches settle
    }
    const int n_all = sp.ns * kPage;
    // sampled entry e is position (off + stride * (e / 64)) * 64 + e % 64;
    // only the last sampled page can reach past the context
    auto valid = [&](int e) { return (sp.off + sp.stride * (e / kPage)) * kPage + e % kPage < ctx; };
    // pass over the sample: histogram of digit (key >> shift) & 2047 of the
    // keys whose top bits (key >> 21) equal `sel` (all keys when sel < 0)
    auto pass = [&](int shift, int sel) {
        for (int i = t; i < kHistBins; i += NT) h[i] = 0u;
        __syncthreads();  // (the first time: also every sampled key is in LDS)
        for (int e = t; e < n_all; e += NT) {
            const uint32_t kk = skey[e];
            if (valid(e) && (sel < 0 || (int)(kk >> 21) == sel)) atomicAdd(&h[(kk >> shift) & (kHistBins - 1)], 1u);
        }
        __syncthreads();
    };
    pass(21, -1);
    uint32_t m = 0;
    bin_from_top<NT>(h, 0, &m, red);
    const float ex = (float)m * (float)a.topk / (float)ctx;
    const uint32_t r = (uint32_t)ceilf(ex + 5.f * sqrtf(ex) + 8.f);
    uint32_t fl = 0u;
    if (r < m) {
        uint32_t above1 = 0;
        const int bin1 = bin_from_top<NT>(h, r, &above1, red);
        pass(10, bin1);
        uint32_t above2 = 0;
        const int bin2 = bin_from_top<NT>(h, r - above1, &above2, red);
        fl = ((uint32_t)bin1 << 21) | ((uint32_t)bin2 << 10);
    }
    return fl;
}

// Sample and floor of query b, one workgroup of kSfThreads per query (the
// three-kernel form of the step, for batches too large for the fused scan).
// Writes the floor (word 2 of the query's counter block) and clears the
// candidate count (word 1) and the unfiltered-flush flag (word 3) -- for
// every query.
template <int HB>
__global__ void __launch_bounds__(kSfThreads)
decode_sample_floor_kernel(DecodeArgs a) {
    __shared__ uint32_t skey[kMaxSamplePages * kPage];
    __shared__ uint32_t h[kHistBins];
    __shared__ __align__(16) uint16_t qsh[64 * kD];
    __shared__ float csh[64];
    __shared__ uint32_t red[kSfThreads / kWave + 2];
    const int b = blockIdx.x;
    const uint32_t fl = sample_floor<HB, kSfThreads>(a, b, skey, h, qsh, csh, red);
    if (threadIdx.x == 0) {
        uint32_t* ctrl = a.ctrl + (size_t)b * kCtrlStride;
        ctrl[1] = 0u;
        ctrl[2] = fl;
        ctrl[3] = 0u;
    }
}

// Fused scan: the query whose floor workgroup j samples (query b goes to
// workgroup floor(b G / B), so the samplers spread evenly over the grid), or
// -1.  Needs 2 B <= G.
__device__ __forceinline__ int sampled_by(int j, int G, int B) {
    const int b = (int)(((int64_t)j * B + G - 1) / G);
    return (b < B && (int)((int64_t)b * G / B) == j) ? b : -1;
}

// Fused scan: a sampling workgroup's share is smaller by kProducerPages, as a
// fraction of the mean share P / G in 1/1024 (at most 0.88).
__device__ __forceinline__ int64_t dq_share(int P, int64_t G) {
    const int64_t dq = P > 0 ? (int64_t)kProducerPages * 1024 * G / P : 0;
    return dq > 900 ? 900 : dq;
}

// The main scan.  A persistent grid (one resident round of workgroups): the
// global list of (query, page) pairs, query-major, is cut into equal
// contiguous shares, one per workgroup, so ragged context lengths leave no
// tail of idle CUs.  Inside a share the 4 waves take interleaved pages (wave
// w: pages w, w+4, ...).  Each wave keeps two pages of loads in flight while
// it multiplies the current one; the (query, position, page id) of its next
// 64 pages sit one per lane, so no load waits on a block-table read.  Query
// operands are reloaded only when a wave's pages cross into the next query.
// Scores whose key reaches the query's floor go to the wave's LDS candidate
// buffer, flushed to the query's candidate list.  The page prefix over
// queries is built in LDS from the context lengths (or read from the
// prologue's output for very large batches).
//
// FUSED: the sampling runs inside this grid instead of a kernel before it.
// Workgroup floor(b G / B) first samples query b and publishes its floor in
// word 2 of the query's counter block with an agent-scope atomic store (floor | 1: the
// floor's low 10 bits are zero, bit 0 marks it published; the words were
// cleared before the launch).  Its share of pages is smaller by about the
// time that takes (kProducerPages).  A wave entering a query reads that word
// with an agent-scope atomic load and, until it finds the floor published,
// keeps every valid score in its buffer, polling once per page; once the
// floor is there it filters the buffer in place and goes on as usual.  A
// buffer that must be flushed (full, or the wave leaves the query) before
// the floor is known is flushed unfiltered and the query is marked (word 3),
// so the final kernel's verification counts only the candidates at or above
// the floor.  Nothing ever waits on another workgroup.
template <int HB, bool FUSED>
__global__ void __launch_bounds__(kThreadsDec)
decode_scan_kernel(DecodeArgs a) {
    __shared__ __align__(16) uint32_t lds_wave[kThreadsDec / kWave][2 * kCandBuf];  // candidate buffer
    __shared__ int32_t prefix_lds[kPrefixLds];
    __shared__ uint32_t wtot[kThreadsDec / kWave];
    constexpr int NW = kThreadsDec / kWave;
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    const int n = lane & 15, g = lane >> 4;
    float* cbuf_s = reinterpret_cast<float*>(lds_wave[wave]);
    int32_t* cbuf_p = reinterpret_cast<int32_t*>(lds_wave[wave] + kCandBuf);

    if constexpr (FUSED) {
        // The producer's sample borrows the candidate buffers' LDS: keys,
        // histogram and the staged query fill exactly its 32 KB.
        static_assert(kMaxSamplePages * kPage + kHistBins + 64 * kD / 2 <= NW * 2 * kCandBuf, "sample LDS");
        __shared__ float csh[64];
        __shared__ uint32_t red[NW + 2];
        const int qs = sampled_by(blockIdx.x, gridDim.x, a.B);
        if (qs >= 0) {
            uint32_t* base = &lds_wave[0][0];
            const uint32_t fl = sample_floor<HB, kThreadsDec>(a, qs, base, base + kMaxSamplePages * kPage,
                                                              reinterpret_cast<uint16_t*>(base + kMaxSamplePages * kPage + kHistBins),
                                                              csh, red);
            if (threadIdx.x == 0)
                __hip_atomic_store(a.ctrl + (size_t)qs * kCtrlStride + 2, fl | 1u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            __syncthreads();  // the LDS goes back to the candidate buffers
        }
    }

    const bool pre_in_lds = a.B + 1 <= kPrefixLds;
    if (pre_in_lds) {
        // exclusive prefix of the per-query page counts, 256 queries a round
        int carry = 0;
        for (int b0 = 0; b0 <= a.B; b0 += kThreadsDec) {
            const int b = b0 + (int)threadIdx.x;
            const uint32_t np = b < a.B ? (uint32_t)((clamp_ctx(a.context_lens[b], a.max_ctx) + kPage - 1) / kPage)
                                        : 0u;
            const uint32_t ip = wave_incl_scan(np);
            if (lane == kWave - 1) wtot[wave] = ip;
            __syncthreads();
            uint32_t rp = (uint32_t)carry + ip - np, tot = 0;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                if (w < wave) rp += wtot[w];
                tot += wtot[w];
            }
            if (b <= a.B) prefix_lds[b] = (int32_t)rp;
            carry += (int)tot;
            __syncthreads();
        }
    }
    auto prefix_at = [&](int i) -> int { return pre_in_lds ? prefix_lds[i] : a.prefix[i]; };
    const int P = prefix_at(a.B);
    const int64_t G = gridDim.x;
    int share_begin, share_end;
    if constexpr (FUSED) {
        // The sampling workgroups (every G/B-th) get weight 1 - d, d =
        // kProducerPages over the mean share (in 1/1024, at most 0.88), the
        // others 1 + d B / (G - B), so the weights of each run of G/B
        // workgroups still sum to G/B and the shares around them keep their
        // usual edges (with whole runs per query, the query boundaries).
        auto edge = [&](int64_t j) -> int {  // start of workgroup j's share
            const int64_t c = (j * a.B + G - 1) / G;  // sampling workgroups below j
            const int64_t num = j * 1024 * (G - a.B) - dq_share(P, G) * (c * (G - a.B) - (j - c) * a.B);
            return (int)((int64_t)P * num / (G * 1024 * (G - a.B)));
        };
        share_begin = edge(blockIdx.x);
        share_end = blockIdx.x + 1 == G ? P : edge(blockIdx.x + 1);
    } else {
        share_begin = (int)((int64_t)blockIdx.x * P / G);
        share_end = (int)((int64_t)(blockIdx.x + 1) * P / G);
    }
    // this wave's pages: share_begin + wave + NW*k for k < nk
    const int nk = share_end - share_begin - wave > 0 ? (share_end - share_begin - wave + NW - 1) / NW : 0;
    if (nk == 0) return;

    // Query of the share's first page (the last b with prefix[b] <= page).
    int lo = 0, hi = a.B;
    {
        const int p0 = share_begin + wave;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (prefix_at(mid) <= p0) lo = mid; else hi = mid;
        }
    }
    // Per-lane description of pages k0 .. k0+63 of this wave.
    int walk_b = lo;  // query of page k0 (wave-uniform)
    auto describe = [&](int k0, int& qb, int& pos0, int& pid) {
        const int k = k0 + lane;
        const int gp = share_begin + wave + NW * k;
        qb = -1; pos0 = 0; pid = 0;
        if (k < nk) {
            int bb = walk_b;
            while (prefix_at(bb + 1) <= gp) ++bb;
            const int j = gp - prefix_at(bb);
            qb = bb;
            pos0 = j * kPage;
            pid = a.block_table[(size_t)bb * a.max_pages + j];
        }
        const int last = min(63, nk - 1 - k0);
        if (last >= 0) walk_b = __builtin_amdgcn_readlane(qb, last);
        // Settle the table loads here (once per 64 pages): left pending, they
        // would make every later step wait for its own prefetches too.
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    };

    const uint32_t lane_off = (uint32_t)(n * kD + 32 * g);
    v8bf A[HB][4];
    float c[HB][4];
    int qcur = -1, ctx_cur = 0;
    uint32_t floor_key = 0u;  // candidates have key >= floor_key
    int nbuf = 0;             // entries in the wave's candidate buffer
    uint32_t* cand_n = a.ctrl + 1;  // word 1 of each query's counter block
    // FUSED: whether the current query's floor is known
    bool fready = !FUSED;
    auto floor_word = [&](int qb) -> uint32_t {
        return __hip_atomic_load(a.ctrl + (size_t)qb * kCtrlStride + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    // keep the buffer's entries whose key reaches fk, in place and in order
    auto compact = [&](uint32_t fk) {
        int o = 0;
        for (int j0 = 0; j0 < nbuf; j0 += kWave) {
            const int j = j0 + lane;
            float sc = 0.f;
            int32_t ps = 0;
            bool keep = false;
            if (j < nbuf) {
                sc = cbuf_s[j];
                ps = cbuf_p[j];
                keep = score_key(sc) >= fk;
            }
            const uint64_t m = wave_ballot(keep);
            if (keep) {
                const int d = o + lanes_below(m);  // d <= j: every entry of this step was read above
                cbuf_s[d] = sc;
                cbuf_p[d] = ps;
            }
            o += __builtin_popcountll(m);
        }
        __builtin_amdgcn_wave_barrier();
        nbuf = o;
    };
    // a flush before the floor is known writes every valid score: mark the query
    auto mark_unfiltered = [&](int qb) {
        if (FUSED && !fready && nbuf > 0 && lane == 0) a.ctrl[(size_t)qb * kCtrlStride + 3] = 1u;
    };
    auto flush_cand = [&](int qb) {
        if (nbuf == 0) return;
        uint32_t base = 0;
        if (lane == 0) base = atomicAdd(&cand_n[(size_t)qb * kCtrlStride], (uint32_t)nbuf);
        base = (uint32_t)__builtin_amdgcn_readfirstlane((int)base);
        float* cs = a.cand_score + (size_t)qb * a.cand_stride + base;
        int32_t* cp = a.cand_pos + (size_t)qb * a.cand_stride + base;
        for (int j = lane; j < nbuf; j += kWave) {
            cs[j] = cbuf_s[j];
            cp[j] = cbuf_p[j];
        }
        __builtin_amdgcn_wave_barrier();
        nbuf = 0;
    };

    int cq, cpos, cpid;   // lanes: pages k0 .. k0+63
    int nq, npos, npid;   // lanes: pages k0+64 .. k0+127
    describe(0, cq, cpos, cpid);
    describe(64, nq, npos, npid);

    // One pipeline step: prefetch page k+2 into `pre`, multiply page k held
    // in `cur` (page k+1 is in flight meanwhile).  Called with three buffers
    // rotating, so no copies.
    auto step = [&](int k, v4i (&cur)[4][2], float ks_c, v4i (&pre)[4][2], float& ks_p) {
        const int i = k & 63;
        const int pb = __builtin_amdgcn_readlane(cq, i);
        const int ppos = __builtin_amdgcn_readlane(cpos, i);
        // FUSED, floor not yet known: poll it now, read the answer after this
        // page's scores (issued ahead of the next prefetch, so that wait covers
        // one page fewer in flight, only on these few steps)
        uint32_t fpoll = 0u;
        if (FUSED && !fready && pb == qcur) fpoll = floor_word(qcur);
        {
            // Unconditional, so every path issues the same loads and the wait
            // for `cur` can leave two pages in flight; past the end of the
            // share the current page is fetched again (unused).
            const int pid_n = i < 62 ? __builtin_amdgcn_readlane(cpid, i + 2) : __builtin_amdgcn_readlane(npid, i - 62);
            const int pid = k + 2 < nk ? pid_n : __builtin_amdgcn_readlane(cpid, i);
            load_page(a, pid, lane_off, lane, pre, ks_p);
        }
        if (i == 63) {  // roll the page descriptions forward
            cq = nq; cpos = npos; cpid = npid;
            describe(k + 65, nq, npos, npid);
        }
        if (pb != qcur) {  // entering a new query
            if (qcur >= 0) {
                mark_unfiltered(qcur);
                flush_cand(qcur);
            }
            qcur = pb;
            ctx_cur = clamp_ctx(a.context_lens[pb], a.max_ctx);
            load_query<HB>(a, pb, n, g, A, c);
            const uint32_t fw = FUSED ? floor_word(pb) : a.ctrl[(size_t)pb * kCtrlStride + 2];
            // Settle the query loads here, on this rare path: otherwise the
            // common path after it inherits their pending count and waits
            // for every page load in flight at each step.
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
            if constexpr (FUSED) {
                fready = (fw & 1u) != 0u;
                floor_key = fready ? (fw & ~1u) : 0u;
            } else {
                floor_key = fw;
            }
        }
        const float score = page_scores<HB>(A, c, cur, ks_c);
        const int s = ppos + lane;
        const uint32_t key = score_key(score);
        if (FUSED && !fready && pb == qcur) {
            // the asm keeps the read of the polled word (and its wait) on this path
            asm volatile("" : "+v"(fpoll));
            if (fpoll & 1u) {  // the floor came out: filter what is buffered
                fready = true;
                floor_key = fpoll & ~1u;
                compact(floor_key);
            }
        }
        if (nbuf > kCandBuf - kWave) {
            mark_unfiltered(qcur);
            flush_cand(qcur);
        }
        const bool take = s < ctx_cur && key >= floor_key;
        const uint64_t m = wave_ballot(take);
        if (take) {
            const int o = nbuf + lanes_below(m);
            cbuf_s[o] = score;
            cbuf_p[o] = s;
        }
        nbuf += __builtin_popcountll(m);
    };

    v4i b0[4][2], b1[4][2], b2[4][2];
    float k0 = 0.f, k1 = 0.f, k2 = 0.f;
    load_page(a, __builtin_amdgcn_readlane(cpid, 0), lane_off, lane, b0, k0);
    load_page(a, __builtin_amdgcn_readlane(cpid, nk > 1 ? 1 : 0), lane_off, lane, b1, k1);
    for (int k = 0; k < nk; k += 3) {
        step(k, b0, k0, b2, k2);
        if (k + 1 < nk) step(k + 1, b1, k1, b0, k0);
        if (k + 2 < nk) step(k + 2, b2, k2, b1, k1);
    }
    if (qcur >= 0) {
        mark_unfiltered(qcur);
        flush_cand(qcur);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // the final page prefetches (unused) settle before exit
}

// Final kernel, one workgroup per query: verification, repair, selection.
// A query whose candidate count fell short of min(k, context) -- its sample
// floor lay above its k-th largest score -- is first rescored in full, every
// position becoming a candidate (plain per-key dot products on the VALU:
// slow, and reached only by inputs whose sampled pages score unlike the rest
// of their context).  Then the exact selection over the candidates.
template <int HB>
__global__ void __launch_bounds__(sel::kThreads)
decode_finish_kernel(DecodeArgs a, SelectArgs sa) {
    constexpr int H = HB * 16;
    extern __shared__ __align__(16) unsigned char smem_raw[];
    sel::SelShared& sh = *reinterpret_cast<sel::SelShared*>(smem_raw);
    const int b = blockIdx.x, t = threadIdx.x;
    // The first candidates are loaded before their count is known (inside the
    // row's stride), so both arrive in one round trip.
    sel::Preload pre;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int j = u * sel::kThreads + t;
        pre.v[u] = j < a.cand_stride ? a.cand_score[(size_t)b * a.cand_stride + j] : 0.f;
        pre.p[u] = j < a.cand_stride ? (uint32_t)a.cand_pos[(size_t)b * a.cand_stride + j] : 0u;
    }
    const int ctx = clamp_ctx(a.context_lens[b], a.max_ctx);
    uint32_t* cnt = a.ctrl + (size_t)b * kCtrlStride + 1;
    const uint32_t need = (uint32_t)min(a.topk, ctx);
    int n_known = (int)*cnt;
    bool rescore = (uint32_t)n_known < need;
    if (!rescore && a.ctrl[(size_t)b * kCtrlStride + 3] != 0u) {
        // Some candidates were flushed before the floor was known: only
        // those at or above the floor prove the selection exact.
        const uint32_t fk = a.ctrl[(size_t)b * kCtrlStride + 2] & ~1u;
        const float* cs = a.cand_score + (size_t)b * a.cand_stride;
        uint32_t c = 0;
        for (int j = t; j < n_known; j += sel::kThreads) c += score_key(cs[j]) >= fk ? 1u : 0u;
        if (t == 0) sh.above = 0u;
        __syncthreads();
        c = wave_sum(c);
        if (lane_id() == 0) atomicAdd(&sh.above, c);
        __syncthreads();
        rescore = sh.above < need;
        __syncthreads();
    }
    if (rescore) {
        // the query and its head coefficients, in the selector's LDS (free until it runs)
        float* qs = reinterpret_cast<float*>(sh.cand_key);  // [H][kD]
        float* cs = reinterpret_cast<float*>(sh.cand_pos);  // [H]
        static_assert(sizeof(sh.cand_key) >= sizeof(float) * H * kD, "query does not fit");
        for (int i = t; i < H * kD; i += sel::kThreads)
            qs[i] = __uint_as_float((uint32_t)a.q[(size_t)b * H * kD + i] << 16);
        for (int i = t; i < H; i += sel::kThreads) cs[i] = a.w[(size_t)b * H + i] * a.inv_sqrt_d;
        __syncthreads();
        float* out_s = a.cand_score + (size_t)b * a.cand_stride;
        int32_t* out_p = a.cand_pos + (size_t)b * a.cand_stride;
        for (int s = t; s < ctx; s += sel::kThreads) {
            const int page = a.block_table[(size_t)b * a.max_pages + s / kPage];
            const uint8_t* row = a.k_cache + ((size_t)page * kPage + (s % kPage)) * kD;
            uint32_t kw[kD / 4];  // the key row stays packed; each head widens it again
#pragma unroll
            for (int j = 0; j < kD / 16; ++j) {
                const uint4 v = reinterpret_cast<const uint4*>(row)[j];
                kw[4 * j] = v.x;
                kw[4 * j + 1] = v.y;
                kw[4 * j + 2] = v.z;
                kw[4 * j + 3] = v.w;
            }
            float acc = 0.f;
#pragma unroll 1
            for (int h = 0; h < H; ++h) {
                const float* qh = qs + h * kD;
                float dot = 0.f;
#pragma unroll 1
                for (int j0 = 0; j0 < kD / 4; j0 += 8)  // 32 dimensions per step, to bound the live LDS reads
#pragma unroll
                    for (int j = j0; j < j0 + 8; ++j) {
                        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)kw[j], false);
                        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)kw[j], true);
                        dot = fmaf(qh[4 * j], lo[0], dot);
                        dot = fmaf(qh[4 * j + 1], lo[1], dot);
                        dot = fmaf(qh[4 * j + 2], hi[0], dot);
                        dot = fmaf(qh[4 * j + 3], hi[1], dot);
                    }
                acc = fmaf(cs[h], fmaxf(dot, 0.f), acc);
            }
            out_s[s] = acc * a.k_scale[(size_t)page * kPage + (s % kPage)];
            out_p[s] = s;
        }
        __syncthreads();  // every rescored candidate is written, and the LDS is free again
        if (t == 0) *cnt = (uint32_t)ctx;
        n_known = ctx;
    }
    sel::select_row(sa, b, sh, n_known, pre, !rescore);  // a rescore rewrote the candidates
}

__global__ void zero_u32_kernel(uint32_t* p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}


template <int HB>
hipError_t launch_decode_hb(const DecodeArgs& a_in, const SelectArgs& s, int64_t max_pages, hipStream_t stream) {
    DecodeArgs a = a_in;
    // Main scan: one resident round of workgroups (occupancy queried once
    // per process; both forms of the scan have the same resources), never
    // more workgroups than pages.
    static PerDevice<int> resident_once;
    int resident = 0;
    hipError_t e = resident_once.get(
        [](int dev, int* v) {
            int per_cu = 0, per_cu_f = 0, cus = 0;
            hipError_t r = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
            if (r != hipSuccess) return r;
            r = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)decode_scan_kernel<HB, false>,
                                                             kThreadsDec, 0);
            if (r != hipSuccess) return r;
            r = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu_f, (const void*)decode_scan_kernel<HB, true>,
                                                             kThreadsDec, 0);
            if (r != hipSuccess) return r;
            if (per_cu_f < per_cu) per_cu = per_cu_f;
            *v = (per_cu < 1 ? 1 : per_cu) * cus;
            return hipSuccess;
        },
        &resident);
    if (e != hipSuccess) return e;
    int64_t grid = resident;
    if (grid > max_pages) grid = max_pages;
    if (grid < 1) grid = 1;
    // The sample runs inside the scan when at most half the grid samples
    // (workgroup b < B samples query b) and the page prefix fits in LDS;
    // otherwise a kernel of its own goes first.
    const bool fused = (int64_t)a.B * 2 <= grid && a.B + 1 <= kPrefixLds;
    if (fused) {
        if ((e = launch_zero_u32(a.ctrl, (size_t)a.B * kCtrlStride, stream)) != hipSuccess) return e;
        hipLaunchKernelGGL((decode_scan_kernel<HB, true>), dim3((unsigned)grid), dim3(kThreadsDec), 0, stream, a);
    } else {
        hipLaunchKernelGGL(decode_sample_floor_kernel<HB>, dim3((unsigned)a.B), dim3(kSfThreads), 0, stream, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL((decode_scan_kernel<HB, false>), dim3((unsigned)grid), dim3(kThreadsDec), 0, stream, a);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    static PerDevice<int> lds_once;
    if ((e = set_lds_limit(lds_once, (const void*)decode_finish_kernel<HB>, (int)sizeof(sel::SelShared))) !=
        hipSuccess)
        return e;
    hipLaunchKernelGGL(decode_finish_kernel<HB>, dim3((unsigned)a.B), dim3(sel::kThreads), sizeof(sel::SelShared),
                       stream, a, s);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_zero_u32(uint32_t* p, size_t n, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    size_t blocks = (n + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    hipLaunchKernelGGL(zero_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n);
    return hipGetLastError();
}

hipError_t launch_decode_scan(const DecodeArgs& a, const SelectArgs& s, int H, hipStream_t stream) {
    hipError_t e;
    if (a.B + 1 > kPrefixLds) {  // the scan's LDS prefix does not fit: build it in global memory
        hipLaunchKernelGGL(decode_prologue_kernel, dim3(1), dim3(1024), 0, stream, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const int hb = H / 16;
    if (hb < 1 || hb > 4) return hipErrorInvalidValue;
    const int64_t max_pages = (int64_t)a.B * ((a.max_ctx + kPage - 1) / kPage);
    switch (hb) {
        case 1: e = launch_decode_hb<1>(a, s, max_pages, stream); break;
        case 2: e = launch_decode_hb<2>(a, s, max_pages, stream); break;
        case 3: e = launch_decode_hb<3>(a, s, max_pages, stream); break;
        default: e = launch_decode_hb<4>(a, s, max_pages, stream); break;
    }
    return e;
}

}  // namespace dsaidx
