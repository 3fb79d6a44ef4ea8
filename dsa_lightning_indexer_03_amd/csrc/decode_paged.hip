// Decode-step scan of a paged FP8 indexer key cache.
//
// One query per decode step scores every position of its cached context
// (the decode walkthrough of "Lightning Indexer explained", section 2: one
// dot of the current query against the whole indexer cache).  The scan is
// bound by the cache bytes it streams (128 fp8 bytes + a 4-byte scale per
// position), so the kernel is laid out for HBM:
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
// * Scores go to a [B][stride] fp32 workspace (4 bytes written per 132
//   bytes read) and into a per-workgroup LDS histogram of the first radix
//   digit, flushed to a per-query global histogram that the selector uses
//   to skip its first pass.
#include "common.h"
#include "kernels.h"

namespace dsaidx {

namespace {

constexpr int kD = 128;
constexpr int kPage = 64;
constexpr int kThreadsDec = 256;

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

// Prologue: per-query page counts -> exclusive prefix over queries (the
// global page list the scan walks; workgroup 0), and clears the histograms
// and per-query counters (all workgroups, 16-byte stores).
__global__ void __launch_bounds__(1024)
decode_prologue_kernel(DecodeArgs a) {
    __shared__ uint32_t wtot[16];
    __shared__ uint32_t carry;
    const int t = threadIdx.x;
    const size_t nz4 = (size_t)a.B * (kHistBins + kCtrlStride) / 4;
    v4i* z = reinterpret_cast<v4i*>(a.hist);
    for (size_t i = (size_t)blockIdx.x * 1024 + t; i < nz4; i += (size_t)gridDim.x * 1024) z[i] = v4i{0, 0, 0, 0};
    if (blockIdx.x != 0) return;
    if (t == 0) carry = 0;
    __syncthreads();
    for (int b0 = 0; b0 < a.B; b0 += 1024) {
        const int b = b0 + t;
        uint32_t np = 0;
        if (b < a.B) {
            int ctx = a.context_lens[b];
            ctx = ctx < 0 ? 0 : (ctx > a.max_ctx ? a.max_ctx : ctx);
            np = (uint32_t)((ctx + kPage - 1) / kPage);
        }
        const uint32_t incl = wave_incl_scan(np);
        if (lane_id() == kWave - 1) wtot[t / kWave] = incl;
        __syncthreads();
        uint32_t run = carry + incl - np;
        for (int w = 0; w < t / kWave; ++w) run += wtot[w];
        if (b < a.B) a.prefix[b] = (int32_t)run;
        __syncthreads();
        if (t == 1023) carry = run + np;
        __syncthreads();
    }
    if (t == 0) a.prefix[a.B] = (int32_t)carry;
}

// The scan.  A persistent grid (one resident round of workgroups): the
// global list of (query, page) pairs, query-major, is cut into equal
// contiguous shares, one per workgroup, so ragged context lengths leave no
// tail of idle CUs.  Inside a share the 4 waves take interleaved pages
// (wave w: pages w, w+4, ...), so a workgroup streams 32 KB of adjacent
// cache per step.  Each wave keeps the next page's loads in flight while it
// multiplies the current one; the (query, position, page id) of its next 64
// pages sit one per lane, so no load waits on a block-table read.  Query
// operands are reloaded only when a wave's pages cross into the next query;
// each wave keeps its own LDS histogram of the first radix digit, flushed to
// the query's global histogram on every query change and at the end.
template <int HB>
__global__ void __launch_bounds__(kThreadsDec)
decode_scan_kernel(DecodeArgs a) {
    __shared__ uint32_t hist_all[kThreadsDec / kWave][kHistBins];
    constexpr int NW = kThreadsDec / kWave;
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    const int n = lane & 15, g = lane >> 4;
    constexpr int H = HB * 16;
    uint32_t* hist = hist_all[wave];
#pragma unroll
    for (int i = 0; i < kHistBins / kWave; ++i) hist[lane + kWave * i] = 0u;

    const int32_t* prefix = a.prefix;
    const int P = prefix[a.B];
    const int64_t G = gridDim.x;
    const int share_begin = (int)((int64_t)blockIdx.x * P / G);
    const int share_end = (int)((int64_t)(blockIdx.x + 1) * P / G);
    // this wave's pages: share_begin + wave + NW*k for k < nk
    const int nk = share_end - share_begin - wave > 0 ? (share_end - share_begin - wave + NW - 1) / NW : 0;
    if (nk == 0) return;

    // Query of the share's first page (the last b with prefix[b] <= page).
    int lo = 0, hi = a.B;
    {
        const int p0 = share_begin + wave;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (prefix[mid] <= p0) lo = mid; else hi = mid;
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
            while (prefix[bb + 1] <= gp) ++bb;
            const int j = gp - prefix[bb];
            qb = bb;
            pos0 = j * kPage;
            pid = a.block_table[(size_t)bb * a.max_pages + j];
        }
        const int last = min(63, nk - 1 - k0);
        if (last >= 0) walk_b = __builtin_amdgcn_readlane(qb, last);
    };

    const uint32_t lane_off = (uint32_t)(n * kD + 32 * g);
    auto load_page = [&](int page, v4i (&dst)[4][2], float& ksc) {
        const uint8_t* pbase = a.k_cache + (size_t)page * kPage * kD;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const uint8_t* rp = pbase + lane_off + st * 16 * kD;
            dst[st][0] = stream_load(reinterpret_cast<const v4i*>(rp));
            dst[st][1] = stream_load(reinterpret_cast<const v4i*>(rp + 16));
        }
        ksc = stream_load(a.k_scale + (size_t)page * kPage + lane);
    };

    v8bf A[HB][4];
    float c[HB][4];
    int qcur = -1, ctx_cur = 0;
    float* out = nullptr;
    auto flush = [&](int qb) {
        uint32_t* gh = a.hist + (size_t)qb * kHistBins;
#pragma unroll 4
        for (int i = 0; i < kHistBins / kWave; ++i) {
            const uint32_t v = hist[lane + kWave * i];
            if (v) {
                atomicAdd(&gh[lane + kWave * i], v);
                hist[lane + kWave * i] = 0u;
            }
        }
    };

    int cq, cpos, cpid;   // lanes: pages k0 .. k0+63
    int nq, npos, npid;   // lanes: pages k0+64 .. k0+127
    describe(0, cq, cpos, cpid);
    describe(64, nq, npos, npid);

    // One pipeline step: prefetch page k+1 into `nxt`, multiply page k held
    // in `cur`.  Called with the two buffers alternating, so no copies.
    auto step = [&](int k, v4i (&cur)[4][2], float ks_c, v4i (&nxt)[4][2], float& ks_n) {
        const int i = k & 63;
        const int pb = __builtin_amdgcn_readlane(cq, i);
        const int ppos = __builtin_amdgcn_readlane(cpos, i);
        if (k + 1 < nk) {
            const int pid = i < 63 ? __builtin_amdgcn_readlane(cpid, i + 1) : __builtin_amdgcn_readlane(npid, 0);
            load_page(pid, nxt, ks_n);
        }
        if (i == 63) {  // roll the page descriptions forward
            cq = nq; cpos = npos; cpid = npid;
            describe(k + 65, nq, npos, npid);
        }
        if (pb != qcur) {  // entering a new query
            if (qcur >= 0) flush(qcur);
            qcur = pb;
            int ctx = a.context_lens[pb];
            ctx_cur = ctx < 0 ? 0 : (ctx > a.max_ctx ? a.max_ctx : ctx);
            out = a.scores + (size_t)pb * a.score_stride;
            const uint16_t* qb = a.q + (size_t)pb * H * kD;
#pragma unroll
            for (int hb = 0; hb < HB; ++hb)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    A[hb][j] = *reinterpret_cast<const v8bf*>(qb + (16 * hb + n) * kD + 32 * g + 8 * j);
#pragma unroll
            for (int hb = 0; hb < HB; ++hb)
#pragma unroll
                for (int ii = 0; ii < 4; ++ii)
                    c[hb][ii] = a.w[(size_t)pb * H + 16 * hb + 4 * g + ii] * a.inv_sqrt_d;
        }
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
        const float score = reduce_scatter4(part) * ks_c;
        const int s = ppos + lane;
        if (s < ctx_cur) {
            out[s] = score;
            atomicAdd(&hist[score_key(score) >> 21], 1u);
        }
    };

    v4i bx[4][2], by[4][2];
    float kx = 0.f, ky = 0.f;
    load_page(__builtin_amdgcn_readlane(cpid, 0), bx, kx);
    for (int k = 0; k < nk; k += 2) {
        step(k, bx, kx, by, ky);
        if (k + 1 < nk) step(k + 1, by, ky, bx, kx);
    }
    if (qcur >= 0) flush(qcur);
}

// Selection, pass 1 of 2: with the first-digit histogram of the whole row
// known, the digit b1 of the k-th largest score follows; every score whose
// digit is above b1 is selected outright (written to the output), the ones
// in bin b1 go to a per-query candidate list for the exact finish.  Many
// workgroups per query, so the row is read at full chip bandwidth.
__global__ void __launch_bounds__(256)
decode_filter_kernel(DecodeFilterArgs a) {
    constexpr int kPer = kFilterChunk / 256;  // entries per thread
    __shared__ uint32_t wtot[4];
    __shared__ int s_bin;
    __shared__ uint32_t s_base_above, s_base_tie;
    const int b = blockIdx.y;
    int ctx = a.context_lens[b];
    ctx = ctx < 0 ? 0 : (ctx > a.max_ctx ? a.max_ctx : ctx);
    const int j0 = blockIdx.x * kFilterChunk;
    if (j0 >= ctx) return;
    const int K = a.topk;
    const int t = threadIdx.x;
    const int w = t / kWave;

    // Block-wide exclusive prefix sum (4 waves) of one value per thread.
    auto block_scan = [&](uint32_t v, uint32_t* total) -> uint32_t {
        const uint32_t incl = wave_incl_scan(v);
        __syncthreads();
        if (lane_id() == kWave - 1) wtot[w] = incl;
        __syncthreads();
        uint32_t run = incl - v;
        for (int i = 0; i < w; ++i) run += wtot[i];
        *total = wtot[0] + wtot[1] + wtot[2] + wtot[3];
        return run;
    };

    int b1 = -1;  // ctx <= K: every entry is selected
    if (ctx > K) {
        const uint32_t* h = a.hist + (size_t)b * kHistBins;
        uint32_t c[8], loc = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) { c[i] = h[kHistBins - 1 - 8 * t - i]; loc += c[i]; }
        uint32_t tot;
        uint32_t run = block_scan(loc, &tot);
        const uint32_t need = (uint32_t)K;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (run < need && need <= run + c[i]) s_bin = kHistBins - 1 - 8 * t - i;
            run += c[i];
        }
        __syncthreads();
        b1 = s_bin;
    }
    if (blockIdx.x == 0 && t == 0) a.pre_count[(size_t)b * kCtrlStride + 2] = (uint32_t)b1;
    const float* sc = a.scores + (size_t)b * a.stride;
    const int j1 = min(ctx, j0 + kFilterChunk);
    // Entry j0 + i*256 + t: thread t, step i.  Output positions are handed
    // out per (step, wave) in step-major order, so each wave's stores of one
    // step go to consecutive slots.
    __shared__ uint32_t cnt[kPer][4];
    float v[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int j = j0 + i * 256 + t;
        v[i] = j < j1 ? sc[j] : -INFINITY;
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int j = j0 + i * 256 + t;
        const int d = j < j1 ? (int)(score_key(v[i]) >> 21) : -2;
        const uint32_t na = (uint32_t)__builtin_popcountll(wave_ballot(d > b1));
        const uint32_t nt = (uint32_t)__builtin_popcountll(wave_ballot(d == b1));
        if (lane_id() == 0) cnt[i][w] = na | (nt << 16);
    }
    __syncthreads();
    if (w == 0) {  // exclusive prefix over the kPer*4 (step, wave) counts
        const int l = lane_id();
        const uint32_t c0 = cnt[(2 * l) / 4][(2 * l) % 4], c1 = cnt[(2 * l + 1) / 4][(2 * l + 1) % 4];
        const uint32_t incl = wave_incl_scan(c0 + c1);
        const uint32_t tot = __shfl(incl, kWave - 1, kWave);
        uint32_t ba = 0, bt = 0;
        if (l == 0) {
            ba = (tot & 0xFFFFu) ? atomicAdd(&a.pre_count[(size_t)b * kCtrlStride], tot & 0xFFFFu) : 0u;
            bt = (tot >> 16) ? atomicAdd(&a.cand_n[(size_t)b * kCtrlStride], tot >> 16) : 0u;
        }
        ba = __shfl(ba, 0, kWave);
        bt = __shfl(bt, 0, kWave);
        const uint32_t e0 = incl - c0 - c1, e1 = incl - c1;
        cnt[(2 * l) / 4][(2 * l) % 4] = e0;
        cnt[(2 * l + 1) / 4][(2 * l + 1) % 4] = e1;
        if (l == 0) { s_base_above = ba; s_base_tie = bt; }
    }
    __syncthreads();
    const uint32_t ba = s_base_above, bt = s_base_tie;
    int32_t* io = a.idx_out + (size_t)b * K;
    float* vo = a.val_out ? a.val_out + (size_t)b * K : nullptr;
    float* cs = a.cand_score + (size_t)b * a.stride;
    int32_t* cp = a.cand_pos + (size_t)b * a.stride;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int j = j0 + i * 256 + t;
        const int d = j < j1 ? (int)(score_key(v[i]) >> 21) : -2;
        const uint64_t ma = wave_ballot(d > b1), mt = wave_ballot(d == b1);
        const uint32_t off = cnt[i][w];
        if (d > b1) {
            const uint32_t o = ba + (off & 0xFFFFu) + (uint32_t)lanes_below(ma);
            if (o < (uint32_t)K) {
                io[o] = j;
                if (vo) vo[o] = v[i];
            }
        } else if (d == b1) {
            const uint32_t o = bt + (off >> 16) + (uint32_t)lanes_below(mt);
            if (o < (uint32_t)a.stride) {
                cs[o] = v[i];
                cp[o] = j;
            }
        }
    }
}

__global__ void zero_u32_kernel(uint32_t* p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

}  // namespace

hipError_t launch_zero_u32(uint32_t* p, size_t n, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    size_t blocks = (n + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    hipLaunchKernelGGL(zero_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n);
    return hipGetLastError();
}

hipError_t launch_decode_filter(const DecodeFilterArgs& a, hipStream_t stream) {
    const dim3 grid((unsigned)((a.max_ctx + kFilterChunk - 1) / kFilterChunk), (unsigned)a.B);
    hipLaunchKernelGGL(decode_filter_kernel, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_decode_scan(const DecodeArgs& a, int H, int max_ctx, hipStream_t stream) {
    (void)max_ctx;
    {
        const size_t nz4 = (size_t)a.B * (kHistBins + kCtrlStride) / 4;
        size_t blocks = (nz4 + 4095) / 4096;
        blocks = blocks < 1 ? 1 : (blocks > 256 ? 256 : blocks);
        hipLaunchKernelGGL(decode_prologue_kernel, dim3((unsigned)blocks), dim3(1024), 0, stream, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // One resident round of workgroups (occupancy queried once per process).
    static int resident[5] = {0, 0, 0, 0, 0};
    const int hb = H / 16;
    if (hb < 1 || hb > 4) return hipErrorInvalidValue;
    const void* fn = hb == 1 ? (const void*)decode_scan_kernel<1> : hb == 2 ? (const void*)decode_scan_kernel<2>
                   : hb == 3 ? (const void*)decode_scan_kernel<3> : (const void*)decode_scan_kernel<4>;
    if (resident[hb] == 0) {
        int dev = 0, per_cu = 0, cus = 0;
        if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
        if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
        if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kThreadsDec, 0)) != hipSuccess) return e;
        resident[hb] = (per_cu < 1 ? 1 : per_cu) * cus;
    }
    // Never more workgroups than pages; the kernel tolerates empty shares.
    const int64_t max_pages = (int64_t)a.B * ((a.max_ctx + kPage - 1) / kPage);
    int64_t grid = resident[hb];
    if (grid > max_pages) grid = max_pages;
    if (grid < 1) grid = 1;
    switch (hb) {
        case 1: hipLaunchKernelGGL(decode_scan_kernel<1>, dim3((unsigned)grid), dim3(kThreadsDec), 0, stream, a); break;
        case 2: hipLaunchKernelGGL(decode_scan_kernel<2>, dim3((unsigned)grid), dim3(kThreadsDec), 0, stream, a); break;
        case 3: hipLaunchKernelGGL(decode_scan_kernel<3>, dim3((unsigned)grid), dim3(kThreadsDec), 0, stream, a); break;
        default: hipLaunchKernelGGL(decode_scan_kernel<4>, dim3((unsigned)grid), dim3(kThreadsDec), 0, stream, a); break;
    }
    return hipGetLastError();
}

}  // namespace dsaidx
