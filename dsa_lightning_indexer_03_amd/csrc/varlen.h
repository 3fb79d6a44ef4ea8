// Row blocks of the fused prefill kernels: a workgroup owns kBlockRows
// consecutive query rows of one sequence.  Whole-sequence calls map
// blockIdx.x to (sequence, block), heaviest block first; variable-length
// chunk calls (B sequences' chunks packed one after another, sequence b's
// rows cu_q[b] .. cu_q[b+1]-1 at positions q_start[b], q_start[b]+1, ...,
// scored against the paged key cache) read the block from a plan built on
// the device, again heaviest first.
#pragma once

#include "common.h"
#include "kernels.h"

namespace dsaidx {
namespace {

constexpr int kBlockRows = 8;

// The rows a workgroup owns.
struct Seg {
    int b;     // sequence
    int blk;   // 8-row block within the sequence
    int row0;  // global row of the sequence's first query
    int Lq;    // query rows of the sequence
    int q0;    // position of its first query
    int Lk;    // keys it sees (its last query's position + 1)
};

template <bool VARLEN>
__device__ __forceinline__ bool block_seg(const PrefillArgs& a, Seg& s) {
    if constexpr (VARLEN) {
        const int2 e = a.plan[blockIdx.x];
        s.b = uniform(e.x);
        if (s.b < 0) return false;
        s.blk = uniform(e.y);
        s.row0 = uniform(a.cu_q[s.b]);
        s.Lq = uniform(a.cu_q[s.b + 1]) - s.row0;
        s.q0 = max(uniform(a.q_start[s.b]), 0);
        s.Lk = min(s.q0 + s.Lq, a.max_kv);
        return s.Lq > 0 && s.Lk > 0;
    } else {
        const int nblk = (a.L + kBlockRows - 1) / kBlockRows;
        s.b = (int)(blockIdx.x % (unsigned)a.B);
        s.blk = nblk - 1 - (int)(blockIdx.x / (unsigned)a.B);  // heaviest first
        s.row0 = s.b * a.L;
        s.Lq = a.L;
        s.q0 = 0;
        s.Lk = a.L;
        return true;
    }
}

// Storage slot (row of k / k_cache) of key r < Lk of sequence b.
template <bool VARLEN>
__device__ __forceinline__ size_t key_slot(const PrefillArgs& a, int b, int r) {
    if constexpr (VARLEN)
        return (size_t)a.block_table[(size_t)b * a.max_pages + (r >> 6)] * 64 + (r & 63);
    else
        return (size_t)b * a.L + r;
}

// Block plan of a variable-length call: every 8-row block (sequence b, block
// j) of every sequence, ordered by the number of key chunks it scans,
// largest first (a counting sort over the 2048 possible chunk counts), then
// (-1, 0) up to n_plan.  One workgroup.
__global__ void __launch_bounds__(1024)
varlen_plan_kernel(PrefillArgs a) {
    __shared__ uint32_t cnt[2048];
    __shared__ uint32_t wtot[16];
    __shared__ uint32_t total;
    const int t = threadIdx.x;
    for (int i = t; i < 2048; i += 1024) cnt[i] = 0u;
    __syncthreads();
    // bucket = the block's last chunk (its last row's position, clamped to the keys)
    auto for_each_block = [&](auto&& f) {
        for (int b = 0; b < a.B; ++b) {
            const int r0 = a.cu_q[b];
            const int Lq = a.cu_q[b + 1] - r0;
            if (Lq <= 0) continue;
            const int q0 = max(a.q_start[b], 0);
            const int Lk = min(q0 + Lq, a.max_kv);
            if (Lk <= 0) continue;
            const int nbk = (Lq + kBlockRows - 1) / kBlockRows;
            for (int j = t; j < nbk; j += 1024) {
                const int lr = min(kBlockRows * j + kBlockRows - 1, Lq - 1);
                const int w = min(min(q0 + lr, Lk - 1) >> 6, 2047);
                f(b, j, w);
            }
        }
    };
    for_each_block([&](int, int, int w) { atomicAdd(&cnt[w], 1u); });
    __syncthreads();
    // thread t owns buckets 2047 - 2t and 2046 - 2t: start offsets from the top
    const uint32_t c0 = cnt[2047 - 2 * t], c1 = cnt[2046 - 2 * t];
    const uint32_t incl = wave_incl_scan(c0 + c1);
    if (lane_id() == kWave - 1) wtot[t / kWave] = incl;
    __syncthreads();
    uint32_t base = incl - (c0 + c1);
    for (int w = 0; w < t / kWave; ++w) base += wtot[w];
    if (t == 1023) total = base + c0 + c1;
    __syncthreads();
    cnt[2047 - 2 * t] = base;
    cnt[2046 - 2 * t] = base + c0;
    __syncthreads();
    for_each_block([&](int b, int j, int w) {
        const uint32_t p = atomicAdd(&cnt[w], 1u);
        if (p < (uint32_t)a.n_plan) a.plan[p] = make_int2(b, j);
    });
    for (uint32_t p = total + (uint32_t)t; p < (uint32_t)a.n_plan; p += 1024u) a.plan[p] = make_int2(-1, 0);
}

}  // namespace
}  // namespace dsaidx
