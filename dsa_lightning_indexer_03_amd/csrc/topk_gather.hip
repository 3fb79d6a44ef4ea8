// The selection's consumer: for every query, the rows of a paged latent
// cache at its selected positions, gathered into one contiguous block.
//
// The pages send the indexer's top-k to the sparse attention, which reads
// the latent cache c^KV only at those positions, k * d_c elements per query
// ("Study MLA Indexer", the data-flow diagram's last step and the first of
// its "three whys").  The latent cache is taken to share the indexer cache's
// paging (block table, 64-token pages); rows are opaque bytes; a padding or
// out-of-table index gives a zero row.
//
// Layout: one wave per four output rows.  Lane l moves 16-byte pieces
// l, l + 64, ... of each row; the wave first reads the four indices, then
// the four page ids, then issues every row load before any store.  HBM
// bound: per selected row row_bytes read and row_bytes written (plus 4
// bytes of index and 4 of page id).
#include "common.h"
#include "kernels.h"

namespace dsaidx {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerWave = 4;
constexpr int kPage = 64;

__global__ void __launch_bounds__(kThreads)
topk_gather_kernel(GatherArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
    const int64_t total = (int64_t)a.B * a.K;
    const int64_t r0 = wave * kRowsPerWave;
    if (r0 >= total) return;
    const int64_t limit = (int64_t)a.max_pages * kPage;
    const int pieces = a.row_bytes / 16;
    int64_t src[kRowsPerWave];
    bool ok[kRowsPerWave], live[kRowsPerWave];
    int s[kRowsPerWave];
#pragma unroll
    for (int u = 0; u < kRowsPerWave; ++u) {
        live[u] = r0 + u < total;
        s[u] = live[u] ? a.idx[r0 + u] : -1;
    }
#pragma unroll
    for (int u = 0; u < kRowsPerWave; ++u) {
        ok[u] = s[u] >= 0 && (int64_t)s[u] < limit;
        const int64_t b = live[u] ? (r0 + u) / a.K : 0;
        src[u] = ok[u] ? ((int64_t)a.block_table[b * a.max_pages + s[u] / kPage] * kPage + s[u] % kPage) *
                             a.row_bytes
                       : 0;
    }
    for (int c = lane; c < pieces; c += 64) {
        v4i v[kRowsPerWave];
#pragma unroll
        for (int u = 0; u < kRowsPerWave; ++u)
            v[u] = ok[u] ? *reinterpret_cast<const v4i*>(a.cache + src[u] + 16 * c) : v4i{0, 0, 0, 0};
#pragma unroll
        for (int u = 0; u < kRowsPerWave; ++u)
            if (live[u]) *reinterpret_cast<v4i*>(a.out + (r0 + u) * a.row_bytes + 16 * c) = v[u];
    }
}

// Index Share: one selection serves several layers ("Lightning Indexer
// explained", section 1, question 4 of the Q&A, and section 3: the top-k
// computed at one layer is reused by the layers that follow it, which skip
// their own indexer).  The consumer side of that reuse is a gather of the
// same positions from every serving layer's latent cache.  One launch does
// them all: blockIdx.y is the layer, and each wave moves four rows of that
// layer exactly as the single-layer gather does; the indices and page ids
// are read once per layer (from L2 after the first).  A wave that moved its
// rows for several layers in turn, the indices read only once, was 4% slower
// (its next layer's loads queue behind the previous layer's stores).
__global__ void __launch_bounds__(kThreads)
topk_gather_layers_kernel(GatherLayersArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
    const int64_t total = (int64_t)a.B * a.K;
    const int64_t r0 = wave * kRowsPerWave;
    if (r0 >= total) return;
    const uint8_t* cache = a.cache[blockIdx.y];
    uint8_t* out = a.out[blockIdx.y];
    const int64_t limit = (int64_t)a.max_pages * kPage;
    const int pieces = a.row_bytes / 16;
    int64_t src[kRowsPerWave];
    bool ok[kRowsPerWave], live[kRowsPerWave];
    int s[kRowsPerWave];
#pragma unroll
    for (int u = 0; u < kRowsPerWave; ++u) {
        live[u] = r0 + u < total;
        s[u] = live[u] ? a.idx[r0 + u] : -1;
    }
#pragma unroll
    for (int u = 0; u < kRowsPerWave; ++u) {
        ok[u] = s[u] >= 0 && (int64_t)s[u] < limit;
        const int64_t b = live[u] ? (r0 + u) / a.K : 0;
        src[u] = ok[u] ? ((int64_t)a.block_table[b * a.max_pages + s[u] / kPage] * kPage + s[u] % kPage) *
                             a.row_bytes
                       : 0;
    }
    for (int c = lane; c < pieces; c += 64) {
        v4i v[kRowsPerWave];
#pragma unroll
        for (int u = 0; u < kRowsPerWave; ++u)
            v[u] = ok[u] ? *reinterpret_cast<const v4i*>(cache + src[u] + 16 * c) : v4i{0, 0, 0, 0};
#pragma unroll
        for (int u = 0; u < kRowsPerWave; ++u)
            if (live[u]) *reinterpret_cast<v4i*>(out + (r0 + u) * a.row_bytes + 16 * c) = v[u];
    }
}

}  // namespace

hipError_t launch_topk_gather_layers(const GatherLayersArgs& a, hipStream_t stream) {
    const int64_t total = (int64_t)a.B * a.K;
    const int64_t waves = (total + kRowsPerWave - 1) / kRowsPerWave;
    const int64_t blocks = (waves * 64 + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(topk_gather_layers_kernel, dim3((unsigned)blocks, (unsigned)a.n_layers), dim3(kThreads), 0,
                       stream, a);
    return hipGetLastError();
}

hipError_t launch_topk_gather(const GatherArgs& a, hipStream_t stream) {
    const int64_t total = (int64_t)a.B * a.K;
    const int64_t waves = (total + kRowsPerWave - 1) / kRowsPerWave;
    const int64_t blocks = (waves * 64 + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(topk_gather_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace dsaidx
