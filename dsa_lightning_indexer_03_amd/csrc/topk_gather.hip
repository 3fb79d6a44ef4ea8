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
// them all: a wave reads its four indices and page ids once, then moves the
// four rows of each layer of its layer group, two layers' loads in flight
// before their stores.  blockIdx.y is the layer group, so a small selection
// still fills the chip when many layers share it.
__global__ void __launch_bounds__(kThreads)
topk_gather_layers_kernel(GatherLayersArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
    const int64_t total = (int64_t)a.B * a.K;
    const int64_t r0 = wave * kRowsPerWave;
    if (r0 >= total) return;
    const int l0 = (int)blockIdx.y * a.layers_per_group;
    const int l1 = min(a.n_layers, l0 + a.layers_per_group);
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
    int l = l0;
    for (; l + 1 < l1; l += 2) {
        const uint8_t* c0 = a.cache[l];
        const uint8_t* c1 = a.cache[l + 1];
        uint8_t* o0 = a.out[l];
        uint8_t* o1 = a.out[l + 1];
        for (int c = lane; c < pieces; c += 64) {
            v4i v[2][kRowsPerWave];
#pragma unroll
            for (int u = 0; u < kRowsPerWave; ++u) {
                v[0][u] = ok[u] ? *reinterpret_cast<const v4i*>(c0 + src[u] + 16 * c) : v4i{0, 0, 0, 0};
                v[1][u] = ok[u] ? *reinterpret_cast<const v4i*>(c1 + src[u] + 16 * c) : v4i{0, 0, 0, 0};
            }
#pragma unroll
            for (int u = 0; u < kRowsPerWave; ++u)
                if (live[u]) {
                    *reinterpret_cast<v4i*>(o0 + (r0 + u) * a.row_bytes + 16 * c) = v[0][u];
                    *reinterpret_cast<v4i*>(o1 + (r0 + u) * a.row_bytes + 16 * c) = v[1][u];
                }
        }
    }
    if (l < l1) {
        const uint8_t* c0 = a.cache[l];
        uint8_t* o0 = a.out[l];
        for (int c = lane; c < pieces; c += 64) {
            v4i v[kRowsPerWave];
#pragma unroll
            for (int u = 0; u < kRowsPerWave; ++u)
                v[u] = ok[u] ? *reinterpret_cast<const v4i*>(c0 + src[u] + 16 * c) : v4i{0, 0, 0, 0};
#pragma unroll
            for (int u = 0; u < kRowsPerWave; ++u)
                if (live[u]) *reinterpret_cast<v4i*>(o0 + (r0 + u) * a.row_bytes + 16 * c) = v[u];
        }
    }
}

}  // namespace

hipError_t launch_topk_gather_layers(const GatherLayersArgs& a_in, hipStream_t stream) {
    GatherLayersArgs a = a_in;
    const int64_t total = (int64_t)a.B * a.K;
    const int64_t waves = (total + kRowsPerWave - 1) / kRowsPerWave;
    const int64_t blocks = (waves * 64 + kThreads - 1) / kThreads;
    // Layer groups: all layers in one group when the rows alone give enough
    // waves; otherwise split the layers until about 8192 waves are in flight
    // (32 per CU), so the indices are re-read only where that buys occupancy.
    constexpr int64_t kWantWaves = 8192;
    int64_t groups = (kWantWaves + waves - 1) / waves;
    if (groups > a.n_layers) groups = a.n_layers;
    if (groups < 1) groups = 1;
    a.layers_per_group = (int)((a.n_layers + groups - 1) / groups);
    groups = (a.n_layers + a.layers_per_group - 1) / a.layers_per_group;
    hipLaunchKernelGGL(topk_gather_layers_kernel, dim3((unsigned)blocks, (unsigned)groups), dim3(kThreads), 0,
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
