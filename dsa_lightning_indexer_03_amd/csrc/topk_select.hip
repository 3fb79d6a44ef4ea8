// Row-wise exact top-k selection over fp32 scores (the token selector): one
// 1024-thread workgroup per row, the radix select of select_row.h.
#include "device_once.h"
#include "select_row.h"

namespace dsaidx {

__global__ void __launch_bounds__(sel::kThreads)
topk_select_kernel(SelectArgs a) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    sel::select_row(a, blockIdx.x, *reinterpret_cast<sel::SelShared*>(smem_raw), -1);
}

size_t topk_select_smem_bytes() { return sizeof(sel::SelShared); }

hipError_t launch_topk_select(const SelectArgs& a, int rows, hipStream_t stream) {
    static PerDevice<int> lds_once;
    hipError_t e = set_lds_limit(lds_once, (const void*)topk_select_kernel, (int)sizeof(sel::SelShared));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_select_kernel, dim3(rows), dim3(sel::kThreads), sizeof(sel::SelShared), stream, a);
    return hipGetLastError();
}

}  // namespace dsaidx
