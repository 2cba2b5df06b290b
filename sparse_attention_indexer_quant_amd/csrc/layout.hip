// decode_layout as its own launch: one workgroup runs the body in layout.h.
#include "launch.h"
#include "layout.h"

namespace dsaidx {

constexpr int kLayoutThreads = 1024;

__global__ __launch_bounds__(kLayoutThreads) void decode_layout_kernel(LayoutArgs a) {
    decode_layout_body<kLayoutThreads>(a);
}

hipError_t launch_decode_layout(const int32_t *seq_lens, const int32_t *query_lens,
                                int64_t num_requests, int64_t num_rows, int dcp_rank,
                                int dcp_world_size, int interleave, int32_t *query_starts,
                                int32_t *row_ends, hipStream_t stream) {
    const LayoutArgs a{seq_lens, query_lens, num_requests, num_rows, dcp_rank,
                       dcp_world_size, interleave, query_starts, row_ends};
    hipLaunchKernelGGL(decode_layout_kernel, dim3(1), dim3(kLayoutThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace dsaidx
