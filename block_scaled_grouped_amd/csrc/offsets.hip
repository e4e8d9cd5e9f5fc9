// Group sizes (int32, device) -> int64 sizes and exclusive prefix-sum offsets.
//
// "[JAX] MXFP8 Grouped Quant+GEMM", Changes list and the review thread on
// cublaslt_grouped_gemm.cu: sizes are widened to int64 with a multiplier and
// scanned into G + 1 offsets, offsets[0] = 0.  The prior art scans with a
// single thread and notes a warp-level scan for large G; here one 256-thread
// block scans all G <= 256 groups in LDS (eight barrier steps), so the cost is
// one kernel's launch latency for any G.  pad_to rounds every size up first
// (the 128-padded columnwise token offsets).
#include "bsg_internal.h"

namespace bsg {

__global__ __launch_bounds__(256) void group_offsets_kernel(const int32_t* __restrict__ sizes,
                                                            int G, int64_t mult, int64_t pad,
                                                            int64_t* __restrict__ sizes_i64,
                                                            int64_t* __restrict__ offsets,
                                                            int64_t cap, uint32_t* status) {
  __shared__ int64_t s[256];
  const int g = threadIdx.x;
  int64_t v = 0;
  uint32_t bad = 0;
  if (g < G) {
    int64_t sz = sizes[g];
    if (sz < 0) {
      bad |= kDevNegativeSize;
      sz = 0;
    }
    v = ((sz + pad - 1) / pad) * pad * mult;
    if (sizes_i64 != nullptr) sizes_i64[g] = sz * mult;
  }
  s[g] = v;
  __syncthreads();
  for (int d = 1; d < 256; d <<= 1) {
    int64_t t = g >= d ? s[g - d] : 0;
    __syncthreads();
    s[g] += t;
    __syncthreads();
  }
  if (g < G) offsets[g + 1] = s[g];
  if (g == 0) offsets[0] = 0;
  if (g == G - 1 && cap > 0 && s[g] > cap) bad |= kDevOverCapacity;
  dev_status_or(status, bad);
}

hipError_t launch_group_offsets(const int32_t* sizes, int G, int64_t multiplier, int64_t pad_to,
                                int64_t* sizes_i64, int64_t* offsets, int64_t capacity,
                                uint32_t* status, hipStream_t stream) {
  hipLaunchKernelGGL(group_offsets_kernel, dim3(1), dim3(256), 0, stream, sizes, G, multiplier,
                     pad_to, sizes_i64, offsets, capacity, status);
  return hipGetLastError();
}

}  // namespace bsg
