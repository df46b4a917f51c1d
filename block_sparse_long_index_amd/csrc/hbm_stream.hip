// A measuring aid: a plain streaming kernel with a chosen read:write byte mix,
// used to find the HBM rate a kernel with that mix can reach on this GPU
// (the Main Branch's attend pass reads about one byte for every two it
// writes; its merge pass almost only reads).  Not part of the method.
//
// Unit u reads 16-byte chunk u of src and writes `ratio` chunks derived from
// it, chunk j * n_units + u of dst for j = 0 .. ratio-1 (ratio 0: read only;
// the loaded values are folded into a conditional store so the loads cannot
// be dropped).  Lanes take consecutive units, so every load and store
// instruction covers 1 KiB of consecutive bytes.  A grid-stride loop keeps the
// launch at a few workgroups per CU whatever the size.
#include "msa_common.h"

namespace msa {

template <int RATIO>
__global__ __launch_bounds__(256) void hbm_stream_kernel(const uint4* __restrict__ src,
                                                         long long n_units, uint4* __restrict__ dst,
                                                         uint32_t* __restrict__ sink) {
  uint32_t fold = 0;
  const long long stride = (long long)gridDim.x * 256;
  for (long long u = (long long)blockIdx.x * 256 + threadIdx.x; u < n_units; u += stride) {
    const uint4 v = src[u];
    if constexpr (RATIO == 0) {
      fold ^= v.x ^ v.y ^ v.z ^ v.w;
    } else {
#pragma unroll
      for (int j = 0; j < RATIO; ++j)
        dst[(long long)j * n_units + u] = make_uint4(v.x ^ j, v.y, v.z, v.w);
    }
  }
  if constexpr (RATIO == 0) {
    // a store that depends on every loaded value (and practically never happens)
    if (fold == 0x9e3779b9u) sink[blockIdx.x] = fold;
  }
}

hipError_t launch_hbm_stream(const void* src, long long n_units, int ratio, void* dst, void* sink,
                             int grid, hipStream_t st) {
  const dim3 g((unsigned)grid), b(256);
  const uint4* s = static_cast<const uint4*>(src);
  uint4* d = static_cast<uint4*>(dst);
  uint32_t* k = static_cast<uint32_t*>(sink);
  switch (ratio) {
    case 0: hipLaunchKernelGGL(hbm_stream_kernel<0>, g, b, 0, st, s, n_units, d, k); break;
    case 1: hipLaunchKernelGGL(hbm_stream_kernel<1>, g, b, 0, st, s, n_units, d, k); break;
    case 2: hipLaunchKernelGGL(hbm_stream_kernel<2>, g, b, 0, st, s, n_units, d, k); break;
    case 3: hipLaunchKernelGGL(hbm_stream_kernel<3>, g, b, 0, st, s, n_units, d, k); break;
    case 4: hipLaunchKernelGGL(hbm_stream_kernel<4>, g, b, 0, st, s, n_units, d, k); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace msa
