// pad.hip -- copies between a caller's tensors and the shapes the kernels run
// at.  The read is the same sum whatever the head or chunk sizes the kernels
// use, so a head size no kernel runs natively (dk != dv, or bf16 d = 16) runs
// zero-padded to a square one, and a token count that is not a multiple of the
// chunk the kernels run runs zero-padded at the end (zero keys and values and
// no decay: the tokens before see nothing of them).
#include "ll_device.hpp"
#include "ll_launch.hpp"

namespace llattn {

// dst[i0][i1][i2][i3] = src[i0][i1][i2][i3] where every index is inside src's
// extents (s1, s2, s3), else 0; dst has extents (d1, d2, d3) and n0 outer rows.
template <typename E>
__global__ void __launch_bounds__(256) ll_pad_copy(const E* src, E* dst, int64_t n0, int s1, int s2, int s3, int d1,
                                                   int d2, int d3) {
  const int64_t total = n0 * d1 * d2 * d3;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int i3 = (int)(i % d3);
    int64_t rest = i / d3;
    const int i2 = (int)(rest % d2);
    rest /= d2;
    const int i1 = (int)(rest % d1);
    const int64_t i0 = rest / d1;
    E v = E(0);
    if (i1 < s1 && i2 < s2 && i3 < s3) v = src[((i0 * s1 + i1) * s2 + i2) * s3 + i3];
    dst[i] = v;
  }
}

hipError_t launch_pad_copy(int esz, const void* src, void* dst, int64_t n0, int s1, int s2, int s3, int d1, int d2,
                           int d3, hipStream_t s) {
  const int64_t total = n0 * d1 * d2 * d3;
  if (total <= 0) return hipSuccess;
  const int grid = (int)((total + 255) / 256 < 65536 ? (total + 255) / 256 : 65536);
  if (esz == 2)
    hipLaunchKernelGGL(ll_pad_copy<uint16_t>, dim3(grid), dim3(256), 0, s, static_cast<const uint16_t*>(src),
                       static_cast<uint16_t*>(dst), n0, s1, s2, s3, d1, d2, d3);
  else if (esz == 4)
    hipLaunchKernelGGL(ll_pad_copy<uint32_t>, dim3(grid), dim3(256), 0, s, static_cast<const uint32_t*>(src),
                       static_cast<uint32_t*>(dst), n0, s1, s2, s3, d1, d2, d3);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace llattn
