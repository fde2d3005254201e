// Device check of the cu_seqlens precondition of the attention calls:
// 0 = c_0 < c_1 < ... < c_n = T.  InternEvo "数据加载与流程", section
// "获取Dataloader数据", describes cu_seqlens as the cumulative document (and
// padding) boundaries of each row, starting at 0 and ending at the packed
// length, so every segment is non-empty and the last boundary is the total.
//
// One workgroup reads the n + 1 boundaries once and writes a bitmask of the
// violations (see psc.h) to flags[0]; it never reads past entry n.
#include "psc_internal.h"

namespace psc {
namespace {

constexpr int kThreads = 256;

__global__ void __launch_bounds__(kThreads) k_check_cu(const int32_t* cu, int32_t n_seg, int32_t T, int32_t* flags) {
  __shared__ int32_t bad;
  if (threadIdx.x == 0) bad = 0;
  __syncthreads();
  int32_t mine = 0;
  if (threadIdx.x == 0) {
    if (cu[0] != 0) mine |= kCuBadStart;
    if (cu[n_seg] != T) mine |= kCuBadEnd;
  }
  for (int32_t i = threadIdx.x; i < n_seg; i += kThreads) {
    if (cu[i + 1] <= cu[i]) mine |= kCuNotIncreasing;
  }
  if (mine) atomicOr(&bad, mine);
  __syncthreads();
  if (threadIdx.x == 0) flags[0] = bad;
}

}  // namespace

hipError_t launch_check_cu(const int32_t* cu, int32_t n_seg, int32_t T, int32_t* flags, hipStream_t stream) {
  k_check_cu<<<1, kThreads, 0, stream>>>(cu, n_seg, T, flags);
  return hipGetLastError();
}

}  // namespace psc
