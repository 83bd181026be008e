// sample_rows kernels for one element type (f32).
#include "dispatch.hpp"

namespace tsr {

hipError_t launch_sample_dt0(const unsigned char* p, int rows, int V, long long stride_bytes,
                              int ragged, const KParams& kp, int32_t* out, const DiagPtrs& dg,
                              hipStream_t s) {
  const int nc = pick_nc(chunks_per_thread(0, V), kRowNcs, 8);
  const int ext = (kp.flags & F_MASK) ? 1 : (kp.flags & F_REP) ? 2 : 0;
  if (nc == 0) {   // wider than the register file: stream
    hipLaunchKernelGGL((sample_kernel_stream<0>), dim3(rows), dim3(kBlock), 0, s, p,
                       stride_bytes, V, kp, out, dg);
    return hipGetLastError();
  }
#define TSR_CASE(N)                                                                            \
  case N:                                                                                      \
    if (ext == 1)                                                                              \
      hipLaunchKernelGGL((sample_kernel<0, N, false, 1>), dim3(rows), dim3(kBlock), 0, s, p,   \
                         stride_bytes, V, ragged, kp, out, dg);                                \
    else if (ext == 2)                                                                         \
      hipLaunchKernelGGL((sample_kernel<0, N, false, 2>), dim3(rows), dim3(kBlock), 0, s, p,   \
                         stride_bytes, V, ragged, kp, out, dg);                                \
    else                                                                                       \
      hipLaunchKernelGGL((sample_kernel<0, N, false, 0>), dim3(rows), dim3(kBlock), 0, s, p,   \
                         stride_bytes, V, ragged, kp, out, dg);                                \
    break;
  switch (nc) {
    TSR_ROW_NCS(TSR_CASE)
    default: return hipErrorInvalidValue;
  }
#undef TSR_CASE
  return hipGetLastError();
}

}  // namespace tsr
