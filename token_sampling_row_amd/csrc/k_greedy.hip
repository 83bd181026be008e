// Greedy argmax kernels (both element types).
#include "dispatch.hpp"

namespace tsr {

hipError_t launch_greedy(const void* logits, int dtype, int rows, int V, long long stride_bytes,
                         int ragged, int32_t* out, int32_t* status, hipStream_t s) {
  const int nc = pick_nc(chunks_per_thread(dtype, V), kRowNcs, 8);
  const unsigned char* p = static_cast<const unsigned char*>(logits);
  if (nc == 0) {   // wider than the register file: stream
    if (dtype == 0)
      hipLaunchKernelGGL((greedy_kernel_stream<0>), dim3(rows), dim3(kBlock), 0, s, p,
                         stride_bytes, V, out, status);
    else
      hipLaunchKernelGGL((greedy_kernel_stream<1>), dim3(rows), dim3(kBlock), 0, s, p,
                         stride_bytes, V, out, status);
    return hipGetLastError();
  }
#define TSR_CASE(N)                                                                      \
  case N:                                                                                \
    if (dtype == 0)                                                                      \
      hipLaunchKernelGGL((greedy_kernel<0, N>), dim3(rows), dim3(kBlock), 0, s, p,       \
                         stride_bytes, V, ragged, out, status);                 \
    else                                                                                 \
      hipLaunchKernelGGL((greedy_kernel<1, N>), dim3(rows), dim3(kBlock), 0, s, p,       \
                         stride_bytes, V, ragged, out, status);                 \
    break;
  switch (nc) {
    TSR_ROW_NCS(TSR_CASE)
    default: return hipErrorInvalidValue;
  }
#undef TSR_CASE
  return hipGetLastError();
}

// Rows stream when they exceed the register file; the bound keeps histogram
// masses (2^40 fixed point, weights <= 1) inside 64 bits.
int max_vocab_sample(int) { return 1 << 23; }
int max_vocab_verify_narrow(int dtype) { return 16 * kBlock * (dtype == 0 ? 4 : 8); }
int max_vocab_verify(int dtype) { return 38 * kBlock * (dtype == 0 ? 4 : 8); }

}  // namespace tsr
