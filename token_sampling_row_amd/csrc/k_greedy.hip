// Greedy argmax kernels (both element types).
#include "dispatch.hpp"

namespace tsr {

hipError_t launch_greedy(const void* logits, int dtype, int rows, int V, long long stride_bytes,
                         int aligned, int ragged, int32_t* out, int32_t* status, hipStream_t s) {
  const int nc = pick_nc(chunks_per_thread(dtype, V), kRowNcs, 7);
  const unsigned char* p = static_cast<const unsigned char*>(logits);
#define TSR_CASE(N)                                                                      \
  case N:                                                                                \
    if (dtype == 0)                                                                      \
      hipLaunchKernelGGL((greedy_kernel<0, N>), dim3(rows), dim3(kBlock), 0, s, p,       \
                         stride_bytes, V, aligned, ragged, out, status);                 \
    else                                                                                 \
      hipLaunchKernelGGL((greedy_kernel<1, N>), dim3(rows), dim3(kBlock), 0, s, p,       \
                         stride_bytes, V, aligned, ragged, out, status);                 \
    break;
  switch (nc) {
    TSR_ROW_NCS(TSR_CASE)
    default: return hipErrorInvalidValue;
  }
#undef TSR_CASE
  return hipGetLastError();
}

int max_vocab_sample(int dtype) { return 19 * kBlock * (dtype == 0 ? 4 : 8); }
int max_vocab_verify(int dtype) { return 8 * kBlock * (dtype == 0 ? 4 : 8); }

}  // namespace tsr
