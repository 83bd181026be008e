// Beam-step kernels (both element types).
#include "dispatch.hpp"

namespace tsr {

hipError_t launch_beam(const void* logits, int dtype, int groups, int beam, int V,
                       long long stride_bytes, int ragged, const double* scores, BeamWs ws,
                       int32_t* out_parent, int32_t* out_tok, double* out_score,
                       int32_t* out_status, hipStream_t s) {
  const int nc = pick_nc(chunks_per_thread(dtype, V), kRowNcs, 8);
  if (nc == 0) return hipErrorInvalidValue;
  const unsigned char* p = static_cast<const unsigned char*>(logits);
  const int rows = groups * beam;
#define TSR_CASE(N)                                                                          \
  case N:                                                                                    \
    if (dtype == 0)                                                                          \
      hipLaunchKernelGGL((beam_kernel<0, N>), dim3(rows), dim3(kBlock), 0, s, p,             \
                         stride_bytes, V, ragged, beam, scores, ws, out_parent, out_tok,     \
                         out_score, out_status);                                             \
    else                                                                                     \
      hipLaunchKernelGGL((beam_kernel<1, N>), dim3(rows), dim3(kBlock), 0, s, p,             \
                         stride_bytes, V, ragged, beam, scores, ws, out_parent, out_tok,     \
                         out_score, out_status);                                             \
    break;
  switch (nc) {
    TSR_ROW_NCS(TSR_CASE)
    default: return hipErrorInvalidValue;
  }
#undef TSR_CASE
  return hipGetLastError();
}

// Rows held in registers only (at most 38 chunks of 16 bytes per thread).
int max_vocab_beam(int dtype) { return 38 * kBlock * (dtype == 0 ? 4 : 8); }

}  // namespace tsr
