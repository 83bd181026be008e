// Verify-step kernels for one element type (f32).
#include "dispatch.hpp"

namespace tsr {

hipError_t launch_verify_dt0(const unsigned char* tp, const unsigned char* dp, const int32_t* xs,
                             int rows, int K, int V, int aligned, int ragged, const KParams& kp,
                             const VerifyWs& ws, int32_t* out_tokens, int32_t* out_acc,
                             int32_t* out_status, hipStream_t s) {
  const int nc = pick_nc(chunks_per_thread(0, V), kVerifyNcs, 5);
  const dim3 grid((unsigned)rows * (unsigned)(K + 1));
#define TSR_CASE(N)                                                                          \
  case N:                                                                                    \
    if (aligned)                                                                             \
      hipLaunchKernelGGL((verify_kernel<0, N, false>), grid, dim3(kBlock), 0, s, tp, dp, xs,  \
                         K, V, aligned, ragged, kp, ws, out_tokens, out_acc, out_status);    \
    else                                                                                     \
      hipLaunchKernelGGL((verify_kernel<0, N, true>), grid, dim3(kBlock), 0, s, tp, dp, xs,   \
                         K, V, aligned, ragged, kp, ws, out_tokens, out_acc, out_status);    \
    break;
  switch (nc) {
    TSR_VERIFY_NCS(TSR_CASE)
    default: return hipErrorInvalidValue;
  }
#undef TSR_CASE
  return hipGetLastError();
}

hipError_t launch_tree_dt0(const unsigned char* tp, const unsigned char* dp,
                           const int32_t* parent, const int32_t* tokens, int rows, int N, int V,
                           int aligned, int ragged, const KParams& kp, const VerifyWs& ws,
                           int32_t* out_tokens, int32_t* out_path, int32_t* out_acc,
                           int32_t* out_status, hipStream_t s) {
  const int nc = pick_nc(chunks_per_thread(0, V), kVerifyNcs, 5);
  const dim3 grid((unsigned)rows * (unsigned)N);
#define TSR_CASE(N_)                                                                         \
  case N_:                                                                                   \
    if (aligned)                                                                             \
      hipLaunchKernelGGL((tree_kernel<0, N_, false>), grid, dim3(kBlock), 0, s, tp, dp,     \
                         parent, tokens, N, V, ragged, kp, ws, out_tokens, out_path, out_acc, \
                         out_status);                                                        \
    else                                                                                     \
      hipLaunchKernelGGL((tree_kernel<0, N_, true>), grid, dim3(kBlock), 0, s, tp, dp,      \
                         parent, tokens, N, V, ragged, kp, ws, out_tokens, out_path, out_acc, \
                         out_status);                                                        \
    break;
  switch (nc) {
    TSR_VERIFY_NCS(TSR_CASE)
    default: return hipErrorInvalidValue;
  }
#undef TSR_CASE
  return hipGetLastError();
}

}  // namespace tsr
