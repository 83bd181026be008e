// Verify-step kernels for one element type (f32).
#include "dispatch.hpp"

namespace tsr {

hipError_t launch_verify_dt0(const unsigned char* tp, const unsigned char* dp, const int32_t* xs,
                             int rows, int K, int V, int ragged, const KParams& kp,
                             const VerifyWs& ws, int32_t* out_tokens, int32_t* out_acc,
                             int32_t* out_status, hipStream_t s) {
  const int need = chunks_per_thread(0, V);
  if (need > 16) {
    // wider rows: one row per workgroup, then one sequence per workgroup
    const int ncw = pick_nc(need, kVerifyWideNcs, 3);
    if (ncw == 0 || !ws.rec) return hipErrorInvalidValue;
    const bool greedy = (kp.flags & F_GREEDY) != 0;
    const dim3 grid_rows((unsigned)rows * (unsigned)(greedy ? K + 1 : 2 * K + 1));
#define TSR_WCASE(N)                                                                         \
  case N:                                                                                    \
    hipLaunchKernelGGL((verify_rows_kernel<0, N, false>), grid_rows, dim3(kBlock), 0, s, tp, dp, \
                       nullptr, K, V, ragged, kp, ws);                                       \
    break;
    switch (ncw) {
      TSR_VERIFY_WIDE_NCS(TSR_WCASE)
      default: return hipErrorInvalidValue;
    }
#undef TSR_WCASE
    // the residual in slices of kSliceRows chunk rows (one slice when greedy)
    VerifyWs wf = ws;
    wf.nseq = rows;
    const int S = greedy ? 1 : (need + kSliceRows - 1) / kSliceRows;
    hipLaunchKernelGGL((verify_finish_kernel<0>), dim3((unsigned)rows * (unsigned)S), dim3(kBlock),
                       0, s, tp, dp, xs, K, V, kp, wf, out_tokens, out_acc, out_status);
    if (!greedy)
      hipLaunchKernelGGL((verify_draw_kernel<0>), dim3(rows), dim3(kBlock), 0, s, tp, dp, K, V, kp,
                         wf, out_tokens);
    return hipGetLastError();
  }
  const int nc = pick_nc(need, kVerifyNcs, 5);
  const dim3 grid((unsigned)rows * (unsigned)(K + 1));
#define TSR_CASE(N)                                                                          \
  case N:                                                                                    \
    hipLaunchKernelGGL((verify_kernel<0, N>), grid, dim3(kBlock), 0, s, tp, dp, xs, K, V, ragged, \
                       kp, ws);                                                               \
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
                           int ragged, const KParams& kp, const VerifyWs& ws,
                           int32_t* out_tokens, int32_t* out_path, int32_t* out_acc,
                           int32_t* out_status, hipStream_t s) {
  const int need = chunks_per_thread(0, V);
  if (need > 16) {
    const int ncw = pick_nc(need, kVerifyWideNcs, 3);
    if (ncw == 0 || !ws.rec) return hipErrorInvalidValue;
    const bool greedy = (kp.flags & F_GREEDY) != 0;
    const dim3 grid_rows((unsigned)rows * (unsigned)(greedy ? N : 2 * N));
#define TSR_WCASE(N_)                                                                        \
  case N_:                                                                                   \
    hipLaunchKernelGGL((verify_rows_kernel<0, N_, true>), grid_rows, dim3(kBlock), 0, s, tp, dp, \
                       parent, N, V, ragged, kp, ws);                                        \
    break;
    switch (ncw) {
      TSR_VERIFY_WIDE_NCS(TSR_WCASE)
      default: return hipErrorInvalidValue;
    }
#undef TSR_WCASE
    hipLaunchKernelGGL((tree_finish_kernel<0>), dim3(rows), dim3(kBlock), 0, s, tp, dp, parent,
                       tokens, N, V, kp, ws, out_tokens, out_path, out_acc, out_status);
    return hipGetLastError();
  }
  const int nc = pick_nc(need, kVerifyNcs, 5);
  const dim3 grid((unsigned)rows * (unsigned)N);
#define TSR_CASE(N_)                                                                         \
  case N_:                                                                                   \
    hipLaunchKernelGGL((tree_kernel<0, N_>), grid, dim3(kBlock), 0, s, tp, dp, parent, tokens, N, \
                       V, ragged, kp, ws, out_tokens, out_path, out_acc, out_status);        \
    break;
  switch (nc) {
    TSR_VERIFY_NCS(TSR_CASE)
    default: return hipErrorInvalidValue;
  }
#undef TSR_CASE
  return hipGetLastError();
}

}  // namespace tsr
