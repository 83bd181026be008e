// The sample_rows and verify front doors (element type dispatch) and the Philox test hook.
#include "dispatch.hpp"

namespace tsr {

hipError_t launch_sample_dt0(const unsigned char* p, int rows, int V, long long stride_bytes,
                             int ragged, const KParams& kp, int32_t* out,
                             const DiagPtrs& dg, hipStream_t s);
hipError_t launch_sample_dt1(const unsigned char* p, int rows, int V, long long stride_bytes,
                             int ragged, const KParams& kp, int32_t* out,
                             const DiagPtrs& dg, hipStream_t s);

hipError_t launch_verify_dt0(const unsigned char* tp, const unsigned char* dp, const int32_t* xs,
                             int rows, int K, int V, int ragged, const KParams& kp,
                             const VerifyWs& ws, int32_t* out_tokens, int32_t* out_acc,
                             int32_t* out_status, hipStream_t s);
hipError_t launch_verify_dt1(const unsigned char* tp, const unsigned char* dp, const int32_t* xs,
                             int rows, int K, int V, int ragged, const KParams& kp,
                             const VerifyWs& ws, int32_t* out_tokens, int32_t* out_acc,
                             int32_t* out_status, hipStream_t s);

hipError_t launch_verify(const void* tgt, const void* dft, int dtype, const int32_t* xs,
                         int rows, int K, int V, int ragged, const KParams& kp,
                         const VerifyWs& ws, int32_t* out_tokens, int32_t* out_acc,
                         int32_t* out_status, hipStream_t s) {
  const unsigned char* tp = static_cast<const unsigned char*>(tgt);
  const unsigned char* dp = static_cast<const unsigned char*>(dft ? dft : tgt);
  return dtype == 0 ? launch_verify_dt0(tp, dp, xs, rows, K, V, ragged, kp, ws,
                                        out_tokens, out_acc, out_status, s)
                    : launch_verify_dt1(tp, dp, xs, rows, K, V, ragged, kp, ws,
                                        out_tokens, out_acc, out_status, s);
}

hipError_t launch_tree_dt0(const unsigned char* tp, const unsigned char* dp,
                           const int32_t* parent, const int32_t* tokens, int rows, int N, int V,
                           int ragged, const KParams& kp, const VerifyWs& ws,
                           int32_t* out_tokens, int32_t* out_path, int32_t* out_acc,
                           int32_t* out_status, hipStream_t s);
hipError_t launch_tree_dt1(const unsigned char* tp, const unsigned char* dp,
                           const int32_t* parent, const int32_t* tokens, int rows, int N, int V,
                           int ragged, const KParams& kp, const VerifyWs& ws,
                           int32_t* out_tokens, int32_t* out_path, int32_t* out_acc,
                           int32_t* out_status, hipStream_t s);

hipError_t launch_tree(const void* tgt, const void* dft, int dtype, const int32_t* parent,
                       const int32_t* tokens, int rows, int N, int V, int ragged,
                       const KParams& kp, const VerifyWs& ws, int32_t* out_tokens,
                       int32_t* out_path, int32_t* out_acc, int32_t* out_status, hipStream_t s) {
  const unsigned char* tp = static_cast<const unsigned char*>(tgt);
  const unsigned char* dp = static_cast<const unsigned char*>(dft ? dft : tgt);
  return dtype == 0 ? launch_tree_dt0(tp, dp, parent, tokens, rows, N, V, ragged, kp, ws,
                                      out_tokens, out_path, out_acc, out_status, s)
                    : launch_tree_dt1(tp, dp, parent, tokens, rows, N, V, ragged, kp, ws,
                                      out_tokens, out_path, out_acc, out_status, s);
}

hipError_t launch_sample(const void* logits, int dtype, int rows, int V, long long stride_bytes,
                         int ragged, const KParams& kp, int32_t* out,
                         const DiagPtrs& dg, hipStream_t s) {
  const unsigned char* p = static_cast<const unsigned char*>(logits);
  return dtype == 0 ? launch_sample_dt0(p, rows, V, stride_bytes, ragged, kp, out, dg, s)
                    : launch_sample_dt1(p, rows, V, stride_bytes, ragged, kp, out, dg, s);
}

static __global__ void fill_u32_kernel(uint32_t* p, int n, uint32_t v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

hipError_t launch_fill_u32(uint32_t* p, int n, uint32_t v, hipStream_t s) {
  const int threads = 256;
  hipLaunchKernelGGL(fill_u32_kernel, dim3((n + threads - 1) / threads), dim3(threads), 0, s, p,
                     n, v);
  return hipGetLastError();
}

hipError_t launch_philox(const uint32_t* ctr, int n, uint32_t k0, uint32_t k1, uint32_t* out,
                         hipStream_t s) {
  const int threads = 256;
  hipLaunchKernelGGL(philox_kernel, dim3((n + threads - 1) / threads), dim3(threads), 0, s, ctr,
                     n, k0, k1, out);
  return hipGetLastError();
}

}  // namespace tsr
