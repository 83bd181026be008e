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

// One wavefront per sequence after the two-row verify kernel [P2 39.4,
// Listing 39.4]: lane q reads position q's results (acceptance, token,
// statuses); the status is the target's of the first position that has one,
// else the draft's, else 3 for a draft token out of range; the accepted prefix
// runs up to the first rejection, whose token (the residual draw, or the
// bonus draw when every position accepted) follows it.
__global__ __launch_bounds__(kWave) void verify_seq_finish_kernel(const int32_t* xs, int K, int V,
                                                                  VerifyWs ws,
                                                                  int32_t* out_tokens,
                                                                  int32_t* out_acc,
                                                                  int32_t* out_status) {
  const int b = blockIdx.x, q = threadIdx.x;
  const int s0 = b * ws.kmax1;
  const bool inq = q <= K, dq = q < K;
  const int qt = inq ? ws.st_t[s0 + q] : 0;
  const int qd = dq ? ws.st_d[s0 + q] : 0;
  const int qa = dq ? ws.acc[s0 + q] : 1;
  const int qk = inq ? ws.tok[s0 + q] : -1;
  const int xq = dq ? xs[(long long)b * K + q] : 0;
  const unsigned long long bt = __ballot(qt != 0), bd = __ballot(qd != 0);
  const unsigned long long bx = __ballot(dq && (xq < 0 || xq >= V));
  const int status = bt ? readlane_u32((uint32_t)qt, __ffsll((long long)bt) - 1)
                        : bd ? readlane_u32((uint32_t)qd, __ffsll((long long)bd) - 1)
                             : (bx ? 3 : 0);
  const unsigned long long rej = __ballot(dq && !qa);
  const int n = rej ? __ffsll((long long)rej) - 1 : K;
  const int tn = readlane_u32((uint32_t)qk, n);
  if (inq) {
    int32_t* o = out_tokens + (long long)b * (K + 1);
    o[q] = status ? -1 : (q < n ? xq : (q == n ? tn : -1));
  }
  if (q == 0) {
    out_acc[b] = status ? 0 : n;
    if (out_status) out_status[b] = status;
  }
}

hipError_t launch_verify(const void* tgt, const void* dft, int dtype, const int32_t* xs,
                         int rows, int K, int V, int ragged, const KParams& kp,
                         const VerifyWs& ws, int32_t* out_tokens, int32_t* out_acc,
                         int32_t* out_status, hipStream_t s) {
  const unsigned char* tp = static_cast<const unsigned char*>(tgt);
  const unsigned char* dp = static_cast<const unsigned char*>(dft ? dft : tgt);
  const hipError_t e = dtype == 0 ? launch_verify_dt0(tp, dp, xs, rows, K, V, ragged, kp, ws,
                                                      out_tokens, out_acc, out_status, s)
                                  : launch_verify_dt1(tp, dp, xs, rows, K, V, ragged, kp, ws,
                                                      out_tokens, out_acc, out_status, s);
  if (e != hipSuccess || rows == 0 || chunks_per_thread(dtype, V) > 16) return e;
  // the two-row kernel's rows: one finishing wavefront per sequence
  hipLaunchKernelGGL(verify_seq_finish_kernel, dim3(rows), dim3(kWave), 0, s, xs, K, V, ws,
                     out_tokens, out_acc, out_status);
  return hipGetLastError();
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

hipError_t launch_philox(const uint32_t* ctr, int n, uint32_t k0, uint32_t k1, uint32_t* out,
                         hipStream_t s) {
  const int threads = 256;
  hipLaunchKernelGGL(philox_kernel, dim3((n + threads - 1) / threads), dim3(threads), 0, s, ctr,
                     n, k0, k1, out);
  return hipGetLastError();
}

}  // namespace tsr
