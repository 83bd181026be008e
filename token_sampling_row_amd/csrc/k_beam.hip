// Beam-step kernels (both element types): one workgroup per beam row, then
// one wavefront per group for the merge.
#include "dispatch.hpp"

namespace tsr {

// One wavefront per group: the group's beam lists (each row's best tokens,
// best first) into LDS, then lane b < beam walks beam b's list, B times the
// best head (ties to the lower beam).
__global__ __launch_bounds__(kWave) void beam_merge_kernel(int beam, BeamWs ws,
                                                           int32_t* out_parent, int32_t* out_tok,
                                                           double* out_score,
                                                           int32_t* out_status) {
  __shared__ double lsc[kBeamMax * kBeamMax];
  __shared__ int ltk[kBeamMax * kBeamMax];
  const int g = blockIdx.x, lane = threadIdx.x;
  const long long base = (long long)g * beam * kBeamMax;
  for (int q = lane; q < beam * kBeamMax; q += kWave) {
    lsc[q] = ws.score[base + q];
    ltk[q] = ws.tok[base + q];
  }
  __syncthreads();
  const bool gbad = __any(lane < beam && lsc[lane * kBeamMax] != lsc[lane * kBeamMax]);
  int ptr = 0;
  auto head = [&](int q) -> double {
    return (lane < beam && q < beam) ? lsc[lane * kBeamMax + q] : (double)kNegInf;
  };
  double hs = head(0);
  int any_finite = 0;
  for (int q = 0; q < beam; ++q) {
    const double best = wave_reduce(hs, [](double a, double b) { return a > b ? a : b; });
    const int w = __ffsll((long long)__ballot(lane < beam && hs == best)) - 1;
    const long long o = (long long)g * beam + q;
    if (lane == w) {
      const bool fin = best > (double)kNegInf;
      const int tk = fin ? ltk[w * kBeamMax + ptr] : -1;
      out_parent[o] = gbad ? -1 : (fin ? w : -1);
      out_tok[o] = gbad ? -1 : tk;
      out_score[o] = gbad ? __builtin_nan("") : best;
      ++ptr;
      hs = head(ptr);
    }
    any_finite |= best > (double)kNegInf;
  }
  if (lane == 0 && out_status) out_status[g] = gbad ? 1 : (any_finite ? 0 : 2);
}

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
                         stride_bytes, V, ragged, beam, scores, ws);                         \
    else                                                                                     \
      hipLaunchKernelGGL((beam_kernel<1, N>), dim3(rows), dim3(kBlock), 0, s, p,             \
                         stride_bytes, V, ragged, beam, scores, ws);                         \
    break;
  switch (nc) {
    TSR_ROW_NCS(TSR_CASE)
    default: return hipErrorInvalidValue;
  }
#undef TSR_CASE
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || groups == 0) return e;
  hipLaunchKernelGGL(beam_merge_kernel, dim3(groups), dim3(kWave), 0, s, beam, ws, out_parent,
                     out_tok, out_score, out_status);
  return hipGetLastError();
}

// Rows held in registers only (at most 38 chunks of 16 bytes per thread).
int max_vocab_beam(int dtype) { return 38 * kBlock * (dtype == 0 ? 4 : 8); }

}  // namespace tsr
