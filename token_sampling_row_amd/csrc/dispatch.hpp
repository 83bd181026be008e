// Chunks per thread compiled for each kernel family; a launch takes the
// smallest count that covers the row.
#pragma once

#include "verify_wide.hpp"

namespace tsr {

#define TSR_ROW_NCS(X) X(1) X(2) X(4) X(8) X(16) X(24) X(32) X(38)
#define TSR_VERIFY_NCS(X) X(1) X(2) X(4) X(8) X(16)
#define TSR_VERIFY_WIDE_NCS(X) X(24) X(32) X(38)

inline int chunks_per_thread(int dtype, int V) {
  const int epc = dtype == 0 ? 4 : 8;
  const long long chunks = ((long long)V + epc - 1) / epc;
  return (int)((chunks + kBlock - 1) / kBlock);
}

inline int pick_nc(int needed, const int* list, int n) {
  for (int i = 0; i < n; ++i)
    if (list[i] >= needed) return list[i];
  return 0;
}

constexpr int kRowNcs[] = {1, 2, 4, 8, 16, 24, 32, 38};
constexpr int kVerifyNcs[] = {1, 2, 4, 8, 16};
constexpr int kVerifyWideNcs[] = {24, 32, 38};

// Each kernel instance is compiled in a translation unit of its own (the
// build generates them), so the units that launch them only declare them.
#define TSR_SAMPLE_ARGS const unsigned char*, long long, int, int, KParams, int32_t*, DiagPtrs
#define TSR_DECLARE_ROW(N)                                                                   \
  extern template __global__ void sample_kernel<0, N, false, 0>(TSR_SAMPLE_ARGS);             \
  extern template __global__ void sample_kernel<1, N, false, 0>(TSR_SAMPLE_ARGS);             \
  extern template __global__ void sample_kernel<1, N, true, 0>(TSR_SAMPLE_ARGS);              \
  extern template __global__ void sample_kernel<0, N, false, 1>(TSR_SAMPLE_ARGS);             \
  extern template __global__ void sample_kernel<0, N, false, 2>(TSR_SAMPLE_ARGS);             \
  extern template __global__ void sample_kernel<1, N, true, 1>(TSR_SAMPLE_ARGS);              \
  extern template __global__ void sample_kernel<1, N, true, 2>(TSR_SAMPLE_ARGS);              \
  extern template __global__ void beam_kernel<0, N>(const unsigned char*, long long, int, int,  \
                                                    int, const double*, BeamWs);              \
  extern template __global__ void beam_kernel<1, N>(const unsigned char*, long long, int, int,  \
                                                    int, const double*, BeamWs);              \
  extern template __global__ void greedy_kernel<0, N>(const unsigned char*, long long, int,  \
                                                      int, int32_t*, int32_t*);               \
  extern template __global__ void greedy_kernel<1, N>(const unsigned char*, long long, int,  \
                                                      int, int32_t*, int32_t*);
#define TSR_DECLARE_VERIFY_DT(D, N)                                                           \
  extern template __global__ void verify_kernel<D, N>(                                        \
      const unsigned char*, const unsigned char*, const int32_t*, int, int, int, KParams,      \
      VerifyWs);                                                                               \
  extern template __global__ void tree_kernel<D, N>(                                          \
      const unsigned char*, const unsigned char*, const int32_t*, const int32_t*, int, int,    \
      int, KParams, VerifyWs, int32_t*, int32_t*, int32_t*, int32_t*);
#define TSR_DECLARE_VERIFY(N) TSR_DECLARE_VERIFY_DT(0, N) TSR_DECLARE_VERIFY_DT(1, N)
#define TSR_DECLARE_VROWS_DT(D, N, T)                                                         \
  extern template __global__ void verify_rows_kernel<D, N, T>(                                \
      const unsigned char*, const unsigned char*, const int32_t*, int, int, int, KParams,      \
      VerifyWs);
#define TSR_DECLARE_VROWS(N)                                                                 \
  TSR_DECLARE_VROWS_DT(0, N, false) TSR_DECLARE_VROWS_DT(1, N, false)                        \
  TSR_DECLARE_VROWS_DT(0, N, true) TSR_DECLARE_VROWS_DT(1, N, true)
#define TSR_DECLARE_VFINISH(D)                                                                \
  extern template __global__ void verify_finish_kernel<D>(                                    \
      const unsigned char*, const unsigned char*, const int32_t*, int, int, KParams, VerifyWs, \
      int32_t*, int32_t*, int32_t*);                                                           \
  extern template __global__ void verify_draw_kernel<D>(                                      \
      const unsigned char*, const unsigned char*, int, int, KParams, VerifyWs, int32_t*);      \
  extern template __global__ void tree_finish_kernel<D>(                                      \
      const unsigned char*, const unsigned char*, const int32_t*, const int32_t*, int, int,    \
      KParams, VerifyWs, int32_t*, int32_t*, int32_t*, int32_t*);
#ifndef TSR_INSTANCE_UNIT
TSR_ROW_NCS(TSR_DECLARE_ROW)
TSR_VERIFY_NCS(TSR_DECLARE_VERIFY)
TSR_VERIFY_WIDE_NCS(TSR_DECLARE_VROWS)
TSR_DECLARE_VFINISH(0)
TSR_DECLARE_VFINISH(1)
extern template __global__ void sample_kernel_stream<0>(const unsigned char*, long long, int,
                                                        KParams, int32_t*, DiagPtrs);
extern template __global__ void sample_kernel_stream<1>(const unsigned char*, long long, int,
                                                        KParams, int32_t*, DiagPtrs);
extern template __global__ void greedy_kernel_stream<0>(const unsigned char*, long long, int,
                                                        int32_t*, int32_t*);
extern template __global__ void greedy_kernel_stream<1>(const unsigned char*, long long, int,
                                                        int32_t*, int32_t*);
#endif

}  // namespace tsr
