// Chunks per thread compiled for each kernel family; a launch takes the
// smallest count that covers the row.
#pragma once

#include "kernels_impl.hpp"

namespace tsr {

#define TSR_ROW_NCS(X) X(1) X(2) X(4) X(8) X(16) X(24) X(32) X(38)
#define TSR_VERIFY_NCS(X) X(1) X(2) X(4) X(8) X(16)

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

}  // namespace tsr
