// Chunks per thread compiled for each kernel family; a launch takes the
// smallest count that covers the row.
#pragma once

#include "kernels_impl.hpp"

namespace tsr {

#define TSR_ROW_NCS(X) X(1) X(2) X(4) X(8) X(12) X(16) X(19)
#define TSR_VERIFY_NCS(X) X(1) X(2) X(4) X(8)

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

constexpr int kRowNcs[] = {1, 2, 4, 8, 12, 16, 19};
constexpr int kVerifyNcs[] = {1, 2, 4, 8};

}  // namespace tsr
