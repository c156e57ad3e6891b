// Device copy of the codec's basis table (see basis.h): each kernel source
// that includes this holds the table in its code object.
#pragma once

#include <hip/hip_runtime.h>

#include "basis.h"

namespace cdattn {

static __device__ const float kBasisDev[kBasisEntries] = {
#include "cdattn_basis_table.inc"
};

// Analysis entry M[j][i] (frequency j < R, token i < R) of block size R: the
// DCT-II basis, or for PNG mode (README "Math", PNG item) the anchor row and
// the first-order differences, x_0 and x_i - x_{i-1}.  The table entry is
// read either way and the PNG value chosen by a select, so there is no
// branch around the load.
__device__ __forceinline__ float analysis_entry(int png, int R, int j, int i) {
  const float t = kBasisDev[basis_index(R, j, i)];
  const float d = i == j ? 1.0f : (j > 0 && i == j - 1 ? -1.0f : 0.0f);
  return png ? d : t;
}

// Synthesis entry A[i][j] (token i < R from row j < R): M^T for the DCT-II,
// the cumulative sum for PNG mode (x_hat_i = x_0 + sum_{j = 1..i} delta_j).
// The table is read in both modes (no branch around the load).
__device__ __forceinline__ float synthesis_entry(int png, int R, int i, int j) {
  const float t = kBasisDev[basis_index(R, j, i)];
  return png ? (j <= i ? 1.0f : 0.0f) : t;
}

}  // namespace cdattn
