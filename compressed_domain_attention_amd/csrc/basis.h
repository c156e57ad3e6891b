// The codec's fp32 DCT-II analysis basis: one table, generated at build time
// (cdattn_basis_table.inc), read by the host (codec_basis) and by every
// kernel that encodes, decodes or materialises, so all of them use the same
// values.  flashcodec-kv README "Math" (JPEG item): M[j][i] = c_j
// cos(pi (2i + 1) j / (2R)), c_0 = sqrt(1/R), c_j = sqrt(2/R), evaluated in
// double precision and rounded to the nearest fp32.  The synthesis matrix is
// its transpose, A[i][j] = M[j][i].
#pragma once

namespace cdattn {

constexpr int kBasisMaxR = 32;
constexpr int kBasisEntries = kBasisMaxR * (kBasisMaxR + 1) * (2 * kBasisMaxR + 1) / 6;   // sum of R^2

// Position of M[j][i] (frequency j, token i) of block size R: the tables of
// block sizes 1 .. R-1 come first, then R rows of R entries.
constexpr int basis_index(int R, int j, int i) { return (R - 1) * R * (2 * R - 1) / 6 + j * R + i; }

}  // namespace cdattn
