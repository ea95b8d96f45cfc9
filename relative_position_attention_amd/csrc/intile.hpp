// In-tile relation products for the attention kernels ([RPA] §6
// "Limitations" and Table 7, row "Projections": every tile computes its own
// relation products instead of reading projections stored in HBM).  [RPA] =
// "Fast and Exact Relative-Position Attention via Structure-Aware Kernels"
// (arXiv 2611.01182).
//
// With in-tile products the plan takes D > N - 1 (every pair is a band pair)
// and D = 15 mod 16, so for a 16-query block starting at qb0 and a 64-key
// tile starting at j0 the rows s = i - j + D the block reaches form the window
// sb = qb0 - j0 - 63 + D .. sb + 78, with sb a multiple of 16.  The window's
// products Z[i, s] = q_i . A~[s] + bt[s] (bt: the expanded bias with b and
// v . A~ folded in, fp32) are one MFMA row block per 16 rows: the lane of
// query column c16 and group g receives rows sb + 16 w + 4 g + t, t = 0..3.
// A pair's entry sits at window position s' = c16 + 63 - (j - j0), a
// different diagonal per query, so the rows go through a per-wave LDS
// scratch ([query][s'] fp32) from which each lane reads the runs its pairs
// need.  The products and their order of accumulation are the same in every
// pass, so the forward and both backward passes see bitwise the same scores.
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace relpos {

// Buffer resources of head h: the expanded table A~^Q [S, 64] (bf16), its
// transpose [64, Sp] (bf16, columns past S zero) and the expanded bias
// bt [S] (fp32).  Loads past a resource return zero; negative rows are sent
// past it (kOob).
struct ItTables {
  Rsrc at, att, bt;
};

__device__ __forceinline__ ItTables it_tables(const AttnArgs& a, int h) {
  const int64_t ht = a.at_shared ? 0 : h;
  ItTables t;
  t.at = make_rsrc(static_cast<const bf16*>(a.at) + ht * a.S * 64, static_cast<uint64_t>(a.S) * 128);
  t.att = make_rsrc(static_cast<const bf16*>(a.att) + ht * 64 * a.Sp,
                    static_cast<uint64_t>(a.Sp) * 128);
  t.bt = make_rsrc(a.bt + static_cast<int64_t>(h) * a.S, static_cast<uint64_t>(a.S) * 4);
  return t;
}

// zw[w] = rows sb + 16 w + 4 g + (0..3) of the lane's query (qf: the query's
// B-operand fragments, K = 32 c + 8 g ..), w < NW: bt as the accumulator's
// initial value, then the two K-steps of q . A~.
template <int NW>
__device__ __forceinline__ void it_rows(const ItTables& tb, int sb, bf16x8 qf0, bf16x8 qf1, int c16,
                                        int g, floatx4 (&zw)[NW]) {
  bf16x8 af[2][NW];
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int r4 = sb + 16 * w + 4 * g;
    zw[w] = __builtin_bit_cast(floatx4, bload16(tb.bt, r4 >= 0 ? static_cast<uint32_t>(r4) * 4 : kOob));
    const int row = sb + 16 * w + c16;
#pragma unroll
    for (int c = 0; c < 2; ++c)
      af[c][w] = __builtin_bit_cast(
          bf16x8, bload16(tb.at, row >= 0 ? static_cast<uint32_t>(row * 64 + 32 * c + 8 * g) * 2 : kOob));
  }
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int w = 0; w < NW; ++w)
      zw[w] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[c][w], c ? qf1 : qf0, zw[w], 0, 0, 0);
}

// The rows into the wave's scratch scr[query c16][s'] (pitch P).
template <int NW>
__device__ __forceinline__ void it_put(float* scr, int P, int c16, int g, const floatx4 (&zw)[NW]) {
#pragma unroll
  for (int w = 0; w < NW; ++w) *reinterpret_cast<floatx4*>(scr + c16 * P + 16 * w + 4 * g) = zw[w];
}

}  // namespace relpos
