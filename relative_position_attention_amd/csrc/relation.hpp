// Relation terms of one score tile, for the two lane layouts of the
// attention kernels.  [RPA] = "Fast and Exact Relative-Position Attention via
// Structure-Aware Kernels" (arXiv 2611.01182).
//
// Offset-aware tiles ([RPA] §4.1 "Constant-Range Reuse", §4.3.1, App. B.2
// saturated-tile lemma): a tile whose offsets all satisfy delta >= D
// (SAT_HI) or delta <= -D (SAT_LO) reads one precomputed entry per query and
// one per key; only BAND tiles read the per-pair projections.  Every pair
// with |delta| >= D takes the fp32 boundary entries, in every kind of tile, so
// the value of a score does not depend on how its tile was classified (the
// forward and both backward passes classify tiles differently).
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace relpos {

enum Region { SAT_HI = 0, BAND = 1, SAT_LO = 2 };

// Query-row layout (forward and query-parallel pass): the lane owns query row
// i; its registers hold keys j1..j1+3.  Adds the relation terms (score units,
// before the scale) of those four pairs to acc[0..3].
template <typename T, int F, int REG>
__device__ __forceinline__ void relation_qrow(const AttnArgs& a, int64_t tok, int h, int i,
                                              float rlo, float rhi, const GroupInfo& giq,
                                              const GroupInfo& gik, int gk0, int j1,
                                              float* acc) {
  using ZT = typename Store<T>::Z;
  const int N = a.N, D = a.D;
  float kl[4], kh[4], km[4];
  if (REG == SAT_HI) {
    load4_guard(a.keyhi + tok, j1, N, kh);
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] += rhi + kh[t];
    return;
  }
  if (REG == SAT_LO) {
    load4_guard(a.keylo + tok, j1, N, kl);
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] += rlo + kl[t];
    return;
  }
  load4_guard(a.keyhi + tok, j1, N, kh);
  load4_guard(a.keylo + tok, j1, N, kl);
  load4_guard(a.keymid + tok, j1, N, km);
  float zq[4] = {0.f, 0.f, 0.f, 0.f};
  if ((F & F_ZQ) && i < N) {
    const ZT* row = reinterpret_cast<const ZT*>(a.zq) + tok / N * a.zq_bh + giq.base +
                    static_cast<int64_t>(i - (i / kGroup) * kGroup) * giq.pitch;
    int c0 = (i - (j1 + 3) + D) - giq.slo + giq.pad;
    float m[4];
    load4(row + clamp_run(c0, giq.pitch), m);
#pragma unroll
    for (int t = 0; t < 4; ++t) zq[t] = m[3 - t];  // descending columns
  }
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int j = j1 + t;
    const int dl = i - j;
    float band = km[t] + zq[t];
    if (F & F_ZK) {
      if (j < N) {
        const ZT* zk = reinterpret_cast<const ZT*>(a.zk) + tok / N * a.zk_bh + gik.base +
                       static_cast<int64_t>(j - gk0) * gik.pitch;
        int c = iclamp((dl + D) - gik.slo + gik.pad, 0, gik.pitch - 1);
        band += to_f(zk[c]);
      }
    }
    if (F & F_BT) band += a.bt[h * a.S + iclamp(dl + D, 0, 2 * D)];
    acc[t] += dl >= D ? (rhi + kh[t]) : (dl <= -D ? (rlo + kl[t]) : band);
  }
}

// Key-row layout (key-parallel pass): the lane owns key row j; its registers
// hold queries i1..i1+3 with per-query boundary entries rlo4/rhi4.
template <typename T, int F, int REG>
__device__ __forceinline__ void relation_krow(const AttnArgs& a, int64_t tok, int h, int j,
                                              float klo, float khi, float kmid,
                                              const float* rlo4, const float* rhi4,
                                              const GroupInfo& giq, int gq0,
                                              const GroupInfo& gik, int i1, float* acc) {
  using ZT = typename Store<T>::Z;
  const int N = a.N, D = a.D;
  if (REG == SAT_HI) {
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] += rhi4[t] + khi;
    return;
  }
  if (REG == SAT_LO) {
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] += rlo4[t] + klo;
    return;
  }
  float zk[4] = {0.f, 0.f, 0.f, 0.f};
  if ((F & F_ZK) && j < N) {
    const ZT* row = reinterpret_cast<const ZT*>(a.zk) + tok / N * a.zk_bh + gik.base +
                    static_cast<int64_t>(j - (j / kGroup) * kGroup) * gik.pitch;
    int c0 = (i1 - j + D) - gik.slo + gik.pad;
    load4(row + clamp_run(c0, gik.pitch), zk);  // ascending columns
  }
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int i = i1 + t;
    const int dl = i - j;
    float band = kmid + zk[t];
    if (F & F_ZQ) {
      if (i < N) {
        const ZT* zq = reinterpret_cast<const ZT*>(a.zq) + tok / N * a.zq_bh + giq.base +
                       static_cast<int64_t>(i - gq0) * giq.pitch;
        int c = iclamp((dl + D) - giq.slo + giq.pad, 0, giq.pitch - 1);
        band += to_f(zq[c]);
      }
    }
    if (F & F_BT) band += a.bt[h * a.S + iclamp(dl + D, 0, 2 * D)];
    acc[t] += dl >= D ? (rhi4[t] + khi) : (dl <= -D ? (rlo4[t] + klo) : band);
  }
}

}  // namespace relpos
