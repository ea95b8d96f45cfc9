// Segment masks and attention dropout for the attention kernels ([RPA]
// appendix "Masks, packing, and dropout": padding masks, packed
// variable-length sequences, and dropout drawn from a counter-based generator
// inside the kernels so that the backward regenerates the forward's mask).
// [RPA] = "Fast and Exact Relative-Position Attention via Structure-Aware
// Kernels" (arXiv 2611.01182).
//
// Segments.  seg[b, t] = (start, end): token t of batch row b lies in the
// segment [start, end) of that row and a pair (i, j) is visible iff j lies
// in i's segment (then i lies in j's).  A padding token has an empty segment
// (start = end).  One segment [0, L) per row is a padding mask of length L;
// several per row are packed sequences.  Offsets stay delta = i - j.
//
// Dropout.  Philox4x32 with 10 rounds (Salmon, Moraes, Dror, Shaw, "Parallel
// random numbers: as easy as 1, 2, 3", SC 2011) keyed by the 64-bit seed.
// Counter (j >> 2, i >> 2, b H + h, 0) gives four words for the 4 x 4 block of
// pairs holding (i, j); byte (j & 3) of word (i & 3) is the pair's uniform
// byte, kept iff >= p8 (drop probability p8 / 256), and kept probabilities are
// multiplied by 256 / (256 - p8).  A lane holding four consecutive keys of
// one query (forward, query pass) reads one word; a lane holding four
// consecutive queries of one key (key pass) reads one byte of each word.
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace relpos {

struct Philox4 {
  uint32_t x[4];
};

__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                                 uint32_t c3, uint32_t k0, uint32_t k1) {
  constexpr uint32_t kM0 = 0xD2511F53u, kM1 = 0xCD9E8D57u;
  constexpr uint32_t kW0 = 0x9E3779B9u, kW1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint32_t hi0 = __umulhi(kM0, c0), lo0 = kM0 * c0;
    const uint32_t hi1 = __umulhi(kM1, c2), lo1 = kM1 * c2;
    const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
    k0 += kW0;
    k1 += kW1;
  }
  return Philox4{{c0, c1, c2, c3}};
}

// Keep factors (0, or `kept`: the keep scale, or 1 where the scale is applied
// to a finished fp32 sum instead of to a bf16 MFMA operand, which it would
// round) of pairs (i, j1 + t), t = 0..3, with j1 a multiple of 4: byte t of
// word (i & 3).
__device__ __forceinline__ void keep_row4(const AttnArgs& a, int bh, int i, int j1, float kept,
                                          float* m) {
  const Philox4 w = philox4x32_10(static_cast<uint32_t>(j1) >> 2, static_cast<uint32_t>(i) >> 2,
                                  static_cast<uint32_t>(bh), 0u, a.seed_lo, a.seed_hi);
  // (selects, not an indexed read: a private array indexed at run time
  // would live in scratch memory)
  const int r = i & 3;
  const uint32_t word = r == 0 ? w.x[0] : (r == 1 ? w.x[1] : (r == 2 ? w.x[2] : w.x[3]));
#pragma unroll
  for (int t = 0; t < 4; ++t)
    m[t] = static_cast<int>((word >> (8 * t)) & 0xffu) >= a.drop_p8 ? kept : 0.f;
}

// Keep factors of pairs (i1 + t, j), t = 0..3, with i1 a multiple of 4:
// byte (j & 3) of word t (0 or `kept`).
__device__ __forceinline__ void keep_col4(const AttnArgs& a, int bh, int i1, int j, float kept,
                                          float* m) {
  const Philox4 w = philox4x32_10(static_cast<uint32_t>(j) >> 2, static_cast<uint32_t>(i1) >> 2,
                                  static_cast<uint32_t>(bh), 0u, a.seed_lo, a.seed_hi);
  const int sh = 8 * (j & 3);
#pragma unroll
  for (int t = 0; t < 4; ++t)
    m[t] = static_cast<int>((w.x[t] >> sh) & 0xffu) >= a.drop_p8 ? kept : 0.f;
}

__device__ __forceinline__ int wave_min_i(int v) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v = imin(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ int wave_max_i(int v) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v = imax(v, __shfl_xor(v, o));
  return v;
}

// Segment bounds [lo, hi) of token t of batch row brow / N (brow = b N), for
// a kernel with a segment mask (a.seg not null).
__device__ __forceinline__ void token_segment(const AttnArgs& a, int64_t brow, int t, int& lo,
                                              int& hi) {
  const int2 s = *reinterpret_cast<const int2*>(a.seg + 2 * (brow + t));
  lo = s.x;
  hi = s.y;
}

// Ranges of a wave's tokens (each lane one or more; tokens past N or not
// owned are skipped): the union [ulo, uhi) of their segments and the
// intersection [ilo, ihi) (empty when a padding token, whose segment is
// empty, is among them).  A tile inside the intersection needs no
// per-pair segment test; a tile outside the union holds no visible pair.
struct SegWave {
  int ulo, uhi, ilo, ihi;
};

__device__ __forceinline__ SegWave seg_wave(const int* lo, const int* hi, const bool* on, int n) {
  int ulo = 0x7fffffff, uhi = -0x7fffffff, ilo = -0x7fffffff, ihi = 0x7fffffff;
  for (int k = 0; k < n; ++k) {
    if (!on[k]) continue;
    if (hi[k] > lo[k]) {
      ulo = imin(ulo, lo[k]);
      uhi = imax(uhi, hi[k]);
    }
    ilo = imax(ilo, lo[k]);
    ihi = imin(ihi, hi[k]);
  }
  // (the reduced values are equal in every lane; readfirstlane makes that
  // known to the compiler, so tests on them are scalar branches)
  return SegWave{__builtin_amdgcn_readfirstlane(wave_min_i(ulo)),
                 __builtin_amdgcn_readfirstlane(wave_max_i(uhi)),
                 __builtin_amdgcn_readfirstlane(wave_max_i(ilo)),
                 __builtin_amdgcn_readfirstlane(wave_min_i(ihi))};
}

// Union of the four waves' unions through `sh` (int[2][4] in LDS), between
// two barriers that every thread of the workgroup reaches.
__device__ __forceinline__ void seg_block(const SegWave& w, int wave, int (*sh)[4], int& blo,
                                          int& bhi) {
  if ((threadIdx.x & 63) == 0) {
    sh[0][wave] = w.ulo;
    sh[1][wave] = w.uhi;
  }
  __syncthreads();
  blo = imin(imin(sh[0][0], sh[0][1]), imin(sh[0][2], sh[0][3]));
  bhi = imax(imax(sh[1][0], sh[1][1]), imax(sh[1][2], sh[1][3]));
  __syncthreads();
}

}  // namespace relpos
