// Layout constants and index formulas shared by the host plan and the kernels.
//
// [RPA] = "Fast and Exact Relative-Position Attention via Structure-Aware
// Kernels" (arXiv 2611.01182).
//
// Expanded offsets.  With saturation radius D, every pair (i, j) has offset
// delta = i - j and expanded row s = clip(delta, -D, D) + D in [0, 2D]
// ([RPA] App. B.1, bucket-copy lemma: the bucketed map becomes a clipping
// map over 2D+1 copied rows).  Rows 0 and 2D are the saturated ones.
//
// Projection rows ([RPA] §4.1 "Reachable Projection Ranges", App. B.2
// reachable-range lemma).  Queries are split in groups of G = 128; a group
// reaches one interval [slo, shi] of expanded rows.  Row i of group g stores
// Z[i, s] at element  base_g + (i - gG) * pitch_g + (s - slo_g + pad_g)
// inside its (batch, head) slice.  The same layout holds the offset
// gradients dZ~ of the backward pass.
//
//  * Query side: pitch = 7 (mod 8).  Then the element address of Z[i, i-j+D]
//    is (pitch+1)(i-gG) - j + const: for four consecutive keys j1..j1+3
//    (j1 = 0 mod 4) the entries are four consecutive elements (descending),
//    and pad_g makes their first element 4-aligned for every row i.  A lane
//    that owns one query row reads or writes them with one 8-byte access.
//  * Key side: pitch = 1 (mod 8): for a key row j and four consecutive
//    queries i1..i1+3 the entries Z^K[j, i-j+D] are four consecutive
//    (ascending) elements, 4-aligned.
//  * pad >= 8 and pitch >= pad + width + 4 leave margins of at least three
//    elements on both sides of every row, so such a 4-run that holds at
//    least one reachable entry never leaves its row.
//  * The pads also make longer runs 16-byte aligned: on the query side the 64
//    entries of one query row and one 64-key tile (j0 = 0 mod 64), on the key
//    side the 128 entries of one key row and one 128-query block, start on an
//    8-element boundary (the kernels stage them into LDS with 16-byte loads).
#pragma once

#include <cstdint>

#ifdef __HIPCC__
#include <hip/hip_runtime.h>
#define RP_HD __host__ __device__ __forceinline__
#else
#define RP_HD inline
#endif

namespace relpos {

constexpr int kHeadDim = 64;
constexpr int kGroup = 128;  // G of [RPA] §4.3.1 (queries per projection group)

struct GroupInfo {
  int32_t slo;    // first expanded row of the group's window
  int32_t pad;    // column of slo inside a row
  int32_t pitch;  // elements per row
  int32_t base;   // element offset of the group's first row in the slice
};

RP_HD int imin(int a, int b) { return a < b ? a : b; }
RP_HD int imax(int a, int b) { return a > b ? a : b; }
RP_HD int iclamp(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// Expanded rows reachable by query row i: offsets delta = i - j over the
// visible keys j (all j < N, or j <= i when causal).
RP_HD void query_s_range(int i, int N, int D, bool causal, int& smin, int& smax) {
  int dmin = causal ? 0 : i - (N - 1);
  int dmax = i;
  smin = iclamp(dmin, -D, D) + D;
  smax = iclamp(dmax, -D, D) + D;
}

// Expanded rows reachable by key row j: delta = i - j over visible queries.
RP_HD void key_s_range(int j, int N, int D, bool causal, int& smin, int& smax) {
  int dmin = causal ? 0 : -j;
  int dmax = (N - 1) - j;
  smin = iclamp(dmin, -D, D) + D;
  smax = iclamp(dmax, -D, D) + D;
}

// Window of query group g: union over its rows.
RP_HD void query_group_window(int g, int N, int D, bool causal, int& slo, int& shi) {
  int first = g * kGroup;
  int last = imin(N - 1, first + kGroup - 1);
  int a, b, c, d;
  query_s_range(first, N, D, causal, a, b);
  query_s_range(last, N, D, causal, c, d);
  slo = imin(a, c);
  shi = imax(b, d);
}

RP_HD void key_group_window(int g, int N, int D, bool causal, int& slo, int& shi) {
  int first = g * kGroup;
  int last = imin(N - 1, first + kGroup - 1);
  int a, b, c, d;
  key_s_range(first, N, D, causal, a, b);
  key_s_range(last, N, D, causal, c, d);
  slo = imin(a, c);
  shi = imax(b, d);
}

RP_HD int mod4(int x) { return ((x % 4) + 4) % 4; }

RP_HD int mod8(int x) { return ((x % 8) + 8) % 8; }

// Column pads making the 4-runs and the tile runs aligned (see the header
// comment); base and gG are multiples of 8.
RP_HD int query_pad(int slo, int D) { return 8 + mod8(7 - D + slo); }
RP_HD int key_pad(int slo, int D) { return 8 + mod8(slo - D); }

// Smallest pitch >= need with pitch = r (mod 8).
RP_HD int pitch_mod8(int need, int r) { return need + ((r - need) % 8 + 8) % 8; }

// Clamp a 4-run start column into [0, pitch - 4] keeping its residue mod 4,
// so the clamped access stays aligned and inside the row.
RP_HD int clamp_run(int c, int pitch) {
  if (c < 0) return c & 3;
  int hi = pitch - 4;
  if (c > hi) return c - ((c - hi + 3) & ~3);
  return c;
}

}  // namespace relpos
