// Forward attention kernel for bf16 inputs ([RPA] Table 9 "Attention"; the
// forward of Algorithm 1).  [RPA] = "Fast and Exact Relative-Position
// Attention via Structure-Aware Kernels" (arXiv 2611.01182).
//
// Layout.  A workgroup of 4 waves owns 128 consecutive queries (one
// projection group); each wave owns 32 of them (two 16-query blocks), which
// keeps a wave within 168 registers so three workgroups share a CU (two
// with a key table, causal pairing or in-tile products) and the MFMA work
// of some waves overlaps the softmax of others.  Key tiles of 64
// keys stream through LDS, double buffered: K and V row-major (the V^T
// operand of P V is read with the gfx950 transposing LDS read), and (when a
// per-key relation term exists) the tile's per-key boundary entries.
// All global reads are buffer loads: 32-bit offsets, and reads past a slice
// return zero, so no lane branches on bounds.  Per tile and wave:
//   S^T = K Q^T on 16x16x32 bf16 MFMA (each lane owns one query column and
//   four consecutive keys per 16-key block);
//   relation terms by tile region: a tile whose offsets delta = i - j all
//   satisfy delta >= D or delta <= -D is saturated and adds one fp32 entry per
//   query (folded into the exponent's offset) and one per key (the initial
//   value of the S accumulator); band tiles
//   read the per-pair projections Z ([RPA] §4.1, App. B saturated-tile lemma),
//   which without causal pairing are the S accumulator's initial value too
//   (with it, and for in-tile products, they are added after the products).
//   Every pair with |delta| >= D takes the boundary entries whatever its tile,
//   exactly as the backward passes do.
//   Online softmax in base 2 with tau log2(e) folded into one FMA ([RPA]
//   "Half-precision numerics"; [RPA] §3.1 Eq. (2)).  The running maximum is
//   raised lazily: only when a tile's maximum exceeds it by more than 8
//   (a factor 256) are O and the row sum rescaled; the result is the same
//   exact quotient.
//   O^T += V^T P^T on MFMA with P in registers (bf16, or a bf16 hi + lo pair
//   under F_SPLIT); the row sums of P are one more MFMA with a ones operand
//   (two under F_SPLIT, one per part).
// The region of each tile is decided per wave from the wave's extreme offsets
// before the loop (the three ranges of [RPA] §4.3.3).
// F_SEG adds segment masks (the key-tile loop covers the union of the
// workgroup's segments; per-pair tests on tiles not inside every query's
// segment), F_DROP dropout (P V takes P times the pair's 0/1 keep mask and O
// the keep scale; the row sums, hence L, keep P itself; segments are then
// taken when given), as defined in extras.hpp.
// F_IT computes the band tiles' Z^Q entries in the tile (intile.hpp)
// instead of reading stored projections.
#pragma once
#include "extras.hpp"
#include "intile.hpp"
#include "relation.hpp"
#include "tiles.hpp"

namespace relpos {

namespace {

constexpr int QB = 2;              // 16-query blocks per wave
constexpr int kWQ = 16 * QB;       // queries per wave
constexpr int kBM = 4 * kWQ;       // queries per workgroup
constexpr int kKP = 80;            // K and V tile pitch (bf16): 160-byte rows (bank-conflict free)
constexpr float kLazy = 8.f;       // rescale threshold, log2 units
constexpr int kZwP = 84;           // in-tile scratch pitch (fp32): 80 window rows
// an MFMA A operand whose 16 rows are all ones (bf16 1.0 = 0x3f80)
#define kOnes8 (__builtin_bit_cast(bf16x8, uint4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u}))

template <int F>
__global__ __launch_bounds__(256, ((F & F_ZK) || (F & F_CAUSAL) || (F & F_U) || (F & F_DROP) || (F & F_IT) ||
                                                  ((F & F_SEG) && (F & F_BT))) ? 2 : 3) void attn_fwd_fast(AttnArgs a, int nqb, int total,
                                                          int xcd_map) {
  constexpr bool CAUSAL = (F & F_CAUSAL) != 0;
  constexpr bool SPLIT = (F & F_SPLIT) != 0;
  constexpr bool EXT = (F & (F_SEG | F_DROP)) != 0;
  constexpr bool IT = (F & F_IT) != 0;
  // raised wave priority around the matrix products (measured at N = 8192:
  // up to 3% faster, never slower, on the four mechanisms)
  constexpr bool PRIO = !IT;
  // per-key relation entries: with a key table (F_ZK) the band value and the
  // two boundary values differ per key; with only the Transformer-XL u term
  // they are one value u . k_j
  constexpr bool KC = (F & (F_ZK | F_U)) != 0;
  constexpr bool KC3 = (F & F_ZK) != 0;
  // key projections of a band tile are staged into LDS once per workgroup
  constexpr bool STZK = (F & F_ZK) != 0;
  // causal masks: pair each 16-query block with its mirror (below)
  constexpr bool PAIR = CAUSAL && !STZK;
  constexpr int kZP = 136;  // szk pitch (fp16)
  // Z^Q runs of band tiles under causal masks (every tile of an identity map
  // is a band tile) and with a key table (two waves per SIMD leave the
  // registers): issued for all blocks at the top of the step, before the
  // next tile's prefetch, so that waiting for them leaves the prefetch in
  // flight.  Elsewhere band tiles are few and the runs are loaded where used.
  constexpr bool HOIST = (F & F_ZQ) && (CAUSAL || (F & F_ZK));
  __shared__ __attribute__((aligned(16))) _Float16 szk[STZK ? 64 * kZP : 8];
  __shared__ __attribute__((aligned(16))) bf16 sk[2][64 * kKP];
  __shared__ __attribute__((aligned(16))) bf16 sv[2][64 * kKP];
  // per key: boundary entries lo, hi and the band constant (row 3: unread
  // copies, written so that the store needs no branch)
  __shared__ __attribute__((aligned(16))) float skc[2][4][64];
  __shared__ int sseg[2][4];
  // in-tile products: one [16 queries][kZwP] window scratch per wave
  __shared__ __attribute__((aligned(16))) float szw[IT ? 4 * 16 * kZwP : 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = wave_index(), g = lane >> 4, c16 = lane & 15;
  const int N = a.N, D = a.D;

  // Work item.  Non-causal: items are head-major and, with xcd_map, each of
  // the 8 XCDs (which receive workgroups round-robin) gets a contiguous range
  // of items, so the query blocks of one head share one L2.  Causal: longest
  // query blocks first.
  int item = static_cast<int>(blockIdx.x);
  if (xcd_map) {
    const int q8 = total / 8, r8 = total % 8;
    const int x = item % 8, slot = item / 8;
    item = (x < r8 ? x * (q8 + 1) : r8 * (q8 + 1) + (x - r8) * q8) + slot;
  }
  const int BH = total / nqb;
  int bh, qblk;
  if (CAUSAL) {
    qblk = PAIR ? item / BH : nqb - 1 - item / BH;
    bh = item % BH;
  } else {
    bh = item / nqb;
    qblk = item % nqb;
  }
  const int h = bh % a.H;
  const int64_t tok = static_cast<int64_t>(bh) * N;
  // The wave's queries: QB blocks of 16 starting at qbase[qb].  Without PAIR
  // they are consecutive (the workgroup owns kBM consecutive queries).  With
  // PAIR (causal masks) wave w of workgroup m owns 16-query block
  // kL = 4m + w and its mirror kH = n16 - 1 - kL: a causal block reaches keys
  // up to its own position, so every wave then has the same work (a lone
  // middle block is taken as block 1).
  static_assert(!PAIR || QB == 2, "pairing takes two 16-query blocks per wave");
  int qbase[QB];
  bool qon[QB];
  int i0, nkt;
  if (PAIR) {
    const int n16 = (N + 15) / 16;
    const int kL = 4 * qblk + wave, kH = n16 - 1 - kL;
    qbase[0] = 16 * kL;
    qbase[QB - 1] = 16 * kH;
    qon[0] = kL < kH;
    qon[QB - 1] = kL <= kH;
    i0 = 0;
    const int kH0 = n16 - 1 - 4 * qblk;  // the workgroup's widest block
    nkt = imin(N - 1, 16 * kH0 + 15) / 64 + 1;
  } else {
    i0 = qblk * kBM;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      qbase[qb] = i0 + kWQ * wave + 16 * qb;
      qon[qb] = true;
    }
    const int ilast_b = imin(N - 1, i0 + kBM - 1);
    nkt = CAUSAL ? (ilast_b / 64 + 1) : (N + 63) / 64;
  }
  const float sl2 = a.scale_log2;
  const uint64_t slice_bytes = static_cast<uint64_t>(N) * 128;
  const Rsrc rq = make_rsrc(reinterpret_cast<const bf16*>(a.q) + tok * 64, slice_bytes);
  const Rsrc rk = make_rsrc(reinterpret_cast<const bf16*>(a.k) + tok * 64, slice_bytes);
  const Rsrc rv = make_rsrc(reinterpret_cast<const bf16*>(a.v) + tok * 64, slice_bytes);

  // queries of this lane: qbase[qb] + c16 (rows past N load as zero)
  bf16x8 qf[QB][2];
  float rlo[QB], rhi[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int i = qbase[qb] + c16;
#pragma unroll
    for (int c = 0; c < 2; ++c)
      qf[qb][c] = __builtin_bit_cast(bf16x8, bload16(rq, static_cast<uint32_t>(i * 128 + 64 * c + 16 * g)));
    const bool ok = i < N && qon[qb];
    rlo[qb] = ok ? a.rowlo[tok + i] : 0.f;
    rhi[qb] = ok ? a.rowhi[tok + i] : 0.f;
  }
  // projection group of each block (a 16-query block lies in one group;
  // without PAIR all of the wave's blocks share one)
  GroupInfo giq[QB];
  int gq0[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qg = qbase[PAIR ? qb : 0] / kGroup;
    gq0[qb] = qg * kGroup;
    giq[qb] = GroupInfo{0, 0, 0, 0};
    if ((F & F_ZQ) && qon[qb]) giq[qb] = a.gq[qg];
  }
  Rsrc rzq = rq, rzk = rq, rbt = rq;
  if (F & F_ZQ)
    rzq = make_rsrc(reinterpret_cast<const _Float16*>(a.zq) + bh * a.zq_bh,
                    static_cast<uint64_t>(a.zq_bh) * 2);
  if (F & F_ZK)
    rzk = make_rsrc(reinterpret_cast<const _Float16*>(a.zk) + bh * a.zk_bh,
                    static_cast<uint64_t>(a.zk_bh) * 2);
  if (F & F_BT) rbt = make_rsrc(a.bt + static_cast<int64_t>(h) * a.S, static_cast<uint64_t>(a.S) * 4);
  ItTables itb;
  if (IT) itb = it_tables(a, h);
  float* const scr = szw + (IT ? wave * 16 * kZwP : 0);

  // key tiles of each block: [0, nkq) visible; region bounds from the
  // block's extreme offsets: tiles [0, n_hi) have delta >= D for every pair,
  // tiles [t_lo, nkq) have delta <= -D (without PAIR every block uses the
  // wave's range)
  int nkq[QB], n_hi[QB], t_lo[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qa = qbase[PAIR ? qb : 0], qz = qbase[PAIR ? qb : QB - 1] + 15;
    nkq[qb] = !qon[qb] ? 0 : (CAUSAL ? imin(nkt, imin(N - 1, qz) / 64 + 1) : nkt);
    const int nh = (qa - D - 63 >= 0) ? (qa - D - 63) / 64 + 1 : 0;
    n_hi[qb] = imin(nh, nkq[qb]);
    const int tl = CAUSAL ? nkq[qb] : (qz + D + 63) / 64;
    t_lo[qb] = imax(n_hi[qb], imin(tl, nkq[qb]));
  }
  const int nkt_w = nkq[QB - 1];  // the last block reaches the most tiles

  // segment masks: each query's segment, the wave's union and intersection,
  // and the workgroup's key tiles [kt_begin, kt_end) (those holding a key of
  // some query's segment)
  const bool SEG = (F & F_SEG) != 0 && a.seg != nullptr;
  const bool DROP = (F & F_DROP) != 0 && a.drop_p8 > 0;
  // (defined on every path: the per-pair tests read them only when SEG)
  int sgl[QB], sgh[QB];
#pragma unroll
  for (int x = 0; x < QB; ++x) {
    sgl[x] = 0;
    sgh[x] = N;
  }
  SegWave sw = {0, N, 0, N};
  int kt_begin = 0, kt_end = nkt;
  if (SEG) {
    bool on[QB];
    const int64_t brow = static_cast<int64_t>(bh / a.H) * N;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int i = qbase[qb] + c16;
      on[qb] = i < N && qon[qb];
      sgl[qb] = sgh[qb] = 0;
      if (on[qb]) token_segment(a, brow, i, sgl[qb], sgh[qb]);
    }
    sw = seg_wave(sgl, sgh, on, QB);
    int blo, bhi;
    seg_block(sw, wave, sseg, blo, bhi);
    kt_begin = blo < bhi ? blo / 64 : 0;
    kt_end = blo < bhi ? imin(nkt, (bhi + 63) / 64) : 0;
  }

  float mu[QB], l[QB];
  floatx4 o[QB][4];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    mu[qb] = -INFINITY;
    l[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < 4; ++db) o[qb][db] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  // tile staging: K and V rows (t>>3) and 32 + (t>>3), chunk t&7, and one
  // per-key value per thread (value tid >> 6 of key tid & 63).  Every load is
  // issued unconditionally (rows past N read zero, indexes are clamped), so
  // each wave issues the same vector loads on every path and the compiler's
  // wait counts stay exact.
  const int kr = tid >> 3, kc8 = (tid & 7) * 8;
  uint4 tk[2], tv[2];
  float tkc = 0.f;
  const int kcx = tid >> 6, kcj = tid & 63;
  const float* const kbase = (KC3 && kcx == 0) ? a.keylo : ((KC3 && kcx == 1) ? a.keyhi : a.keymid);
  auto load_tile = [&](int j0) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      tk[u] = bload16(rk, static_cast<uint32_t>((j0 + kr + 32 * u) * 128 + kc8 * 2));
      tv[u] = bload16(rv, static_cast<uint32_t>((j0 + kr + 32 * u) * 128 + kc8 * 2));
    }
    if (KC) tkc = kbase[tok + imin(j0 + kcj, N - 1)];
  };
  auto store_tile = [&](int buf, int j0) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      *reinterpret_cast<uint4*>(&sk[buf][(kr + 32 * u) * kKP + kc8]) = tk[u];
      *reinterpret_cast<uint4*>(&sv[buf][(kr + 32 * u) * kKP + kc8]) = tv[u];
    }
    if (KC) skc[buf][kcx][kcj] = j0 + kcj < N ? tkc : 0.f;
  };

  load_tile(64 * kt_begin);
  store_tile(0, 64 * kt_begin);
  wait_vm_all();
  __syncthreads();

  for (int kt = kt_begin; kt < kt_end; ++kt) {
    const int buf = (kt - kt_begin) & 1;
    const int j0 = kt * 64;
    if (STZK) {
      // band for some wave of the workgroup: stage Z^K of the tile's keys
      // (before the next tile's prefetch is issued, so the staging's waits
      // do not cover it; the group record comes through the scalar cache)
      const bool blk_sat = (i0 - (j0 + 63) >= D) || (i0 + kBM - 1 - j0 <= -D);
      if (!blk_sat && j0 < N) {
        const GroupInfo gk = sload_uniform16(a.gk + j0 / kGroup);
        stage_zk_rows(rzk, gk.base, gk.slo, gk.pad, gk.pitch, (j0 / kGroup) * kGroup, j0, i0, D,
                      szk, kZP);
        __syncthreads();
      }
    }
    // Z^Q runs of this tile's band blocks, then the next tile's prefetch: in
    // this order the wait for the runs leaves the prefetch in flight, and the
    // runs of all blocks are in flight together.  Lane (c16, g) of block qb
    // reads Z^Q[i][i - j1 - t + D], t = 0..3, i = qbase + c16,
    // j1 = j0 + 16 kb + 4g (a run in descending column order).
    uint2 zqr[QB][4];
    // (with a key table most tiles are saturated: the runs are requested
    // only on tiles where some block is in the band, a uniform branch)
    bool anyband = !STZK;
    if (STZK) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        anyband = anyband || (kt < nkt_w && !(kt < n_hi[qb] || kt >= t_lo[qb]));
    }
    if (HOIST && anyband) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const bool bandq = kt < nkt_w && (PAIR ? kt < nkq[qb] : true) &&
                           !(kt < n_hi[qb] || kt >= t_lo[qb]);
        const int i = qbase[qb] + c16;
        const bool iok = bandq && i < N;
        const int zrow = giq[qb].base + (i - gq0[qb]) * giq[qb].pitch;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const int j1 = j0 + 16 * kb + 4 * g;
          const int c0 = clamp_run((i - (j1 + 3) + D) - giq[qb].slo + giq[qb].pad, giq[qb].pitch);
          zqr[qb][kb] = bload8(rzq, iok ? static_cast<uint32_t>((zrow + c0) * 2) : kOob);
        }
      }
    }
    if (HOIST) __builtin_amdgcn_sched_barrier(0);
    load_tile(j0 + 64);

    if (kt < nkt_w && (!SEG || (j0 < sw.uhi && j0 + 64 > sw.ulo))) {
      const bf16* Ks = sk[buf];
      const bf16* Vs = sv[buf];
      // per block (uniform): does the tile reach it, and its region (1:
      // delta >= D, row 2D; 0: delta <= -D); on saturated tiles the key's
      // boundary entry is the initial value of the S accumulator.  A block
      // the tile does not reach is block 0 (the last block is the widest).
      bool act[QB], sat[QB];
      int side[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        act[qb] = PAIR ? kt < nkq[qb] : true;
        sat[qb] = kt < n_hi[qb] || kt >= t_lo[qb];
        side[qb] = kt < n_hi[qb] ? 1 : 0;
      }
      floatx4 s[QB][4];
      // the saturated tiles' initial value of the S accumulator: the key's
      // boundary entry (with per-key entries), else zero
      auto sat_init = [&]() {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          if (!PAIR) {
            floatx4 kx = floatx4{0.f, 0.f, 0.f, 0.f};
            if (KC && sat[0])
              kx = *reinterpret_cast<const floatx4*>(&skc[buf][KC3 ? side[0] : 2][16 * kb + 4 * g]);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) s[qb][kb] = kx;
          } else {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
              floatx4 kx = floatx4{0.f, 0.f, 0.f, 0.f};
              if (KC && sat[qb])
                kx = *reinterpret_cast<const floatx4*>(&skc[buf][KC3 ? side[qb] : 2][16 * kb + 4 * g]);
              s[qb][kb] = kx;
            }
          }
        }
      };
      // S^T = K Q^T added to the accumulator's initial value
      auto products = [&]() {
        prio_matrix<PRIO>();
#pragma unroll
        for (int c = 0; c < 2; ++c) {
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            const bf16x8 kf = *reinterpret_cast<const bf16x8*>(Ks + (16 * kb + c16) * kKP + 32 * c + 8 * g);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
              if (qb == 0 && !act[0]) continue;
              s[qb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[qb][c], s[qb][kb], 0, 0, 0);
            }
          }
        }
        prio_normal<PRIO>();
      };
      // ---- relation terms: s becomes S plus the per-pair terms (score
      // units); off[qb] is the row's constant term (scaled) on saturated tiles
      float off[QB];
      // band tile: per-pair terms; pairs with |delta| >= D take the boundary
      // entries (PURE: the tile holds no such pair, as every tile of an
      // identity map does, and the selects are skipped)
      auto band_terms = [&](int qb, auto PURE, auto ASSIGN) {
        const int i = qbase[qb] + c16;
        const bool iok = i < N;
        const int zrow = giq[qb].base + (i - gq0[qb]) * giq[qb].pitch;
        if constexpr (IT) {
          // the block's 80-row window on MFMA, into the wave's scratch
          floatx4 zw[5];
          it_rows<5>(itb, qbase[qb] - j0 - 63 + D, qf[qb][0], qf[qb][1], c16, g, zw);
          it_put<5>(scr, kZwP, c16, g, zw);
        }
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const int j1 = j0 + 16 * kb + 4 * g;
          float zq[4] = {0.f, 0.f, 0.f, 0.f};
          if constexpr (IT) {
            // pair (i, j1 + t) at window row c16 + 63 - 16 kb - 4 g - t
            const float* zr = scr + c16 * kZwP + c16 + 60 - 16 * kb - 4 * g;
#pragma unroll
            for (int t = 0; t < 4; ++t) zq[t] = zr[3 - t];
          }
          if (F & F_ZQ) {
            uint2 w;
            if (HOIST) {
              w = zqr[qb][kb];
            } else {
              const int c0 = clamp_run((i - (j1 + 3) + D) - giq[qb].slo + giq[qb].pad, giq[qb].pitch);
              w = bload8(rzq, iok ? static_cast<uint32_t>((zrow + c0) * 2) : kOob);
            }
            const halfx4 hv = __builtin_bit_cast(halfx4, w);
#pragma unroll
            for (int t = 0; t < 4; ++t) zq[t] = static_cast<float>(hv[3 - t]);  // descending
          }
          floatx4 km = floatx4{0.f, 0.f, 0.f, 0.f}, klo4 = km, khi4 = km;
          if (KC) km = *reinterpret_cast<const floatx4*>(&skc[buf][2][16 * kb + 4 * g]);
          if (KC3 && !PURE) {
            klo4 = *reinterpret_cast<const floatx4*>(&skc[buf][0][16 * kb + 4 * g]);
            khi4 = *reinterpret_cast<const floatx4*>(&skc[buf][1][16 * kb + 4 * g]);
          }
          halfx4 zk4 = halfx4{0, 0, 0, 0};
          if (STZK)  // Z^K[j1 + t][i - j1 - t + D], t = 0..3
            zk4 = __builtin_bit_cast(halfx4, lds_tr4(reinterpret_cast<const bf16*>(szk), kZP,
                                                     16 * kb + 4 * g, qbase[qb] - i0, c16));
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int j = j1 + t;
            const int dl = i - j;
            float band = km[t] + zq[t];
            if (F & F_ZK) band += static_cast<float>(zk4[t]);
            if (F & F_BT) band += bloadf(rbt, static_cast<uint32_t>(iclamp(dl + D, 0, 2 * D) * 4));
            float add;
            if constexpr (PURE) {
              add = band;
            } else {
              // boundary pairs: the row's entry plus the key's
              const float kedge = KC3 ? (dl >= D ? khi4[t] : klo4[t]) : km[t];
              add = dl >= D ? (rhi[qb] + kedge) : (dl <= -D ? (rlo[qb] + kedge) : band);
            }
            if constexpr (ASSIGN)
              s[qb][kb][t] = add;
            else
              s[qb][kb][t] += add;
          }
        }
      };
      auto mask_block = [&](int qb) {
        const int i = qbase[qb] + c16;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int j = j0 + 16 * kb + 4 * g + t;
            const bool off_seg = SEG && (j < sgl[qb] || j >= sgh[qb]);
            s[qb][kb][t] = (j >= N || (CAUSAL && j > i) || off_seg) ? -INFINITY : s[qb][kb][t];
          }
      };
      if (!PAIR && !IT) {
        // the wave's blocks share one region and one edge test.  Each branch
        // makes its own products: a band tile's terms are the accumulator's
        // initial value, so both branches leave S in the registers of their
        // own MFMA results (with the terms added after the products, the
        // saturated branch copied every score into the band branch's
        // registers: 3-5% slower)
        if (sat[0]) {
          sat_init();
          products();
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) off[qb] = (side[0] ? rhi[qb] : rlo[qb]) * sl2;
        } else {
          const bool pure = qbase[0] - (j0 + 63) > -D && qbase[QB - 1] + 15 - j0 < D;
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            off[qb] = 0.f;
            if (pure)
              band_terms(qb, std::true_type{}, std::true_type{});
            else
              band_terms(qb, std::false_type{}, std::true_type{});
          }
          products();
        }
        if ((j0 + 64 > N) || (CAUSAL && j0 + 63 > qbase[0]) ||
            (SEG && (j0 < sw.ilo || j0 + 64 > sw.ihi))) {
          // (the empty asm keeps this a branch taken by the edge tiles only)
          asm volatile("");
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) mask_block(qb);
        }
      } else {
        // causal pairing (per-block regions) and in-tile products: the terms
        // are added after the products, as in the backward passes
        sat_init();
        products();
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          off[qb] = 0.f;
          if (!act[qb]) continue;
          if (sat[qb])
            off[qb] = (side[qb] ? rhi[qb] : rlo[qb]) * sl2;
          else if (IT || (qbase[qb] - (j0 + 63) > -D && qbase[qb] + 15 - j0 < D))
            band_terms(qb, std::true_type{}, std::false_type{});
          else
            band_terms(qb, std::false_type{}, std::false_type{});
          if (PAIR && ((j0 + 64 > N) || (j0 + 63 > qbase[qb]) ||
                       (SEG && (j0 < sw.ilo || j0 + 64 > sw.ihi)))) {
            asm volatile("");
            mask_block(qb);
          }
        }
        if (!PAIR && ((j0 + 64 > N) || (CAUSAL && j0 + 63 > qbase[0]) ||
                      (SEG && (j0 < sw.ilo || j0 + 64 > sw.ihi)))) {
          asm volatile("");
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) mask_block(qb);
        }
      }

      // ---- online softmax (base 2, lazy rescale)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        if (!act[qb]) continue;
        float mx = s[qb][0][0];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int t = 0; t < 4; ++t) mx = fmaxf(mx, s[qb][kb][t]);
        mx = wave_max_g(mx);
        const float mxs = mx * sl2 + off[qb];  // scaled tile maximum
        if (mxs > mu[qb] + kLazy) {
          const float alpha = fast_exp2(mu[qb] - mxs);
          mu[qb] = mxs;
          l[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < 4; ++db) o[qb][db] *= alpha;
        }
        // (a segment mask can leave a row without any key so far: its P is 0)
        const float bias = (SEG && mu[qb] == -INFINITY) ? 0.f : off[qb] - mu[qb];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int t = 0; t < 4; ++t) s[qb][kb][t] = fast_exp2(fmaf(s[qb][kb][t], sl2, bias));
      }

      // ---- O^T += V^T P^T (keys in the permuted order of frag_regs); the
      // row sums of P come from the same MFMA with a row of ones for V^T, so
      // they add exactly the bf16 weights that multiply V (with split
      // operands both parts, hi and lo, go through the ones product)
      floatx4 ls[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) ls[qb] = floatx4{0.f, 0.f, 0.f, 0.f};
      prio_matrix<PRIO>();
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        bf16x8 pf[QB], pl[QB], pd[QB], pdl[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          // dropout: keep factors of the lane's query and keys 32 c + 4 g
          // (+ 0..3) and 32 c + 16 + 4 g (+ 0..3)
          float mk[2][4] = {{1.f, 1.f, 1.f, 1.f}, {1.f, 1.f, 1.f, 1.f}};
          // (0 or 1: the keep scale multiplies the finished O in fp32)
          if (DROP) {
            keep_row4(a, bh, qbase[qb] + c16, j0 + 32 * c + 4 * g, 1.f, mk[0]);
            keep_row4(a, bh, qbase[qb] + c16, j0 + 32 * c + 16 + 4 * g, 1.f, mk[1]);
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float x = s[qb][2 * c + (e >> 2)][e & 3];
            pf[qb][e] = static_cast<bf16>(x);
            if (SPLIT) pl[qb][e] = static_cast<bf16>(x - static_cast<float>(pf[qb][e]));
            if constexpr ((F & F_DROP) != 0) {
              const float xd = x * mk[e >> 2][e & 3];
              pd[qb][e] = static_cast<bf16>(xd);
              if (SPLIT) pdl[qb][e] = static_cast<bf16>(xd - static_cast<float>(pd[qb][e]));
            }
          }
        }
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          // V^T rows 16 db + c16, keys 32 c + 4 g + (0..3) and + 16
          const bf16x4 lo = lds_tr4(Vs, kKP, 32 * c + 4 * g, 16 * db, c16);
          const bf16x4 hi = lds_tr4(Vs, kKP, 32 * c + 16 + 4 * g, 16 * db, c16);
          bf16x8 vf;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            vf[e] = lo[e];
            vf[e + 4] = hi[e];
          }
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            if (qb == 0 && !act[0]) continue;
            // (with F_DROP P V takes the dropped probabilities)
            o[qb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, (F & F_DROP) ? pd[qb] : pf[qb], o[qb][db], 0, 0, 0);
            if (SPLIT)
              o[qb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, (F & F_DROP) ? pdl[qb] : pl[qb], o[qb][db], 0, 0, 0);
          }
        }
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          if (qb == 0 && !act[0]) continue;
          ls[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kOnes8, pf[qb], ls[qb], 0, 0, 0);
          if (SPLIT) ls[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kOnes8, pl[qb], ls[qb], 0, 0, 0);
        }
      }
      prio_normal<PRIO>();
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        if (act[qb]) l[qb] += ls[qb][0];
    }

    // buffer buf ^ 1 was last read in iteration kt - 1, which every wave
    // finished before the previous barrier (stored also after the last tile,
    // into the buffer no one reads again)
    store_tile(buf ^ 1, j0 + 64);
    __syncthreads();
  }

#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float ls = l[qb];  // the full row sum in every lane of the column
    const int i = qbase[qb] + c16;
    if (i >= N || !qon[qb]) continue;
    // (a query whose segment is empty has no key: O = 0, L = -inf)
    const float inv = (EXT && !(ls > 0.f)) ? 0.f : (DROP ? a.drop_scale : 1.f) / ls;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      float vals[4] = {o[qb][db][0] * inv, o[qb][db][1] * inv, o[qb][db][2] * inv,
                       o[qb][db][3] * inv};
      store_out4(a.o, (tok + i) * 64 + 16 * db + 4 * g, a.out_f32 != 0, vals);
    }
    if (g == 0) a.lse[tok + i] = (EXT && !(ls > 0.f)) ? -INFINITY : mu[qb] * kLn2 + logf(ls);
  }
}

template <int F>
hipError_t launch_fast(const AttnArgs& a, int B, hipStream_t s) {
  constexpr bool PAIR = (F & F_CAUSAL) && !(F & F_ZK);
  // PAIR: workgroup m owns 16-query blocks 4m .. 4m+3 and their mirrors
  const int n16 = (a.N + 15) / 16;
  const int nqb = PAIR ? ((n16 + 1) / 2 + 3) / 4 : (a.N + kBM - 1) / kBM;
  const int total = nqb * B * a.H;
  const int xcd_map = (F & F_CAUSAL) ? 0 : 1;
  hipLaunchKernelGGL((attn_fwd_fast<F>), dim3(total), dim3(256), 0, s, a, nqb, total, xcd_map);
  return hipGetLastError();
}

template <int SPL>
hipError_t dispatch_fast(int flags, const AttnArgs& a, int B, hipStream_t s) {
  const int f = flags & (F_ZQ | F_ZK | F_BT | F_U | F_CAUSAL);
  switch (f) {
#define RP_CASE(X)                                        \
  case X:                                                 \
    return launch_fast<(X) | SPL>(a, B, s);               \
  case (X) | F_CAUSAL:                                    \
    return launch_fast<(X) | F_CAUSAL | SPL>(a, B, s);
    RP_CASE(0)
    RP_CASE(F_ZQ)
    RP_CASE(F_ZK)
    RP_CASE(F_BT)
    RP_CASE(F_ZQ | F_ZK)
    RP_CASE(F_ZK | F_BT)
    RP_CASE(F_U)
    RP_CASE(F_ZQ | F_U)
    RP_CASE(F_ZK | F_U)
    RP_CASE(F_BT | F_U)
    RP_CASE(F_ZQ | F_ZK | F_U)
    RP_CASE(F_ZK | F_BT | F_U)
#undef RP_CASE
    default:
      return hipErrorInvalidValue;
  }
}

// in-tile products (F_IT): A^Q with or without the u term
template <int SPL>
hipError_t dispatch_it(int flags, const AttnArgs& a, int B, hipStream_t s) {
  switch (flags & (F_IT | F_U | F_CAUSAL)) {
    case F_IT:
      return launch_fast<F_IT | SPL>(a, B, s);
    case F_IT | F_CAUSAL:
      return launch_fast<F_IT | F_CAUSAL | SPL>(a, B, s);
    case F_IT | F_U:
      return launch_fast<F_IT | F_U | SPL>(a, B, s);
    case F_IT | F_U | F_CAUSAL:
      return launch_fast<F_IT | F_U | F_CAUSAL | SPL>(a, B, s);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace

}  // namespace relpos
