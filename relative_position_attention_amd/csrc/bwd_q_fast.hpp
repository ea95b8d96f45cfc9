// Query-parallel backward pass for bf16 inputs ([RPA] Table 9 "Query-parallel
// pass", Algorithm 2).  [RPA] = "Fast and Exact Relative-Position Attention
// via Structure-Aware Kernels" (arXiv 2611.01182).
//
// A workgroup of 4 waves owns 128 queries (one projection group), 32 per
// wave.  Key tiles of 64 keys (K, V row-major; per-key boundary entries)
// stream through double-buffered LDS.  Per tile and wave the pass rebuilds
// the scores as the forward does (same relation terms, same boundary-entry
// rule; the band terms enter as the S accumulator's initial value with a key
// table, else after the products, so without one a band score may differ
// from the forward's in its last bit) and, from the saved logsumexp L and
// D = rowdot(dO, O)
// ([RPA] §3.1 Eq. (3), App. B tile-locality lemma):
//   S^T = K Q^T and dP^T = V dO^T on MFMA (A from LDS rows, B in registers),
//   P = exp2(S tau log2 e - L log2 e), G' = P (dP - D) (the gradient of the
//   scores is G = tau G'; tau multiplies the finished sums instead),
//   dQ^T += K^T G'^T on MFMA (K^T read with the transposing LDS read; G' as
//   bf16, or bf16 hi + lo under F_SPLIT).
// Offset gradients ([RPA] §4.2): a band pair (|delta| < D) writes its G to
// dZ~^Q[i, delta + D] -- one entry per (query, offset), a single writer,
// written as aligned 4-entry runs; pairs with |delta| >= D add into two fp32
// per-query boundary sums kept on chip ("Local Boundary Sums").  No atomics.
// F_SEG adds segment masks (key tiles limited to the union of the
// workgroup's segments, per-pair tests elsewhere), F_DROP dropout (dP takes
// the pair's keep factor: G' = P (dP keep - D); segments are then taken when
// given), as defined in extras.hpp.
// F_IT computes the band tiles' Z^Q entries in the tile and adds the
// relation part of dQ, sum over the window rows of G A~[s], on MFMA in the
// tile (intile.hpp), instead of reading projections and writing dZ~^Q.
#pragma once
#include "extras.hpp"
#include "intile.hpp"
#include "relation.hpp"
#include "tiles.hpp"

namespace relpos {

namespace {

// tile pitch (bf16): 160-byte rows, a 40-dword stride that puts eight
// consecutive rows on distinct 8-bank groups (no bank conflict in the
// transposing reads; 144 bytes had two rows of eight sharing banks)
constexpr int kP = 80;
// in-tile scratch pitch (fp32): 80 window rows, or a G' row with its zero
// margins (32 + 64 + 16 entries)
constexpr int kQwP = 116;

template <int F>
__global__ __launch_bounds__(256, 2) void bwd_q_fast(AttnArgs a, int nqb, int total, int xcd_map) {
  constexpr bool CAUSAL = (F & F_CAUSAL) != 0;
  constexpr bool SPLIT = (F & F_SPLIT) != 0;
  constexpr bool EXT = (F & (F_SEG | F_DROP)) != 0;
  constexpr bool HOISTQ = (F & F_ZQ) && !(F & F_ZK);
  constexpr bool DZ = (F & F_DZQ) != 0;
  constexpr bool KC = (F & (F_ZK | F_U)) != 0;
  constexpr bool KC3 = (F & F_ZK) != 0;
  constexpr bool IT = (F & F_IT) != 0;
  // raised wave priority around the matrix products (measured at N = 8192:
  // up to 7% faster without a key table, 2% slower with one)
  constexpr bool PRIO = !IT && !(F & F_ZK);
  // with a key table, band terms as the initial value of the S accumulator
  // (8% faster: see below); without one the Z^Q runs, then requested before
  // the products, cost more than that saves
  constexpr bool BAND_INIT = (F & F_ZK) != 0;
  // band terms added to the scores as 4-vectors, so that the saturated and
  // band branches merge the scores in register pairs (bias or key table: 2%
  // faster; query table alone: 3% slower, the scalar adds stay)
  constexpr bool VEC_ADD = (F & (F_ZK | F_BT)) != 0;
  using GT = std::conditional_t<(F & F_DZ16) != 0, _Float16,
                                typename DzType<bf16, (F & F_DZ32) != 0>::type>;
  // key projections of a band tile are staged into LDS once per workgroup
  constexpr bool STZK = (F & F_ZK) != 0;
  // causal masks: pair each 16-query block with its mirror (below)
  constexpr bool PAIR = CAUSAL && !STZK;
  constexpr int kZP = 136;  // szk pitch (fp16)
  __shared__ __attribute__((aligned(16))) _Float16 szk[STZK ? 64 * kZP : 8];
  __shared__ __attribute__((aligned(16))) bf16 sk[2][64 * kP];
  __shared__ __attribute__((aligned(16))) bf16 sv[2][64 * kP];
  __shared__ __attribute__((aligned(16))) float skc[2][3][64];
  __shared__ int sseg[2][4];
  // in-tile products: one [16 queries][kQwP] scratch per wave
  __shared__ __attribute__((aligned(16))) float szw[IT ? 4 * 16 * kQwP : 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = wave_index(), g = lane >> 4, c16 = lane & 15;
  const int N = a.N, D = a.D;

  int item = static_cast<int>(blockIdx.x);
  if (xcd_map) {
    const int q8 = total / 8, r8 = total % 8;
    const int x = item % 8, slot = item / 8;
    item = (x < r8 ? x * (q8 + 1) : r8 * (q8 + 1) + (x - r8) * q8) + slot;
  }
  const int BH = total / nqb;
  int bh, qblk;
  if (CAUSAL) {
    qblk = item / BH;
    bh = item % BH;
  } else {
    bh = item / nqb;
    qblk = item % nqb;
  }
  const int h = bh % a.H;
  const int64_t tok = static_cast<int64_t>(bh) * N;
  const float sl2 = a.scale_log2, tau = a.scale;
  const uint64_t slice_bytes = static_cast<uint64_t>(N) * 128;
  const Rsrc rq = make_rsrc(reinterpret_cast<const bf16*>(a.q) + tok * 64, slice_bytes);
  const Rsrc rdo = make_rsrc(reinterpret_cast<const bf16*>(a.dout) + tok * 64, slice_bytes);
  const Rsrc rk = make_rsrc(reinterpret_cast<const bf16*>(a.k) + tok * 64, slice_bytes);
  const Rsrc rv = make_rsrc(reinterpret_cast<const bf16*>(a.v) + tok * 64, slice_bytes);

  // The wave's queries: two blocks of 16 starting at qbase[0], qbase[1].
  // Without PAIR they are consecutive (the workgroup owns 128 consecutive
  // queries, one projection group).  With PAIR (causal masks) wave w of
  // workgroup m owns 16-query block kL = 4m + w and its mirror
  // kH = n16 - 1 - kL: a causal block reaches keys up to its own position,
  // so every wave then has the same work, kL + kH + 2 key blocks of 16
  // (a lone middle block is taken as block 1).
  int qbase[2];
  bool qon[2];
  int i0;  // first query of the workgroup's key-tile range owner (non-PAIR)
  int nkt;
  if (PAIR) {
    const int n16 = (N + 15) / 16;
    const int kL = 4 * qblk + wave, kH = n16 - 1 - kL;
    qbase[0] = 16 * kL;
    qbase[1] = 16 * kH;
    qon[0] = kL < kH;
    qon[1] = kL <= kH;
    i0 = 0;
    // the workgroup's widest block is wave 0's mirror
    const int kH0 = n16 - 1 - 4 * qblk;
    nkt = imin(N - 1, 16 * kH0 + 15) / 64 + 1;
  } else {
    i0 = qblk * 128;
    qbase[0] = i0 + 32 * wave;
    qbase[1] = qbase[0] + 16;
    qon[0] = qon[1] = true;
    const int ilast_b = imin(N - 1, i0 + 127);
    nkt = CAUSAL ? (ilast_b / 64 + 1) : (N + 63) / 64;
  }

  bf16x8 qf[2][2], df[2][2];
  float rlo[2], rhi[2], l2[2], dd[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int i = qbase[qb] + c16;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const uint32_t off = static_cast<uint32_t>(i * 128 + 64 * c + 16 * g);
      qf[qb][c] = __builtin_bit_cast(bf16x8, bload16(rq, off));
      df[qb][c] = __builtin_bit_cast(bf16x8, bload16(rdo, off));
    }
    const bool ok = i < N && qon[qb];
    rlo[qb] = ok ? a.rowlo[tok + i] : 0.f;
    rhi[qb] = ok ? a.rowhi[tok + i] : 0.f;
    l2[qb] = ok ? a.lse[tok + i] * kLog2e : INFINITY;  // P = 0 on padding rows
    if (EXT && !(l2[qb] > -INFINITY)) l2[qb] = INFINITY;  // a row with no key
    dd[qb] = ok ? a.dvec[tok + i] : 0.f;
  }
  // projection group of each block (a 16-query block lies in one group)
  GroupInfo giq[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
  int gq0[2];
  if (PAIR) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      gq0[qb] = (qbase[qb] / kGroup) * kGroup;
      if (((F & F_ZQ) || DZ) && qon[qb]) giq[qb] = sload_uniform16(a.gq + qbase[qb] / kGroup);
    }
  } else {
    // both blocks in the workgroup's group (group records come through the
    // scalar cache: they stay in scalar registers)
    gq0[0] = gq0[1] = i0;
    if ((F & F_ZQ) || DZ) giq[0] = giq[1] = sload_uniform16(a.gq + i0 / kGroup);
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
  float* const scr = szw + (IT ? wave * 16 * kQwP : 0);
  // offset gradients through a buffer resource: 32-bit element offsets (no
  // 64-bit row pointers to keep in registers) and range-checked stores
  const Rsrc rdz = make_rsrc(DZ ? reinterpret_cast<GT*>(a.dz) + static_cast<int64_t>(bh) * a.dz_bh : nullptr,
                             DZ ? static_cast<uint64_t>(a.dz_bh) * sizeof(GT) : 0);

  // key-tile ranges of each block: tiles [0, nkq) are visible; [0, n_hi) have
  // delta >= D for every pair of the block, [t_lo, nkq) delta <= -D
  // (without PAIR the two blocks share the wave's 32-query ranges)
  int nkq[2], n_hi[2], t_lo[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qa = qbase[PAIR ? qb : 0], qz = qbase[PAIR ? qb : 1] + 15;
    nkq[qb] = !qon[qb] ? 0 : (CAUSAL ? imin(nkt, imin(N - 1, qz) / 64 + 1) : nkt);
    int nh = (qa - D - 63 >= 0) ? (qa - D - 63) / 64 + 1 : 0;
    n_hi[qb] = imin(nh, nkq[qb]);
    const int tl = CAUSAL ? nkq[qb] : (qz + D + 63) / 64;
    t_lo[qb] = imax(n_hi[qb], imin(tl, nkq[qb]));
  }
  const int nkt_w = imax(nkq[0], nkq[1]);

  // segment masks: each query's segment, the wave's union and intersection,
  // and the workgroup's key tiles [kt_begin, kt_end)
  const bool SEG = (F & F_SEG) != 0 && a.seg != nullptr;
  const bool DROP = (F & F_DROP) != 0 && a.drop_p8 > 0;
  // (defined on every path: the per-pair tests read them only when SEG)
  int sgl[2], sgh[2];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    sgl[x] = 0;
    sgh[x] = N;
  }
  SegWave sw = {0, N, 0, N};
  int kt_begin = 0, kt_end = nkt;
  if (SEG) {
    bool on[2];
    const int64_t brow = static_cast<int64_t>(bh / a.H) * N;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int i = qbase[qb] + c16;
      on[qb] = i < N && qon[qb];
      sgl[qb] = sgh[qb] = 0;
      if (on[qb]) token_segment(a, brow, i, sgl[qb], sgh[qb]);
    }
    sw = seg_wave(sgl, sgh, on, 2);
    int blo, bhi;
    seg_block(sw, wave, sseg, blo, bhi);
    kt_begin = blo < bhi ? blo / 64 : 0;
    kt_end = blo < bhi ? imin(nkt, (bhi + 63) / 64) : 0;
  }

  floatx4 dq[2][4];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < 4; ++db) dq[qb][db] = floatx4{0.f, 0.f, 0.f, 0.f};
  float blo[2] = {0.f, 0.f}, bhi[2] = {0.f, 0.f};

  const int kr = tid >> 3, kc8 = (tid & 7) * 8;
  uint4 tk[2], tv[2];
  float tkc[3] = {0.f, 0.f, 0.f};
  auto load_tile = [&](int j0) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint32_t off = static_cast<uint32_t>((j0 + kr + 32 * u) * 128 + kc8 * 2);
      tk[u] = bload16(rk, off);
      tv[u] = bload16(rv, off);
    }
    if (KC && tid < 64) {
      const int j = j0 + tid;
      const bool ok = j < N;
      tkc[2] = ok ? a.keymid[tok + j] : 0.f;
      if (KC3) {
        tkc[0] = ok ? a.keylo[tok + j] : 0.f;
        tkc[1] = ok ? a.keyhi[tok + j] : 0.f;
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      *reinterpret_cast<uint4*>(&sk[buf][(kr + 32 * u) * kP + kc8]) = tk[u];
      *reinterpret_cast<uint4*>(&sv[buf][(kr + 32 * u) * kP + kc8]) = tv[u];
    }
    if (KC && tid < 64) {
      skc[buf][2][tid] = tkc[2];
      if (KC3) {
        skc[buf][0][tid] = tkc[0];
        skc[buf][1][tid] = tkc[1];
      }
    }
  };

  load_tile(64 * kt_begin);
  store_tile(0);
  __syncthreads();

  for (int kt = kt_begin; kt < kt_end; ++kt) {
    const int buf = (kt - kt_begin) & 1;
    const int j0 = kt * 64;
    // With a key table the pass sits at the register limit: the lane index
    // is made opaque each tile so the per-lane LDS addresses derived from it
    // are recomputed in the tile (a few adds) instead of being kept across the
    // loop, where they spilled to scratch and were reloaded every tile.
    int lane_t = lane;
    if constexpr (STZK) asm volatile("" : "+v"(lane_t));
    const int g = lane_t >> 4, c16 = lane_t & 15;
    if (STZK) {
      // band for some wave of the workgroup: stage Z^K of the tile's keys
      // (before the next tile's prefetch is issued: loads complete in order,
      // so the staging's wait would otherwise cover the prefetch too)
      const bool blk_sat = (i0 - (j0 + 63) >= D) || (i0 + 127 - j0 <= -D);
      if (!blk_sat && j0 < N) {
        const GroupInfo gk = sload_uniform16(a.gk + j0 / kGroup);
        stage_zk_rows(rzk, gk.base, gk.slo, gk.pad, gk.pitch, (j0 / kGroup) * kGroup, j0, i0, D,
                      szk, kZP);
        __syncthreads();
      }
    }
    if (kt + 1 < kt_end) load_tile(j0 + 64);

    if (kt < nkt_w && (!SEG || (j0 < sw.uhi && j0 + 64 > sw.ulo))) {
      const bf16* Ks = sk[buf];
      const bf16* Vs = sv[buf];
      // per block (uniform): does the tile reach it, and its region; on
      // saturated tiles the key's entry is the initial value of the S
      // accumulator and the query's entry goes into off
      bool act[2], sat[2];
      int side[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        act[qb] = PAIR ? kt < nkq[qb] : true;
        sat[qb] = kt < n_hi[qb] || kt >= t_lo[qb];
        side[qb] = kt < n_hi[qb] ? 1 : 0;
      }
      // a block that the tile does not reach is always block 0 (block 1 is
      // the wider one), so block 1's products are always made
      const bool both = act[0];
      floatx4 s[2][4], dp[2][4];
      // initial values: dP zero; S the key's boundary entry on saturated
      // tiles (with per-key entries), else zero
      auto sat_init = [&](int qb) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          floatx4 kx = floatx4{0.f, 0.f, 0.f, 0.f};
          if (KC && sat[qb])
            kx = *reinterpret_cast<const floatx4*>(&skc[buf][KC3 ? side[qb] : 2][16 * kb + 4 * g]);
          s[qb][kb] = kx;
        }
      };
      if constexpr (!BAND_INIT) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            floatx4 kx = floatx4{0.f, 0.f, 0.f, 0.f};
            if (KC && sat[qb])
              kx = *reinterpret_cast<const floatx4*>(&skc[buf][KC3 ? side[qb] : 2][16 * kb + 4 * g]);
            s[qb][kb] = kx;
            dp[qb][kb] = floatx4{0.f, 0.f, 0.f, 0.f};
          }
        }
      } else {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) dp[qb][kb] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
      // S^T = K Q^T and dP^T = V dO^T added to the accumulators' initial
      // values
      auto products = [&]() {
        prio_matrix<PRIO>();
#pragma unroll
        for (int c = 0; c < 2; ++c) {
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            const bf16x8 kf = *reinterpret_cast<const bf16x8*>(Ks + (16 * kb + c16) * kP + 32 * c + 8 * g);
            const bf16x8 vf = *reinterpret_cast<const bf16x8*>(Vs + (16 * kb + c16) * kP + 32 * c + 8 * g);
            if (both) {
              s[0][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[0][c], s[0][kb], 0, 0, 0);
              dp[0][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, df[0][c], dp[0][kb], 0, 0, 0);
            }
            s[1][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[1][c], s[1][kb], 0, 0, 0);
            dp[1][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, df[1][c], dp[1][kb], 0, 0, 0);
          }
        }
        prio_normal<PRIO>();
      };
      if constexpr (!BAND_INIT) products();

      // relation terms (same values as the forward); off = the row's
      // constant on saturated tiles.  pure: a band tile without any pair
      // |delta| >= D (every tile of an identity map), whose selects are
      // skipped
      bool pure[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const int qa = qbase[PAIR ? qb : 0], qz = qbase[PAIR ? qb : 1] + 15;
        pure[qb] = IT || (qa - (j0 + 63) > -D && qz - j0 < D);
      }
      float off[2];
      // transposing-read address of this lane in szk (lds_tr4 with row0 = 4g)
      const _Float16* szk_lane = szk + (4 * g + (c16 >> 2)) * kZP + 4 * (c16 & 3);
      auto band_q = [&](int qb, auto PURE, auto ASSIGN) {
        const int i = qbase[qb] + c16;
        const bool iok = i < N;
        const int zrow = giq[qb].base + (i - gq0[qb]) * giq[qb].pitch;
        // without a key table (room in the registers): the block's four Z^Q
        // runs are requested together, one memory round trip per block
        // instead of four (every tile of an identity map is a band tile)
        if constexpr (IT) {
          // the block's 80-row window on MFMA, into the wave's scratch
          floatx4 zt[5];
          it_rows<5>(itb, qbase[qb] - j0 - 63 + D, qf[qb][0], qf[qb][1], c16, g, zt);
          it_put<5>(scr, kQwP, c16, g, zt);
        }
        uint2 zw[4];
        if constexpr (HOISTQ) {
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            const int j1 = j0 + 16 * kb + 4 * g;
            const int c0 = clamp_run((i - (j1 + 3) + D) - giq[qb].slo + giq[qb].pad, giq[qb].pitch);
            zw[kb] = bload8(rzq, iok ? static_cast<uint32_t>((zrow + c0) * 2) : kOob);
          }
        }
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const int j1 = j0 + 16 * kb + 4 * g;
          float zq[4] = {0.f, 0.f, 0.f, 0.f};
          if constexpr (IT) {
            // pair (i, j1 + t) at window row c16 + 63 - 16 kb - 4 g - t
            const float* zr = scr + c16 * kQwP + c16 + 60 - 16 * kb - 4 * g;
#pragma unroll
            for (int t = 0; t < 4; ++t) zq[t] = zr[3 - t];
          }
          if (F & F_ZQ) {
            uint2 w;
            if constexpr (HOISTQ) {
              w = zw[kb];
            } else {
              const int c0 = clamp_run((i - (j1 + 3) + D) - giq[qb].slo + giq[qb].pad, giq[qb].pitch);
              w = bload8(rzq, iok ? static_cast<uint32_t>((zrow + c0) * 2) : kOob);
            }
            const halfx4 hv = __builtin_bit_cast(halfx4, w);
#pragma unroll
            for (int t = 0; t < 4; ++t) zq[t] = static_cast<float>(hv[3 - t]);
          }
          floatx4 km = floatx4{0.f, 0.f, 0.f, 0.f}, klo4 = km, khi4 = km;
          if (KC) km = *reinterpret_cast<const floatx4*>(&skc[buf][2][16 * kb + 4 * g]);
          if (KC3 && !PURE) {
            klo4 = *reinterpret_cast<const floatx4*>(&skc[buf][0][16 * kb + 4 * g]);
            khi4 = *reinterpret_cast<const floatx4*>(&skc[buf][1][16 * kb + 4 * g]);
          }
          halfx4 zk4 = halfx4{0, 0, 0, 0};
          if (STZK)  // Z^K[j1 + t][i - j1 - t + D], t = 0..3 (the lane's base, plus rows 16 kb and the block's columns)
            zk4 = __builtin_bit_cast(halfx4, lds_tr4_at(szk_lane + (16 * kb) * kZP + (qbase[qb] - i0)));
          floatx4 add4;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int j = j1 + t;
            const int dl = i - j;
            float band = km[t] + zq[t];
            if (F & F_ZK) band += static_cast<float>(zk4[t]);
            if (F & F_BT) band += bloadf(rbt, static_cast<uint32_t>(iclamp(dl + D, 0, 2 * D) * 4));
            if constexpr (PURE) {
              add4[t] = band;
            } else {
              const float kedge = KC3 ? (dl >= D ? khi4[t] : klo4[t]) : km[t];
              add4[t] = dl >= D ? (rhi[qb] + kedge) : (dl <= -D ? (rlo[qb] + kedge) : band);
            }
            if constexpr (!ASSIGN && !VEC_ADD) s[qb][kb][t] += add4[t];
          }
          if constexpr (ASSIGN)
            s[qb][kb] = add4;  // the initial value of the accumulator
          else if constexpr (VEC_ADD)
            s[qb][kb] += add4;
          // keep each 4-run's loads next to their use (register pressure)
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      if constexpr (BAND_INIT) {
        // (no causal pairing with a key table) each branch makes its own
        // products: a band tile's terms are the accumulator's initial value,
        // so both branches leave S in the registers of their own MFMA
        // results (with the terms added after the products, the saturated
        // branch copied every score into the band branch's registers)
        if (sat[0] && sat[1]) {
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            sat_init(qb);
            off[qb] = side[qb] ? rhi[qb] : rlo[qb];
          }
          products();
        } else {
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            off[qb] = 0.f;
            if (sat[qb]) {
              sat_init(qb);
              off[qb] = side[qb] ? rhi[qb] : rlo[qb];
            } else if (pure[qb]) {
              band_q(qb, std::true_type{}, std::true_type{});
            } else {
              band_q(qb, std::false_type{}, std::true_type{});
            }
          }
          products();
        }
      } else {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          off[qb] = 0.f;
          if (!act[qb]) continue;
          if (sat[qb])
            off[qb] = side[qb] ? rhi[qb] : rlo[qb];
          else if (pure[qb])
            band_q(qb, std::true_type{}, std::false_type{});
          else
            band_q(qb, std::false_type{}, std::false_type{});
        }
      }

      // P, then G' = P (dP - D) in place of s; tau is applied to the sums
      // of G' (dQ, the boundary sums) and to the band entries as written
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        if (!act[qb]) continue;
        const float bias = off[qb] * sl2 - l2[qb];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int t = 0; t < 4; ++t) s[qb][kb][t] = fast_exp2(fmaf(s[qb][kb][t], sl2, bias));
      }
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        if (!act[qb]) continue;
        if ((j0 + 64 > N) || (CAUSAL && j0 + 63 > qbase[qb]) ||
            (SEG && (j0 < sw.ilo || j0 + 64 > sw.ihi))) {
          // (the empty asm keeps this a branch: without it the compiler turns
          // the rare masked pass into selects on every tile)
          asm volatile("");
          const int i = qbase[qb] + c16;
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const int j = j0 + 16 * kb + 4 * g + t;
              const bool off_seg = SEG && (j < sgl[qb] || j >= sgh[qb]);
              s[qb][kb][t] = (j >= N || (CAUSAL && j > i) || off_seg) ? 0.f : s[qb][kb][t];
            }
        }
      }
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        if (!act[qb]) continue;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          // dropout: dP of a dropped pair is 0, of a kept one times the scale
          float mk[4] = {1.f, 1.f, 1.f, 1.f};
          if (DROP) keep_row4(a, bh, qbase[qb] + c16, j0 + 16 * kb + 4 * g, a.drop_scale, mk);
#pragma unroll
          for (int t = 0; t < 4; ++t)
            s[qb][kb][t] *= (F & F_DROP) ? fmaf(dp[qb][kb][t], mk[t], -dd[qb]) : dp[qb][kb][t] - dd[qb];
        }
      }

      // offset gradients of the queries
      if (DZ) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          if (!act[qb]) continue;
          if (sat[qb]) {
            float acc = 0.f;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
              acc += (s[qb][kb][0] + s[qb][kb][1]) + (s[qb][kb][2] + s[qb][kb][3]);
            if (side[qb])
              bhi[qb] += acc;
            else
              blo[qb] += acc;
            continue;
          }
          const int i = qbase[qb] + c16;
          const int rowe = giq[qb].base + (i - gq0[qb]) * giq[qb].pitch - giq[qb].slo + giq[qb].pad;
          auto dz_band = [&](auto PURE) {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
              const int j1 = j0 + 16 * kb + 4 * g;
              float run[4];
              bool any = false;
#pragma unroll
              for (int t = 0; t < 4; ++t) {
                const int j = j1 + t;
                const int dl = i - j;
                const float gg = s[qb][kb][t];
                float bandv = 0.f;  // tau G' for the band entry
                if (!PURE && dl >= D)
                  bhi[qb] += gg;
                else if (!PURE && dl <= -D)
                  blo[qb] += gg;
                else {
                  bandv = tau * gg;
                  any = any || (i < N && j < N && (!CAUSAL || j <= i));
                }
                run[3 - t] = bandv;  // descending columns
              }
              // (issued whether or not the run holds a band pair: a run
              // without one stores nothing)
              bstore4(rdz, any ? static_cast<uint32_t>(rowe + (i - (j1 + 3) + D)) * sizeof(GT) : kOob, run,
                      static_cast<GT*>(nullptr));
            }
          };
          if (pure[qb])
            dz_band(std::true_type{});
          else
            dz_band(std::false_type{});
        }
      }

      // in-tile: dQ^T += A~_window^T G'_window^T.  Block qb's G' goes into
      // the scratch as rows [query][32 + key] between zero margins, so that
      // window row s'' = 32 k + 8 g + e (e = 0..7) of query c16, which holds
      // the pair with key j0 + 63 + c16 - s'', is column 95 + c16 - s''; the
      // table side is A~^T[16 db + c16][sb + 32 k + 8 g ..] (sb = the
      // window's first row, a multiple of 16: aligned 16-byte loads)
      if constexpr (IT) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          if (!act[qb]) continue;
          float* row = scr + c16 * kQwP;
          const floatx4 z4 = floatx4{0.f, 0.f, 0.f, 0.f};
          *reinterpret_cast<floatx4*>(row + 8 * g) = z4;
          *reinterpret_cast<floatx4*>(row + 8 * g + 4) = z4;
          *reinterpret_cast<floatx4*>(row + 96 + 4 * g) = z4;
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) *reinterpret_cast<floatx4*>(row + 32 + 16 * kb + 4 * g) = s[qb][kb];
          const int sb = qbase[qb] - j0 - 63 + D;
#pragma unroll
          for (int k = 0; k < 3; ++k) {
            const float* gr = row + 88 + c16 - 32 * k - 8 * g;  // e = 7 .. 0
            bf16x8 gw;
#pragma unroll
            for (int e = 0; e < 8; ++e) gw[e] = static_cast<bf16>(gr[7 - e]);
            const int col = sb + 32 * k + 8 * g;
#pragma unroll
            for (int db = 0; db < 4; ++db) {
              const bf16x8 at8 = __builtin_bit_cast(
                  bf16x8, bload16(itb.att, col >= 0 ? static_cast<uint32_t>((16 * db + c16) * a.Sp + col) * 2 : kOob));
              dq[qb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(at8, gw, dq[qb][db], 0, 0, 0);
            }
          }
        }
      }

      // dQ^T += K^T G'^T
      prio_matrix<PRIO>();
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        bf16x8 gf[2], gl[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float x = s[qb][2 * c + (e >> 2)][e & 3];
            gf[qb][e] = static_cast<bf16>(x);
            if (SPLIT) gl[qb][e] = static_cast<bf16>(x - static_cast<float>(gf[qb][e]));
          }
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const bf16x4 lo = lds_tr4(Ks, kP, 32 * c + 4 * g, 16 * db, c16);
          const bf16x4 hi = lds_tr4(Ks, kP, 32 * c + 16 + 4 * g, 16 * db, c16);
          bf16x8 kt8;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            kt8[e] = lo[e];
            kt8[e + 4] = hi[e];
          }
          if (both) {
            dq[0][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kt8, gf[0], dq[0][db], 0, 0, 0);
            if (SPLIT)
              dq[0][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kt8, gl[0], dq[0][db], 0, 0, 0);
          }
          dq[1][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kt8, gf[1], dq[1][db], 0, 0, 0);
          if (SPLIT)
            dq[1][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kt8, gl[1], dq[1][db], 0, 0, 0);
        }
      }
    }

    prio_normal<PRIO>();
    if (kt + 1 < kt_end) store_tile(buf ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int i = qbase[qb] + c16;
    const float lo = tau * wave_sum_g(blo[qb]);
    const float hi = tau * wave_sum_g(bhi[qb]);
    if (i >= N || !qon[qb]) continue;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      float vals[4] = {tau * dq[qb][db][0], tau * dq[qb][db][1], tau * dq[qb][db][2],
                       tau * dq[qb][db][3]};
      store4(a.dqacc + (tok + i) * 64 + 16 * db + 4 * g, vals);
    }
    if (DZ && g == 0) {
      a.bndq[(tok + i) * 2 + 0] = lo;
      a.bndq[(tok + i) * 2 + 1] = hi;
    }
  }
}

template <int F>
hipError_t launch_qf(const AttnArgs& a, int B, hipStream_t s) {
  constexpr bool PAIR = (F & F_CAUSAL) && !(F & F_ZK);
  // PAIR: workgroup m owns 16-query blocks 4m .. 4m+3 and their mirrors
  const int n16 = (a.N + 15) / 16;
  const int nqb = PAIR ? ((n16 + 1) / 2 + 3) / 4 : (a.N + 127) / 128;
  const int total = nqb * B * a.H;
  const int xcd_map = (F & F_CAUSAL) ? 0 : 1;
  hipLaunchKernelGGL((bwd_q_fast<F>), dim3(total), dim3(256), 0, s, a, nqb, total, xcd_map);
  return hipGetLastError();
}

// term combinations: Shaw (ZQ), T5 (BT), DeBERTa (ZQ+ZK), Transformer-XL
// (ZQ+U), and the other mixes of the descriptor's terms
#define RP_QF_FLAGS(X)                                                                    \
  X(0) X(F_U) X(F_ZK) X(F_ZK | F_U) X(F_ZQ | F_DZQ) X(F_ZQ | F_ZK | F_DZQ)               \
  X(F_ZQ | F_DZQ | F_DZ32) X(F_ZQ | F_ZK | F_DZQ | F_DZ32) X(F_ZQ | F_U | F_DZQ)         \
  X(F_ZQ | F_U | F_DZQ | F_DZ32) X(F_ZQ | F_ZK | F_U | F_DZQ) X(F_ZQ | F_ZK | F_U | F_DZQ | F_DZ32) \
  X(F_BT | F_DZQ | F_DZ32) X(F_BT | F_U | F_DZQ | F_DZ32) X(F_ZK | F_BT | F_DZQ | F_DZ32)  \
  X(F_ZK | F_BT | F_U | F_DZQ | F_DZ32) X(F_ZQ | F_DZQ | F_DZ16) X(F_ZQ | F_U | F_DZQ | F_DZ16) \
  X(F_ZQ | F_ZK | F_DZQ | F_DZ16) X(F_ZQ | F_ZK | F_U | F_DZQ | F_DZ16)

template <int SPL>
hipError_t dispatch_qf(int flags, const AttnArgs& a, int B, hipStream_t s) {
  const int f = flags & (F_ZQ | F_ZK | F_BT | F_U | F_CAUSAL | F_DZQ | F_DZ32 | F_DZ16);
  switch (f) {
#define RP_CASE(X)                                   \
  case X:                                            \
    return launch_qf<(X) | SPL>(a, B, s);            \
  case (X) | F_CAUSAL:                               \
    return launch_qf<(X) | F_CAUSAL | SPL>(a, B, s);
    RP_QF_FLAGS(RP_CASE)
#undef RP_CASE
    default:
      return hipErrorInvalidValue;
  }
}

// in-tile products (F_IT): A^Q with or without the u term
template <int SPL>
hipError_t dispatch_qit(int flags, const AttnArgs& a, int B, hipStream_t s) {
  switch (flags & (F_IT | F_U | F_CAUSAL)) {
    case F_IT:
      return launch_qf<F_IT | SPL>(a, B, s);
    case F_IT | F_CAUSAL:
      return launch_qf<F_IT | F_CAUSAL | SPL>(a, B, s);
    case F_IT | F_U:
      return launch_qf<F_IT | F_U | SPL>(a, B, s);
    case F_IT | F_U | F_CAUSAL:
      return launch_qf<F_IT | F_U | F_CAUSAL | SPL>(a, B, s);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace

}  // namespace relpos
