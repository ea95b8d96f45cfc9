// Key-parallel backward pass for bf16 inputs ([RPA] Table 9 "Key-parallel
// pass", Algorithm 2).  [RPA] = "Fast and Exact Relative-Position Attention
// via Structure-Aware Kernels" (arXiv 2611.01182).
//
// A workgroup of 4 waves owns 128 keys (one projection group), 32 per wave.
// Query tiles of 32 queries (Q, dO row-major, and per query L, D and the two
// boundary entries) stream through double-buffered LDS; the short tile keeps
// a wave's scores, score gradients and four accumulators within 256
// registers.  Per tile and wave:
//   S = Q K^T and dP = dO V^T on MFMA (A from LDS rows, K and V of the
//   wave's keys in registers), each lane owning one key column and four
//   consecutive queries per 16-query block;
//   relation terms exactly as the forward (same boundary-entry rule);
//   P = exp2(S tau log2 e - L log2 e), G' = P (dP - D) (G = tau G'; tau
//   multiplies the finished sums instead);
//   dV^T += dO^T P and dK^T += Q^T G' on MFMA (dO^T and Q^T read with the
//   transposing LDS read; P and G' as bf16).  Under F_SPLIT (a strongly
//   peaked softmax) G' enters dK as a bf16 pair hi + lo (~16 significant
//   bits) and P enters dV as fp16 (11 bits, against dO and, for dP, V
//   converted to fp16 when staged): an 11-bit P moves dV by ~2^-12 |dO|,
//   well inside the tolerance, where an 8-bit one does not, and costs one
//   product instead of the pair's two.
// Key offset gradients ([RPA] §4.2): a band pair writes G to
// dZ~^K[j, delta + D] (single writer, aligned 4-entry runs); pairs with
// |delta| >= D add into two fp32 per-key boundary sums; with the
// Transformer-XL u term the column sums of G are kept too.  No atomics.
// F_SEG adds segment masks (query tiles limited to the union of the
// workgroup's keys' segments, per-pair tests elsewhere), F_DROP dropout
// (G' = P (dP keep - D), dV takes P keep; segments are then taken when
// given), as defined in extras.hpp.
// F_IT computes the tiles' Z^Q entries in the tile (intile.hpp) instead of
// staging stored projections.
#pragma once
#include "extras.hpp"
#include "intile.hpp"
#include "relation.hpp"
#include "tiles.hpp"

namespace relpos {

namespace {

// tile pitch (bf16): 160-byte rows, a 40-dword stride that puts eight
// consecutive rows on distinct 8-bank groups, so the transposing reads of
// 16 rows (and the row reads of 8) meet no bank conflict (at 144 bytes two
// of the eight rows shared banks)
constexpr int kP = 80;
constexpr int kT = 32;  // queries per tile
constexpr int kKwP = 36;  // in-tile scratch pitch (fp32): 32 window rows

template <int F>
__global__ __launch_bounds__(256, 2) void bwd_k_fast(AttnArgs a, int nkb, int total, int xcd_map) {
  constexpr bool CAUSAL = (F & F_CAUSAL) != 0;
  constexpr bool SPLIT = (F & F_SPLIT) != 0;
  constexpr bool EXT = (F & (F_SEG | F_DROP)) != 0;
  // fp16 P in dV = P^T dO (under F_SPLIT): dO and V as fp16 words
  constexpr bool HP = SPLIT;
  constexpr bool DZ = (F & F_DZK) != 0;
  constexpr bool CS = (F & F_U) != 0;
  constexpr bool KC = (F & (F_ZK | F_U)) != 0;
  constexpr bool IT = (F & F_IT) != 0;
  // query projections of a band tile are staged into LDS once per workgroup
  constexpr bool STZQ = (F & F_ZQ) != 0;
  // causal masks: pair each 16-key block with its mirror (below)
  constexpr bool PAIR = CAUSAL && !(F & F_ZK) && !DZ;
  constexpr int kZP = 136;  // szq pitch (fp16)
  __shared__ __attribute__((aligned(16))) _Float16 szq[2][STZQ ? kT * kZP : 8];
  __shared__ __attribute__((aligned(16))) bf16 sq[2][kT * kP];
  __shared__ __attribute__((aligned(16))) bf16 sd[2][kT * kP];
  // l2, D, rowlo, rowhi (rows 4..7: unread copies, written by threads 128..255
  // so that the store needs no branch)
  __shared__ __attribute__((aligned(16))) float sqs[2][8][kT];
  __shared__ int sseg[2][4];
  // in-tile products: one [16 queries][kKwP] window scratch per wave
  __shared__ __attribute__((aligned(16))) float szw[IT ? 4 * 16 * kKwP : 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = wave_index(), g = lane >> 4, c16 = lane & 15;
  const int N = a.N, D = a.D;

  int item = static_cast<int>(blockIdx.x);
  if (xcd_map) {
    const int q8 = total / 8, r8 = total % 8;
    const int x = item % 8, slot = item / 8;
    item = (x < r8 ? x * (q8 + 1) : r8 * (q8 + 1) + (x - r8) * q8) + slot;
  }
  const int BH = total / nkb;
  int bh, kblk;
  if (CAUSAL) {
    // causal: the first key blocks see the most queries
    kblk = item / BH;
    bh = item % BH;
  } else {
    bh = item / nkb;
    kblk = item % nkb;
  }
  const int h = bh % a.H;
  const int64_t tok = static_cast<int64_t>(bh) * N;
  // The wave's keys: two blocks of 16 starting at jbase[0], jbase[1]; jloc is
  // their column in the staged Z^Q rows.  Without PAIR the workgroup owns 128
  // consecutive keys (one projection group).  With PAIR (causal masks) wave w
  // of workgroup m owns 16-key block kH = 4m + w and its mirror
  // kL = n16 - 1 - kH: a key is seen by the queries at or after it, so every
  // wave then has the same work (a lone middle block is taken as block 0).
  // The staged key ranges are then [64m, 64m + 64) and the 64 keys ending
  // with block n16 - 1 - 4m.
  int jbase[2], jloc[2];
  bool kon[2];
  int j0b, jrB = 0;
  if (PAIR) {
    const int n16 = (N + 15) / 16;
    const int kH = 4 * kblk + wave, kL = n16 - 1 - kH;
    jbase[0] = 16 * kH;
    jbase[1] = 16 * kL;
    kon[0] = kH <= kL;
    kon[1] = kH < kL;
    j0b = 64 * kblk;
    jrB = 16 * (n16 - 4 - 4 * kblk);
    jloc[0] = 16 * wave;
    jloc[1] = 64 + 16 * (3 - wave);
  } else {
    j0b = kblk * 128;
    jbase[0] = j0b + 32 * wave;
    jbase[1] = jbase[0] + 16;
    kon[0] = kon[1] = true;
    jloc[0] = 32 * wave;
    jloc[1] = 32 * wave + 16;
  }
  const float sl2 = a.scale_log2, tau = a.scale;
  const uint64_t slice_bytes = static_cast<uint64_t>(N) * 128;
  const Rsrc rq = make_rsrc(reinterpret_cast<const bf16*>(a.q) + tok * 64, slice_bytes);
  const Rsrc rdo = make_rsrc(reinterpret_cast<const bf16*>(a.dout) + tok * 64, slice_bytes);
  const Rsrc rk = make_rsrc(reinterpret_cast<const bf16*>(a.k) + tok * 64, slice_bytes);
  const Rsrc rv = make_rsrc(reinterpret_cast<const bf16*>(a.v) + tok * 64, slice_bytes);

  // keys of this lane: jbase[kb] + c16
  bf16x8 kf[2][2], vf[2][2];
  float klo[2], khi[2], kmid[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int j = jbase[kb] + c16;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const uint32_t off = static_cast<uint32_t>(j * 128 + 64 * c + 16 * g);
      kf[kb][c] = __builtin_bit_cast(bf16x8, bload16(rk, off));
      vf[kb][c] = __builtin_bit_cast(bf16x8, stage16<HP>(bload16(rv, off)));
    }
    const bool ok = j < N && kon[kb];
    klo[kb] = (KC && ok) ? a.keylo[tok + j] : 0.f;
    khi[kb] = (KC && ok) ? a.keyhi[tok + j] : 0.f;
    kmid[kb] = (KC && ok) ? a.keymid[tok + j] : 0.f;
  }
  GroupInfo gik = {0, 0, 0, 0};
  const int gk0 = (j0b / kGroup) * kGroup;  // (used without PAIR only)
  if ((F & F_ZK) || DZ) gik = sload_uniform16(a.gk + j0b / kGroup);
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
  float* const scr = szw + (IT ? wave * 16 * kKwP : 0);

  // query tiles: causal starts at the workgroup's first key; a block's tiles
  // before its own first key are fully masked and skipped.  Regions from the
  // block's extreme offsets: [itk, n_lo) all delta <= -D, [t_hi, nqt) all
  // delta >= D (without PAIR both blocks use the wave's 32-key range).
  const int nqt = (N + kT - 1) / kT;
  const int it0 = CAUSAL ? j0b / kT : 0;
  int itk[2], n_lo[2], t_hi[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int ja = jbase[PAIR ? kb : 0], jz = jbase[PAIR ? kb : 1] + 15;
    itk[kb] = !kon[kb] ? nqt : (CAUSAL ? ja / kT : 0);
    int nl = (ja - D - (kT - 1) >= 0) ? (ja - D - (kT - 1)) / kT + 1 : 0;
    n_lo[kb] = CAUSAL ? itk[kb] : imax(itk[kb], imin(nl, nqt));
    const int th = (jz + D + kT - 1) / kT;
    t_hi[kb] = imax(n_lo[kb], imin(th, nqt));
  }
  const int itw = itk[0];  // block 0 starts first (PAIR: the earlier keys)

  // segment masks: each key's segment (the queries that see it), the wave's
  // union and intersection, and the workgroup's query tiles [it_first, it_end)
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
  int it_first = it0, it_end = nqt;
  if (SEG) {
    bool on[2];
    const int64_t brow = static_cast<int64_t>(bh / a.H) * N;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int j = jbase[kb] + c16;
      on[kb] = j < N && kon[kb];
      sgl[kb] = sgh[kb] = 0;
      if (on[kb]) token_segment(a, brow, j, sgl[kb], sgh[kb]);
    }
    sw = seg_wave(sgl, sgh, on, 2);
    int blo, bhi;
    seg_block(sw, wave, sseg, blo, bhi);
    it_first = blo < bhi ? imax(it0, blo / kT) : nqt;
    it_end = blo < bhi ? imin(nqt, (bhi + kT - 1) / kT) : 0;
  }

  floatx4 dk[2][4], dv[2][4];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      dk[kb][db] = floatx4{0.f, 0.f, 0.f, 0.f};
      dv[kb][db] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
  float blo[2] = {0.f, 0.f}, bhi[2] = {0.f, 0.f}, csum[2] = {0.f, 0.f};

  const int kr = tid >> 3, kc8 = (tid & 7) * 8;
  // a query tile in registers on its way to LDS: Q and dO rows (t >> 3), chunk
  // t & 7, and one per-query value: thread t < 128 holds value (t >> 5) (L, D
  // and the two boundary entries) of query t & 31 (threads past 128 repeat
  // those loads).  Every load is issued unconditionally, rows past N reading
  // zero or a clamped index, so that each wave issues the same vector loads on
  // every path and the compiler's wait counts stay exact.
  const int sx = (tid >> 5) & 3, sqi = tid & 31;
  const float* const sbase = sx == 0 ? a.lse : (sx == 1 ? a.dvec : (sx == 2 ? a.rowlo : a.rowhi));
  struct TileRegs {
    uint4 q, d;
    float st;
  };
  auto load_tile = [&](TileRegs& r, int i0) {
    const uint32_t off = static_cast<uint32_t>((i0 + kr) * 128 + kc8 * 2);
    r.q = bload16(rq, off);
    r.d = bload16(rdo, off);
    r.st = sbase[tok + imin(i0 + sqi, N - 1)];
  };
  auto store_tile = [&](const TileRegs& r, int buf, int i0) {
    *reinterpret_cast<uint4*>(&sq[buf][kr * kP + kc8]) = r.q;
    *reinterpret_cast<uint4*>(&sd[buf][kr * kP + kc8]) = stage16<HP>(r.d);
    // L enters log2 units; padding rows get L = inf (P = 0) and zeros
    const bool ok = i0 + sqi < N;
    const float v = sx == 0 ? (ok ? r.st * kLog2e : INFINITY) : (ok ? r.st : 0.f);
    sqs[buf][tid >> 5][sqi] = v;
  };

  // Z^Q of a tile's queries for the workgroup's keys (band tiles), staged as
  // szq[query][key column]: a query row holds 64 consecutive keys in
  // descending order from a 16-byte boundary (the query-side pad), so each
  // chunk is reversed.  Columns 0..63 are keys j0b.., 64..127 keys j0b + 64..
  // (PAIR: keys jrB..).  The loads of tile t + 1 are issued during tile t
  // (before that step's tile prefetch) and written at its end.
  // (a tile that needs no Z^Q loads and stores none: its LDS copy is never
  // read)
  uint4 zr[2] = {uint4{0, 0, 0, 0}, uint4{0, 0, 0, 0}};
  bool zq_need = false;
  auto load_zq = [&](int t) {
    const int i0 = t * kT;
    const int jr0 = j0b, jr1 = PAIR ? jrB : j0b + 64;
    const bool sat0 = (i0 - (jr0 + 63) >= D) || (i0 + kT - 1 - jr0 <= -D);
    const bool sat1 = (i0 - (jr1 + 63) >= D) || (i0 + kT - 1 - jr1 <= -D);
    const bool need = t < nqt && !(sat0 && sat1);
    // (a uniform branch: a tile saturated for both halves reads no Z^Q, and
    // out-of-range loads still cost; its LDS copy is then never read)
    zq_need = need;
    if (!need) return;
    const GroupInfo gq = sload_uniform16(a.gq + i0 / kGroup);
    const int gq0s = (i0 / kGroup) * kGroup;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int idx = tid + 256 * u;
      const int r = idx >> 4, ch = idx & 15;
      const int half = ch >> 3, chl = ch & 7;
      const int jtop = (half ? jr1 : jr0) + 63;
      const int i = i0 + r;
      const int col = (i - jtop + D) - gq.slo + gq.pad + 8 * chl;
      const int e = gq.base + (i - gq0s) * gq.pitch + col;
      zr[u] = bload16(rzq, (i < N && e >= 0) ? static_cast<uint32_t>(e) * 2 : kOob);
    }
  };
  auto store_zq = [&](int buf) {
    if (!zq_need) return;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int idx = tid + 256 * u;
      const int r = idx >> 4, ch = idx & 15;
      const int half = ch >> 3, chl = ch & 7;
      // entries 8 chl .. 8 chl + 7 of the run are keys jtop - 8 chl - (0..7)
      const uint4 w = zr[u];
      uint4 rev;
      rev.x = __builtin_amdgcn_perm(w.w, w.w, 0x01000302u);
      rev.y = __builtin_amdgcn_perm(w.z, w.z, 0x01000302u);
      rev.z = __builtin_amdgcn_perm(w.y, w.y, 0x01000302u);
      rev.w = __builtin_amdgcn_perm(w.x, w.x, 0x01000302u);
      *reinterpret_cast<uint4*>(szq[buf] + r * kZP + (64 * half + 56 - 8 * chl)) = rev;
    }
  };

  // Tiles are loaded two ahead: while tile t is computed from LDS, tile t + 1
  // is in flight in one register set and tile t + 2 is requested into the
  // other (the loads of a tile get two tiles' time to arrive).
  TileRegs ra, rb;
  load_tile(ra, it_first * kT);
  store_tile(ra, 0, it_first * kT);
  if (STZQ) {
    load_zq(it_first);
    store_zq(0);
  }
  wait_vm_all();
  load_tile(rb, (it_first + 1) * kT);
  __syncthreads();

  // one tile step: rl held tile it (already in LDS) and now receives tile
  // it + 2; rs holds tile it + 1, stored to the other LDS buffer at the end
  auto tile_step = [&](int it, TileRegs& rl, TileRegs& rs) {
    const int buf = (it - it_first) & 1;
    const int i0 = it * kT;
    // Z^K runs of this band tile (key tables): issued first, so that waiting
    // for them leaves the prefetches below in flight.  Lane (c16, g) of
    // blocks (qb, kb) reads Z^K[j][i1 - j + D], i1 = i0 + 16 qb + 4g + t,
    // t = 0..3, j = jbase[kb] + c16 (an ascending run).
    uint2 zkr[2][2];
    // (requested on band tiles only, a uniform branch: most tiles of a key
    // table's map are saturated, and out-of-range loads still cost)
    const bool bandk = (F & F_ZK) && it >= itw && !(it < n_lo[0] || it >= t_hi[0]);
    if (bandk) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int i1 = i0 + 16 * qb + 4 * g;
          const int j = jbase[kb] + c16;
          const int c0 = clamp_run((i1 - j + D) - gik.slo + gik.pad, gik.pitch);
          zkr[qb][kb] = bload8(rzk, j < N
              ? static_cast<uint32_t>((gik.base + (j - gk0) * gik.pitch + c0) * 2) : kOob);
        }
    }
    if (STZQ) load_zq(it + 1);
    load_tile(rl, i0 + 2 * kT);

    const bool computed = it >= itw && (!SEG || (i0 < sw.uhi && i0 + kT > sw.ulo));
    if (computed) {
      const bf16* Qs = sq[buf];
      const bf16* Ds = sd[buf];
      // per block (uniform): does the tile reach it, and its region; on
      // saturated tiles the key's boundary entry is the initial value of the
      // S accumulator.  A block the tile does not reach is block 1 (block 0
      // starts first), so block 0's products are always made.
      bool sat_lo[2], sat_hi[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sat_lo[kb] = it < n_lo[kb];
        sat_hi[kb] = it >= t_hi[kb];
      }
      const bool both = PAIR ? it >= itk[1] : true;
      floatx4 s[2][2], dp[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const float k0 = (KC && (sat_lo[kb] || sat_hi[kb])) ? (sat_hi[kb] ? khi[kb] : klo[kb]) : 0.f;
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          s[qb][kb] = floatx4{k0, k0, k0, k0};
          dp[qb][kb] = floatx4{0.f, 0.f, 0.f, 0.f};
        }
      }
#pragma unroll
      for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const bf16x8 qa = *reinterpret_cast<const bf16x8*>(Qs + (16 * qb + c16) * kP + 32 * c + 8 * g);
          const bf16x8 da = *reinterpret_cast<const bf16x8*>(Ds + (16 * qb + c16) * kP + 32 * c + 8 * g);
          s[qb][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa, kf[0][c], s[qb][0], 0, 0, 0);
          dp[qb][0] = mma16<HP>(da, vf[0][c], dp[qb][0]);
          if (both) {
            s[qb][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa, kf[1][c], s[qb][1], 0, 0, 0);
            dp[qb][1] = mma16<HP>(da, vf[1][c], dp[qb][1]);
          }
        }
      }

      // pure: a band tile without any pair |delta| >= D (every tile of an
      // identity map), whose selects are skipped
      bool pure[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int ja = jbase[PAIR ? kb : 0], jz = jbase[PAIR ? kb : 1] + 15;
        pure[kb] = IT || (i0 - jz > -D && i0 + kT - 1 - ja < D);
      }
      bool need_mask[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        need_mask[kb] = (i0 + kT > N) || (jbase[PAIR ? kb : 1] + 16 > N) ||
                        (CAUSAL && i0 < jbase[PAIR ? kb : 1] + 15) ||
                        (SEG && (i0 < sw.ilo || i0 + kT > sw.ihi));
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const int i1 = i0 + 16 * qb + 4 * g;
        const int qo = 16 * qb + 4 * g;
        const floatx4 ql2 = *reinterpret_cast<const floatx4*>(&sqs[buf][0][qo]);
        const floatx4 qrl = *reinterpret_cast<const floatx4*>(&sqs[buf][2][qo]);
        const floatx4 qrh = *reinterpret_cast<const floatx4*>(&sqs[buf][3][qo]);
        if (!PAIR && (sat_lo[0] || sat_hi[0])) {
          // saturated tile (both blocks): the query's entry and L fold into
          // one offset per query (the key's entry is already in the
          // accumulator)
          float cq[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) cq[t] = fmaf(sat_hi[0] ? qrh[t] : qrl[t], sl2, -ql2[t]);
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int t = 0; t < 4; ++t) s[qb][kb][t] = fast_exp2(fmaf(s[qb][kb][t], sl2, cq[t]));
          continue;
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          if (kb == 1 && !both) continue;
          if (PAIR && (sat_lo[kb] || sat_hi[kb])) {
            // saturated tile: the query's entry and L fold into one offset
            // per query (the key's entry is already in the accumulator)
            float cq[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) cq[t] = fmaf(sat_hi[kb] ? qrh[t] : qrl[t], sl2, -ql2[t]);
#pragma unroll
            for (int t = 0; t < 4; ++t) s[qb][kb][t] = fast_exp2(fmaf(s[qb][kb][t], sl2, cq[t]));
            continue;
          }
          const int j = jbase[kb] + c16;
          float rel[4];
          {
            float zk[4] = {0.f, 0.f, 0.f, 0.f};
            if (F & F_ZK) {
              const halfx4 hv = __builtin_bit_cast(halfx4, zkr[qb][kb]);
#pragma unroll
              for (int t = 0; t < 4; ++t) zk[t] = static_cast<float>(hv[t]);  // ascending
            }
            halfx4 zq4 = halfx4{0, 0, 0, 0};
            if (STZQ)  // Z^Q[i1 + t][i1 + t - j + D], t = 0..3
              zq4 = __builtin_bit_cast(halfx4, lds_tr4(reinterpret_cast<const bf16*>(szq[buf]), kZP,
                                                       16 * qb + 4 * g, jloc[kb], c16));
            float zi[4] = {0.f, 0.f, 0.f, 0.f};
            if constexpr (IT) {
              // the 32-row window of query block qb against key block kb
              // (rows sb + 0..31, sb = i0 + 16 qb - jbase[kb] - 15 + D) on
              // MFMA, through the wave's scratch; pair (i1 + t, j) sits at
              // window row 4 g + t - c16 + 15 of query row 4 g + t
              bf16x8 q2[2];
#pragma unroll
              for (int c = 0; c < 2; ++c)
                q2[c] = *reinterpret_cast<const bf16x8*>(Qs + (16 * qb + c16) * kP + 32 * c + 8 * g);
              floatx4 zw[2];
              it_rows<2>(itb, i0 + 16 * qb - jbase[kb] - 15 + D, q2[0], q2[1], c16, g, zw);
              it_put<2>(scr, kKwP, c16, g, zw);
              const float* zr = scr + (4 * g) * (kKwP + 1) + 15 - c16;
#pragma unroll
              for (int t = 0; t < 4; ++t) zi[t] = zr[t * (kKwP + 1)];
            }
            if (pure[kb]) {
#pragma unroll
              for (int t = 0; t < 4; ++t) {
                float band = kmid[kb] + zk[t];
                if (F & F_ZQ) band += static_cast<float>(zq4[t]);
                if (IT) band += zi[t];
                if (F & F_BT)
                  band += bloadf(rbt, static_cast<uint32_t>(iclamp(i1 + t - j + D, 0, 2 * D) * 4));
                rel[t] = band;
              }
            } else {
#pragma unroll
              for (int t = 0; t < 4; ++t) {
                const int i = i1 + t;
                const int dl = i - j;
                float band = kmid[kb] + zk[t];
                if (F & F_ZQ) band += static_cast<float>(zq4[t]);
                if (F & F_BT) band += bloadf(rbt, static_cast<uint32_t>(iclamp(dl + D, 0, 2 * D) * 4));
                rel[t] = dl >= D ? (qrh[t] + khi[kb]) : (dl <= -D ? (qrl[t] + klo[kb]) : band);
              }
            }
          }
#pragma unroll
          for (int t = 0; t < 4; ++t) s[qb][kb][t] = fast_exp2(fmaf(s[qb][kb][t] + rel[t], sl2, -ql2[t]));
        }
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (kb == 1 && (!PAIR || !both)) continue;
        if (need_mask[kb]) {
          // (the empty asm keeps this a branch: without it the compiler turns
          // the rare masked pass into selects on every tile)
          asm volatile("");
#pragma unroll
          for (int kx = 0; kx < 2; ++kx) {
            if (PAIR && kx != kb) continue;  // without PAIR one pass masks both blocks
            const int j = jbase[kx] + c16;
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
#pragma unroll
              for (int t = 0; t < 4; ++t) {
                const int i = i0 + 16 * qb + 4 * g + t;
                const bool off_seg = SEG && (i < sgl[kx] || i >= sgh[kx]);
                s[qb][kx][t] = (j >= N || (CAUSAL && j > i) || off_seg) ? 0.f : s[qb][kx][t];
              }
          }
        }
      }
      // G' = P (dP - D)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const floatx4 qdd = *reinterpret_cast<const floatx4*>(&sqs[buf][1][16 * qb + 4 * g]);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          if constexpr ((F & F_DROP) != 0) {
            // dropout: G' = P (dP keep scale - D), and dV takes P keep (0 or
            // 1; the keep scale multiplies the finished dV in fp32)
            float mk[4] = {1.f, 1.f, 1.f, 1.f};
            if (DROP) keep_col4(a, bh, i0 + 16 * qb + 4 * g, jbase[kb] + c16, 1.f, mk);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              dp[qb][kb][t] = s[qb][kb][t] * fmaf(dp[qb][kb][t], mk[t] * a.drop_scale, -qdd[t]);
              s[qb][kb][t] *= mk[t];
            }
          } else {
#pragma unroll
            for (int t = 0; t < 4; ++t) dp[qb][kb][t] = s[qb][kb][t] * (dp[qb][kb][t] - qdd[t]);
          }
        }
      }

      // with key offset gradients the next tiles go to the other LDS buffers
      // (last read in the previous step, before its closing barrier) here,
      // ahead of the offset-gradient stores, so the waits for their loads do
      // not count those stores
      if (DZ) {
        store_tile(rs, buf ^ 1, i0 + kT);
        if (STZQ) store_zq(buf ^ 1);
      }

      // key offset gradients and column sums
      if (DZ && !CS && !PAIR && (sat_lo[0] || sat_hi[0])) {
        // a saturated tile (both blocks: without pairing they share the
        // wave's range): every key's sum of G' goes to one boundary entry,
        // one uniform branch instead of a three-way branch per block
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const float g0 = (dp[0][kb][0] + dp[0][kb][1]) + (dp[0][kb][2] + dp[0][kb][3]);
          const float g1 = (dp[1][kb][0] + dp[1][kb][1]) + (dp[1][kb][2] + dp[1][kb][3]);
          if (sat_lo[0])
            blo[kb] += g0 + g1;
          else
            bhi[kb] += g0 + g1;
        }
      } else if (DZ || CS) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          if (kb == 1 && !both) continue;
          const int j = jbase[kb] + c16;
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            const int i1 = i0 + 16 * qb + 4 * g;
            const float gs = (dp[qb][kb][0] + dp[qb][kb][1]) + (dp[qb][kb][2] + dp[qb][kb][3]);
            if (CS) csum[kb] += gs;
            if (DZ) {
              if (sat_lo[kb]) {
                blo[kb] += gs;
              } else if (sat_hi[kb]) {
                bhi[kb] += gs;
              } else {
                float run[4];
                bool any = false;
                if (pure[kb]) {
#pragma unroll
                  for (int t = 0; t < 4; ++t) {
                    const int i = i1 + t;
                    run[t] = tau * dp[qb][kb][t];  // ascending columns
                    any = any || (i < N && j < N && (!CAUSAL || j <= i));
                  }
                } else {
#pragma unroll
                  for (int t = 0; t < 4; ++t) {
                    const int i = i1 + t;
                    const int dl = i - j;
                    const float gg = dp[qb][kb][t];
                    float bandv = 0.f;
                    if (dl >= D)
                      bhi[kb] += gg;
                    else if (dl <= -D)
                      blo[kb] += gg;
                    else {
                      bandv = tau * gg;
                      any = any || (i < N && j < N && (!CAUSAL || j <= i));
                    }
                    run[t] = bandv;  // ascending columns
                  }
                }
                if (any) {
                  bf16* row = reinterpret_cast<bf16*>(a.dz) + static_cast<int64_t>(bh) * a.dz_bh +
                              gik.base + static_cast<int64_t>(j - gk0) * gik.pitch;
                  store4(row + ((i1 - j + D) - gik.slo + gik.pad), run);
                }
              }
            }
          }
        }
      }

      // dV^T += dO^T P ; dK^T += Q^T G  (K axis: the tile's 32 queries, in the
      // order 4g + e, 16 + 4g + e of the lanes' own values)
      {
        bf16x8 pf[2], gf[2], gl[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float x = s[e >> 2][kb][e & 3];
            const float y = dp[e >> 2][kb][e & 3];
            pf[kb][e] = op16<HP>(x);
            gf[kb][e] = static_cast<bf16>(y);
            if (SPLIT) gl[kb][e] = static_cast<bf16>(y - static_cast<float>(gf[kb][e]));
          }
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const bf16x4 dlo = lds_tr4(Ds, kP, 4 * g, 16 * db, c16);
          const bf16x4 dhi = lds_tr4(Ds, kP, 16 + 4 * g, 16 * db, c16);
          const bf16x4 qlo = lds_tr4(Qs, kP, 4 * g, 16 * db, c16);
          const bf16x4 qhi = lds_tr4(Qs, kP, 16 + 4 * g, 16 * db, c16);
          bf16x8 dt8, qt8;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            dt8[e] = dlo[e];
            dt8[e + 4] = dhi[e];
            qt8[e] = qlo[e];
            qt8[e + 4] = qhi[e];
          }
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            if (kb == 1 && !both) continue;
            dv[kb][db] = mma16<HP>(dt8, pf[kb], dv[kb][db]);
            dk[kb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qt8, gf[kb], dk[kb][db], 0, 0, 0);
            if (SPLIT)
              dk[kb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qt8, gl[kb], dk[kb][db], 0, 0, 0);
          }
        }
      }
    }

    // (stored also after the last tile, into the buffer no one reads again:
    // with no branch around them the compiler's wait counts stay exact)
    if (!DZ || !computed) {
      store_tile(rs, buf ^ 1, i0 + kT);
      if (STZQ) store_zq(buf ^ 1);
    }
    __syncthreads();
  };
  // two steps per iteration so the register sets swap roles without copies;
  // the loop is left from either step, so the back edge carries exact counts
  for (int it = it_first; it < it_end;) {
    tile_step(it, ra, rb);
    if (++it >= it_end) break;
    tile_step(it, rb, ra);
    if (++it >= it_end) break;
  }

#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int j = jbase[kb] + c16;
    const float lo = tau * wave_sum_g(blo[kb]);
    const float hi = tau * wave_sum_g(bhi[kb]);
    const float cs = tau * wave_sum_g(csum[kb]);
    if (j >= N || !kon[kb]) continue;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const float dsc = DROP ? a.drop_scale : 1.f;
      float dvv[4] = {dsc * dv[kb][db][0], dsc * dv[kb][db][1], dsc * dv[kb][db][2],
                      dsc * dv[kb][db][3]};
      store_out4(a.dv, (tok + j) * 64 + 16 * db + 4 * g, a.out_f32 != 0, dvv);
      float dkv[4] = {tau * dk[kb][db][0], tau * dk[kb][db][1], tau * dk[kb][db][2],
                      tau * dk[kb][db][3]};
      store4(a.dkacc + (tok + j) * 64 + 16 * db + 4 * g, dkv);
    }
    if (g == 0) {
      if (DZ) {
        a.bndk[(tok + j) * 2 + 0] = lo;
        a.bndk[(tok + j) * 2 + 1] = hi;
      }
      if (CS) a.colsum[tok + j] = cs;
    }
  }
}

template <int F>
hipError_t launch_kf(const AttnArgs& a, int B, hipStream_t s) {
  constexpr bool PAIR = (F & F_CAUSAL) && !(F & F_ZK) && !(F & F_DZK);
  // PAIR: workgroup m owns 16-key blocks 4m .. 4m+3 and their mirrors
  const int n16 = (a.N + 15) / 16;
  const int nkb = PAIR ? ((n16 + 1) / 2 + 3) / 4 : (a.N + 127) / 128;
  const int total = nkb * B * a.H;
  const int xcd_map = (F & F_CAUSAL) ? 0 : 1;
  hipLaunchKernelGGL((bwd_k_fast<F>), dim3(total), dim3(256), 0, s, a, nkb, total, xcd_map);
  return hipGetLastError();
}

#define RP_KF_FLAGS(X)                                                                    \
  X(0) X(F_ZQ) X(F_BT) X(F_ZQ | F_ZK | F_DZK) X(F_ZK | F_DZK) X(F_ZK | F_BT | F_DZK)     \
  X(F_U) X(F_ZQ | F_U) X(F_BT | F_U) X(F_ZQ | F_ZK | F_DZK | F_U) X(F_ZK | F_DZK | F_U)   \
  X(F_ZK | F_BT | F_DZK | F_U)

template <int SPL>
hipError_t dispatch_kf(int flags, const AttnArgs& a, int B, hipStream_t s) {
  const int f = flags & (F_ZQ | F_ZK | F_BT | F_CAUSAL | F_DZK | F_U);
  switch (f) {
#define RP_CASE(X)                                   \
  case X:                                            \
    return launch_kf<(X) | SPL>(a, B, s);            \
  case (X) | F_CAUSAL:                               \
    return launch_kf<(X) | F_CAUSAL | SPL>(a, B, s);
    RP_KF_FLAGS(RP_CASE)
#undef RP_CASE
    default:
      return hipErrorInvalidValue;
  }
}

// in-tile products (F_IT): A^Q with or without the u term
template <int SPL>
hipError_t dispatch_kit(int flags, const AttnArgs& a, int B, hipStream_t s) {
  switch (flags & (F_IT | F_U | F_CAUSAL)) {
    case F_IT:
      return launch_kf<F_IT | SPL>(a, B, s);
    case F_IT | F_CAUSAL:
      return launch_kf<F_IT | F_CAUSAL | SPL>(a, B, s);
    case F_IT | F_U:
      return launch_kf<F_IT | F_U | SPL>(a, B, s);
    case F_IT | F_U | F_CAUSAL:
      return launch_kf<F_IT | F_U | F_CAUSAL | SPL>(a, B, s);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace

}  // namespace relpos
