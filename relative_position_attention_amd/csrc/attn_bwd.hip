// Backward attention passes for fp32 inputs ([RPA] Table 9 "Query-parallel
// pass" and "Key-parallel pass", Algorithm 2; bf16 inputs run bwd_q_fast.hip
// and bwd_k_fast.hip).
// F_SEG adds segment masks (tested on every pair), F_DROP dropout
// (G = tau P (dP keep - D), dV takes P keep), as defined in extras.hpp.  [RPA] = "Fast and Exact Relative-
// Position Attention via Structure-Aware Kernels" (arXiv 2611.01182).
//
// Both passes rebuild each score tile from the saved logsumexp L and
// D = rowdot(dO, O): P = exp(S - L), dS = P * (dO V^T - D) ([RPA] §3.1
// Eq. (3), App. B.2 tile-locality lemma).  With G = tau dS:
//
//  * query pass: one workgroup owns 128 queries and writes dQ_acc = G K and
//    the query offset gradients dZ~^Q[i, s] = G_ij, s = i - j + D, one entry
//    per (query, offset) and a single writer each ([RPA] §4.2, Prop. B.9);
//    pairs with delta >= D / delta <= -D go to two fp32 on-chip boundary sums
//    per query ([RPA] §4.2 "Local Boundary Sums").
//  * key pass: one workgroup owns 128 keys and writes dV = P^T dO,
//    dK_acc = G^T Q, the key offset gradients dZ~^K[j, s] and boundary sums,
//    and (Transformer-XL u term) the key column sums of G.
// No atomics anywhere: every output element has one writer and a fixed
// summation order, so the results are bitwise reproducible.
#include "extras.hpp"
#include "relation.hpp"
#include "tiles.hpp"

namespace relpos {

namespace {

// ------------------------------------------------------------------------
// Query-parallel pass
// ------------------------------------------------------------------------
template <typename T, int F>
__global__ __launch_bounds__(256) void attn_bwd_q_kernel(AttnArgs a) {
  using M = Mma<T>;
  using Frag = typename M::frag;
  // offset gradients whose plain sums are needed (a scalar bias, or the
  // Transformer-XL v term) cancel (rows of dS sum to zero): kept in fp32
  using GT = typename DzType<T, (F & F_DZ32) != 0>::type;
  constexpr int E = M::E;
  constexpr int KS = M::KS;
  constexpr int NST = 64 / KS;
  constexpr int P = TileP<T>::P;
  constexpr bool CAUSAL = (F & F_CAUSAL) != 0;
  constexpr bool DZ = (F & F_DZQ) != 0;
  constexpr bool EXT = (F & (F_SEG | F_DROP)) != 0;
  __shared__ __attribute__((aligned(16))) T lds[2][3][64 * P];  // K rows, K^T, V rows

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = wave_index(), g = lane >> 4, c16 = lane & 15;
  const int N = a.N, D = a.D;
  const int nqb = (N + 127) / 128;
  const int qblk = CAUSAL ? (nqb - 1 - static_cast<int>(blockIdx.x)) : static_cast<int>(blockIdx.x);
  const int bh = blockIdx.y;
  const int h = bh % a.H;
  const int64_t tok = static_cast<int64_t>(bh) * N;
  const int i0 = qblk * 128;
  const int ilast = imin(N - 1, i0 + 127);
  const int iw = i0 + 32 * wave;
  const T* q = reinterpret_cast<const T*>(a.q) + tok * 64;
  const T* k = reinterpret_cast<const T*>(a.k) + tok * 64;
  const T* v = reinterpret_cast<const T*>(a.v) + tok * 64;
  const T* dout = reinterpret_cast<const T*>(a.dout) + tok * 64;

  Frag qf[2][NST], df[2][NST];
  float rlo[2], rhi[2], l2[2], dd[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int i = iw + 16 * qb + c16;
    const bool ok = i < N;
#pragma unroll
    for (int c = 0; c < NST; ++c) {
      qf[qb][c] = ok ? M::load(q + static_cast<int64_t>(i) * 64 + c * KS + g * E) : M::zero();
      df[qb][c] = ok ? M::load(dout + static_cast<int64_t>(i) * 64 + c * KS + g * E) : M::zero();
    }
    rlo[qb] = ok ? a.rowlo[tok + i] : 0.f;
    rhi[qb] = ok ? a.rowhi[tok + i] : 0.f;
    l2[qb] = ok ? a.lse[tok + i] * kLog2e : INFINITY;  // P = 0 on padding rows
    if (EXT && !(l2[qb] > -INFINITY)) l2[qb] = INFINITY;  // a row with no key
    dd[qb] = ok ? a.dvec[tok + i] : 0.f;
  }
  GroupInfo giq = {0, 0, 0, 0};
  if ((F & F_ZQ) || DZ) giq = a.gq[i0 / kGroup];
  const bool SEG = (F & F_SEG) != 0 && a.seg != nullptr;
  const bool DROP = (F & F_DROP) != 0 && a.drop_p8 > 0;
  int sgl[2] = {0, 0}, sgh[2] = {0, 0};
  if (SEG) {
    const int64_t brow = static_cast<int64_t>(bh / a.H) * N;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int i = iw + 16 * qb + c16;
      if (i < N) token_segment(a, brow, i, sgl[qb], sgh[qb]);
    }
  }

  const int nkt = CAUSAL ? (ilast / 64 + 1) : (N + 63) / 64;
  int n_hi = (i0 - D - 63 >= 0) ? (i0 - D - 63) / 64 + 1 : 0;
  n_hi = imin(n_hi, nkt);
  int t_lo = CAUSAL ? nkt : (ilast + D + 63) / 64;
  t_lo = imax(n_hi, imin(t_lo, nkt));

  floatx4 dq[2][4];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < 4; ++db) dq[qb][db] = floatx4{0.f, 0.f, 0.f, 0.f};
  float blo[2] = {0.f, 0.f}, bhi[2] = {0.f, 0.f};

  Stage<T> sk, sv;
  sk.init(tid);
  sv.init(tid);
  sk.load(k, 0, N);
  sv.load(v, 0, N);
  sk.store_rows(lds[0][0]);
  sk.store_trans(lds[0][1]);
  sv.store_rows(lds[0][2]);
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    const int j0 = kt * 64;
    if (kt + 1 < nkt) {
      sk.load(k, j0 + 64, N);
      sv.load(v, j0 + 64, N);
    }
    const T* Ks = lds[buf][0];
    const T* Kt = lds[buf][1];
    const T* Vs = lds[buf][2];

    floatx4 s[2][4], dp[2][4];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        s[qb][kb] = floatx4{0.f, 0.f, 0.f, 0.f};
        dp[qb][kb] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
    for (int c = 0; c < NST; ++c) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        Frag kf = frag_rows<T>(Ks, 16 * kb + c16, c, g);
        Frag vf = frag_rows<T>(Vs, 16 * kb + c16, c, g);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          s[qb][kb] = M::run(kf, qf[qb][c], s[qb][kb]);    // S^T = K Q^T
          dp[qb][kb] = M::run(vf, df[qb][c], dp[qb][kb]);  // dP^T = V dO^T
        }
      }
    }

    GroupInfo gik = {0, 0, 0, 0};
    const int gk0 = (j0 / kGroup) * kGroup;
    if (F & F_ZK) gik = a.gk[j0 / kGroup];
    const bool need_mask = (j0 + 64 > N) || (CAUSAL && j0 + 63 > iw) || SEG;
    const int region = kt < n_hi ? SAT_HI : (kt < t_lo ? BAND : SAT_LO);
    float gv[2][4][4];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int i = iw + 16 * qb + c16;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int j1 = j0 + 16 * kb + 4 * g;
        float acc[4] = {s[qb][kb][0], s[qb][kb][1], s[qb][kb][2], s[qb][kb][3]};
        if (region == SAT_HI)
          relation_qrow<T, F, SAT_HI>(a, tok, h, i, rlo[qb], rhi[qb], giq, gik, gk0, j1, acc);
        else if (region == BAND)
          relation_qrow<T, F, BAND>(a, tok, h, i, rlo[qb], rhi[qb], giq, gik, gk0, j1, acc);
        else
          relation_qrow<T, F, SAT_LO>(a, tok, h, i, rlo[qb], rhi[qb], giq, gik, gk0, j1, acc);
        // dropout: dP of a dropped pair is 0, of a kept one times the scale
        float mk[4] = {1.f, 1.f, 1.f, 1.f};
        if (DROP) keep_row4(a, bh, i, j1, a.drop_scale, mk);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          float xv = acc[t] * a.scale_log2;
          if (need_mask) {
            const int j = j1 + t;
            if (j >= N || (CAUSAL && j > i) || (SEG && (j < sgl[qb] || j >= sgh[qb])))
              xv = -INFINITY;
          }
          const float p = fast_exp2(xv - l2[qb]);
          gv[qb][kb][t] = a.scale * p * (dp[qb][kb][t] * mk[t] - dd[qb]);
        }
        if (DZ) {
          if (region == SAT_HI) {
            bhi[qb] += gv[qb][kb][0] + gv[qb][kb][1] + gv[qb][kb][2] + gv[qb][kb][3];
          } else if (region == SAT_LO) {
            blo[qb] += gv[qb][kb][0] + gv[qb][kb][1] + gv[qb][kb][2] + gv[qb][kb][3];
          } else {
            float run[4];
            bool any = false;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const int j = j1 + t;
              const int dl = i - j;
              const float gg = gv[qb][kb][t];
              const bool valid = i < N && j < N && (!CAUSAL || j <= i);
              float bandv = 0.f;
              if (dl >= D)
                bhi[qb] += gg;
              else if (dl <= -D)
                blo[qb] += gg;
              else {
                bandv = gg;
                any = any || valid;
              }
              run[3 - t] = bandv;  // descending columns
            }
            if (any) {
              GT* row = reinterpret_cast<GT*>(a.dz) + static_cast<int64_t>(bh) * a.dz_bh +
                        giq.base + static_cast<int64_t>(i - i0) * giq.pitch;
              const int c0 = (i - (j1 + 3) + D) - giq.slo + giq.pad;
              store4(row + c0, run);
            }
          }
        }
      }
    }

    // dQ^T += K^T G^T
#pragma unroll
    for (int c = 0; c < NST; ++c) {
      Frag gf[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) gf[qb] = frag_regs<T, 4>(gv[qb], c);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        Frag kf = frag_perm<T>(Kt, 16 * db + c16, c, g);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) dq[qb][db] = M::run(kf, gf[qb], dq[qb][db]);
      }
    }

    if (kt + 1 < nkt) {
      sk.store_rows(lds[buf ^ 1][0]);
      sk.store_trans(lds[buf ^ 1][1]);
      sv.store_rows(lds[buf ^ 1][2]);
    }
    __syncthreads();
  }

#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int i = iw + 16 * qb + c16;
    const float lo = wave_sum_g(blo[qb]);
    const float hi = wave_sum_g(bhi[qb]);
    if (i >= N) continue;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      float vals[4] = {dq[qb][db][0], dq[qb][db][1], dq[qb][db][2], dq[qb][db][3]};
      store4(a.dqacc + (tok + i) * 64 + 16 * db + 4 * g, vals);
    }
    if (DZ && g == 0) {
      a.bndq[(tok + i) * 2 + 0] = lo;
      a.bndq[(tok + i) * 2 + 1] = hi;
    }
  }
}

// ------------------------------------------------------------------------
// Key-parallel pass
// ------------------------------------------------------------------------
template <typename T, int F>
__global__ __launch_bounds__(256) void attn_bwd_k_kernel(AttnArgs a) {
  using M = Mma<T>;
  using Frag = typename M::frag;
  using GT = typename Store<T>::G;
  constexpr int E = M::E;
  constexpr int KS = M::KS;
  constexpr int NST = 64 / KS;
  constexpr int P = TileP<T>::P;
  constexpr bool CAUSAL = (F & F_CAUSAL) != 0;
  constexpr bool DZ = (F & F_DZK) != 0;
  constexpr bool CS = (F & F_U) != 0;
  constexpr bool EXT = (F & (F_SEG | F_DROP)) != 0;
  __shared__ __attribute__((aligned(16))) T lds[2][4][64 * P];  // Q rows, Q^T, dO rows, dO^T

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = wave_index(), g = lane >> 4, c16 = lane & 15;
  const int N = a.N, D = a.D;
  const int bh = blockIdx.y;
  const int h = bh % a.H;
  const int64_t tok = static_cast<int64_t>(bh) * N;
  const int j0b = static_cast<int>(blockIdx.x) * 128;
  const int jlast = imin(N - 1, j0b + 127);
  const int jw = j0b + 32 * wave;
  const T* q = reinterpret_cast<const T*>(a.q) + tok * 64;
  const T* k = reinterpret_cast<const T*>(a.k) + tok * 64;
  const T* v = reinterpret_cast<const T*>(a.v) + tok * 64;
  const T* dout = reinterpret_cast<const T*>(a.dout) + tok * 64;

  Frag kf[2][NST], vf[2][NST];
  float klo[2], khi[2], kmid[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int j = jw + 16 * kb + c16;
    const bool ok = j < N;
#pragma unroll
    for (int c = 0; c < NST; ++c) {
      kf[kb][c] = ok ? M::load(k + static_cast<int64_t>(j) * 64 + c * KS + g * E) : M::zero();
      vf[kb][c] = ok ? M::load(v + static_cast<int64_t>(j) * 64 + c * KS + g * E) : M::zero();
    }
    klo[kb] = ok ? a.keylo[tok + j] : 0.f;
    khi[kb] = ok ? a.keyhi[tok + j] : 0.f;
    kmid[kb] = ok ? a.keymid[tok + j] : 0.f;
  }
  GroupInfo gik = {0, 0, 0, 0};
  if ((F & F_ZK) || DZ) gik = a.gk[j0b / kGroup];
  const bool SEG = (F & F_SEG) != 0 && a.seg != nullptr;
  const bool DROP = (F & F_DROP) != 0 && a.drop_p8 > 0;
  int sgl[2] = {0, 0}, sgh[2] = {0, 0};
  if (SEG) {
    const int64_t brow = static_cast<int64_t>(bh / a.H) * N;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int j = jw + 16 * kb + c16;
      if (j < N) token_segment(a, brow, j, sgl[kb], sgh[kb]);
    }
  }

  // query tiles, ascending: saturated-low, band, saturated-high
  const int nqt = (N + 63) / 64;
  const int it0 = CAUSAL ? j0b / 64 : 0;
  int n_lo = CAUSAL ? it0 : ((j0b - D - 63 >= 0) ? (j0b - D - 63) / 64 + 1 : 0);
  n_lo = imax(it0, imin(n_lo, nqt));
  int t_hi = (jlast + D + 63) / 64;
  t_hi = imax(n_lo, imin(t_hi, nqt));

  floatx4 dvacc[2][4], dkacc[2][4];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      dvacc[kb][db] = floatx4{0.f, 0.f, 0.f, 0.f};
      dkacc[kb][db] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
  float blo[2] = {0.f, 0.f}, bhi[2] = {0.f, 0.f}, csum[2] = {0.f, 0.f};

  Stage<T> sq, sd;
  sq.init(tid);
  sd.init(tid);
  if (it0 < nqt) {
    sq.load(q, it0 * 64, N);
    sd.load(dout, it0 * 64, N);
    sq.store_rows(lds[0][0]);
    sq.store_trans(lds[0][1]);
    sd.store_rows(lds[0][2]);
    sd.store_trans(lds[0][3]);
  }
  __syncthreads();

  for (int it = it0; it < nqt; ++it) {
    const int buf = (it - it0) & 1;
    const int i0 = it * 64;
    if (it + 1 < nqt) {
      sq.load(q, i0 + 64, N);
      sd.load(dout, i0 + 64, N);
    }
    const T* Qs = lds[buf][0];
    const T* Qt = lds[buf][1];
    const T* Ds = lds[buf][2];
    const T* Dt = lds[buf][3];

    floatx4 s[4][2], dp[4][2];  // [qb][kb], S = Q K^T, dP = dO V^T
#pragma unroll
    for (int qb = 0; qb < 4; ++qb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[qb][kb] = floatx4{0.f, 0.f, 0.f, 0.f};
        dp[qb][kb] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
    for (int c = 0; c < NST; ++c) {
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) {
        Frag qa = frag_rows<T>(Qs, 16 * qb + c16, c, g);
        Frag da = frag_rows<T>(Ds, 16 * qb + c16, c, g);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          s[qb][kb] = M::run(qa, kf[kb][c], s[qb][kb]);
          dp[qb][kb] = M::run(da, vf[kb][c], dp[qb][kb]);
        }
      }
    }

    GroupInfo giq = {0, 0, 0, 0};
    const int gq0 = (i0 / kGroup) * kGroup;
    if (F & F_ZQ) giq = a.gq[i0 / kGroup];
    const bool need_mask = (i0 + 64 > N) || (j0b + 128 > N) || (CAUSAL && i0 < jw + 31) || SEG;
    const int region = it < n_lo ? SAT_LO : (it < t_hi ? BAND : SAT_HI);
    float pv[2][4][4], gv[2][4][4];  // [kb][qb][t]
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      const int i1 = i0 + 16 * qb + 4 * g;
      float l2[4], dd[4], rl[4], rh[4];
      load4_guard(a.lse + tok, i1, N, l2);
      load4_guard(a.dvec + tok, i1, N, dd);
      load4_guard(a.rowlo + tok, i1, N, rl);
      load4_guard(a.rowhi + tok, i1, N, rh);
#pragma unroll
      for (int t = 0; t < 4; ++t) l2[t] = (i1 + t < N) ? l2[t] * kLog2e : INFINITY;
      if (EXT) {  // a row with no key (L = -inf): P = 0
#pragma unroll
        for (int t = 0; t < 4; ++t) l2[t] = l2[t] > -INFINITY ? l2[t] : INFINITY;
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int j = jw + 16 * kb + c16;
        float acc[4] = {s[qb][kb][0], s[qb][kb][1], s[qb][kb][2], s[qb][kb][3]};
        if (region == SAT_HI)
          relation_krow<T, F, SAT_HI>(a, tok, h, j, klo[kb], khi[kb], kmid[kb], rl, rh, giq, gq0,
                                      gik, i1, acc);
        else if (region == BAND)
          relation_krow<T, F, BAND>(a, tok, h, j, klo[kb], khi[kb], kmid[kb], rl, rh, giq, gq0,
                                    gik, i1, acc);
        else
          relation_krow<T, F, SAT_LO>(a, tok, h, j, klo[kb], khi[kb], kmid[kb], rl, rh, giq, gq0,
                                      gik, i1, acc);
        // dropout: G = tau P (dP keep - D), and dV takes P keep
        float mk[4] = {1.f, 1.f, 1.f, 1.f};
        if (DROP) keep_col4(a, bh, i1, j, a.drop_scale, mk);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          float xv = acc[t] * a.scale_log2;
          if (need_mask) {
            const int i = i1 + t;
            if (j >= N || i >= N || (CAUSAL && j > i) || (SEG && (i < sgl[kb] || i >= sgh[kb])))
              xv = -INFINITY;
          }
          const float p = fast_exp2(xv - l2[t]);
          pv[kb][qb][t] = p * mk[t];
          gv[kb][qb][t] = a.scale * p * (dp[qb][kb][t] * mk[t] - dd[t]);
        }
        if (CS) csum[kb] += gv[kb][qb][0] + gv[kb][qb][1] + gv[kb][qb][2] + gv[kb][qb][3];
        if (DZ) {
          if (region == SAT_HI) {
            bhi[kb] += gv[kb][qb][0] + gv[kb][qb][1] + gv[kb][qb][2] + gv[kb][qb][3];
          } else if (region == SAT_LO) {
            blo[kb] += gv[kb][qb][0] + gv[kb][qb][1] + gv[kb][qb][2] + gv[kb][qb][3];
          } else {
            float run[4];
            bool any = false;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const int i = i1 + t;
              const int dl = i - j;
              const float gg = gv[kb][qb][t];
              const bool valid = i < N && j < N && (!CAUSAL || j <= i);
              float bandv = 0.f;
              if (dl >= D)
                bhi[kb] += gg;
              else if (dl <= -D)
                blo[kb] += gg;
              else {
                bandv = gg;
                any = any || valid;
              }
              run[t] = bandv;  // ascending columns
            }
            if (any) {
              GT* row = reinterpret_cast<GT*>(a.dz) + static_cast<int64_t>(bh) * a.dz_bh +
                        gik.base + static_cast<int64_t>(j - j0b) * gik.pitch;
              const int c0 = (i1 - j + D) - gik.slo + gik.pad;
              store4(row + c0, run);
            }
          }
        }
      }
    }

    // dV^T += dO^T P ; dK^T += Q^T G
#pragma unroll
    for (int c = 0; c < NST; ++c) {
      Frag pf[2], gf[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        pf[kb] = frag_regs<T, 4>(pv[kb], c);
        gf[kb] = frag_regs<T, 4>(gv[kb], c);
      }
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        Frag da = frag_perm<T>(Dt, 16 * db + c16, c, g);
        Frag qa = frag_perm<T>(Qt, 16 * db + c16, c, g);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          dvacc[kb][db] = M::run(da, pf[kb], dvacc[kb][db]);
          dkacc[kb][db] = M::run(qa, gf[kb], dkacc[kb][db]);
        }
      }
    }

    if (it + 1 < nqt) {
      sq.store_rows(lds[buf ^ 1][0]);
      sq.store_trans(lds[buf ^ 1][1]);
      sd.store_rows(lds[buf ^ 1][2]);
      sd.store_trans(lds[buf ^ 1][3]);
    }
    __syncthreads();
  }

#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int j = jw + 16 * kb + c16;
    const float lo = wave_sum_g(blo[kb]);
    const float hi = wave_sum_g(bhi[kb]);
    const float cs = wave_sum_g(csum[kb]);
    if (j >= N) continue;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      float dvv[4] = {dvacc[kb][db][0], dvacc[kb][db][1], dvacc[kb][db][2], dvacc[kb][db][3]};
      store_out4(a.dv, (tok + j) * 64 + 16 * db + 4 * g, a.out_f32 != 0, dvv);
      float dkv[4] = {dkacc[kb][db][0], dkacc[kb][db][1], dkacc[kb][db][2], dkacc[kb][db][3]};
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

template <typename T, int F>
hipError_t launch_q(const AttnArgs& a, int B, hipStream_t s) {
  dim3 grid((a.N + 127) / 128, B * a.H);
  hipLaunchKernelGGL((attn_bwd_q_kernel<T, F>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename T, int F>
hipError_t launch_k(const AttnArgs& a, int B, hipStream_t s) {
  dim3 grid((a.N + 127) / 128, B * a.H);
  hipLaunchKernelGGL((attn_bwd_k_kernel<T, F>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

// The term combinations of the mechanisms: Shaw (ZQ), T5 (BT), DeBERTa
// (ZQ+ZK), Transformer-XL (ZQ+U), each with and without the causal mask,
// plus the plain and bias-with-key-table variants.
#define RP_QFLAGS(X)                                                         \
  X(0) X(F_ZQ | F_DZQ) X(F_ZQ | F_ZK | F_DZQ) X(F_ZK)                        \
  X(F_ZQ | F_DZQ | F_DZ32) X(F_BT | F_DZQ | F_DZ32) X(F_ZQ | F_ZK | F_DZQ | F_DZ32) \
  X(F_ZK | F_BT | F_DZQ | F_DZ32)

template <typename T, int EXTF>
hipError_t dispatch_q(int flags, const AttnArgs& a, int B, hipStream_t s) {
  const int f = flags & (F_ZQ | F_ZK | F_BT | F_CAUSAL | F_DZQ | F_DZ32);
  switch (f) {
#define RP_CASE(X)                                   \
  case X:                                            \
    return launch_q<T, (X) | EXTF>(a, B, s);          \
  case (X) | F_CAUSAL:                               \
    return launch_q<T, (X) | F_CAUSAL | EXTF>(a, B, s);
    RP_QFLAGS(RP_CASE)
#undef RP_CASE
    default:
      return hipErrorInvalidValue;
  }
}

#define RP_KFLAGS(X)                                                              \
  X(0) X(F_ZQ) X(F_BT) X(F_ZQ | F_ZK | F_DZK) X(F_ZK | F_DZK) X(F_ZK | F_BT | F_DZK) \
  X(F_U) X(F_ZQ | F_U) X(F_BT | F_U) X(F_ZQ | F_ZK | F_DZK | F_U) X(F_ZK | F_DZK | F_U) \
  X(F_ZK | F_BT | F_DZK | F_U)

template <typename T, int EXTF>
hipError_t dispatch_k(int flags, const AttnArgs& a, int B, hipStream_t s) {
  const int f = flags & (F_ZQ | F_ZK | F_BT | F_CAUSAL | F_DZK | F_U);
  switch (f) {
#define RP_CASE(X)                                   \
  case X:                                            \
    return launch_k<T, (X) | EXTF>(a, B, s);          \
  case (X) | F_CAUSAL:                               \
    return launch_k<T, (X) | F_CAUSAL | EXTF>(a, B, s);
    RP_KFLAGS(RP_CASE)
#undef RP_CASE
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_attn_bwd_q_f32(int flags, const AttnArgs& a, int B, hipStream_t s) {
  if (flags & (F_SEG | F_DROP)) return dispatch_q<float, F_SEG | F_DROP>(flags, a, B, s);
  return dispatch_q<float, 0>(flags, a, B, s);
}

hipError_t launch_attn_bwd_k_f32(int flags, const AttnArgs& a, int B, hipStream_t s) {
  if (flags & (F_SEG | F_DROP)) return dispatch_k<float, F_SEG | F_DROP>(flags, a, B, s);
  return dispatch_k<float, 0>(flags, a, B, s);
}

}  // namespace relpos
