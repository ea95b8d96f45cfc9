// Forward attention kernel for fp32 inputs ([RPA] Table 9 "Attention"; the
// forward of Algorithm 1; bf16 inputs run fwd_fast.hip).
// [RPA] = "Fast and Exact Relative-Position Attention via Structure-Aware
// Kernels" (arXiv 2611.01182).
//
// One workgroup of 4 waves owns 128 consecutive queries (one projection
// group: [RPA] §4.3.1 makes the group as large as the largest tile);
// each wave owns 32 of them.  Key tiles of 64 keys stream through LDS
// (double buffered: K row-major, V transposed).  Per tile:
//   S^T = K Q^T on MFMA (keys on rows, so every lane owns one query column),
//   relation terms by tile region (saturated tiles: one entry per query and
//   per key; band tiles: per-pair projections, [RPA] §4.1),
//   online softmax in base 2 with log2(e) folded into tau ([RPA] "Half-
//   precision numerics"; update of [RPA] §3.1 Eq. (2)),
//   O^T += V^T P^T on MFMA with P kept in registers.
// The key loop is split into its three ranges (saturated-high, band,
// saturated-low) once per workgroup from the tile's extreme offsets
// ([RPA] §4.3.3: the ranges are fixed before the loop instead of testing
// every tile).  F_SEG adds segment masks (tested on every pair), F_DROP dropout
// (P V takes P times the pair's keep factor), as defined in extras.hpp.
#include "extras.hpp"
#include "relation.hpp"
#include "tiles.hpp"

namespace relpos {

namespace {

template <typename T, int F>
__global__ __launch_bounds__(256) void attn_fwd_kernel(AttnArgs a) {
  using M = Mma<T>;
  using Frag = typename M::frag;
  constexpr int E = M::E;
  constexpr int KS = M::KS;
  constexpr int NST = 64 / KS;
  constexpr int P = TileP<T>::P;
  constexpr bool CAUSAL = (F & F_CAUSAL) != 0;
  constexpr bool EXT = (F & (F_SEG | F_DROP)) != 0;
  __shared__ __attribute__((aligned(16))) T lds[2][2][64 * P];

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

  Frag qf[2][NST];
  float rlo[2], rhi[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int i = iw + 16 * qb + c16;
#pragma unroll
    for (int c = 0; c < NST; ++c)
      qf[qb][c] = i < N ? M::load(q + static_cast<int64_t>(i) * 64 + c * KS + g * E) : M::zero();
    rlo[qb] = i < N ? a.rowlo[tok + i] : 0.f;
    rhi[qb] = i < N ? a.rowhi[tok + i] : 0.f;
  }
  GroupInfo giq = {0, 0, 0, 0};
  if (F & F_ZQ) giq = a.gq[i0 / kGroup];
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

  // key-tile ranges from the workgroup's extreme offsets
  const int nkt = CAUSAL ? (ilast / 64 + 1) : (N + 63) / 64;
  int n_hi = (i0 - D - 63 >= 0) ? (i0 - D - 63) / 64 + 1 : 0;
  n_hi = imin(n_hi, nkt);
  int t_lo = CAUSAL ? nkt : (ilast + D + 63) / 64;
  t_lo = imax(n_hi, imin(t_lo, nkt));

  float m[2] = {-INFINITY, -INFINITY};
  float l[2] = {0.f, 0.f};
  floatx4 o[2][4];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < 4; ++db) o[qb][db] = floatx4{0.f, 0.f, 0.f, 0.f};

  Stage<T> sk, sv;
  sk.init(tid);
  sv.init(tid);
  sk.load(k, 0, N);
  sv.load(v, 0, N);
  sk.store_rows(lds[0][0]);
  sv.store_trans(lds[0][1]);
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    const int j0 = kt * 64;
    if (kt + 1 < nkt) {
      sk.load(k, j0 + 64, N);
      sv.load(v, j0 + 64, N);
    }
    const T* Ks = lds[buf][0];
    const T* Vt = lds[buf][1];

    floatx4 s[2][4];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) s[qb][kb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NST; ++c) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        Frag kf = frag_rows<T>(Ks, 16 * kb + c16, c, g);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) s[qb][kb] = M::run(kf, qf[qb][c], s[qb][kb]);
      }
    }

    GroupInfo gik = {0, 0, 0, 0};
    const int gk0 = (j0 / kGroup) * kGroup;
    if (F & F_ZK) gik = a.gk[j0 / kGroup];
    const bool need_mask = (j0 + 64 > N) || (CAUSAL && j0 + 63 > iw) || SEG;
    float x[2][4][4];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int i = iw + 16 * qb + c16;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int j1 = j0 + 16 * kb + 4 * g;
        float acc[4] = {s[qb][kb][0], s[qb][kb][1], s[qb][kb][2], s[qb][kb][3]};
        if (kt < n_hi)
          relation_qrow<T, F, SAT_HI>(a, tok, h, i, rlo[qb], rhi[qb], giq, gik, gk0, j1, acc);
        else if (kt < t_lo)
          relation_qrow<T, F, BAND>(a, tok, h, i, rlo[qb], rhi[qb], giq, gik, gk0, j1, acc);
        else
          relation_qrow<T, F, SAT_LO>(a, tok, h, i, rlo[qb], rhi[qb], giq, gik, gk0, j1, acc);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          float xv = acc[t] * a.scale_log2;
          if (need_mask) {
            const int j = j1 + t;
            if (j >= N || (CAUSAL && j > i) || (SEG && (j < sgl[qb] || j >= sgh[qb])))
              xv = -INFINITY;
          }
          x[qb][kb][t] = xv;
        }
      }
    }

    // online softmax (base 2), per query row
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int t = 0; t < 4; ++t) mx = fmaxf(mx, x[qb][kb][t]);
      mx = wave_max_g(mx);
      const float mnew = fmaxf(m[qb], mx);
      const float muse = mnew == -INFINITY ? 0.f : mnew;
      const float alpha = fast_exp2(m[qb] - muse);
      m[qb] = mnew;
      float ls = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float p = fast_exp2(x[qb][kb][t] - muse);
          x[qb][kb][t] = p;
          ls += p;
        }
      l[qb] = l[qb] * alpha + ls;
#pragma unroll
      for (int db = 0; db < 4; ++db) o[qb][db] *= alpha;
    }
    if (DROP) {
      // P V takes the dropped probabilities (the row sums above keep P)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          float mk[4];
          keep_row4(a, bh, iw + 16 * qb + c16, j0 + 16 * kb + 4 * g, a.drop_scale, mk);
#pragma unroll
          for (int t = 0; t < 4; ++t) x[qb][kb][t] *= mk[t];
        }
    }

    // O^T += V^T P^T
#pragma unroll
    for (int c = 0; c < NST; ++c) {
      Frag pf[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) pf[qb] = frag_regs<T, 4>(x[qb], c);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        Frag vf = frag_perm<T>(Vt, 16 * db + c16, c, g);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) o[qb][db] = M::run(vf, pf[qb], o[qb][db]);
      }
    }

    if (kt + 1 < nkt) {
      sk.store_rows(lds[buf ^ 1][0]);
      sv.store_trans(lds[buf ^ 1][1]);
    }
    __syncthreads();
  }

#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float ls = wave_sum_g(l[qb]);
    const int i = iw + 16 * qb + c16;
    if (i >= N) continue;
    // (a query whose segment is empty has no key: O = 0, L = -inf)
    const float inv = (EXT && !(ls > 0.f)) ? 0.f : 1.f / ls;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      float vals[4] = {o[qb][db][0] * inv, o[qb][db][1] * inv, o[qb][db][2] * inv,
                       o[qb][db][3] * inv};
      store_out4(a.o, (tok + i) * 64 + 16 * db + 4 * g, a.out_f32 != 0, vals);
    }
    if (g == 0) a.lse[tok + i] = (EXT && !(ls > 0.f)) ? -INFINITY : m[qb] * kLn2 + logf(ls);
  }
}

template <typename T, int F>
hipError_t launch_one(const AttnArgs& a, int B, hipStream_t s) {
  dim3 grid((a.N + 127) / 128, B * a.H);
  hipLaunchKernelGGL((attn_fwd_kernel<T, F>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename T, int EXTF>
hipError_t dispatch(int flags, const AttnArgs& a, int B, hipStream_t s) {
  const int f = flags & (F_ZQ | F_ZK | F_BT | F_CAUSAL);
  switch (f) {
#define RP_CASE(X) \
  case X:          \
    return launch_one<T, (X) | EXTF>(a, B, s);
    RP_CASE(0)
    RP_CASE(F_ZQ)
    RP_CASE(F_ZK)
    RP_CASE(F_BT)
    RP_CASE(F_ZQ | F_ZK)
    RP_CASE(F_ZK | F_BT)
    RP_CASE(F_CAUSAL)
    RP_CASE(F_ZQ | F_CAUSAL)
    RP_CASE(F_ZK | F_CAUSAL)
    RP_CASE(F_BT | F_CAUSAL)
    RP_CASE(F_ZQ | F_ZK | F_CAUSAL)
    RP_CASE(F_ZK | F_BT | F_CAUSAL)
#undef RP_CASE
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_attn_fwd_f32(int flags, const AttnArgs& a, int B, hipStream_t s) {
  // (one variant takes both extras, each switched on at run time)
  if (flags & (F_SEG | F_DROP)) return dispatch<float, F_SEG | F_DROP>(flags, a, B, s);
  return dispatch<float, 0>(flags, a, B, s);
}

}  // namespace relpos
