// Offset-parallel pass of the backward with in-tile relation products: the
// table and bias gradients without a stored offset-gradient buffer.  [RPA] =
// "Fast and Exact Relative-Position Attention via Structure-Aware Kernels"
// (arXiv 2611.01182).
//
// The gradient of expanded row s = delta + D is a sum along one diagonal of
// the score-gradient matrix ([RPA] §3.3, the many-to-one reduction of the
// table gradients; §4.2 "Relation-Row Reduction"):
//   P1[s] = sum_i G[i, i - delta] q_i,   P2[s] = sum_i G[i, i - delta],
// G = tau dS.  With stored projections these sums come from the query pass's
// single-writer entries dZ~^Q[i, s] ([RPA] Table 9); with in-tile products
// nothing quadratic is stored, so this pass gives each workgroup 64
// consecutive rows s (one batch row and head) and walks their diagonals over
// every query, recomputing the scores exactly as the other passes do (same
// MFMA products, same order of additions, so bitwise the same P), and keeps
// the sums on chip.  Each row has one owner and the four waves' partials are
// added in a fixed order: deterministic, no atomics.  The results are the
// chunk partials of the table-gradient fold (one chunk per batch row), which
// the fold kernels then sum and map to table rows as in the stored path.
//
// Per step a wave takes 16 queries i = qw + c16 and the block's 64 offsets:
// the keys j = i - delta span an 80-key rectangle starting at
// jb = qw - delta0 - 63.  S = K Q^T and dP = V dO^T are made on MFMA over the
// rectangle (lane: query c16, keys 16 kb + 4 g + t) and moved to the
// (query, offset) layout through the wave's LDS scratch (key kk of query c16
// is offset delta0 + c16 + 63 - kk); the relation entries q_i . A~[s] + bt[s]
// come straight in that layout (rows s0 + 16 w + 4 g + t).  Then
// P = exp2(S tau log2 e - L log2 e), G' = P (dP - D), and
// P1 += G'^T Q on 16x16x16 fp16 MFMA (the reduction axis is the wave's 16
// queries: G'^T through the scratch, Q^T by the transposing LDS read).  The
// operands are fp16 ([RPA] "Half-precision numerics"): G' keeps 11
// significant bits instead of bf16's 8 (a clipped map folds thousands of
// offsets into its edge rows, whose sums would otherwise carry the larger
// rounding), and the bf16 queries convert to fp16 exactly.
// EXT adds segment masks (a pair outside its query's segment is masked) and
// dropout (dP takes the pair's keep factor, as in the query pass, applied in
// the rectangle order, whose key runs start on multiples of 4), as defined in
// extras.hpp.
#include "common.hpp"
#include "extras.hpp"
#include "intile.hpp"
#include "kernels.hpp"

namespace relpos {

namespace {

constexpr int kOP = 84;    // scratch pitch (fp32): 80 keys or 64 offsets per query row
constexpr int kOQP = 72;   // query tile pitch (bf16)

// Offset block of the k-th workgroup along the offset axis: blocks in order of
// distance from the block holding delta = 0, alternating sides, so the longest
// diagonals start first.
__device__ __forceinline__ int block_order(int k, int nob, int center) {
  const int right = nob - center;  // blocks center .. nob - 1
  const int left = center;         // blocks 0 .. center - 1
  const int both = imin(left, right);
  if (k < 2 * both) return (k & 1) ? center - 1 - (k >> 1) : center + (k >> 1);
  const int r = k - 2 * both;
  return right > left ? center + both + r : center - 1 - both - r;
}

template <bool CAUSAL, bool U, bool EXT>
__global__ __launch_bounds__(256, 2) void offset_pass(AttnArgs a, float* p1, float* p2, int nob,
                                                      int BH, int nchunk) {
  // During the loop: the step's K and V rectangle (128 keys, shared by the
  // four waves) and its keys' u . k entries, and per wave a scratch and its
  // query tile (fp16 words).  After the loop the same memory holds the four
  // waves' partials.
  constexpr int kWave = 16 * kOP + 16 * kOQP / 2;  // floats per wave
  struct Loop {
    bf16 sk[128 * kOQP];
    bf16 sv[128 * kOQP];
    bf16 sa[64 * kOQP];  // the block's table rows s0 .. s0 + 63
    float sbt[64];       // and their expanded bias
    float skm[128];
    float w[4][kWave];
  };
  union Mem {
    Loop l;
    float red[4][64 * 64];
  };
  __shared__ __attribute__((aligned(16))) Mem mem;
  __shared__ float sdb[4][64];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = wave_index(), g = lane >> 4, c16 = lane & 15;
  const int N = a.N, D = a.D, S = a.S;

  const int center = D / 64;
  const int ob = block_order(static_cast<int>(blockIdx.x) / BH, nob, center);
  const int bh = static_cast<int>(blockIdx.x) % BH;
  const int b = bh / a.H, h = bh % a.H;
  const int64_t tok = static_cast<int64_t>(bh) * N;
  const int s0 = 64 * ob, dl0 = s0 - D;
  const int dmin = CAUSAL ? 0 : -(N - 1);
  const int dlo = imax(dl0, dmin), dhi = imin(dl0 + 63, N - 1);
  const float sl2 = a.scale_log2;
  const bool SEG = EXT && a.seg != nullptr;
  const bool DROP = EXT && a.drop_p8 > 0;
  const int64_t brow = static_cast<int64_t>(b) * N;

  const uint64_t slice_bytes = static_cast<uint64_t>(N) * 128;
  const Rsrc rq = make_rsrc(reinterpret_cast<const bf16*>(a.q) + tok * 64, slice_bytes);
  const Rsrc rdo = make_rsrc(reinterpret_cast<const bf16*>(a.dout) + tok * 64, slice_bytes);
  const Rsrc rk = make_rsrc(reinterpret_cast<const bf16*>(a.k) + tok * 64, slice_bytes);
  const Rsrc rv = make_rsrc(reinterpret_cast<const bf16*>(a.v) + tok * 64, slice_bytes);
  // per-token values of the slice (reads past N return zero)
  const uint64_t row_bytes = static_cast<uint64_t>(N) * 4;
  const Rsrc rlse = make_rsrc(a.lse + tok, row_bytes);
  const Rsrc rdd = make_rsrc(a.dvec + tok, row_bytes);
  const Rsrc rkm = make_rsrc(a.keymid + tok, row_bytes);
  const ItTables itb = it_tables(a, h);

  float* const scr = &mem.l.w[wave][0];
  bf16* const sq = reinterpret_cast<bf16*>(&mem.l.w[wave][16 * kOP]);

  floatx4 acc[4][4];
#pragma unroll
  for (int w = 0; w < 4; ++w)
#pragma unroll
    for (int db = 0; db < 4; ++db) acc[w][db] = floatx4{0.f, 0.f, 0.f, 0.f};
  float dbs[4] = {0.f, 0.f, 0.f, 0.f};

  if (dlo <= dhi) {
    // the block's table rows s0 .. s0 + 63 (A operand of the relation
    // entries) and their expanded bias, the same for every step: into LDS
    // once (written before the first step's barrier)
    {
      const int r = tid >> 2, ch = (tid & 3) * 16;
#pragma unroll
      for (int u = 0; u < 2; ++u)
        *reinterpret_cast<uint4*>(&mem.l.sa[r * kOQP + ch + 8 * u]) =
            bload16(itb.at, static_cast<uint32_t>((s0 + r) * 64 + ch + 8 * u) * 2);
      if (tid < 64) mem.l.sbt[tid] = bloadf(itb.bt, static_cast<uint32_t>(s0 + tid) * 4);
    }

    // queries with a pair in the block: i in [max(0, dlo), min(N - 1, N - 1 + dhi)]
    const int i_lo = imax(0, dlo), i_hi = imin(N - 1, N - 1 + dhi);
    // Step at ib: the workgroup's 64 queries ib .. ib + 63 (wave w: 16 from
    // ib + 16 w) and keys jw = ib - dl0 - 63 .. jw + 127 (wave w's 80-key
    // rectangle starts at row 16 w).  Tile staging: K and V rows (t >> 3) and
    // 32 + (t >> 3) (+ 64, + 96), chunk t & 7; the keys' u . k by threads < 128.
    const int kr = tid >> 3, kc8 = (tid & 7) * 8;
    uint4 tk[4], tv[4];
    float tkm = 0.f;
    auto load_tile = [&](int ib) {
      const int jw = ib - dl0 - 63;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = jw + kr + 32 * u;
        const uint32_t off = j >= 0 ? static_cast<uint32_t>(j * 128 + kc8 * 2) : kOob;
        tk[u] = bload16(rk, off);
        tv[u] = bload16(rv, off);
      }
      if (U) {
        const int j = jw + (tid & 127);
        tkm = bloadf(rkm, j >= 0 ? static_cast<uint32_t>(j) * 4 : kOob);
      }
    };
    auto store_tile = [&]() {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        *reinterpret_cast<uint4*>(&mem.l.sk[(kr + 32 * u) * kOQP + kc8]) = tk[u];
        *reinterpret_cast<uint4*>(&mem.l.sv[(kr + 32 * u) * kOQP + kc8]) = tv[u];
      }
      if (U && tid < 128) mem.l.skm[tid] = tkm;
    };
    // the wave's queries of a step: Q, dO fragments, L and D
    bf16x8 qf[2], df[2], qn[2], dn[2];
    float lse_i, dd_i, lse_n, dd_n;
    auto load_queries = [&](int ib, bf16x8 (&q2)[2], bf16x8 (&d2)[2], float& ls, float& dv) {
      const int i = ib + 16 * wave + c16;
      ls = bloadf(rlse, static_cast<uint32_t>(i) * 4);
      dv = bloadf(rdd, static_cast<uint32_t>(i) * 4);
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const uint32_t off = static_cast<uint32_t>(i * 128 + 64 * c + 16 * g);
        q2[c] = __builtin_bit_cast(bf16x8, bload16(rq, off));
        d2[c] = __builtin_bit_cast(bf16x8, bload16(rdo, off));
      }
    };

    const int ib0 = i_lo & ~63;
    load_queries(ib0, qf, df, lse_i, dd_i);
    load_tile(ib0);
    store_tile();
    __syncthreads();
    for (int ib = ib0; ib <= i_hi; ib += 64) {
      const bool more = ib + 64 <= i_hi;
      if (more) {
        load_queries(ib + 64, qn, dn, lse_n, dd_n);
        load_tile(ib + 64);
      }
      const int qw = ib + 16 * wave;
      // (uniform per wave: a wave without a query in the range computes
      // nothing but still meets the barriers)
      if (!(qw > i_hi || qw + 15 < i_lo)) {
        const int i = qw + c16;
        const bool iok = i < N;
        float l2 = iok ? lse_i * kLog2e : INFINITY;
        if (EXT && !(l2 > -INFINITY)) l2 = INFINITY;  // a row with no key: P = 0
        const float dd = dd_i;
        // the query's segment (keys outside it are masked)
        int sgl = 0, sgh = N;
        if (SEG) {
          sgl = sgh = 0;
          if (iok) token_segment(a, brow, i, sgl, sgh);
        }
        const bf16* Ks = mem.l.sk + (16 * wave) * kOQP;
        const bf16* Vs = mem.l.sv + (16 * wave) * kOQP;

        // S and dP over the wave's 80-key rectangle (keys jb + 16 kb + 4 g
        // + t, jb = qw - dl0 - 63)
        floatx4 sr[5], pr[5];
#pragma unroll
        for (int kb = 0; kb < 5; ++kb) {
          sr[kb] = floatx4{0.f, 0.f, 0.f, 0.f};
          pr[kb] = floatx4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int kb = 0; kb < 5; ++kb) {
            const bf16x8 kf = *reinterpret_cast<const bf16x8*>(Ks + (16 * kb + c16) * kOQP + 32 * c + 8 * g);
            const bf16x8 vf = *reinterpret_cast<const bf16x8*>(Vs + (16 * kb + c16) * kOQP + 32 * c + 8 * g);
            sr[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[c], sr[kb], 0, 0, 0);
            pr[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, df[c], pr[kb], 0, 0, 0);
          }
        if (DROP) {
          // dP of a dropped pair is 0, of a kept one times the keep scale;
          // the rectangle's keys jb + 16 kb + 4 g (+ 0..3) start on a multiple
          // of 4 (jb = qw - dl0 - 63 is a multiple of 16)
#pragma unroll
          for (int kb = 0; kb < 5; ++kb) {
            float mk[4];
            keep_row4(a, bh, i, qw - dl0 - 63 + 16 * kb + 4 * g, a.drop_scale, mk);
#pragma unroll
            for (int t = 0; t < 4; ++t) pr[kb][t] *= mk[t];
          }
        }
        // relation entries of the block's rows (lane: query c16, offsets
        // 16 w + 4 g + t): bt, then the two K-steps, as in every pass
        floatx4 zd[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) zd[w] = *reinterpret_cast<const floatx4*>(&mem.l.sbt[16 * w + 4 * g]);
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const bf16x8 af = *reinterpret_cast<const bf16x8*>(&mem.l.sa[(16 * w + c16) * kOQP + 32 * c + 8 * g]);
            zd[w] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, qf[c], zd[w], 0, 0, 0);
          }

        // the query tile as fp16 words for the transposing reads
#pragma unroll
        for (int c = 0; c < 2; ++c)
          *reinterpret_cast<uint4*>(sq + c16 * kOQP + 32 * c + 8 * g) =
              bf16x8_to_f16x8(__builtin_bit_cast(uint4, qf[c]));

        // rectangle -> (query, offset): offset 16 w + 4 g + t of query c16 is
        // key kk = c16 + 63 - 16 w - 4 g - t
        float sv[4][4], pv[4][4];
#pragma unroll
        for (int kb = 0; kb < 5; ++kb) *reinterpret_cast<floatx4*>(scr + c16 * kOP + 16 * kb + 4 * g) = sr[kb];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float* r = scr + c16 * kOP + c16 + 60 - 16 * w - 4 * g;
#pragma unroll
          for (int t = 0; t < 4; ++t) sv[w][t] = r[3 - t];
        }
#pragma unroll
        for (int kb = 0; kb < 5; ++kb) *reinterpret_cast<floatx4*>(scr + c16 * kOP + 16 * kb + 4 * g) = pr[kb];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float* r = scr + c16 * kOP + c16 + 60 - 16 * w - 4 * g;
#pragma unroll
          for (int t = 0; t < 4; ++t) pv[w][t] = r[3 - t];
        }

        // P and G' = P (dP - D) per pair (query i, offset dl0 + 16 w + 4 g + t)
#pragma unroll
        for (int w = 0; w < 4; ++w)
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int dlt = dl0 + 16 * w + 4 * g + t;
            const int j = i - dlt;
            float km = 0.f;
            if (U) km = mem.l.skm[16 * wave + c16 + 63 - 16 * w - 4 * g - t];
            const float band = km + zd[w][t];
            const float sc = sv[w][t] + band;
            float p = fast_exp2(fmaf(sc, sl2, -l2));
            // (computed in every lane, then selected: kept out of branches)
            asm volatile("" : "+v"(p));
            const bool ok = iok && j >= 0 && j < N && dlt >= dmin && dlt <= N - 1 &&
                            (!SEG || (j >= sgl && j < sgh));
            p = ok ? p : 0.f;
            zd[w][t] = p * (pv[w][t] - dd);  // G' in place
          }

        // G'^T through the scratch: lane (c16, g) of row block w takes
        // G'[query 4 g + e][offset 16 w + c16], e = 0..3
#pragma unroll
        for (int w = 0; w < 4; ++w) *reinterpret_cast<floatx4*>(scr + c16 * kOP + 16 * w + 4 * g) = zd[w];
        halfx4 ga[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          float x[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = scr[(4 * g + e) * kOP + 16 * w + c16];
          dbs[w] += (x[0] + x[1]) + (x[2] + x[3]);
          halfx4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = static_cast<_Float16>(x[e]);
          ga[w] = v;
        }
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          // Q^T: lane (c16, g) takes q[query 4 g + e][16 db + c16]
          const halfx4 qt = __builtin_bit_cast(halfx4, lds_tr4(sq, kOQP, 4 * g, 16 * db, c16));
#pragma unroll
          for (int w = 0; w < 4; ++w)
            acc[w][db] = __builtin_amdgcn_mfma_f32_16x16x16f16(ga[w], qt, acc[w][db], 0, 0, 0);
        }
      }
      // every wave is done with this step's rectangle: the next one goes in
      __syncthreads();
      if (more) {
        store_tile();
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          qf[c] = qn[c];
          df[c] = dn[c];
        }
        lse_i = lse_n;
        dd_i = dd_n;
      }
      __syncthreads();
    }
  }

  // the waves' partials, added in a fixed order (wave 0 + 1 + 2 + 3); tau
  // (G = tau G') multiplies the finished sums.  (The loop's last barrier
  // leaves the memory free.)
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float dsum = wave_sum_g(dbs[w]);
    if (g == 0) sdb[wave][16 * w + c16] = dsum;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int t = 0; t < 4; ++t) mem.red[wave][(16 * w + 4 * g + t) * 64 + 16 * db + c16] = acc[w][db][t];
  }
  __syncthreads();
  const int64_t pbase = (static_cast<int64_t>(h) * nchunk + b) * S + s0;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int e = tid + 256 * k;
    const int r = e >> 6;
    if (s0 + r < S)
      p1[(pbase + r) * 64 + (e & 63)] =
          a.scale * (((mem.red[0][e] + mem.red[1][e]) + mem.red[2][e]) + mem.red[3][e]);
  }
  if (tid < 64 && s0 + tid < S)
    p2[pbase + tid] = a.scale * (((sdb[0][tid] + sdb[1][tid]) + sdb[2][tid]) + sdb[3][tid]);
}

}  // namespace

template <bool C, bool U>
hipError_t launch_op(const AttnArgs& a, int B, int ext, float* p1, float* p2, hipStream_t s) {
  const int BH = B * a.H;
  const int nob = (a.S + 63) / 64;
  const dim3 grid(static_cast<unsigned>(nob * BH));
  if (ext)
    hipLaunchKernelGGL((offset_pass<C, U, true>), grid, dim3(256), 0, s, a, p1, p2, nob, BH, B);
  else
    hipLaunchKernelGGL((offset_pass<C, U, false>), grid, dim3(256), 0, s, a, p1, p2, nob, BH, B);
  return hipGetLastError();
}

hipError_t launch_offset_pass_it(const AttnArgs& a, int B, int causal, int u, int ext, float* p1,
                                 float* p2, hipStream_t s) {
  if (causal) return u ? launch_op<true, true>(a, B, ext, p1, p2, s) : launch_op<true, false>(a, B, ext, p1, p2, s);
  return u ? launch_op<false, true>(a, B, ext, p1, p2, s) : launch_op<false, false>(a, B, ext, p1, p2, s);
}

}  // namespace relpos
