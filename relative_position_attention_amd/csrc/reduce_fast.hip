// Reductions of the offset gradients for bf16 inputs ([RPA] Table 9 "Query
// reduction" / "Key reduction"; [RPA] §4.2 and the table-gradient lemma of
// App. B.1).  [RPA] = "Fast and Exact Relative-Position Attention via
// Structure-Aware Kernels" (arXiv 2611.01182).
//
// The offset gradients dZ~[i, s] sit in the skewed per-group rows of the
// projection layout: row i of group g holds expanded rows s in [slo_g, shi_g]
// at column s - slo_g + pad_g.  Both kernels stage (64 tokens x 64 rows s)
// tiles of it into LDS with aligned 16-byte loads (each token row's segment
// is contiguous; entries a token cannot reach, and the two boundary rows, are
// written as zero).  The tile is kept in fp32 with each token row shifted by
// its own misalignment (e0 mod the chunk width), so the LDS writes stay whole
// 16-byte chunks; the readers add the row's shift, kept beside the tile, and
// round to bf16 when they build the MFMA operands:
//   finalize_fast:  out = acc + dZ~ A~ (band rows) + the two boundary sums
//                   times A~[0], A~[2D] in fp32 (+ column sums times u);
//                   dQ = tau dS K + dZ^Q A^Q of the table-gradient lemma, the
//                   bucket fold implicit (copies multiply the same row);
//   partials_fast:  P1[h][c][s] = sum over the tokens of chunk c of
//                   dZ~[i, s] x_i and P2[h][c][s] = sum of dZ~[i, s]: the
//                   fixed-order chunk partials of [RPA] "Deterministic table
//                   gradients" (the chunk sums and the fold follow).
#include "kernels.hpp"
#include "tiles.hpp"

namespace relpos {

namespace {

constexpr int kRP = 72;   // LDS pitch of bf16 tiles (144-byte rows)
constexpr int kSP = 76;   // LDS pitch of the row-shifted fp32 dZ~ tiles

// One (64 tokens x 64 expanded rows s0 .. s0+63) tile of dZ~, moved in two
// phases so the next tile's loads overlap the current tile's products: load()
// issues the aligned 16-byte chunk loads of this thread's token row into
// registers, store() writes them to LDS as fp32 chunks at their memory
// alignment: entry s0 + p of token row r sits at zf[r][p + so[r]], so[r] =
// e0 mod VEC.  Entries outside the token's reachable band rows
// [max(smin, 1), min(smax, 2D-1)] are written as zero.  Thread t moves token
// row t / 4, chunks t % 4, t % 4 + 4, ...  W > 1: 64 W entries per token
// row (rows s0 .. s0 + 64 W - 1), LDS pitch SP.
template <typename GT, int W = 1, int SP = kSP>
struct DzTile {
  static constexpr int VEC = 16 / sizeof(GT);
  static constexpr int NCH = 64 * W / VEC + 1;  // aligned chunks covering 64 W entries
  static constexpr int PER = (NCH + 3) / 4;
  uint4 w[PER];
  int e0;      // element index of s0 in the token's row
  int lo, hi;  // reachable positions s - s0 of the token (empty past N)

  __device__ __forceinline__ void load(const Rsrc& rz, const GroupInfo& gi, int g0, int r0, int s0,
                                       int N, int D, bool key_side, bool causal) {
    const int tid = threadIdx.x, r = tid >> 2, tq = tid & 3;
    const int i = r0 + r;
    int smin = 1, smax = 0;
    if (i < N) {
      if (key_side)
        key_s_range(i, N, D, causal, smin, smax);
      else
        query_s_range(i, N, D, causal, smin, smax);
    }
    lo = imax(smin, 1) - s0;
    hi = imin(smax, 2 * D - 1) - s0;
    e0 = gi.base + (i - g0) * gi.pitch + (s0 - gi.slo + gi.pad);
    const int cf = e0 & ~(VEC - 1);
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int ch = tq + 4 * u;
      const int ce = cf + ch * VEC;
      const bool ok = ch < NCH && ce >= 0 && ce <= e0 + 64 * W - 1 && hi >= 0 && lo <= 64 * W - 1 && lo <= hi;
      w[u] = bload16(rz, ok ? static_cast<uint32_t>(ce * static_cast<int>(sizeof(GT))) : kOob);
    }
  }

  __device__ __forceinline__ void store(float* zf, int* so) const {
    const int tid = threadIdx.x, r = tid >> 2, tq = tid & 3;
    const int o = e0 & (VEC - 1);
    if (tq == 0) so[r] = o;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int ch = tq + 4 * u;
      if (ch >= NCH) continue;
      const int p0 = VEC * ch - o;  // position s - s0 of the chunk's first entry
      float f[VEC];
      if constexpr (sizeof(GT) == 4) {
        __builtin_memcpy(f, &w[u], 16);
      } else if constexpr (std::is_same_v<GT, _Float16>) {
        _Float16 hv[8];
        __builtin_memcpy(hv, &w[u], 16);
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = static_cast<float>(hv[e]);
      } else {
        const uint32_t wd[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          f[2 * k] = __uint_as_float(wd[k] << 16);
          f[2 * k + 1] = __uint_as_float(wd[k] & 0xffff0000u);
        }
      }
      if (!(p0 >= lo && p0 + VEC - 1 <= hi)) {
#pragma unroll
        for (int e = 0; e < VEC; ++e)
          if (p0 + e < lo || p0 + e > hi) f[e] = 0.f;
      }
#pragma unroll
      for (int k = 0; k < VEC / 4; ++k)
        *reinterpret_cast<floatx4*>(&zf[r * SP + VEC * ch + 4 * k]) =
            floatx4{f[4 * k], f[4 * k + 1], f[4 * k + 2], f[4 * k + 3]};
    }
  }
};

__device__ __forceinline__ bf16x8 pack_bf16x8(const float* v) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = static_cast<bf16>(v[e]);
  return r;
}

// ---------------------------------------------------------------- finalize

// W: stages of 64 W expanded rows (see partials_fast for why wider runs
// fetch fewer lines per entry)
template <typename GT, int W>
__global__ __launch_bounds__(256) void finalize_fast(FinalizeArgs f) {
  constexpr int SP = 64 * W + 12;
  __shared__ __attribute__((aligned(16))) float zf[64 * SP];
  __shared__ int so[64];
  __shared__ __attribute__((aligned(16))) bf16 at[64 * W * kRP];
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index(), g = lane >> 4, c16 = lane & 15;
  const int bh = blockIdx.y;
  const int h = bh % f.H;
  const int64_t tok = static_cast<int64_t>(bh) * f.N;
  // one 64-token block: rows r0 .. r0 + 63
  auto run_block = [&](int r0) {
    const int D = f.D;
    floatx4 acc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) acc[db] = floatx4{0.f, 0.f, 0.f, 0.f};
    const bf16* atab = nullptr;
    if (f.at != nullptr)
      atab = reinterpret_cast<const bf16*>(f.at) + static_cast<int64_t>(f.at_shared ? 0 : h) * f.S * 64;

    if (f.dz != nullptr && D >= 1) {
      const int grp = r0 / kGroup;
      const GroupInfo gi = f.gi[grp];
      int slo, shi;
      if (f.key_side)
        key_group_window(grp, f.N, D, f.causal != 0, slo, shi);
      else
        query_group_window(grp, f.N, D, f.causal != 0, slo, shi);
      const int sa = imax(1, slo), sb = imin(2 * D - 1, shi);
      const Rsrc rz = make_rsrc(reinterpret_cast<const GT*>(f.dz) + static_cast<int64_t>(bh) * f.dz_bh,
                                static_cast<uint64_t>(f.dz_bh) * sizeof(GT));
      const Rsrc ra = make_rsrc(atab, static_cast<uint64_t>(f.S) * 128);
      // A~ rows s0 .. s0+63, row-major (rows past the table read zero)
      const int ar = tid >> 2, ac = (tid & 3) * 16;
      DzTile<GT, W, SP> dt;
      uint4 ta[2 * W];
      auto load_stage = [&](int s0) {
        dt.load(rz, gi, grp * kGroup, r0, s0, f.N, D, f.key_side != 0, f.causal != 0);
#pragma unroll
        for (int u = 0; u < 2 * W; ++u)
          ta[u] = bload16(ra, static_cast<uint32_t>((s0 + ar + 64 * (u >> 1)) * 128 + (ac + 8 * (u & 1)) * 2));
      };
      if (sa <= sb) load_stage(sa);
      for (int s0 = sa; s0 <= sb; s0 += 64 * W) {
        dt.store(zf, so);
#pragma unroll
        for (int u = 0; u < 2 * W; ++u)
          *reinterpret_cast<uint4*>(&at[(ar + 64 * (u >> 1)) * kRP + ac + 8 * (u & 1)]) = ta[u];
        __syncthreads();
        if (s0 + 64 * W <= sb) load_stage(s0 + 64 * W);
#pragma unroll
        for (int c = 0; c < 2 * W; ++c) {
          // K axis (rows s) in the order 32c + 4g + e, 32c + 16 + 4g + e
          const int tr = 16 * wave + c16;
          const float* zr = zf + tr * SP + so[tr] + 32 * c + 4 * g;
          float v[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[e] = zr[e];
            v[e + 4] = zr[16 + e];
          }
          const bf16x8 a8 = pack_bf16x8(v);
#pragma unroll
          for (int db = 0; db < 4; ++db) {
            const bf16x4 blo = lds_tr4(at, kRP, 32 * c + 4 * g, 16 * db, c16);
            const bf16x4 bhi = lds_tr4(at, kRP, 32 * c + 16 + 4 * g, 16 * db, c16);
            bf16x8 b8;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              b8[e] = blo[e];
              b8[e + 4] = bhi[e];
            }
            acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a8, b8, acc[db], 0, 0, 0);
          }
        }
        __syncthreads();
      }
    }

    // epilogue: lane holds rows 16 wave + 4g + t, column 16 db + c16
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int i = r0 + 16 * wave + 4 * g + t;
      if (i >= f.N) continue;
      const int64_t row = tok + i;
      float b0 = 0.f, b1 = 0.f, cs = 0.f;
      if (atab != nullptr && f.bnd != nullptr) {
        b0 = f.bnd[row * 2 + 0];
        b1 = f.bnd[row * 2 + 1];
      }
      if (f.colsum != nullptr) cs = f.colsum[row];
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int d = 16 * db + c16;
        float v = acc[db][t] + f.acc[row * 64 + d];
        if (atab != nullptr)
          v += b0 * static_cast<float>(atab[d]) + b1 * static_cast<float>(atab[static_cast<int64_t>(2 * D) * 64 + d]);
        if (f.colsum != nullptr) v += cs * static_cast<float>(reinterpret_cast<const bf16*>(f.u)[h * 64 + d]);
        if (f.out_f32)
          reinterpret_cast<float*>(f.out)[row * 64 + d] = v;
        else
          reinterpret_cast<bf16*>(f.out)[row * 64 + d] = static_cast<bf16>(v);
      }
    }
  };
  const int nrb = (f.N + 63) / 64;
  if (f.causal) {
    // a causal map gives the token blocks windows of linearly growing (query
    // side) or shrinking (key side) width: each workgroup takes block b and
    // block nrb - 1 - b, so every workgroup does the same work
    const int b = static_cast<int>(blockIdx.x);
    run_block(b * 64);
    if (nrb - 1 - b != b) run_block((nrb - 1 - b) * 64);
  } else {
    run_block(static_cast<int>(blockIdx.x) * 64);
  }
}
// ---------------------------------------------------------------- partials

// W: 64-row tiles of s per workgroup.  A token row's run of 64 W entries
// starts at an arbitrary element, so it touches about 64 W / 64 + 1 cache
// lines of 64 entries: two tiles per stage read three lines where two
// workgroups of one tile each read four.
template <typename GT, int W>
__global__ __launch_bounds__(256) void partials_fast(PartialArgs p) {
  constexpr int SP = 64 * W + 12;  // LDS pitch of the row-shifted fp32 tile
  __shared__ __attribute__((aligned(16))) float zf[64 * SP];   // [token][s + shift]
  __shared__ __attribute__((aligned(16))) int so[64];
  __shared__ __attribute__((aligned(16))) bf16 xt[64 * kRP];   // [token][d]
  __shared__ float bsh[2][64];
  __shared__ float bred[4][2][64];  // boundary sums per token quarter
  __shared__ float p2red[4][64 * W];
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index(), g = lane >> 4, c16 = lane & 15;
  const int D = p.D;
  // s tiles from the one holding offset 0 (s = D) outwards: those reach the
  // most tokens, so the longest blocks start first.  Workgroups are numbered
  // rank-major (every head and chunk of one tile rank before the next rank),
  // so the longest blocks of all heads start first, not those of the first
  // head only (a causal map's central tiles take 32 stages per chunk where
  // its outer ones take none: the last head's central tiles, dispatched
  // last, ran alone at the end)
  int tile;
  const int lin = static_cast<int>(blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z));
  const int nhz = static_cast<int>(gridDim.y * gridDim.z);
  const int rank = lin / nhz, hz = lin % nhz;
  {
    const int T = static_cast<int>(gridDim.x), c = imin(D / (64 * W), T - 1);
    const int below = c, above = T - 1 - c, mm = imin(below, above);
    // the two last tiles of the centre-out order (the outermost, which hold
    // the boundary rows 0 and 2D and so visit every token block of their
    // chunk) move to ranks 1 and 2
    const int r = T <= 3 ? rank : (rank == 0 ? 0 : (rank <= 2 ? T - 3 + rank : rank - 2));
    const int k = r - 1;
    if (k < 0)
      tile = c;
    else if (k < 2 * mm)
      tile = (k & 1) ? c - (k / 2 + 1) : c + (k / 2 + 1);
    else
      tile = above > below ? c + mm + 1 + (k - 2 * mm) : c - mm - 1 - (k - 2 * mm);
  }
  const int s0 = tile * 64 * W;
  const int h = hz % static_cast<int>(gridDim.y);
  const int chunk = hz / static_cast<int>(gridDim.y);
  const int nrb = (p.N + 63) / 64;
  const int total = p.B * nrb;
  const int per = (total + p.nchunk - 1) / p.nchunk;
  const int sb0 = chunk * per, sb1 = imin(total, sb0 + per);
  const bool has0 = s0 == 0;
  const bool has2 = (2 * D >= s0) && (2 * D < s0 + 64 * W);
  const bool want_p1 = p.p1 != nullptr;
  const bool want_p2 = p.p2 != nullptr;

  floatx4 acc[W][4];
#pragma unroll
  for (int st = 0; st < W; ++st)
#pragma unroll
    for (int db = 0; db < 4; ++db) acc[st][db] = floatx4{0.f, 0.f, 0.f, 0.f};
  float p2acc[W];              // thread (s = 64 st + (tid & 63), quarter tid >> 6)
#pragma unroll
  for (int st = 0; st < W; ++st) p2acc[st] = 0.f;
  // boundary P1: thread (d = tid & 63, token quarter tid >> 6); boundary P2:
  // thread tid < 64 sums token tid over the stages (both summed in a fixed
  // order at the end)
  float bx0 = 0.f, bx1 = 0.f;
  float bs0 = 0.f, bs1 = 0.f;

  // does row block sb reach this block's band rows (uniform)
  auto band_hit = [&](int sb) {
    const int grp = ((sb % nrb) * 64) / kGroup;
    int slo, shi;
    if (p.key_side)
      key_group_window(grp, p.N, D, p.causal != 0, slo, shi);
    else
      query_group_window(grp, p.N, D, p.causal != 0, slo, shi);
    const int sa = imax(1, slo), se = imin(2 * D - 1, shi);
    return D >= 1 && sa <= se && s0 <= se && s0 + 64 * W - 1 >= sa;
  };
  auto next_stage = [&](int sb) {
    while (sb < sb1 && !(has0 || has2 || band_hit(sb))) ++sb;
    return sb;
  };

  DzTile<GT, W, SP> dt;
  uint4 tx[2];
  float tb[2] = {0.f, 0.f};
  bool hit_next = false;
  const int xr = tid >> 2, xc = (tid & 3) * 16;
  auto load_stage = [&](int sb) {
    const int b = sb / nrb, r0 = (sb % nrb) * 64;
    const int grp = r0 / kGroup;
    const int64_t bhs = static_cast<int64_t>(b) * p.H + h;
    const int64_t tok = bhs * p.N;
    if (want_p1) {
      const Rsrc rx = make_rsrc(reinterpret_cast<const bf16*>(p.x) + tok * 64,
                                static_cast<uint64_t>(p.N) * 128);
#pragma unroll
      for (int u = 0; u < 2; ++u)
        tx[u] = bload16(rx, static_cast<uint32_t>((r0 + xr) * 128 + (xc + 8 * u) * 2));
    }
    hit_next = band_hit(sb);
    if (hit_next) {
      const Rsrc rz = make_rsrc(reinterpret_cast<const GT*>(p.dz) + bhs * p.dz_bh,
                                static_cast<uint64_t>(p.dz_bh) * sizeof(GT));
      dt.load(rz, p.gi[grp], grp * kGroup, r0, s0, p.N, D, p.key_side != 0, p.causal != 0);
    }
    if ((has0 || has2) && tid < 64) {
      const int i = r0 + tid;
      tb[0] = i < p.N ? p.bnd[(tok + i) * 2 + 0] : 0.f;
      tb[1] = i < p.N ? p.bnd[(tok + i) * 2 + 1] : 0.f;
    }
  };

  int sb = next_stage(sb0);
  if (sb < sb1) load_stage(sb);
  while (sb < sb1) {
    const bool hit = hit_next;
    if (want_p1) {
#pragma unroll
      for (int u = 0; u < 2; ++u) *reinterpret_cast<uint4*>(&xt[xr * kRP + xc + 8 * u]) = tx[u];
    }
    if (hit) dt.store(zf, so);
    if ((has0 || has2) && tid < 64) {
      bsh[0][tid] = tb[0];
      bsh[1][tid] = tb[1];
    }
    __syncthreads();
    const int nsb = next_stage(sb + 1);
    if (nsb < sb1) load_stage(nsb);
    if (hit) {
      if (want_p1) {
        // P1 (s x d) += Z^T (s x tokens) X (tokens x d); K axis (tokens) in
        // the order 32c + 4g + e, 32c + 16 + 4g + e
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const int t0 = 32 * c + 4 * g;
          const int4 oa = *reinterpret_cast<const int4*>(&so[t0]);
          const int4 ob = *reinterpret_cast<const int4*>(&so[t0 + 16]);
          const int oo[8] = {oa.x, oa.y, oa.z, oa.w, ob.x, ob.y, ob.z, ob.w};
          bf16x8 b8[4];
#pragma unroll
          for (int db = 0; db < 4; ++db) {
            const bf16x4 blo = lds_tr4(xt, kRP, 32 * c + 4 * g, 16 * db, c16);
            const bf16x4 bhi = lds_tr4(xt, kRP, 32 * c + 16 + 4 * g, 16 * db, c16);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              b8[db][e] = blo[e];
              b8[db][e + 4] = bhi[e];
            }
          }
#pragma unroll
          for (int st = 0; st < W; ++st) {
            const int sc = 64 * st + 16 * wave + c16;
            float v[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              v[e] = zf[(t0 + e) * SP + oo[e] + sc];
              v[e + 4] = zf[(t0 + 16 + e) * SP + oo[e + 4] + sc];
            }
            const bf16x8 a8 = pack_bf16x8(v);
#pragma unroll
            for (int db = 0; db < 4; ++db)
              acc[st][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a8, b8[db], acc[st][db], 0, 0, 0);
          }
        }
      }
      if (want_p2) {
        // columns s = 64 st + (tid & 63), tokens 16 (tid >> 6) .. +15, in order
        const int q = tid >> 6;
#pragma unroll
        for (int st = 0; st < W; ++st) {
          const int s = 64 * st + (tid & 63);
          float part = 0.f;
#pragma unroll
          for (int e = 0; e < 16; ++e) part += zf[(16 * q + e) * SP + so[16 * q + e] + s];
          p2acc[st] += part;
        }
      }
    }
    if (has0 || has2) {
      if (want_p1) {
        const int d = tid & 63, q = tid >> 6;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int tk = 16 * q + e;
          const float xv = static_cast<float>(xt[tk * kRP + d]);
          bx0 = fmaf(bsh[0][tk], xv, bx0);
          bx1 = fmaf(bsh[1][tk], xv, bx1);
        }
      }
      if (want_p2 && tid < 64) {
        bs0 += bsh[0][tid];
        bs1 += bsh[1][tid];
      }
    }
    __syncthreads();
    sb = nsb;
  }

  // write the chunk's partials
  const int64_t pbase = (static_cast<int64_t>(h) * p.nchunk + chunk) * p.S;
  if (want_p1) {
#pragma unroll
    for (int st = 0; st < W; ++st)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int s = s0 + 64 * st + 16 * wave + 4 * g + t;
        if (s >= p.S) continue;
#pragma unroll
        for (int db = 0; db < 4; ++db) p.p1[(pbase + s) * 64 + 16 * db + c16] = acc[st][db][t];
      }
    if (has0 || has2) {
      bred[tid >> 6][0][tid & 63] = bx0;
      bred[tid >> 6][1][tid & 63] = bx1;
    }
    __syncthreads();
    if ((has0 || has2) && tid < 64) {
      // boundary rows: added in a fixed order after the band part
      const float t0 = ((bred[0][0][tid] + bred[1][0][tid]) + bred[2][0][tid]) + bred[3][0][tid];
      const float t1 = ((bred[0][1][tid] + bred[1][1][tid]) + bred[2][1][tid]) + bred[3][1][tid];
      if (has0) p.p1[(pbase + 0) * 64 + tid] += t0 + (2 * D == 0 ? t1 : 0.f);
      if (has2 && D > 0) p.p1[(pbase + 2 * D) * 64 + tid] += t1;
    }
  }
  if (want_p2) {
#pragma unroll
    for (int st = 0; st < W; ++st) p2red[tid >> 6][64 * st + (tid & 63)] = p2acc[st];
    // (bred is free again: its only readers in the P1 epilogue are these
    // same threads, which read it before they write it here)
    if ((has0 || has2) && tid < 64) {
      bred[0][0][tid] = bs0;
      bred[0][1][tid] = bs1;
    }
    __syncthreads();
    if ((has0 || has2) && tid < 64) {
      // every writer thread of P2 forms the same totals in the same order
      // (the row s = 2D is written by thread 2D - s0)
      bs0 = 0.f;
      bs1 = 0.f;
      for (int tk = 0; tk < 64; ++tk) {
        bs0 += bred[0][0][tk];
        bs1 += bred[0][1][tk];
      }
    }
    if (tid < 64) {
#pragma unroll
      for (int st = 0; st < W; ++st) {
        const int sl = 64 * st + tid;
        const int s = s0 + sl;
        if (s < p.S) {
          float v = ((p2red[0][sl] + p2red[1][sl]) + p2red[2][sl]) + p2red[3][sl];
          if (has0 && s == 0) v += bs0 + (2 * D == 0 ? bs1 : 0.f);
          if (has2 && D > 0 && s == 2 * D) v += bs1;
          p.p2[pbase + s] = v;
        }
      }
    }
  }
}

inline unsigned nblk(int64_t n, int b) { return static_cast<unsigned>((n + b - 1) / b); }

}  // namespace

hipError_t launch_finalize_bf16(const FinalizeArgs& f, int BH, hipStream_t s) {
  const unsigned nrb = nblk(f.N, 64);
  dim3 grid(f.causal ? (nrb + 1) / 2 : nrb, BH);
  // fp16 entries (the causal Transformer-XL query side: few workgroups, long
  // rows) take stages of two 64-row tiles; bf16 entries keep one, where the
  // occupancy of the wider stage (3 workgroups per CU instead of 5) costs more
  // than its fewer cache lines save
  if (f.dz_f32)
    hipLaunchKernelGGL((finalize_fast<float, 1>), grid, dim3(256), 0, s, f);
  else if (f.dz_f16)
    hipLaunchKernelGGL((finalize_fast<_Float16, 2>), grid, dim3(256), 0, s, f);
  else
    hipLaunchKernelGGL((finalize_fast<bf16, 1>), grid, dim3(256), 0, s, f);
  return hipGetLastError();
}

hipError_t launch_partials_bf16(const PartialArgs& p, hipStream_t s) {
  // 16-bit entries: two 64-row tiles of s per workgroup
  if (p.dz_f32)
    hipLaunchKernelGGL((partials_fast<float, 1>), dim3(nblk(p.S, 64), p.H, p.nchunk), dim3(256), 0, s, p);
  else if (p.dz_f16)
    hipLaunchKernelGGL((partials_fast<_Float16, 2>), dim3(nblk(p.S, 128), p.H, p.nchunk), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((partials_fast<bf16, 2>), dim3(nblk(p.S, 128), p.H, p.nchunk), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace relpos
