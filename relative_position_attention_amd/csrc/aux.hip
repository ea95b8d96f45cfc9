// Auxiliary kernels: plan metadata, bucket copies, projections, boundary
// entries, and the reductions of the backward pass.
// [RPA] = "Fast and Exact Relative-Position Attention via Structure-Aware
// Kernels" (arXiv 2611.01182).
#include "common.hpp"
#include "kernels.hpp"
#include "relpos.h"
#include "tiles.hpp"

namespace relpos {

namespace {

// ---------------------------------------------------------------- metadata

// Per-group windows, pads, pitches and row bases of both projection sides
// (the formulas of layout.hpp; the host plan evaluates the same ones).
__global__ __launch_bounds__(256) void meta_groups_kernel(MetaArgs m) {
  __shared__ int64_t part[256];
  const int t = threadIdx.x;
  for (int side = 0; side < 2; ++side) {
    GroupInfo* out = side == 0 ? m.gq : m.gk;
    if (out == nullptr) continue;  // uniform
    const int per = (m.NG + 255) / 256;
    const int g0 = t * per, g1 = imin(m.NG, g0 + per);
    int64_t local = 0;
    for (int g = g0; g < g1; ++g) {
      int slo, shi;
      if (side == 0)
        query_group_window(g, m.N, m.D, m.causal != 0, slo, shi);
      else
        key_group_window(g, m.N, m.D, m.causal != 0, slo, shi);
      const int pad = side == 0 ? query_pad(slo, m.D) : key_pad(slo, m.D);
      const int pitch = pitch_mod8(pad + (shi - slo + 1) + 4, side == 0 ? 7 : 1);
      const int rows = imin(kGroup, m.N - g * kGroup);
      GroupInfo gi;
      gi.slo = slo;
      gi.pad = pad;
      gi.pitch = pitch;
      gi.base = 0;
      out[g] = gi;
      local += (static_cast<int64_t>(rows) * pitch + 7) & ~static_cast<int64_t>(7);
    }
    part[t] = local;
    __syncthreads();
    if (t == 0) {
      int64_t run = 0;
      for (int k = 0; k < 256; ++k) {
        int64_t v = part[k];
        part[k] = run;
        run += v;
      }
    }
    __syncthreads();
    int64_t base = part[t];
    for (int g = g0; g < g1; ++g) {
      const int rows = imin(kGroup, m.N - g * kGroup);
      out[g].base = static_cast<int32_t>(base);
      base += (static_cast<int64_t>(rows) * out[g].pitch + 7) & ~static_cast<int64_t>(7);
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void meta_fill_kernel(MetaChunk c) {
  for (int k = threadIdx.x; k < c.count; k += 256) c.dst[k] = c.vals[k];
}

__global__ __launch_bounds__(256) void meta_affine_kernel(AffineMapArgs m) {
  const int s = blockIdx.x * 256 + threadIdx.x;
  if (s >= m.S) return;
  const int dl = s - m.D;
  int row = -1;
  // (offsets beyond N - 1 in magnitude belong to no pair)
  if (!(m.causal && dl < 0) && dl <= m.N - 1 && dl >= -(m.N - 1)) {
    const int x = m.sign * dl;
    row = m.kind == RELPOS_MAP_IDENTITY ? x + m.offset : iclamp(x, -m.clip, m.clip) + m.clip;
  }
  m.beta[s] = row;
}

__global__ __launch_bounds__(256) void fold_init_kernel(int32_t* fold, int R) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r < R) {
    fold[2 * r] = 1;
    fold[2 * r + 1] = 0;
  }
}

// Each table row's expanded rows form one interval of s (map contiguity);
// its ends are where beta changes.
__global__ __launch_bounds__(256) void fold_scan_kernel(const int32_t* beta, int32_t* fold,
                                                        int S) {
  const int s = blockIdx.x * 256 + threadIdx.x;
  if (s >= S) return;
  const int r = beta[s];
  if (r < 0) return;
  if (s == 0 || beta[s - 1] != r) fold[2 * r] = s;
  if (s == S - 1 || beta[s + 1] != r) fold[2 * r + 1] = s;
}

// ---------------------------------------------------------- bucket copies

// Expanded table A~[ht][s] = A[beta(s)][ht] ([RPA] "Kernel structure": the
// bucket copies copy table rows, A~ = E A); unreachable rows are zero.
template <typename T>
__global__ __launch_bounds__(256) void expand_kernel(ExpandArgs e) {
  constexpr int VEC = 16 / sizeof(T);
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t total = static_cast<int64_t>(e.Ht) * e.S * (64 / VEC);
  if (idx >= total) return;
  const int chunk = static_cast<int>(idx % (64 / VEC));
  const int64_t rowid = idx / (64 / VEC);
  const int s = static_cast<int>(rowid % e.S);
  const int ht = static_cast<int>(rowid / e.S);
  const int r = e.beta[s];
  uint4 val = make_uint4(0, 0, 0, 0);
  if (r >= 0)
    val = *reinterpret_cast<const uint4*>(reinterpret_cast<const T*>(e.table) +
                                          r * e.row_stride + ht * e.head_stride + chunk * VEC);
  *reinterpret_cast<uint4*>(reinterpret_cast<T*>(e.out) + rowid * 64 + chunk * VEC) = val;
}

// b~[h][s] = b[beta_b(s), h] + v_h . A~^Q[s]  (the position bias folded as a
// scalar bias over A^Q's map, [RPA] "Kernel structure")
template <typename T>
__global__ __launch_bounds__(256) void bias_expand_kernel(BiasExpandArgs e) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= e.H * e.S) return;
  const int h = idx / e.S, s = idx % e.S;
  float acc = 0.f;
  if (e.bias != nullptr) {
    const int r = e.beta_b[s];
    if (r >= 0) acc += to_f(reinterpret_cast<const T*>(e.bias)[r * e.row_stride + h * e.head_stride]);
  }
  if (e.vb != nullptr) {
    const T* vb = reinterpret_cast<const T*>(e.vb) + h * 64;
    const T* at = reinterpret_cast<const T*>(e.atq) +
                  (static_cast<int64_t>(e.htq_shared ? 0 : h) * e.S + s) * 64;
    float d = 0.f;
    for (int c = 0; c < 64; ++c) d += to_f(vb[c]) * to_f(at[c]);
    acc += d;
  }
  e.bt[idx] = acc;
}

// ------------------------------------------------------------- projection

// Z[i, c] = x_i . A~[s(c)] (+ b~[s(c)]) over each group's reachable window
// ([RPA] Table 9 "Projection", §4.1 "Reachable Projection Ranges"): one MFMA
// product per 64 rows x 64 columns, stored fp16 (clamped) / fp32.
template <typename T>
__global__ __launch_bounds__(256) void project_kernel(ProjectArgs p) {
  using M = Mma<T>;
  using Frag = typename M::frag;
  using ZT = typename Store<T>::Z;
  constexpr int E = M::E, KS = M::KS, NST = 64 / KS;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index(), g = lane >> 4, c16 = lane & 15;
  const int bh = blockIdx.z;
  const int h = bh % p.H;
  const int r0 = blockIdx.y * 64;
  const int grp = r0 / kGroup;
  const GroupInfo gi = p.gi[grp];
  const int c0 = blockIdx.x * 64;
  if (c0 >= gi.pitch) return;
  const int64_t tok = static_cast<int64_t>(bh) * p.N;
  const T* x = reinterpret_cast<const T*>(p.x) + tok * 64;
  const T* at = reinterpret_cast<const T*>(p.at) +
                static_cast<int64_t>(p.at_shared ? 0 : h) * p.S * 64;
  const int rw = r0 + 16 * wave;
  const int ia = rw + c16;
  Frag af[NST];
#pragma unroll
  for (int c = 0; c < NST; ++c)
    af[c] = ia < p.N ? M::load(x + static_cast<int64_t>(ia) * 64 + c * KS + g * E) : M::zero();
  floatx4 acc[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
    acc[cb] = floatx4{0.f, 0.f, 0.f, 0.f};
    const int col = c0 + 16 * cb + c16;
    const int s = iclamp(col - gi.pad + gi.slo, 0, 2 * p.D);
#pragma unroll
    for (int c = 0; c < NST; ++c) {
      Frag bf = M::load(at + static_cast<int64_t>(s) * 64 + c * KS + g * E);
      acc[cb] = M::run(af[c], bf, acc[cb]);
    }
  }
  ZT* z = reinterpret_cast<ZT*>(p.z) + static_cast<int64_t>(bh) * p.z_bh + gi.base;
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
    const int col = c0 + 16 * cb + c16;
    if (col >= gi.pitch) continue;
    const int s = iclamp(col - gi.pad + gi.slo, 0, 2 * p.D);
    const float add = p.bt != nullptr ? p.bt[h * p.S + s] : 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int i = rw + 4 * g + t;
      if (i < p.N) z[static_cast<int64_t>(i - grp * kGroup) * gi.pitch + col] = from_f<ZT>(acc[cb][t] + add);
    }
  }
}

// D_i = <dO_i, O_i> ([RPA] Table 9 "Preprocessing")
// Eight lanes per row, eight consecutive elements each (one or two 16-byte
// loads per operand, so a wave reads eight whole rows); the eight partial
// sums meet in a fixed butterfly, so the result is the same on every call.
template <typename T>
__device__ __forceinline__ void load8f(const T* p, float* v) {
  if constexpr (sizeof(T) == 4) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    const uint4 w = *reinterpret_cast<const uint4*>(p);
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = __uint_as_float(wd[k] << 16);
      v[2 * k + 1] = __uint_as_float(wd[k] & 0xffff0000u);
    }
  }
}

template <typename T, typename TO>
__global__ __launch_bounds__(256) void rowdot_kernel(const TO* o, const T* dout, float* dvec,
                                                     int64_t rows) {
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t row = gid >> 3;
  const int part = static_cast<int>(gid & 7);
  float acc = 0.f;
  if (row < rows) {
    float a[8], b[8];
    load8f(o + row * 64 + part * 8, a);
    load8f(dout + row * 64 + part * 8, b);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += a[e] * b[e];
  }
  acc += __shfl_xor(acc, 1);
  acc += __shfl_xor(acc, 2);
  acc += __shfl_xor(acc, 4);
  if (row < rows && part == 0) dvec[row] = acc;
}

// the sum of a value over the eight lanes of a row (fixed butterfly)
__device__ __forceinline__ float sum8(float v) {
  v += __shfl_xor(v, 1);
  v += __shfl_xor(v, 2);
  v += __shfl_xor(v, 4);
  return v;
}

// Per-token boundary entries (fp32): the saturated rows 0 and 2D of Z^Q and
// Z^K, with the scalar biases and the Transformer-XL u term folded in; they
// are all that saturated tiles read ([RPA] App. B.2 saturated-tile lemma).
// Eight lanes per row as in rowdot, each lane's eight products summed in
// order, then the fixed butterfly.
template <typename T>
__global__ __launch_bounds__(256) void rowkey_kernel(RowKeyArgs a, int64_t rows) {
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t row = gid >> 3;
  const int part = static_cast<int>(gid & 7);
  const bool ok = row < rows;
  const int64_t rr = ok ? row : 0;
  const int h = static_cast<int>((rr / a.N) % a.H);
  const int D2 = a.S - 1;
  float q[8], k[8];
  if (a.atq != nullptr) load8f(reinterpret_cast<const T*>(a.q) + rr * 64 + part * 8, q);
  if (a.atk != nullptr || a.u != nullptr) load8f(reinterpret_cast<const T*>(a.k) + rr * 64 + part * 8, k);
  float s0 = 0.f, s1 = 0.f, kl = 0.f, kh = 0.f, km = 0.f;
  if (a.atq != nullptr) {
    const T* at = reinterpret_cast<const T*>(a.atq) +
                  static_cast<int64_t>(a.atq_shared ? 0 : h) * a.S * 64 + part * 8;
    float t0[8], t1[8];
    load8f(at, t0);
    load8f(at + static_cast<int64_t>(D2) * 64, t1);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      s0 += q[e] * t0[e];
      s1 += q[e] * t1[e];
    }
  }
  if (a.atk != nullptr) {
    const T* at = reinterpret_cast<const T*>(a.atk) +
                  static_cast<int64_t>(a.atk_shared ? 0 : h) * a.S * 64 + part * 8;
    float t0[8], t1[8];
    load8f(at, t0);
    load8f(at + static_cast<int64_t>(D2) * 64, t1);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      kl += k[e] * t0[e];
      kh += k[e] * t1[e];
    }
  }
  if (a.u != nullptr) {
    float uu[8];
    load8f(reinterpret_cast<const T*>(a.u) + h * 64 + part * 8, uu);
#pragma unroll
    for (int e = 0; e < 8; ++e) km += uu[e] * k[e];
  }
  s0 = sum8(s0);
  s1 = sum8(s1);
  kl = sum8(kl);
  kh = sum8(kh);
  km = sum8(km);
  if (ok && part == 0) {
    a.rowlo[row] = a.bt[h * a.S + 0] + s0;
    a.rowhi[row] = a.bt[h * a.S + D2] + s1;
    a.keylo[row] = kl + km;
    a.keyhi[row] = kh + km;
    a.keymid[row] = km;
  }
}

// ---------------------------------------------------------- dQ / dK finish

template <typename T>
struct RedP {
  static constexpr int KC = 32;                        // expanded rows per chunk
  static constexpr int P = sizeof(T) == 4 ? 36 : 40;   // LDS pitch of a 32-wide tile
};

// out = acc + sum over reachable band rows s of dZ~[i, s] A~[s] (MFMA) +
// boundary sums x A~[0], A~[2D] in fp32 (+ colsum u on the key side):
// [RPA] App. B.1 table-gradient lemma, dQ = tau dS K + dZ^Q A^Q.  The bucket
// fold is implicit: copies of one bucket multiply the same table row.
template <typename T, typename GT>
__global__ __launch_bounds__(256) void finalize_kernel(FinalizeArgs f) {
  using M = Mma<T>;
  using Frag = typename M::frag;
  constexpr int E = M::E, KS = M::KS, KC = RedP<T>::KC, LP = RedP<T>::P;
  __shared__ __attribute__((aligned(16))) T zs[64 * LP];
  __shared__ __attribute__((aligned(16))) T as[64 * LP];
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index(), g = lane >> 4, c16 = lane & 15;
  const int bh = blockIdx.y;
  const int h = bh % f.H;
  const int r0 = blockIdx.x * 64;
  const int64_t tok = static_cast<int64_t>(bh) * f.N;
  const int D = f.D;
  floatx4 acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) acc[db] = floatx4{0.f, 0.f, 0.f, 0.f};
  const T* at = nullptr;
  if (f.at != nullptr)
    at = reinterpret_cast<const T*>(f.at) + static_cast<int64_t>(f.at_shared ? 0 : h) * f.S * 64;

  if (f.dz != nullptr && D >= 1) {
    const int grp = r0 / kGroup;
    const GroupInfo gi = f.gi[grp];
    int slo, shi;
    if (f.key_side)
      key_group_window(grp, f.N, D, f.causal != 0, slo, shi);
    else
      query_group_window(grp, f.N, D, f.causal != 0, slo, shi);
    const int sa = imax(1, slo), sb = imin(2 * D - 1, shi);
    const GT* dz = reinterpret_cast<const GT*>(f.dz) + static_cast<int64_t>(bh) * f.dz_bh + gi.base;
    // staging roles
    const int zrow = tid >> 2, zk0 = (tid & 3) * 8;
    const int zi = r0 + zrow;
    int smin = 1, smax = 0;
    if (zi < f.N) {
      if (f.key_side)
        key_s_range(zi, f.N, D, f.causal != 0, smin, smax);
      else
        query_s_range(zi, f.N, D, f.causal != 0, smin, smax);
    }
    const GT* zrowp = dz + static_cast<int64_t>(zi - grp * kGroup) * gi.pitch;
    const int arow = tid >> 3, ad0 = (tid & 7) * 8;
    for (int s0 = sa; s0 <= sb; s0 += KC) {
      // dZ~ rows -> zs[row][kk]
      T zv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int s = s0 + zk0 + e;
        float val = 0.f;
        if (zi < f.N && s <= sb && s >= smin && s <= smax)
          val = to_f(zrowp[s - gi.slo + gi.pad]);
        zv[e] = from_f<T>(val);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) zs[zrow * LP + zk0 + e] = zv[e];
      // A~ rows -> as[d][kk] (transposed)
      {
        const int s = s0 + arow;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          T val = from_f<T>(0.f);
          if (s <= sb) val = at[static_cast<int64_t>(s) * 64 + ad0 + e];
          as[(ad0 + e) * LP + arow] = val;
        }
      }
      __syncthreads();
#pragma unroll
      for (int c = 0; c < KC / KS; ++c) {
        Frag a = M::load(zs + (16 * wave + c16) * LP + c * KS + g * E);
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          Frag b = M::load(as + (16 * db + c16) * LP + c * KS + g * E);
          acc[db] = M::run(a, b, acc[db]);
        }
      }
      __syncthreads();
    }
  }

  // epilogue: lane holds rows 16*wave + 4g + t, column 16*db + c16
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int i = r0 + 16 * wave + 4 * g + t;
    if (i >= f.N) continue;
    const int64_t row = tok + i;
    float b0 = 0.f, b1 = 0.f, cs = 0.f;
    if (at != nullptr && f.bnd != nullptr) {
      b0 = f.bnd[row * 2 + 0];
      b1 = f.bnd[row * 2 + 1];
    }
    if (f.colsum != nullptr) cs = f.colsum[row];
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int d = 16 * db + c16;
      float v = acc[db][t] + f.acc[row * 64 + d];
      if (at != nullptr) v += b0 * to_f(at[d]) + b1 * to_f(at[static_cast<int64_t>(2 * D) * 64 + d]);
      if (f.colsum != nullptr) v += cs * to_f(reinterpret_cast<const T*>(f.u)[h * 64 + d]);
      if (f.out_f32)
        reinterpret_cast<float*>(f.out)[row * 64 + d] = v;
      else
        reinterpret_cast<bf16*>(f.out)[row * 64 + d] = static_cast<bf16>(v);
    }
  }
}

// ------------------------------------------------- table-gradient partials

// P1[h][c][s][:] = sum_i dZ~[i,s] x_i and P2[h][c][s] = sum_i dZ~[i,s] over
// the tokens of chunk c (fp32, written once per chunk; [RPA] "Deterministic
// table gradients").  Band rows on MFMA from the input-precision entries;
// the two boundary rows in fp32 from the boundary sums.
template <typename T, typename GT>
__global__ __launch_bounds__(256) void partials_kernel(PartialArgs p) {
  using M = Mma<T>;
  using Frag = typename M::frag;
  constexpr int E = M::E, KS = M::KS, NST = 64 / KS;
  constexpr int P = TileP<T>::P;
  constexpr int ZP = 68;  // fp32 row pitch: 16-byte rows, staggered banks
  __shared__ __attribute__((aligned(16))) float zt[64 * ZP];  // [s][token]
  __shared__ __attribute__((aligned(16))) T xt[64 * P];       // [d][token]
  __shared__ float bsh[2][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index(), g = lane >> 4, c16 = lane & 15;
  const int s0 = blockIdx.x * 64;
  const int h = blockIdx.y;
  const int chunk = blockIdx.z;
  const int D = p.D;
  const int nrb = (p.N + 63) / 64;
  const int total = p.B * nrb;
  const int per = (total + p.nchunk - 1) / p.nchunk;
  const int sb0 = chunk * per, sb1 = imin(total, sb0 + per);
  const bool has0 = s0 == 0;
  const bool has2 = (2 * D >= s0) && (2 * D < s0 + 64);
  const bool want_p1 = p.p1 != nullptr;

  floatx4 acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) acc[db] = floatx4{0.f, 0.f, 0.f, 0.f};
  float p2acc = 0.f;               // thread (s = tid/4, quarter tid%4)
  float bx0 = 0.f, bx1 = 0.f;      // boundary P1 (threads < 64: d = tid)
  float bs0 = 0.f, bs1 = 0.f;      // boundary P2 (thread 0)
  Stage<T> sx;
  sx.init(tid);

  for (int sb = sb0; sb < sb1; ++sb) {
    const int b = sb / nrb, rb = sb % nrb;
    const int r0 = rb * 64;
    const int grp = r0 / kGroup;
    int slo, shi;
    if (p.key_side)
      key_group_window(grp, p.N, D, p.causal != 0, slo, shi);
    else
      query_group_window(grp, p.N, D, p.causal != 0, slo, shi);
    const int sa = imax(1, slo), se = imin(2 * D - 1, shi);
    const bool band_hit = D >= 1 && sa <= se && s0 <= se && s0 + 63 >= sa;
    if (!band_hit && !has0 && !has2) continue;  // uniform
    const int64_t tok = (static_cast<int64_t>(b) * p.H + h) * p.N;
    const GroupInfo gi = p.gi[grp];
    if (want_p1) {
      sx.load(reinterpret_cast<const T*>(p.x) + tok * 64, r0, p.N);
      sx.store_trans(xt);
    }
    // dZ~ band entries -> zt[s][token]
    {
      const int tkn = tid >> 2, q4 = (tid & 3) * 16;
      const int i = r0 + tkn;
      int smin = 1, smax = 0;
      if (i < p.N) {
        if (p.key_side)
          key_s_range(i, p.N, D, p.causal != 0, smin, smax);
        else
          query_s_range(i, p.N, D, p.causal != 0, smin, smax);
      }
      smin = imax(smin, sa);
      smax = imin(smax, se);
      const GT* row = reinterpret_cast<const GT*>(p.dz) + static_cast<int64_t>(b * p.H + h) * p.dz_bh +
                      gi.base + static_cast<int64_t>(i - grp * kGroup) * gi.pitch;
#pragma unroll 4
      for (int e = 0; e < 16; ++e) {
        const int s = s0 + q4 + e;
        float val = 0.f;
        if (band_hit && i < p.N && s >= smin && s <= smax) val = to_f(row[s - gi.slo + gi.pad]);
        zt[(q4 + e) * ZP + tkn] = val;
      }
    }
    __syncthreads();
    if (want_p1 && band_hit) {
#pragma unroll
      for (int c = 0; c < NST; ++c) {
        Frag a = frag_f32<T>(zt + (16 * wave + c16) * ZP + c * KS + g * E);
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          Frag bb = M::load(xt + (16 * db + c16) * P + c * KS + g * E);
          acc[db] = M::run(a, bb, acc[db]);
        }
      }
    }
    if (p.p2 != nullptr && band_hit) {
      const int s = tid >> 2, q = (tid & 3) * 16;
      float part = 0.f;
      for (int e = 0; e < 16; ++e) part += zt[s * ZP + q + e];
      part += __shfl_xor(part, 1);
      part += __shfl_xor(part, 2);
      p2acc += part;
    }
    if (has0 || has2) {
      if (tid < 64) bsh[0][tid] = 0.f, bsh[1][tid] = 0.f;
      __syncthreads();
      if (tid < 64) {
        const int i = r0 + tid;
        if (i < p.N) {
          bsh[0][tid] = p.bnd[(tok + i) * 2 + 0];
          bsh[1][tid] = p.bnd[(tok + i) * 2 + 1];
        }
      }
      __syncthreads();
      if (want_p1 && tid < 64) {
        for (int tk = 0; tk < 64; ++tk) {
          const float xv = to_f(xt[tid * P + tk]);
          bx0 += bsh[0][tk] * xv;
          bx1 += bsh[1][tk] * xv;
        }
      }
      if (tid == 0) {
        for (int tk = 0; tk < 64; ++tk) {
          bs0 += bsh[0][tk];
          bs1 += bsh[1][tk];
        }
      }
    }
    __syncthreads();
  }

  // write the chunk's partials
  const int64_t pbase = (static_cast<int64_t>(h) * p.nchunk + chunk) * p.S;
  if (want_p1) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int s = s0 + 16 * wave + 4 * g + t;
      if (s >= p.S) continue;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int d = 16 * db + c16;
        p.p1[(pbase + s) * 64 + d] = acc[db][t];
      }
    }
    __syncthreads();
    if (tid < 64) {
      // boundary rows: add in a fixed order after the band part
      if (has0) p.p1[(pbase + 0) * 64 + tid] += bx0 + (2 * D == 0 ? bx1 : 0.f);
      if (has2 && D > 0) p.p1[(pbase + 2 * D) * 64 + tid] += bx1;
    }
  }
  if (p.p2 != nullptr) {
    const int s = s0 + (tid >> 2);
    if ((tid & 3) == 0 && s < p.S) p.p2[pbase + s] = p2acc;
    __syncthreads();
    if (tid == 0) {
      if (has0) p.p2[pbase + 0] += bs0 + (2 * D == 0 ? bs1 : 0.f);
      if (has2 && D > 0) p.p2[pbase + 2 * D] += bs1;
    }
  }
}

// Fixed-order sums over chunks (and heads for a shared table) of the
// partials, then the bucket fold over the table row's expanded rows.  The
// row's items (s, h, c), in that nesting order, are dealt round robin to the
// four waves (four loads in flight each); the four wave sums are added in
// wave order, so the result is the same on every call.
__global__ __launch_bounds__(256) void fold_table_kernel(FoldArgs f, int dtype) {
  __shared__ float red[4][64];
  const int r = blockIdx.x, ht = blockIdx.y, d = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int sa = f.fold[2 * r], sb = f.fold[2 * r + 1];
  const int h0 = f.shared ? 0 : ht, nh = f.shared ? f.H : 1;
  const int n = sb >= sa ? (sb - sa + 1) * nh * f.nchunk : 0;
  auto item = [&](int it) {
    const int c = it % f.nchunk, rest = it / f.nchunk;
    const int h = h0 + rest % nh, pos = sa + rest / nh;
    const int s = f.list != nullptr ? f.list[pos] : pos;
    const int64_t base = (static_cast<int64_t>(h) * f.nchunk + c) * f.S + s;
    float v = f.p1[base * 64 + d];
    if (f.vb != nullptr) {
      const float vb = dtype == 0 ? reinterpret_cast<const float*>(f.vb)[h * 64 + d]
                                  : static_cast<float>(reinterpret_cast<const bf16*>(f.vb)[h * 64 + d]);
      v += vb * f.p2[base];
    }
    return v;
  };
  float sum = 0.f;
  int it = w;
  for (; it + 12 < n; it += 16) {
    const float v0 = item(it), v1 = item(it + 4), v2 = item(it + 8), v3 = item(it + 12);
    sum += v0;
    sum += v1;
    sum += v2;
    sum += v3;
  }
  for (; it < n; it += 4) sum += item(it);
  red[w][d] = sum;
  __syncthreads();
  if (w == 0)
    f.out[r * f.row_stride + ht * f.head_stride + d] = ((red[0][d] + red[1][d]) + red[2][d]) + red[3][d];
}

// db[h][s] = sum over chunks c (ascending) of P2[h][c][s]
__global__ __launch_bounds__(256) void p2_sum_kernel(const float* p2, float* db, int H, int S,
                                                     int nchunk) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= H * S) return;
  const int h = idx / S, s = idx % S;
  float sum = 0.f;
  for (int c = 0; c < nchunk; ++c) sum += p2[(static_cast<int64_t>(h) * nchunk + c) * S + s];
  db[idx] = sum;
}

// dbias[r, h] = sum over the copies s of row r (ascending) of db[h][s]: the
// bucket fold of [RPA] App. B.1 (bucket-copy lemma), db = E^T db~; the copies
// are an interval of s, or listed when the row's offsets are not contiguous
__global__ __launch_bounds__(256) void fold_bias_kernel(FoldBiasArgs f) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= f.R * f.H) return;
  const int r = idx / f.H, h = idx % f.H;
  const int sa = f.fold[2 * r], sb = f.fold[2 * r + 1];
  float sum = 0.f;
  for (int pos = sa; pos <= sb; ++pos)
    sum += f.db[static_cast<int64_t>(h) * f.S + (f.list != nullptr ? f.list[pos] : pos)];
  f.out[r * f.row_stride + h * f.head_stride] = sum;
}

constexpr int kSplit = 64;  // partial sums per head in the two-phase row sums

// Both first phases give a row r (an expanded table row, or a token) to a
// group of eight lanes holding eight consecutive columns each (16-byte
// loads); 32 rows are in flight per step, and the 32 row sums of each
// column are added in row-group order through LDS, so the result is the same
// on every call.
template <typename T>
__device__ __forceinline__ void load8(const T* p, float* v) {
  if constexpr (sizeof(T) == 4) {
    const float4 x = *reinterpret_cast<const float4*>(p);
    const float4 y = *reinterpret_cast<const float4*>(p + 4);
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
    v[4] = y.x; v[5] = y.y; v[6] = y.z; v[7] = y.w;
  } else {
    const uint4 w = *reinterpret_cast<const uint4*>(p);
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = __uint_as_float(wd[k] << 16);
      v[2 * k + 1] = __uint_as_float(wd[k] & 0xffff0000u);
    }
  }
}

// the 32 row groups' sums of column c8 * 8 + e (threads t: c8 = t & 7,
// group t >> 3), reduced in group order, written by threads < 64
__device__ __forceinline__ void reduce_groups(float (&acc)[8], float* out) {
  __shared__ float red[32][65];
  const int t = threadIdx.x, c8 = t & 7, grp = t >> 3;
#pragma unroll
  for (int e = 0; e < 8; ++e) red[grp][c8 * 8 + e] = acc[e];
  __syncthreads();
  if (t < 64) {
    float s = 0.f;
    for (int k = 0; k < 32; ++k) s += red[k][t];
    out[t] = s;
  }
}

// dv, first phase: part[h][sp][d] = sum over the rows s of split sp of
// db[h][s] A~^Q[s][d]
template <typename T>
__global__ __launch_bounds__(256) void dv_part_kernel(DvArgs a) {
  const int h = blockIdx.x, sp = blockIdx.y, c8 = threadIdx.x & 7, grp = threadIdx.x >> 3;
  const int per = (a.S + kSplit - 1) / kSplit;
  const int s0 = sp * per, s1 = imin(a.S, s0 + per);
  const T* at = reinterpret_cast<const T*>(a.atq) +
                static_cast<int64_t>(a.at_shared ? 0 : h) * a.S * 64;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s = s0 + grp; s < s1; s += 32) {
    float v[8];
    load8(at + static_cast<int64_t>(s) * 64 + c8 * 8, v);
    const float w = a.db[static_cast<int64_t>(h) * a.S + s];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += w * v[e];
  }
  reduce_groups(acc, a.part + (static_cast<int64_t>(h) * kSplit + sp) * 64);
}

// du, first phase: part[h][sp][d] = sum over the tokens (b, j) of split sp of
// colsum[b, h, j] k[b, h, j, d]
template <typename T>
__global__ __launch_bounds__(256) void du_part_kernel(DuArgs a) {
  const int h = blockIdx.x, sp = blockIdx.y, c8 = threadIdx.x & 7, grp = threadIdx.x >> 3;
  const int64_t total = static_cast<int64_t>(a.B) * a.N;
  const int64_t per = (total + kSplit - 1) / kSplit;
  const int64_t t0 = sp * per, t1 = t0 + per < total ? t0 + per : total;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int64_t t = t0 + grp; t < t1; t += 32) {
    const int64_t b = t / a.N, j = t % a.N;
    const int64_t row = (b * a.H + h) * a.N + j;
    float v[8];
    load8(reinterpret_cast<const T*>(a.k) + row * 64 + c8 * 8, v);
    const float w = a.colsum[row];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += w * v[e];
  }
  reduce_groups(acc, a.part + (static_cast<int64_t>(h) * kSplit + sp) * 64);
}

// second phase: out[h][d] = sum over splits (ascending) of part[h][sp][d]
__global__ __launch_bounds__(64) void split_sum_kernel(const float* part, float* out) {
  const int h = blockIdx.x, d = threadIdx.x;
  float sum = 0.f;
  for (int sp = 0; sp < kSplit; ++sp) sum += part[(static_cast<int64_t>(h) * kSplit + sp) * 64 + d];
  out[h * 64 + d] = sum;
}

inline unsigned nblk(int64_t n, int b) { return static_cast<unsigned>((n + b - 1) / b); }

}  // namespace

hipError_t launch_meta_groups(const MetaArgs& m, hipStream_t s) {
  hipLaunchKernelGGL(meta_groups_kernel, dim3(1), dim3(256), 0, s, m);
  return hipGetLastError();
}

hipError_t launch_meta_fill(const MetaChunk& c, hipStream_t s) {
  hipLaunchKernelGGL(meta_fill_kernel, dim3(1), dim3(256), 0, s, c);
  return hipGetLastError();
}

// 64 x 64 tile transpose through LDS (bf16 words): block (cb, h) moves table
// rows c = 64 cb .. +63 of head h into columns c of dst.
__global__ __launch_bounds__(256) void transpose_rows_kernel(const u16* src, u16* dst, int S, int Sp) {
  __shared__ u16 t[64][66];
  const int cb = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const u16* sh = src + static_cast<int64_t>(h) * S * 64;
  u16* dh = dst + static_cast<int64_t>(h) * 64 * Sp;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int idx = tid + 256 * k, r = idx >> 6, e = idx & 63;
    const int c = 64 * cb + r;
    t[r][e] = c < S ? sh[static_cast<int64_t>(c) * 64 + e] : u16(0);
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int idx = tid + 256 * k, e = idx >> 6, r = idx & 63;
    const int c = 64 * cb + r;
    if (c < Sp) dh[static_cast<int64_t>(e) * Sp + c] = t[r][e];
  }
}

hipError_t launch_transpose_rows(const void* src, void* dst, int Ht, int S, int Sp, hipStream_t s) {
  hipLaunchKernelGGL(transpose_rows_kernel, dim3(nblk(Sp, 64), Ht), dim3(256), 0, s,
                     static_cast<const u16*>(src), static_cast<u16*>(dst), S, Sp);
  return hipGetLastError();
}

hipError_t launch_meta_affine(const AffineMapArgs& m, hipStream_t s) {
  hipLaunchKernelGGL(meta_affine_kernel, dim3(nblk(m.S, 256)), dim3(256), 0, s, m);
  return hipGetLastError();
}

hipError_t launch_fold_meta(const int32_t* beta, int32_t* fold, int S, int R, hipStream_t s) {
  hipLaunchKernelGGL(fold_init_kernel, dim3(nblk(R, 256)), dim3(256), 0, s, fold, R);
  hipLaunchKernelGGL(fold_scan_kernel, dim3(nblk(S, 256)), dim3(256), 0, s, beta, fold, S);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void zero_kernel(uint4* p, int64_t n16) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  for (int64_t k = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; k < n16; k += stride)
    p[k] = uint4{0u, 0u, 0u, 0u};
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s) {
  const int64_t n16 = static_cast<int64_t>(bytes / 16);
  if (n16 == 0) return hipSuccess;
  const unsigned grid = static_cast<unsigned>(std::min<int64_t>(nblk(n16, 256), 4096));
  hipLaunchKernelGGL(zero_kernel, dim3(grid), dim3(256), 0, s, reinterpret_cast<uint4*>(p), n16);
  return hipGetLastError();
}

hipError_t launch_expand(int dtype, const ExpandArgs& e, hipStream_t s) {
  const int vec = dtype == 0 ? 4 : 8;
  const int64_t total = static_cast<int64_t>(e.Ht) * e.S * (64 / vec);
  if (dtype == 0)
    hipLaunchKernelGGL(expand_kernel<float>, dim3(nblk(total, 256)), dim3(256), 0, s, e);
  else
    hipLaunchKernelGGL(expand_kernel<bf16>, dim3(nblk(total, 256)), dim3(256), 0, s, e);
  return hipGetLastError();
}

hipError_t launch_bias_expand(int dtype, const BiasExpandArgs& e, hipStream_t s) {
  const unsigned g = nblk(static_cast<int64_t>(e.H) * e.S, 256);
  if (dtype == 0)
    hipLaunchKernelGGL(bias_expand_kernel<float>, dim3(g), dim3(256), 0, s, e);
  else
    hipLaunchKernelGGL(bias_expand_kernel<bf16>, dim3(g), dim3(256), 0, s, e);
  return hipGetLastError();
}

hipError_t launch_project_f32(const ProjectArgs& p, int BH, int max_pitch, hipStream_t s) {
  dim3 grid(nblk(max_pitch, 64), nblk(p.N, 64), BH);
  hipLaunchKernelGGL(project_kernel<float>, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_rowkey(int dtype, const RowKeyArgs& a, int BH, hipStream_t s) {
  const int64_t rows = static_cast<int64_t>(BH) * a.N;
  if (dtype == 0)
    hipLaunchKernelGGL(rowkey_kernel<float>, dim3(nblk(rows * 8, 256)), dim3(256), 0, s, a, rows);
  else
    hipLaunchKernelGGL(rowkey_kernel<bf16>, dim3(nblk(rows * 8, 256)), dim3(256), 0, s, a, rows);
  return hipGetLastError();
}

hipError_t launch_rowdot(int dtype, int out_f32, const void* o, const void* dout, float* dvec,
                         int64_t rows, hipStream_t s) {
  dim3 grid(nblk(rows * 8, 256));
  if (dtype == 0 && out_f32)
    hipLaunchKernelGGL((rowdot_kernel<float, float>), grid, dim3(256), 0, s,
                       reinterpret_cast<const float*>(o), reinterpret_cast<const float*>(dout), dvec, rows);
  else if (dtype == 0)
    hipLaunchKernelGGL((rowdot_kernel<float, bf16>), grid, dim3(256), 0, s,
                       reinterpret_cast<const bf16*>(o), reinterpret_cast<const float*>(dout), dvec, rows);
  else if (out_f32)
    hipLaunchKernelGGL((rowdot_kernel<bf16, float>), grid, dim3(256), 0, s,
                       reinterpret_cast<const float*>(o), reinterpret_cast<const bf16*>(dout), dvec, rows);
  else
    hipLaunchKernelGGL((rowdot_kernel<bf16, bf16>), grid, dim3(256), 0, s,
                       reinterpret_cast<const bf16*>(o), reinterpret_cast<const bf16*>(dout), dvec, rows);
  return hipGetLastError();
}

hipError_t launch_finalize_f32(const FinalizeArgs& f, int BH, hipStream_t s) {
  dim3 grid(nblk(f.N, 64), BH);
  hipLaunchKernelGGL((finalize_kernel<float, float>), grid, dim3(256), 0, s, f);
  return hipGetLastError();
}

hipError_t launch_partials_f32(const PartialArgs& p, hipStream_t s) {
  dim3 grid(nblk(p.S, 64), p.H, p.nchunk);
  hipLaunchKernelGGL((partials_kernel<float, float>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_fold_table(int dtype, const FoldArgs& f, hipStream_t s) {
  hipLaunchKernelGGL(fold_table_kernel, dim3(f.R, f.Ht), dim3(256), 0, s, f, dtype);
  return hipGetLastError();
}

hipError_t launch_p2_sum(const float* p2, float* db, int H, int S, int nchunk, hipStream_t s) {
  hipLaunchKernelGGL(p2_sum_kernel, dim3(nblk(static_cast<int64_t>(H) * S, 256)), dim3(256), 0, s,
                     p2, db, H, S, nchunk);
  return hipGetLastError();
}

hipError_t launch_fold_bias(const FoldBiasArgs& f, hipStream_t s) {
  hipLaunchKernelGGL(fold_bias_kernel, dim3(nblk(static_cast<int64_t>(f.R) * f.H, 256)), dim3(256),
                     0, s, f);
  return hipGetLastError();
}

hipError_t launch_dv(int dtype, const DvArgs& a, hipStream_t s) {
  if (dtype == 0)
    hipLaunchKernelGGL(dv_part_kernel<float>, dim3(a.H, kSplit), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(dv_part_kernel<bf16>, dim3(a.H, kSplit), dim3(256), 0, s, a);
  hipLaunchKernelGGL(split_sum_kernel, dim3(a.H), dim3(64), 0, s, a.part, a.out);
  return hipGetLastError();
}

hipError_t launch_du(int dtype, const DuArgs& a, hipStream_t s) {
  if (dtype == 0)
    hipLaunchKernelGGL(du_part_kernel<float>, dim3(a.H, kSplit), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(du_part_kernel<bf16>, dim3(a.H, kSplit), dim3(256), 0, s, a);
  hipLaunchKernelGGL(split_sum_kernel, dim3(a.H), dim3(64), 0, s, a.part, a.out);
  return hipGetLastError();
}

}  // namespace relpos
