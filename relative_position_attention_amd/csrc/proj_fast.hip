// Projection kernel for bf16 inputs ([RPA] Table 9 "Projection"; §4.1
// "Reachable Projection Ranges").  [RPA] = "Fast and Exact Relative-Position
// Attention via Structure-Aware Kernels" (arXiv 2611.01182).
//
// Z[i, c] = x_i . A~[s(c)] + b~[s(c)] over each group's reachable window
// (s(c) = c - pad + slo, clamped to the expanded table), stored fp16 with the
// overflow clamp.  The kernel is bound by its stores, so a workgroup owns 64
// rows (one wave per 16 rows, their x fragments held in registers for the
// whole row) and walks the row's column tiles of 64 in order: consecutive
// tiles of one row fill the same cache lines back to back, and the next
// tile's 64 table rows are loaded into registers while the current tile is
// multiplied, then put into LDS (double buffered), where the four waves read
// them as MFMA B operands.  Rows longer than 16 tiles are split into
// segments of equal tile counts, one workgroup each (a causal identity map's
// last rows hold 2N/64 tiles: walked by one workgroup, they set the kernel's
// time alone).  Workgroups are ordered widest group first.
//
// Stores.  A row of Z starts at an arbitrary element (rows are packed at a
// pitch of 7 or 1 mod 8), so the results of a middle tile go through LDS:
// each row's 64 values are written shifted by the row's misalignment m, and
// threads store whole aligned 16-byte chunks (eight per row and tile instead
// of 64 2-byte stores).  The chunk that runs into the next tile (the row's
// last m values) is carried over in LDS and stored with the next tile's
// first chunk.  The first and the last tile of a row segment store their
// entries one by one, as does the carried part that the last tile takes
// over.
#include "kernels.hpp"
#include "tiles.hpp"

namespace relpos {

namespace {

constexpr int kTP = 72;  // LDS pitch of a table tile (bf16), 144-byte rows
constexpr int kZT = 88;  // LDS pitch of the staged result tile (fp16): 64 + 8 + carry room
typedef unsigned int v4u32 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void project_fast(ProjectArgs p, int nrb, int nseg, int seg_tiles) {
  __shared__ __attribute__((aligned(16))) bf16 st[2][64 * kTP];
  __shared__ float sb[2][64];
  __shared__ __attribute__((aligned(16))) _Float16 zt[64 * kZT];
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index(), g = lane >> 4, c16 = lane & 15;
  const int bh = blockIdx.x;
  const int rb = nrb - 1 - static_cast<int>(blockIdx.y) / nseg;
  const int seg = static_cast<int>(blockIdx.y) % nseg;
  const int h = bh % p.H;
  const int r0 = rb * 64;
  const int grp = r0 / kGroup;
  const GroupInfo gi = p.gi[grp];
  // this workgroup's column tiles: [t0, t0 + nct) of the row's tiles
  const int t0 = seg * seg_tiles;
  const int nct_row = (gi.pitch + 63) / 64;
  if (t0 >= nct_row) return;
  const int nct = imin(seg_tiles, nct_row - t0);
  const int cb0 = 64 * t0;  // first column
  const int D2 = 2 * p.D;
  const int64_t tok = static_cast<int64_t>(bh) * p.N;
  const Rsrc rx = make_rsrc(reinterpret_cast<const bf16*>(p.x) + tok * 64,
                            static_cast<uint64_t>(p.N) * 128);
  const Rsrc ra = make_rsrc(reinterpret_cast<const bf16*>(p.at) +
                                static_cast<int64_t>(p.at_shared ? 0 : h) * p.S * 64,
                            static_cast<uint64_t>(p.S) * 128);
  // (no bias table: a resource of size zero, whose loads all read zero)
  const Rsrc rbt = make_rsrc(p.bt != nullptr ? p.bt + static_cast<int64_t>(h) * p.S : nullptr,
                             p.bt != nullptr ? static_cast<uint64_t>(p.S) * 4 : 0);

  // A operand: rows r0 + 16 wave + c16 (rows past N read zero)
  const int rw = r0 + 16 * wave;
  bf16x8 af[2];
#pragma unroll
  for (int c = 0; c < 2; ++c)
    af[c] = __builtin_bit_cast(bf16x8, bload16(rx, static_cast<uint32_t>((rw + c16) * 128 + 64 * c + 16 * g)));

  // table tile staging: row tid >> 2 of the tile, 16 elements at (tid & 3) * 16,
  // and the bias of column tid & 63 (threads past 64 repeat those loads).
  // Every load and store below is issued unconditionally (clamped rows,
  // out-of-range buffer offsets for entries past the window), so each wave
  // issues the same memory instructions on every path: the wait for the next
  // table tile then never covers the stores still in flight.
  // Table tiles are requested two tiles ahead, into two register sets that
  // alternate (the tile loop is unrolled twice so each set keeps its role):
  // a tile's loads then have two tiles of work to arrive in.
  const int ar = tid >> 2, ac = (tid & 3) * 16;
  struct TabRegs {
    uint4 a[2];
    float b;
  };
  TabRegs ra0, ra1;
  auto load_tab = [&](TabRegs& R, int c0) {
    const int s = iclamp(cb0 + c0 + ar - gi.pad + gi.slo, 0, D2);
#pragma unroll
    for (int u = 0; u < 2; ++u) R.a[u] = bload16(ra, static_cast<uint32_t>(s * 128 + (ac + 8 * u) * 2));
    const int sc = iclamp(cb0 + c0 + (tid & 63) - gi.pad + gi.slo, 0, D2);
    R.b = bloadf(rbt, static_cast<uint32_t>(sc) * 4);
  };
  auto store_tab = [&](const TabRegs& R, int buf) {
#pragma unroll
    for (int u = 0; u < 2; ++u) *reinterpret_cast<uint4*>(&st[buf][ar * kTP + ac + 8 * u]) = R.a[u];
    if (tid < 64) sb[buf][tid] = R.b;
  };

  const Rsrc rz = make_rsrc(reinterpret_cast<_Float16*>(p.z) + static_cast<int64_t>(bh) * p.z_bh,
                            static_cast<uint64_t>(p.z_bh) * 2);
  const int g0 = grp * kGroup;

  // MFMA tile of columns c0 .. c0+63 (lane: rows rw + 4g + e, column 16 cb +
  // c16), bias added, as fp32
  auto tile_products = [&](int buf, float (&val)[4][4]) {
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const bf16x8 bfr =
            *reinterpret_cast<const bf16x8*>(&st[buf][(16 * cb + c16) * kTP + 32 * c + 8 * g]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[c], bfr, acc, 0, 0, 0);
      }
      const float add = sb[buf][16 * cb + c16];
#pragma unroll
      for (int e = 0; e < 4; ++e) val[cb][e] = acc[e] + add;
    }
  };
  // entries one by one (entries past the row's pitch or past N are dropped
  // by the buffer range check)
  auto store_each = [&](int c0, const float (&val)[4][4]) {
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const int col = cb0 + c0 + 16 * cb + c16;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = rw + 4 * g + e;
        const bool ok = col < gi.pitch && i < p.N;
        const uint32_t off = ok ? static_cast<uint32_t>(gi.base + (i - g0) * gi.pitch + col) * 2 : kOob;
        const _Float16 v = from_f<_Float16>(val[cb][e]);
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, v), rz, off, 0, 0);
      }
    }
  };
  // the tile into LDS, row r at columns c + m(r) (+ the carry in front)
  int mis[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) mis[e] = (gi.base + (rw + 4 * g + e - g0) * gi.pitch) & 7;
  auto put_lds = [&](const float (&val)[4][4]) {
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * wave + 4 * g + e;
        zt[r * kZT + 16 * cb + c16 + mis[e]] = from_f<_Float16>(val[cb][e]);
      }
  };
  // thread (row zr, quarter zq) stores chunks zq and zq + 4 of its row, and
  // quarter 0 moves the carried chunk (LDS columns 64 .. 71) to the front
  const int zr = tid >> 2, zq = tid & 3;
  const int zi = r0 + zr;
  const int zm = (gi.base + (zi - g0) * gi.pitch) & 7;
  const int zstart = gi.base + (zi - g0) * gi.pitch - zm;  // aligned chunk base
  auto store_chunks = [&](int c0) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int k = zq + 4 * u;
      const uint4 w = *reinterpret_cast<const uint4*>(&zt[zr * kZT + 8 * k]);
      const uint32_t off = zi < p.N ? static_cast<uint32_t>(zstart + cb0 + c0 + 8 * k) * 2 : kOob;
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u32, w), rz, off, 0, 0);
    }
    if (zq == 0)
      *reinterpret_cast<uint4*>(&zt[zr * kZT]) = *reinterpret_cast<const uint4*>(&zt[zr * kZT + 64]);
  };

  load_tab(ra0, 0);
  store_tab(ra0, 0);
  wait_vm_all();
  __syncthreads();
  load_tab(ra1, 64);
  float val[4][4];
  // first tile: entries one by one, and into LDS for the carry
  load_tab(ra0, 128);
  tile_products(0, val);
  store_each(0, val);
  if (nct > 2) put_lds(val);
  store_tab(ra1, 1);
  __syncthreads();
  if (nct > 2) {
    if (zq == 0)
      *reinterpret_cast<uint4*>(&zt[zr * kZT]) = *reinterpret_cast<const uint4*>(&zt[zr * kZT + 64]);
    __syncthreads();
  }
  // middle tiles: aligned 16-byte chunks.  Tile t + 1 sits in the set loaded
  // during tile t - 1, and tile t + 2 goes into the other one (tiles past the
  // window read clamped rows, staged into the buffer no one reads)
  auto middle = [&](int t, TabRegs& next2, const TabRegs& next1) {
    const int buf = t & 1;
    const int c0 = t * 64;
    load_tab(next2, c0 + 128);
    tile_products(buf, val);
    put_lds(val);
    __syncthreads();
    store_chunks(c0);
    store_tab(next1, buf ^ 1);
    __syncthreads();
  };
  int t = 1;
  for (;;) {
    if (t + 1 >= nct) break;
    middle(t, ra1, ra0);
    ++t;
    if (t + 1 >= nct) break;
    middle(t, ra0, ra1);
    ++t;
  }
  // last tile: entries one by one, and the carried entries of the tile before
  // (LDS columns 0 .. m - 1) when that tile stored chunks
  if (nct > 1) {
    tile_products(t & 1, val);
    store_each(t * 64, val);
    if (nct > 2) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int k = zq + 4 * u;  // carried entry k of row zr (k < m)
        const bool ok = k < zm && zi < p.N;
        const uint32_t off = ok ? static_cast<uint32_t>(zstart + cb0 + t * 64 + k) * 2 : kOob;
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, zt[zr * kZT + k]), rz, off, 0, 0);
      }
    }
  }
}

inline unsigned nblk(int64_t n, int b) { return static_cast<unsigned>((n + b - 1) / b); }

}  // namespace

hipError_t launch_project_bf16(const ProjectArgs& p, int BH, int max_pitch, hipStream_t s) {
  const int nrb = static_cast<int>(nblk(p.N, 64));
  // rows of up to 16 tiles take one workgroup; longer ones split into nseg
  // segments of seg_tiles tiles
  const int nct_max = static_cast<int>(nblk(max_pitch, 64));
  const int nseg = static_cast<int>(nblk(nct_max, 16));
  const int seg_tiles = static_cast<int>(nblk(nct_max, nseg));
  hipLaunchKernelGGL(project_fast, dim3(BH, nrb * nseg), dim3(256), 0, s, p, nrb, nseg, seg_tiles);
  return hipGetLastError();
}

}  // namespace relpos
