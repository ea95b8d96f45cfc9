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
// them as MFMA B operands.  Workgroups are ordered widest group first, which
// balances the jagged windows of causal identity maps.
#include "kernels.hpp"
#include "tiles.hpp"

namespace relpos {

namespace {

constexpr int kTP = 72;  // LDS pitch of a table tile (bf16), 144-byte rows

__global__ __launch_bounds__(256) void project_fast(ProjectArgs p, int nrb) {
  __shared__ __attribute__((aligned(16))) bf16 st[2][64 * kTP];
  __shared__ float sb[2][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index(), g = lane >> 4, c16 = lane & 15;
  const int bh = blockIdx.x;
  const int rb = nrb - 1 - static_cast<int>(blockIdx.y);
  const int h = bh % p.H;
  const int r0 = rb * 64;
  const int grp = r0 / kGroup;
  const GroupInfo gi = p.gi[grp];
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
  const int ar = tid >> 2, ac = (tid & 3) * 16;
  uint4 ta[2];
  float tb = 0.f;
  auto load_tab = [&](int c0) {
    const int s = iclamp(c0 + ar - gi.pad + gi.slo, 0, D2);
#pragma unroll
    for (int u = 0; u < 2; ++u) ta[u] = bload16(ra, static_cast<uint32_t>(s * 128 + (ac + 8 * u) * 2));
    const int sc = iclamp(c0 + (tid & 63) - gi.pad + gi.slo, 0, D2);
    tb = bloadf(rbt, static_cast<uint32_t>(sc) * 4);
  };
  auto store_tab = [&](int buf) {
#pragma unroll
    for (int u = 0; u < 2; ++u) *reinterpret_cast<uint4*>(&st[buf][ar * kTP + ac + 8 * u]) = ta[u];
    if (tid < 64) sb[buf][tid] = tb;
  };

  const Rsrc rz = make_rsrc(reinterpret_cast<_Float16*>(p.z) + static_cast<int64_t>(bh) * p.z_bh,
                            static_cast<uint64_t>(p.z_bh) * 2);
  const int nct = (gi.pitch + 63) / 64;
  load_tab(0);
  store_tab(0);
  wait_vm_all();
  __syncthreads();
  for (int t = 0; t < nct; ++t) {
    const int buf = t & 1;
    const int c0 = t * 64;
    load_tab(c0 + 64);
    floatx4 acc[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      acc[cb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const bf16x8 bfr =
            *reinterpret_cast<const bf16x8*>(&st[buf][(16 * cb + c16) * kTP + 32 * c + 8 * g]);
        acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[c], bfr, acc[cb], 0, 0, 0);
      }
    }
    // lane holds rows rw + 4g + e, column c0 + 16 cb + c16 (entries past the
    // row's window or past N are dropped by the buffer range check)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const int cl = 16 * cb + c16;
      const int col = c0 + cl;
      const float add = sb[buf][cl];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = rw + 4 * g + e;
        const bool ok = col < gi.pitch && i < p.N;
        const uint32_t off = ok ? static_cast<uint32_t>(gi.base + (i - grp * kGroup) * gi.pitch + col) * 2 : kOob;
        const _Float16 v = from_f<_Float16>(acc[cb][e] + add);
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, v), rz, off, 0, 0);
      }
    }
    // (the tile after the last is staged too, into the buffer no one reads)
    store_tab(buf ^ 1);
    __syncthreads();
  }
}

inline unsigned nblk(int64_t n, int b) { return static_cast<unsigned>((n + b - 1) / b); }

}  // namespace

hipError_t launch_project_bf16(const ProjectArgs& p, int BH, hipStream_t s) {
  const int nrb = static_cast<int>(nblk(p.N, 64));
  hipLaunchKernelGGL(project_fast, dim3(BH, nrb), dim3(256), 0, s, p, nrb);
  return hipGetLastError();
}

}  // namespace relpos
