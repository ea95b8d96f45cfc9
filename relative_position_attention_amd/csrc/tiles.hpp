// LDS tile staging for the attention kernels: 64 rows x 64 columns of the
// input type, loaded from global memory with 16-byte vector loads (rows past
// the sequence read as zero) and written to LDS row-major and/or transposed.
#pragma once

#include "common.hpp"

namespace relpos {

template <typename T>
struct TileP {
  // LDS row pitch in elements: 16-byte rows, staggered banks.
  static constexpr int P = sizeof(T) == 4 ? 68 : 72;
};

template <typename T>
struct Stage {
  static constexpr int VEC = 16 / sizeof(T);           // elements per 16 bytes
  static constexpr int CPR = 64 / VEC;                 // chunks per row
  static constexpr int RPT = 64 * 64 / (256 * VEC);    // rows per thread
  uint4 r[RPT];
  int rb, c0;

  __device__ __forceinline__ void init(int tid) {
    rb = tid / CPR;
    c0 = (tid % CPR) * VEC;
  }
  // rows [row0, row0 + 64) of a dense [*, 64] matrix; rows >= nrows -> 0
  __device__ __forceinline__ void load(const T* src, int row0, int nrows) {
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
      int grow = row0 + rb * RPT + k;
      if (grow < nrows)
        r[k] = *reinterpret_cast<const uint4*>(src + static_cast<int64_t>(grow) * 64 + c0);
      else
        r[k] = make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void store_rows(T* lds) const {
    constexpr int P = TileP<T>::P;
#pragma unroll
    for (int k = 0; k < RPT; ++k)
      *reinterpret_cast<uint4*>(lds + (rb * RPT + k) * P + c0) = r[k];
  }
  // lds[col][row]: element (row, col) of the tile at lds[col * P + row]
  __device__ __forceinline__ void store_trans(T* lds) const {
    constexpr int P = TileP<T>::P;
    if constexpr (sizeof(T) == 2) {
      const u16* a = reinterpret_cast<const u16*>(&r[0]);
      const u16* b = reinterpret_cast<const u16*>(&r[1]);
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        uint32_t pair = static_cast<uint32_t>(a[e]) | (static_cast<uint32_t>(b[e]) << 16);
        *reinterpret_cast<uint32_t*>(lds + (c0 + e) * P + rb * RPT) = pair;
      }
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        uint4 col;
        col.x = reinterpret_cast<const uint32_t*>(&r[0])[e];
        col.y = reinterpret_cast<const uint32_t*>(&r[1])[e];
        col.z = reinterpret_cast<const uint32_t*>(&r[2])[e];
        col.w = reinterpret_cast<const uint32_t*>(&r[3])[e];
        *reinterpret_cast<uint4*>(lds + (c0 + e) * P + rb * RPT) = col;
      }
    }
  }
};

// A-operand fragment of a row-major LDS tile: row `row`, K-step c.
template <typename T>
__device__ __forceinline__ typename Mma<T>::frag frag_rows(const T* lds, int row, int c, int g) {
  constexpr int P = TileP<T>::P;
  return Mma<T>::load(lds + row * P + c * Mma<T>::KS + g * Mma<T>::E);
}

// Fragment over the 64-entry K axis of a transposed LDS tile (lds[m][k]) for
// the permuted order used with register-held probabilities: K-step c covers
// the lane's values idx = c*E + e, idx -> k = 16*(idx/4) + 4*g + idx%4.
template <typename T>
__device__ __forceinline__ typename Mma<T>::frag frag_perm(const T* lds, int m, int c, int g) {
  constexpr int P = TileP<T>::P;
  if constexpr (sizeof(T) == 2) {
    const T* row = lds + m * P + 32 * c + 4 * g;
    bf16x4 lo = *reinterpret_cast<const bf16x4*>(row);
    bf16x4 hi = *reinterpret_cast<const bf16x4*>(row + 16);
    bf16x8 f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[e] = lo[e];
      f[e + 4] = hi[e];
    }
    return f;
  } else {
    return lds[m * P + 16 * (c >> 2) + 4 * g + (c & 3)];
  }
}

// Register values v[blk][t] (blk = 16-row block of the K axis, t = 0..3) as
// the matching B fragment of K-step c.
template <typename T, int NB>
__device__ __forceinline__ typename Mma<T>::frag frag_regs(const float (&v)[NB][4], int c) {
  if constexpr (sizeof(T) == 2) {
    bf16x8 f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = static_cast<bf16>(v[2 * c + (e >> 2)][e & 3]);
    return f;
  } else {
    return v[c >> 2][c & 3];
  }
}

// The rounding residue v - bf16(v) of the same values, as a bf16 fragment:
// with frag_regs it forms a two-term (hi + lo) operand carrying about 16
// significant bits, for products whose operand must not be cut to 8 bits.
template <typename T, int NB>
__device__ __forceinline__ typename Mma<T>::frag frag_regs_lo(const float (&v)[NB][4], int c) {
  bf16x8 f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float x = v[2 * c + (e >> 2)][e & 3];
    f[e] = static_cast<bf16>(x - static_cast<float>(static_cast<bf16>(x)));
  }
  return f;
}

// An fp32 LDS run as an MFMA fragment (rounded once to bf16 for bf16 MFMA).
template <typename T>
__device__ __forceinline__ typename Mma<T>::frag frag_f32(const float* p) {
  if constexpr (sizeof(T) == 2) {
    floatx4 a = *reinterpret_cast<const floatx4*>(p);
    floatx4 b = *reinterpret_cast<const floatx4*>(p + 4);
    bf16x8 f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[e] = static_cast<bf16>(a[e]);
      f[e + 4] = static_cast<bf16>(b[e]);
    }
    return f;
  } else {
    return *p;
  }
}

}  // namespace relpos
