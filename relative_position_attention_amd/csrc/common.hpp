// Device helpers shared by the gfx950 kernels: element types, MFMA fragments,
// small vector loads/stores, wave reductions.
//
// MFMA usage.  Every product uses the 16x16 output tile of
// v_mfma_f32_16x16x32_bf16 (bf16 inputs) or v_mfma_f32_16x16x4_f32 (fp32
// inputs).  Both share the output layout: lane l holds rows 4*(l>>4)+t,
// t = 0..3, of column l&15.  Lane l supplies, for A, row l&15 and for B,
// column l&15, with E consecutive K-elements starting at E*(l>>4) (E = 8 for
// bf16, 1 for fp32); one MFMA covers K = 4E.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "layout.hpp"

namespace relpos {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef _Float16 halfx4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <typename T>
struct Mma;

template <>
struct Mma<bf16> {
  static constexpr int E = 8;
  static constexpr int KS = 32;
  using frag = bf16x8;
  static __device__ __forceinline__ floatx4 run(frag a, frag b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ frag load(const bf16* p) {
    return *reinterpret_cast<const bf16x8*>(p);
  }
  static __device__ __forceinline__ frag zero() {
    frag f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = (bf16)0.f;
    return f;
  }
};

template <>
struct Mma<float> {
  static constexpr int E = 1;
  static constexpr int KS = 4;
  using frag = float;
  static __device__ __forceinline__ floatx4 run(frag a, frag b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ frag load(const float* p) { return *p; }
  static __device__ __forceinline__ frag zero() { return 0.f; }
};

// Storage type of the projections Z (fp16 for bf16 inputs, [RPA] "Half-
// precision numerics") and of the offset gradients (input precision).
template <typename T>
struct Store;
template <>
struct Store<bf16> {
  using Z = _Float16;
  using G = bf16;
};
template <>
struct Store<float> {
  using Z = float;
  using G = float;
};

// Element type of the offset gradients dZ~ written by the backward passes:
// the input precision ([RPA] "Half-precision numerics"), except fp32 for a
// scalar bias without a query table, whose per-row sums cancel (every row of
// dS sums to zero) and would lose the 8-bit entries' precision.
template <typename T, bool BIAS_ONLY>
struct DzType {
  using type = typename Store<T>::G;
};
template <typename T>
struct DzType<T, true> {
  using type = float;
};

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(bf16 x) { return static_cast<float>(x); }
__device__ __forceinline__ float to_f(_Float16 x) { return static_cast<float>(x); }

template <typename T>
__device__ __forceinline__ T from_f(float x);
template <>
__device__ __forceinline__ float from_f<float>(float x) {
  return x;
}
template <>
__device__ __forceinline__ bf16 from_f<bf16>(float x) {
  return static_cast<bf16>(x);
}
template <>
__device__ __forceinline__ _Float16 from_f<_Float16>(float x) {
  // clamp to the fp16 range so an outlier cannot overflow to infinity
  x = fminf(fmaxf(x, -65504.f), 65504.f);
  return static_cast<_Float16>(x);
}

// 4 consecutive elements (aligned run) -> float[4]
__device__ __forceinline__ void load4(const _Float16* p, float* out) {
  halfx4 v = *reinterpret_cast<const halfx4*>(p);
#pragma unroll
  for (int t = 0; t < 4; ++t) out[t] = static_cast<float>(v[t]);
}
__device__ __forceinline__ void load4(const float* p, float* out) {
  floatx4 v = *reinterpret_cast<const floatx4*>(p);
#pragma unroll
  for (int t = 0; t < 4; ++t) out[t] = v[t];
}
__device__ __forceinline__ void store4(bf16* p, const float* in) {
  bf16x4 v;
#pragma unroll
  for (int t = 0; t < 4; ++t) v[t] = static_cast<bf16>(in[t]);
  *reinterpret_cast<bf16x4*>(p) = v;
}
__device__ __forceinline__ void store4(_Float16* p, const float* in) {
  halfx4 v;
#pragma unroll
  for (int t = 0; t < 4; ++t) v[t] = static_cast<_Float16>(in[t]);
  *reinterpret_cast<halfx4*>(p) = v;
}
__device__ __forceinline__ void store4(float* p, const float* in) {
  floatx4 v;
#pragma unroll
  for (int t = 0; t < 4; ++t) v[t] = in[t];
  *reinterpret_cast<floatx4*>(p) = v;
}

// Four consecutive fp32 values at p[idx..idx+3]; entries at or past `n` read 0.
// One 16-byte load when in range and aligned, else scalar loads.
__device__ __forceinline__ void load4_guard(const float* p, int idx, int n, float* out) {
  if (idx + 3 < n && (reinterpret_cast<uintptr_t>(p + idx) & 15) == 0) {
    floatx4 v = *reinterpret_cast<const floatx4*>(p + idx);
#pragma unroll
    for (int t = 0; t < 4; ++t) out[t] = v[t];
  } else {
#pragma unroll
    for (int t = 0; t < 4; ++t) out[t] = (idx + t < n) ? p[idx + t] : 0.f;
  }
}

// Reductions over the four lane groups l>>4 that share l&15, with the gfx950
// lane-swap instructions: permlane16_swap pairs every lane with lane l^16 and
// permlane32_swap with l^32 (each returns the pair of values, in an order
// that depends on the lane, so the symmetric max / sum of the two is taken).
__device__ __forceinline__ float xor16_pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_pair_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_pair_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float wave_max_g(float v) { return xor32_pair_max(xor16_pair_max(v)); }
// (the two operands of each add are the same pair in both lanes, so all four
// lanes of a column get bitwise the same sum)
__device__ __forceinline__ float wave_sum_g(float v) { return xor32_pair_sum(xor16_pair_sum(v)); }

// Transposing LDS read (ds_read_b64_tr_b16).  Within each 16-lane group, lane
// m receives tile[row0 + e][col0 + m] for e = 0..3 from a row-major bf16 tile
// of pitch `pitch`: the instruction hands lane m element m%4 of the 8-byte
// blocks addressed by lanes m/4 + 4e, so lane r addresses row row0 + r/4,
// columns col0 + 4 (r%4) .. +3.  row0 may differ between the four groups.
typedef short shortx4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x4 lds_tr4(const bf16* tile, int pitch, int row0, int col0, int m) {
  const bf16* p = tile + (row0 + (m >> 2)) * pitch + col0 + 4 * (m & 3);
  const shortx4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) shortx4*)(p));
  return __builtin_bit_cast(bf16x4, v);
}

// The same read at a lane address computed by the caller (lane r addresses
// row r/4 of its group, columns 4 (r%4) .. +3, as above).
__device__ __forceinline__ bf16x4 lds_tr4_at(const void* p) {
  const shortx4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) shortx4*)(p));
  return __builtin_bit_cast(bf16x4, v);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---- fp16 operands.  fp16 and bf16 words are both 16-bit, so a tile keeps
// its LDS layout and a fragment its registers whichever it holds: the words
// are converted when a tile is staged, and mma16<H> picks the instruction.
// fp16 keeps 11 significant bits against bf16's 8.
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));

// Eight bf16 values as fp16 (round to nearest even, clamped to +-65504).
__device__ __forceinline__ uint4 bf16x8_to_f16x8(uint4 v) {
  const uint32_t in[4] = {v.x, v.y, v.z, v.w};
  uint32_t out[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float a = __builtin_amdgcn_fmed3f(__uint_as_float(in[k] << 16), -65504.f, 65504.f);
    const float b = __builtin_amdgcn_fmed3f(__uint_as_float(in[k] & 0xffff0000u), -65504.f, 65504.f);
    const _Float16 ha = static_cast<_Float16>(a), hb = static_cast<_Float16>(b);
    out[k] = static_cast<uint32_t>(__builtin_bit_cast(u16, ha)) |
             (static_cast<uint32_t>(__builtin_bit_cast(u16, hb)) << 16);
  }
  return make_uint4(out[0], out[1], out[2], out[3]);
}
template <bool H>
__device__ __forceinline__ uint4 stage16(uint4 v) {
  if constexpr (H)
    return bf16x8_to_f16x8(v);
  else
    return v;
}
// a 16-bit MFMA over bf16-typed fragments holding bf16 (H = false) or fp16
// (H = true) words
template <bool H>
__device__ __forceinline__ floatx4 mma16(bf16x8 a, bf16x8 b, floatx4 c) {
  if constexpr (H)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(halfx8, a),
                                                  __builtin_bit_cast(halfx8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// an fp32 value as a 16-bit operand word (round to nearest even)
template <bool H>
__device__ __forceinline__ bf16 op16(float x) {
  if constexpr (H)
    return __builtin_bit_cast(bf16, static_cast<_Float16>(x));
  else
    return static_cast<bf16>(x);
}

// Index of the calling wave in its workgroup, as a wave-uniform (scalar)
// value: everything derived from it stays in scalar registers, so branches on
// it are scalar branches.  (Derived from the lane id alone, the compiler
// treats it as varying per lane and turns such branches into EXEC-masked
// regions, which must not hold matrix instructions.)
__device__ __forceinline__ int wave_index() {
  return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
}

// Wave priority around a run of matrix products (ON selects it per kernel
// variant): a wave about to issue MFMAs is preferred by the SIMD's issue
// arbiter, so the matrix core is fed while the SIMD's other wave runs its
// vector work in the gaps.  It changes no result, only the issue order.
template <bool ON>
__device__ __forceinline__ void prio_matrix() {
  if constexpr (ON) __builtin_amdgcn_s_setprio(1);
}
template <bool ON>
__device__ __forceinline__ void prio_normal() {
  if constexpr (ON) __builtin_amdgcn_s_setprio(0);
}

// Wait for every outstanding vector memory load of the wave (s_waitcnt
// vmcnt(0), the other counters left free).  Used once after the loads that
// precede a tile loop on a conditional path: without it the compiler cannot
// prove those loads done at the loop header and waits for vmcnt(0) inside
// the loop, where the count then covers the loop's own prefetches.
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Scalar-memory load of a 16-byte record at a wave-uniform address, waited for
// in place.  Scalar loads are counted apart from vector loads, so a loop that
// needs such a record every tile does not wait for its own vector prefetches.
template <typename T>
__device__ __forceinline__ T sload_uniform16(const T* p) {
  static_assert(sizeof(T) == 16, "16-byte records only");
  typedef int v4i __attribute__((ext_vector_type(4)));
  // (readfirstlane returns int: each half goes through uint32 before the
  // widening, so the low half is zero-extended, not sign-extended)
  const unsigned long long u = reinterpret_cast<unsigned long long>(p);
  const unsigned lo = static_cast<unsigned>(__builtin_amdgcn_readfirstlane(static_cast<int>(u & 0xffffffffu)));
  const unsigned hi = static_cast<unsigned>(__builtin_amdgcn_readfirstlane(static_cast<int>(u >> 32)));
  const unsigned long long q = (static_cast<unsigned long long>(hi) << 32) | static_cast<unsigned long long>(lo);
  v4i v;
  asm volatile("s_load_dwordx4 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(q) : "memory");
  return __builtin_bit_cast(T, v);
}

// ---- buffer resources: 32-bit offsets, loads past `bytes` return zero (the
// hardware range check replaces per-lane bounds branches)
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr uint32_t kOob = 0x80000000u;  // an offset past every resource used here

__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint64_t bytes) {
  const uint32_t n = bytes > 0x7fffffffull ? 0x7fffffffu : static_cast<uint32_t>(bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(n), 0x00020000);
}
__device__ __forceinline__ uint4 bload16(Rsrc r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ uint2 bload8(Rsrc r, uint32_t off) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
__device__ __forceinline__ float bloadf(Rsrc r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ __forceinline__ _Float16 bloadh(Rsrc r, uint32_t off) {
  return __builtin_bit_cast(_Float16, __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0));
}

// Four values as a range-checked buffer store of the element type (offset in
// bytes; kOob stores nothing).
__device__ __forceinline__ void bstore4(Rsrc r, uint32_t off, const float* in, bf16*) {
  bf16x4 v;
#pragma unroll
  for (int t = 0; t < 4; ++t) v[t] = static_cast<bf16>(in[t]);
  typedef unsigned int v2u __attribute__((ext_vector_type(2)));
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2u, v), r, off, 0, 0);
}
__device__ __forceinline__ void bstore4(Rsrc r, uint32_t off, const float* in, _Float16*) {
  halfx4 v;
#pragma unroll
  for (int t = 0; t < 4; ++t) v[t] = static_cast<_Float16>(in[t]);
  typedef unsigned int v2u __attribute__((ext_vector_type(2)));
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2u, v), r, off, 0, 0);
}
__device__ __forceinline__ void bstore4(Rsrc r, uint32_t off, const float* in, float*) {
  floatx4 v;
#pragma unroll
  for (int t = 0; t < 4; ++t) v[t] = in[t];
  typedef unsigned int v4u __attribute__((ext_vector_type(4)));
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, v), r, off, 0, 0);
}

// Output element store (O, dQ, dK, dV) in the output dtype.
__device__ __forceinline__ void store_out4(void* base, int64_t idx, bool f32, const float* v) {
  if (f32)
    store4(reinterpret_cast<float*>(base) + idx, v);
  else
    store4(reinterpret_cast<bf16*>(base) + idx, v);
}

// Stage the key-side projections Z^K of keys j0 .. j0+63 for queries
// i0 .. i0+127 (one 128-query block) into szk[key][query] (fp16, pitch
// `pitch`): key row j holds them as 128 consecutive entries (ascending in i)
// starting on a 16-byte boundary (the key-side pad), so each thread moves four
// aligned 16-byte chunks.  Rows past the slice read zero.
__device__ __forceinline__ void stage_zk_rows(const Rsrc& rzk, int gbase, int gslo, int gpad,
                                              int gpitch, int gk0, int j0, int i0, int D,
                                              _Float16* szk, int pitch) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int idx = tid + 256 * u;
    const int r = idx >> 4, ch = idx & 15;
    const int j = j0 + r;
    const int col = (i0 - j + D) - gslo + gpad + 8 * ch;
    const int e = gbase + (j - gk0) * gpitch + col;
    const uint4 w = bload16(rzk, e >= 0 ? static_cast<uint32_t>(e) * 2 : kOob);
    *reinterpret_cast<uint4*>(szk + r * pitch + 8 * ch) = w;
  }
}

}  // namespace relpos
