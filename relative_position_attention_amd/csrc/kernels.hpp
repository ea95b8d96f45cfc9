// Kernel argument blocks and host-side launch entry points.
// [RPA] = "Fast and Exact Relative-Position Attention via Structure-Aware
// Kernels" (arXiv 2611.01182).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "layout.hpp"

namespace relpos {

// Template flags of the attention kernels (compile-time specialisation per
// active term, map class and mask, [RPA] §4.3.3).
enum : int {
  F_ZQ = 1,      // read the query projections Z^Q (A^Q, with b and v folded in)
  F_ZK = 2,      // read the key projections Z^K
  F_BT = 4,      // read the expanded bias table directly (no Z^Q)
  F_CAUSAL = 8,  // j > i masked
  F_DZQ = 16,    // backward: query-side offset gradients (A^Q, b or v present)
  F_DZK = 32,    // backward: key-side offset gradients (A^K present)
  F_U = 64,      // backward: key column sums of G (Transformer-XL u term)
  F_SPLIT = 128,  // bf16: P and G enter their MFMA products as bf16 hi + lo
  F_DZ32 = 256,   // backward: query-side offset gradients stored in fp32
  F_DZ16 = 512,   // backward: query-side offset gradients stored in fp16
  F_SEG = 1024,   // segment masks (extras.hpp)
  F_DROP = 2048,  // attention dropout, with segment masks when given (extras.hpp)
  F_IT = 4096,    // in-tile products q . A~^Q from the expanded table (intile.hpp)
};

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  const void* zq;  // projection slices (Z element type)
  const void* zk;
  int64_t zq_bh, zk_bh;  // elements per (b, h) slice
  const GroupInfo* gq;
  const GroupInfo* gk;
  const float* rowlo;
  const float* rowhi;
  const float* keylo;
  const float* keyhi;
  const float* keymid;
  const float* bt;  // [H, S] expanded bias (b and v folded), fp32
  // F_IT (in-tile products): the expanded table A~^Q [Ht, S, 64] and its
  // transpose [Ht, 64, Sp] (bf16), Ht = 1 when shared by the heads
  const void* at;
  const void* att;
  int at_shared, Sp;
  void* o;          // forward output / backward input (out dtype)
  float* lse;       // natural-log logsumexp
  const float* dvec;  // backward: D = rowdot(dO, O)
  float* dqacc;       // backward: tau dS K, fp32 [BH, N, 64]
  float* dkacc;       // backward: tau dS^T Q, fp32
  void* dv;           // backward: dV (out dtype)
  void* dz;           // backward: offset gradients (input precision)
  int64_t dz_bh;
  float* bndq;    // [BH, N, 2] boundary sums (rows 0 and 2D) of the queries
  float* bndk;    // [BH, N, 2] of the keys
  float* colsum;  // [BH, N] sum_i G_ij
  int N, H, D, S;
  float scale;       // tau
  float scale_log2;  // tau * log2(e)
  int out_f32;
  // F_SEG / F_DROP kernels: segment bounds [B, N, 2] (null: no segment mask) and the
  // dropout byte threshold p8 (0: no dropout), keep scale and Philox key
  const int32_t* seg;
  int drop_p8;
  float drop_scale;
  uint32_t seed_lo, seed_hi;
};

// Each launcher returns the hipError_t of its launch.
// fp32 inputs: 16x16x4 fp32 MFMA, plain loads (attn_fwd.hip, attn_bwd.hip)
hipError_t launch_attn_fwd_f32(int flags, const AttnArgs& a, int B, hipStream_t s);
// bf16 forward: 64 queries per wave, 256 per workgroup (fwd_fast.hip)
hipError_t launch_attn_fwd_bf16(int flags, const AttnArgs& a, int B, hipStream_t s);
hipError_t launch_attn_bwd_q_f32(int flags, const AttnArgs& a, int B, hipStream_t s);
hipError_t launch_attn_bwd_k_f32(int flags, const AttnArgs& a, int B, hipStream_t s);
// bf16 backward passes: 32 tokens per wave, buffer loads, transposing LDS
// reads (bwd_q_fast.hip, bwd_k_fast.hip)
hipError_t launch_bwd_q_bf16(int flags, const AttnArgs& a, int B, hipStream_t s);
hipError_t launch_bwd_k_bf16(int flags, const AttnArgs& a, int B, hipStream_t s);
// the segment-mask (F_SEG: fwd_seg.hip, bwd_q_seg.hip, bwd_k_seg.hip) and
// dropout (F_DROP | F_SEG: fwd_drop.hip, bwd_q_drop.hip, bwd_k_drop.hip)
// variants of the three bf16 kernels; the launchers above forward such
// calls to them
hipError_t launch_attn_fwd_bf16_seg(int flags, const AttnArgs& a, int B, hipStream_t s);
hipError_t launch_bwd_q_bf16_seg(int flags, const AttnArgs& a, int B, hipStream_t s);
hipError_t launch_bwd_k_bf16_seg(int flags, const AttnArgs& a, int B, hipStream_t s);
hipError_t launch_attn_fwd_bf16_drop(int flags, const AttnArgs& a, int B, hipStream_t s);
// in-tile products (F_IT: fwd_it.hip, bwd_q_it.hip, bwd_k_it.hip, off_pass.hip)
hipError_t launch_attn_fwd_bf16_it(int flags, const AttnArgs& a, int B, hipStream_t s);
hipError_t launch_bwd_k_bf16_it(int flags, const AttnArgs& a, int B, hipStream_t s);
hipError_t launch_bwd_q_bf16_it(int flags, const AttnArgs& a, int B, hipStream_t s);
hipError_t launch_attn_fwd_bf16_it_ext(int flags, const AttnArgs& a, int B, hipStream_t s);
hipError_t launch_bwd_q_bf16_it_ext(int flags, const AttnArgs& a, int B, hipStream_t s);
hipError_t launch_bwd_k_bf16_it_ext(int flags, const AttnArgs& a, int B, hipStream_t s);
// offset-parallel pass (off_pass.hip): chunk partials P1 [H, B, S, 64] and
// P2 [H, B, S] of the table- and bias-gradient fold, one chunk per batch row
hipError_t launch_offset_pass_it(const AttnArgs& a, int B, int causal, int u, int ext, float* p1,
                                 float* p2, hipStream_t s);
hipError_t launch_bwd_q_bf16_drop(int flags, const AttnArgs& a, int B, hipStream_t s);
hipError_t launch_bwd_k_bf16_drop(int flags, const AttnArgs& a, int B, hipStream_t s);

// ---- auxiliary kernels (aux.hip)

// Plan metadata built on the device (no host-to-device copies).
struct MetaArgs {
  GroupInfo* gq;  // may be null
  GroupInfo* gk;  // may be null
  int N, NG, D;
  int causal;
};
hipError_t launch_meta_groups(const MetaArgs& m, hipStream_t s);

// A small block of host-built int32 metadata, passed by value and written to
// device memory by one launch (kernel-argument upload, fully asynchronous).
constexpr int kMetaChunk = 896;
struct MetaChunk {
  int32_t* dst;
  int count;
  int32_t vals[kMetaChunk];
};
hipError_t launch_meta_fill(const MetaChunk& c, hipStream_t s);

// Affine maps (identity / clipped): beta and fold intervals on the device.
struct AffineMapArgs {
  int32_t* beta;      // [S]
  int kind;           // RELPOS_MAP_IDENTITY or RELPOS_MAP_CLIPPED
  int sign, offset, clip;
  int D, S, R, causal, N;
};
hipError_t launch_meta_affine(const AffineMapArgs& m, hipStream_t s);

// dst[h][e][c] = src[h][c][e] for c < S (bf16 rows of 64), zero for
// S <= c < Sp: the transposed expanded table of the in-tile products
hipError_t launch_transpose_rows(const void* src, void* dst, int Ht, int S, int Sp, hipStream_t s);

// fold[r] = first and last expanded row s with beta(s) = r ([1, 0] if none)
hipError_t launch_fold_meta(const int32_t* beta, int32_t* fold, int S, int R, hipStream_t s);

struct ExpandArgs {
  const void* table;  // original table (input dtype)
  int64_t row_stride, head_stride;
  const int32_t* beta;
  void* out;  // [Ht, S, 64] input dtype
  int Ht, S;
};
hipError_t launch_expand(int dtype, const ExpandArgs& e, hipStream_t s);

struct BiasExpandArgs {
  const void* bias;  // [R, H] with strides (input dtype), may be null
  int64_t row_stride, head_stride;
  const int32_t* beta_b;
  const void* vb;    // [H, 64] v bias (input dtype), may be null
  const void* atq;   // expanded A^Q [Htq, S, 64], needed with vb
  int htq_shared;
  float* bt;         // [H, S]
  int H, S;
};
hipError_t launch_bias_expand(int dtype, const BiasExpandArgs& e, hipStream_t s);

struct ProjectArgs {
  const void* x;       // queries or keys [BH, N, 64]
  const void* at;      // expanded table [Ht, S, 64]
  int at_shared;
  const float* bt;     // [H, S] added to every entry (query side), or null
  const GroupInfo* gi;
  void* z;             // Z slices
  int64_t z_bh;
  int N, H, D, S, NG;
};
hipError_t launch_project_f32(const ProjectArgs& p, int BH, int max_pitch, hipStream_t s);
// bf16 inputs: row-walking projection with LDS-staged table tiles (rows
// longer than 16 column tiles split over several workgroups)
hipError_t launch_project_bf16(const ProjectArgs& p, int BH, int max_pitch, hipStream_t s);

struct RowKeyArgs {
  const void* q;
  const void* k;
  const void* atq;  // [Htq, S, 64] or null
  const void* atk;  // [Htk, S, 64] or null
  int atq_shared, atk_shared;
  const float* bt;  // [H, S]
  const void* u;    // [H, 64] or null
  float* rowlo;
  float* rowhi;
  float* keylo;
  float* keyhi;
  float* keymid;
  int N, H, S;
};
hipError_t launch_rowkey(int dtype, const RowKeyArgs& a, int BH, hipStream_t s);

// Zeroes `bytes` bytes at p (16-byte aligned; bytes a multiple of 16).
hipError_t launch_zero(void* p, size_t bytes, hipStream_t s);

hipError_t launch_rowdot(int dtype, int out_f32, const void* o, const void* dout, float* dvec,
                         int64_t rows, hipStream_t s);

// Completion of dQ (query side) or dK (key side):
//   out = acc + sum_s dZ~[i, s] A~[s] (band rows, MFMA) + boundary rows in fp32
//         (+ colsum * u on the key side).
struct FinalizeArgs {
  const float* acc;  // [BH, N, 64]
  const void* dz;    // offset gradients, null if the side has no table
  int64_t dz_bh;
  const GroupInfo* gi;
  const float* bnd;  // [BH, N, 2]
  const void* at;    // expanded table [Ht, S, 64] (input dtype), null if none
  int at_shared;
  const float* colsum;  // key side with u, else null
  const void* u;        // [H, 64]
  void* out;            // out dtype
  int N, H, D, S, key_side, causal, out_f32;
  int dz_f32;  // entries are fp32
  int dz_f16;  // entries are fp16
};
hipError_t launch_finalize_f32(const FinalizeArgs& f, int BH, hipStream_t s);
// bf16: aligned 16-byte staging of the offset gradients (reduce_fast.hip)
hipError_t launch_finalize_bf16(const FinalizeArgs& f, int BH, hipStream_t s);

// Table-gradient partials per (head, token chunk) ([RPA] "Deterministic table
// gradients", first kernel): P1[h][c][s][:] = sum_i dZ~[i,s] x_i,
// P2[h][c][s] = sum_i dZ~[i,s].
struct PartialArgs {
  const void* dz;
  int64_t dz_bh;
  const GroupInfo* gi;
  const float* bnd;
  const void* x;  // q or k [BH, N, 64] (input dtype)
  float* p1;      // [H, nchunk, S, 64] or null
  float* p2;      // [H, nchunk, S] or null
  int B, N, H, D, S, nchunk, key_side, causal;
  int dz_f32;     // entries are fp32 (scalar bias without a query table)
  int dz_f16;     // entries are fp16 (the Transformer-XL v term)
};
hipError_t launch_partials_f32(const PartialArgs& p, hipStream_t s);
hipError_t launch_partials_bf16(const PartialArgs& p, hipStream_t s);

// Second kernel: fixed-order sums over chunks (and heads of a shared table),
// then the bucket fold dA[r] = sum over copies s of r ([RPA] App. B.1
// bucket-copy lemma), written with the table's strides.  A row's copies are
// the interval fold[r] of s, or, with a list, list[fold[r]] (ascending s).
struct FoldArgs {
  const float* p1;
  const float* p2;
  const int32_t* fold;  // [R, 2] intervals of expanded rows, or of positions in list
  const int32_t* list;  // null, or expanded rows grouped by table row
  const void* vb;       // v bias [H, 64] (query side with V), else null
  float* out;
  int64_t row_stride, head_stride;
  int H, Ht, R, S, nchunk, shared;
};
hipError_t launch_fold_table(int dtype, const FoldArgs& f, hipStream_t s);

// db[h][s] = sum over chunks of P2 (fixed order)
hipError_t launch_p2_sum(const float* p2, float* db, int H, int S, int nchunk, hipStream_t s);

// dbias[r, h] = sum over the copies of row r of db[h][s] (bucket fold)
struct FoldBiasArgs {
  const float* db;      // [H, S]
  const int32_t* fold;  // [R, 2] intervals of expanded rows, or of positions in list
  const int32_t* list;  // null, or expanded rows grouped by table row
  float* out;
  int64_t row_stride, head_stride;
  int H, R, S;
};
hipError_t launch_fold_bias(const FoldBiasArgs& f, hipStream_t s);

// dv[h] = sum_s db[h][s] A~^Q[s], two phases through part [H, 64, 64]
struct DvArgs {
  const float* db;
  const void* atq;
  int at_shared;
  float* part;
  float* out;
  int H, S;
};
hipError_t launch_dv(int dtype, const DvArgs& a, hipStream_t s);

// du[h] = sum_{b,j} colsum[b,h,j] k[b,h,j], two phases through part
struct DuArgs {
  const float* colsum;
  const void* k;
  float* part;
  float* out;
  int B, H, N;
};
hipError_t launch_du(int dtype, const DuArgs& a, hipStream_t s);

}  // namespace relpos
