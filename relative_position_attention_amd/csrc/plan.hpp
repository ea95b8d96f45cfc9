// Host plan of one call: validation, relation-map expansion, per-group
// projection layouts and buffer offsets.  Pure host C++ (no HIP calls), so the
// validation path runs without a GPU.
//
// Method: "Fast and Exact Relative-Position Attention via Structure-Aware
// Kernels" (arXiv 2611.01182), cited as [RPA].
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include "relpos.h"
#include "layout.hpp"

namespace relpos {

struct SideLayout {
  bool present = false;
  std::vector<GroupInfo> groups;  // one per group of G rows
  int64_t bh_elems = 0;           // elements per (batch, head) slice
};

struct Plan {
  int B = 0, H = 0, N = 0, BH = 0;
  int delta = 0;  // saturation radius D ([RPA] §4.1 "Constant-Range Reuse")
  int S = 0;      // expanded rows 2D+1
  int G = kGroup, NG = 0;
  int R = 0;
  bool causal = false;
  float scale = 1.f;
  int dtype = 0, out_dtype = 0;
  bool aq = false, ak = false, bias = false, u = false, v = false;
  bool aq_shared = false, ak_shared = false;
  int Htq = 0, Htk = 0;  // heads of the expanded A^Q / A^K
  // beta_X[s]: original table row of expanded row s, -1 if unreachable
  std::vector<int32_t> beta_q, beta_k, beta_b;
  // map kind: identity and clipped maps get beta computed on the device
  bool affine_map = false;
  int map_kind = 0, map_offset = 0, map_clip = 0;
  int sign_q = 1, sign_k = 1, sign_b = 1;
  SideLayout zq, zk;  // projection / offset-gradient layouts (query side, key side)
  bool need_qside = false;  // query-side offset gradients exist (AQ, bias or v)
  size_t t_size = 2, z_size = 2, g_size = 2;
  bool dzq_f32 = false;    // query-side offset gradients in fp32 (a scalar bias)
  bool dzq_f16 = false;    // query-side offset gradients in fp16 (v without a bias)
  size_t dz_entry = 2;     // bytes per entry of the shared offset-gradient buffer
  bool split = false;  // P and G as bf16 hi + lo pairs in their MFMA products
  bool segmented = false;  // segment mask (tensors->seg)
  int drop_p8 = 0;         // dropout probability in units of 1/256
  bool in_tile = false;    // relation products computed per tile (no stored Z)
  int Sp = 0;              // row pitch of the transposed expanded table (S rounded up to 8)
  int nchunk = 1;  // token chunks per head in the table-gradient reduction
  // Per table (A^Q, A^K, b): rows that are not one interval of expanded rows
  // fold through an index list (fold_rows: [R, 2] first / last position of
  // each row in fold_list; fold_list: expanded rows grouped by table row).
  bool fold_listed[3] = {false, false, false};
  std::vector<int32_t> fold_rows[3], fold_list[3];

  // ---- byte offsets inside z ----
  size_t z_gq = 0, z_gk = 0, z_zq = 0, z_zk = 0, z_rowlo = 0, z_rowhi = 0, z_keylo = 0, z_keyhi = 0,
         z_keymid = 0, z_bt = 0, z_atq = 0, z_atqt = 0, z_bytes = 0;
  // ---- byte offsets inside ws (forward part) ----
  size_t ws_beta_q = 0, ws_beta_k = 0, ws_beta_b = 0, ws_fold = 0, ws_fold_list = 0,
         ws_atq = 0, ws_atk = 0, ws_fwd_end = 0;
  // ---- byte offsets inside ws (backward part, after ws_fwd_end) ----
  size_t ws_D = 0, ws_dqacc = 0, ws_dkacc = 0, ws_dz = 0, ws_bndq = 0, ws_bndk = 0,
         ws_colsum = 0, ws_p1 = 0, ws_p2 = 0, ws_db = 0, ws_red = 0, ws_bwd_end = 0;
};

// Builds the plan; returns RELPOS_OK or an error code with `detail` set.
int make_plan(const relpos_desc* desc, const relpos_shape* shape, Plan& plan,
              std::string& detail);

// Map row of signed argument x (the map's own argument, sign already applied);
// returns false if the descriptor's map is malformed.
bool map_row(const relpos_map& mp, int64_t x, int64_t& row);

}  // namespace relpos
