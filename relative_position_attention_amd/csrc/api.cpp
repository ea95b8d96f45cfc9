// C ABI of the library (include/relpos.h): validation, buffer carving and
// the launch sequence of each entry point on the caller's stream.
// [RPA] = "Fast and Exact Relative-Position Attention via Structure-Aware
// Kernels" (arXiv 2611.01182), Table 9 gives the kernel order.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <exception>
#include <mutex>
#include <string>

#include "kernels.hpp"
#include "plan.hpp"
#include "relpos.h"

namespace relpos {
namespace {

thread_local std::string g_last_error;

// Stage events (instrumentation): hipEvent_t handles the entry points record
// on their stream around their kernels, for timing single kernels.
constexpr int kMaxStageEvents = 8;
thread_local void* g_stage_events[kMaxStageEvents] = {};
thread_local int g_stage_event_count = 0;

int mark(int k, hipStream_t s) {
  if (k < g_stage_event_count && g_stage_events[k] != nullptr) {
    hipError_t e = hipEventRecord(static_cast<hipEvent_t>(g_stage_events[k]), s);
    if (e != hipSuccess) {
      g_last_error = std::string("hipEventRecord: ") + hipGetErrorString(e);
      return RELPOS_E_HIP;
    }
  }
  return RELPOS_OK;
}
#define RP_MARK(k)                                      \
  do {                                                  \
    int rc_ = mark((k), s);                             \
    if (rc_ != RELPOS_OK) return rc_;                   \
  } while (0)

// Host plans are cached per thread, keyed by the descriptor's contents (the
// explicit map rows included) and the shape: building one evaluates the map
// over every offset, far more host time than enqueuing the kernels.
struct PlanCache {
  std::vector<std::pair<std::string, Plan>> entries;  // most recent last
};
thread_local PlanCache g_plans;
constexpr size_t kPlanCacheSize = 16;

// The key is built field by field, so padding bytes of the caller's structs
// (uninitialised in C) never enter it.
template <typename T>
void put(std::string& key, T v) {
  key.append(reinterpret_cast<const char*>(&v), sizeof v);
}

std::string plan_key(const relpos_desc* d, const relpos_shape* sh) {
  std::string key;
  key.reserve(160);
  put(key, sh->B);
  put(key, sh->H);
  put(key, sh->N);
  put(key, sh->d);
  put(key, d->abi_version);
  put(key, d->terms);
  put(key, d->causal);
  put(key, d->scale);
  put(key, d->dtype);
  put(key, d->out_dtype);
  put(key, d->num_rows);
  put(key, d->sign_q);
  put(key, d->sign_k);
  put(key, d->sign_b);
  put(key, d->split_operands);
  const relpos_map& m = d->map;
  put(key, m.kind);
  put(key, m.clip);
  put(key, m.identity_offset);
  put(key, m.num_buckets);
  put(key, m.max_distance);
  put(key, m.bidirectional);
  put(key, m.bucket_size);
  put(key, m.max_position);
  put(key, d->aq_row_stride);
  put(key, d->aq_head_stride);
  put(key, d->ak_row_stride);
  put(key, d->ak_head_stride);
  put(key, d->bias_row_stride);
  put(key, d->bias_head_stride);
  put(key, d->segmented);
  put(key, d->dropout_p8);  // (the seed is read per call, not planned)
  put(key, d->in_tile);
  if (m.kind == RELPOS_MAP_EXPLICIT && m.explicit_rows != nullptr && m.clip >= 0)
    key.append(reinterpret_cast<const char*>(m.explicit_rows),
               sizeof(int32_t) * (2 * static_cast<size_t>(m.clip) + 1));
  return key;
}

// The plan of (desc, shape), from the cache or built; nullptr on error.
const Plan* get_plan(const relpos_desc* desc, const relpos_shape* shape, int& rc) {
  rc = RELPOS_OK;
  if (desc == nullptr || shape == nullptr) {
    rc = RELPOS_E_INVALID_ARG;
    g_last_error = "null descriptor or shape";
    return nullptr;
  }
  // the key needs a readable descriptor: validate the ABI version first
  if (desc->abi_version != RELPOS_ABI_VERSION) {
    rc = RELPOS_E_ABI;
    g_last_error = "abi_version mismatch";
    return nullptr;
  }
  const std::string key = plan_key(desc, shape);
  auto& E = g_plans.entries;
  for (size_t k = 0; k < E.size(); ++k) {
    if (E[k].first == key) {
      if (k + 1 != E.size()) {
        auto hit = std::move(E[k]);
        E.erase(E.begin() + k);
        E.push_back(std::move(hit));
      }
      return &E.back().second;
    }
  }
  Plan p;
  std::string detail;
  rc = make_plan(desc, shape, p, detail);
  if (rc != RELPOS_OK) {
    g_last_error = detail;
    return nullptr;
  }
  if (E.size() >= kPlanCacheSize) E.erase(E.begin());
  E.emplace_back(key, std::move(p));
  return &E.back().second;
}

int fail(int code, const std::string& detail) {
  g_last_error = detail;
  return code;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

template <typename P>
P* at_off(void* base, size_t off) {
  return reinterpret_cast<P*>(reinterpret_cast<char*>(base) + off);
}

#define RP_HIP(expr)                                                                   \
  do {                                                                                 \
    hipError_t e_ = (expr);                                                            \
    if (e_ != hipSuccess) return fail(RELPOS_E_HIP, std::string(#expr) + ": " +        \
                                                        hipGetErrorString(e_));        \
  } while (0)

struct ZView {
  void* zq;
  void* zk;
  float *rowlo, *rowhi, *keylo, *keyhi, *keymid, *bt;
};

ZView z_view(const Plan& p, void* z) {
  ZView v;
  v.zq = p.aq ? at_off<char>(z, p.z_zq) : nullptr;
  v.zk = p.ak ? at_off<char>(z, p.z_zk) : nullptr;
  v.rowlo = at_off<float>(z, p.z_rowlo);
  v.rowhi = at_off<float>(z, p.z_rowhi);
  v.keylo = at_off<float>(z, p.z_keylo);
  v.keyhi = at_off<float>(z, p.z_keyhi);
  v.keymid = at_off<float>(z, p.z_keymid);
  v.bt = at_off<float>(z, p.z_bt);
  return v;
}

int check_inputs(const Plan& p, const relpos_tensors* in) {
  if (in == nullptr) return fail(RELPOS_E_INVALID_ARG, "null tensors");
  if (!in->q || !in->k || !in->v) return fail(RELPOS_E_INVALID_ARG, "null q, k or v");
  if (!aligned16(in->q) || !aligned16(in->k) || !aligned16(in->v))
    return fail(RELPOS_E_MISALIGNED, "q, k, v must be 16-byte aligned");
  if (p.aq && (!in->aq || !aligned16(in->aq)))
    return fail(in->aq ? RELPOS_E_MISALIGNED : RELPOS_E_INVALID_ARG, "A^Q missing or misaligned");
  if (p.ak && (!in->ak || !aligned16(in->ak)))
    return fail(in->ak ? RELPOS_E_MISALIGNED : RELPOS_E_INVALID_ARG, "A^K missing or misaligned");
  if (p.bias && !in->bias) return fail(RELPOS_E_INVALID_ARG, "bias missing");
  if (p.u && !in->u) return fail(RELPOS_E_INVALID_ARG, "u missing");
  if (p.v && !in->vbias) return fail(RELPOS_E_INVALID_ARG, "v missing");
  if (p.segmented && (in->seg == nullptr || (reinterpret_cast<uintptr_t>(in->seg) & 7)))
    return fail(in->seg ? RELPOS_E_MISALIGNED : RELPOS_E_INVALID_ARG,
                "segment bounds missing or not 8-byte aligned");
  return RELPOS_OK;
}

// Group tables of the projection layout, built on the device into z (the
// attention kernels read them from there, so a forward with retained z
// launches nothing else).
int build_groups(const Plan& p, void* z, hipStream_t s) {
  MetaArgs m;
  m.gq = p.need_qside ? at_off<GroupInfo>(z, p.z_gq) : nullptr;
  m.gk = p.ak ? at_off<GroupInfo>(z, p.z_gk) : nullptr;
  m.N = p.N;
  m.NG = p.NG;
  m.D = p.delta;
  m.causal = p.causal;
  if (m.gq || m.gk) RP_HIP(launch_meta_groups(m, s));
  return RELPOS_OK;
}

// Host-built int32 metadata written to device memory as kernel arguments
// (no host-to-device copy).
int upload(const std::vector<int32_t>& v, int32_t* dst, hipStream_t s) {
  const int n = static_cast<int>(v.size());
  for (int k0 = 0; k0 < n; k0 += kMetaChunk) {
    MetaChunk c;
    c.dst = dst + k0;
    c.count = std::min(kMetaChunk, n - k0);
    std::memcpy(c.vals, v.data() + k0, sizeof(int32_t) * c.count);
    RP_HIP(launch_meta_fill(c, s));
  }
  return RELPOS_OK;
}

const int32_t* fold_ptr(const Plan& p, void* ws, int idx) {
  return at_off<int32_t>(ws, p.ws_fold) + static_cast<size_t>(idx) * std::max(p.R, 1) * 2;
}

// Index list of table idx's fold, or null when its rows are intervals.
int32_t* fold_list_ptr(const Plan& p, void* ws, int idx) {
  if (!p.fold_listed[idx]) return nullptr;
  return at_off<int32_t>(ws, p.ws_fold_list) + static_cast<size_t>(idx) * p.S;
}

// Expanded row maps and (with_fold: only the backward's table-gradient folds
// read them) fold intervals or index lists, written into ws.
int build_maps(const Plan& p, void* ws, hipStream_t s, bool with_fold) {
  int rc;
  struct Tab {
    bool on;
    const std::vector<int32_t>* beta;
    size_t beta_off;
    int sign;
    int fold_idx;
  } tabs[3] = {{p.aq, &p.beta_q, p.ws_beta_q, p.sign_q, 0},
               {p.ak, &p.beta_k, p.ws_beta_k, p.sign_k, 1},
               {p.bias, &p.beta_b, p.ws_beta_b, p.sign_b, 2}};
  const int R = std::max(p.R, 1);
  for (auto& t : tabs) {
    if (!t.on) continue;
    int32_t* beta = at_off<int32_t>(ws, t.beta_off);
    if (p.affine_map) {  // identity and clipped rows are always intervals
      AffineMapArgs a;
      a.beta = beta;
      a.kind = p.map_kind;
      a.sign = t.sign;
      a.offset = p.map_offset;
      a.clip = p.map_clip;
      a.D = p.delta;
      a.S = p.S;
      a.R = R;
      a.causal = p.causal;
      a.N = p.N;
      RP_HIP(launch_meta_affine(a, s));
    } else {
      // bucketed / explicit maps: the host-built rows travel as kernel
      // arguments (no host-to-device copy)
      if ((rc = upload(*t.beta, beta, s)) != RELPOS_OK) return rc;
    }
    if (with_fold) {
      int32_t* fold = at_off<int32_t>(ws, p.ws_fold) + static_cast<size_t>(t.fold_idx) * R * 2;
      if (p.fold_listed[t.fold_idx]) {
        // rows that are not intervals: the host-built positions and list
        if ((rc = upload(p.fold_rows[t.fold_idx], fold, s)) != RELPOS_OK) return rc;
        if ((rc = upload(p.fold_list[t.fold_idx], fold_list_ptr(p, ws, t.fold_idx), s)) != RELPOS_OK)
          return rc;
      } else {
        RP_HIP(launch_fold_meta(beta, fold, p.S, R, s));
      }
    }
  }
  return RELPOS_OK;
}

// The expanded table A~^Q: in the workspace, or (in-tile products) in z,
// next to its transpose.
char* atq_ptr(const Plan& p, void* z, void* ws) {
  return p.in_tile ? at_off<char>(z, p.z_atq) : at_off<char>(ws, p.ws_atq);
}

int expand_tables(const Plan& p, const relpos_desc* desc, const relpos_tensors* in, void* z,
                  void* ws, hipStream_t s) {
  const int dt = p.dtype == RELPOS_DTYPE_F32 ? 0 : 1;
  if (p.aq) {
    ExpandArgs e;
    e.table = in->aq;
    e.row_stride = desc->aq_row_stride;
    e.head_stride = desc->aq_head_stride;
    e.beta = at_off<int32_t>(ws, p.ws_beta_q);
    e.out = atq_ptr(p, z, ws);
    e.Ht = p.Htq;
    e.S = p.S;
    RP_HIP(launch_expand(dt, e, s));
    if (p.in_tile)
      RP_HIP(launch_transpose_rows(e.out, at_off<char>(z, p.z_atqt), p.Htq, p.S, p.Sp, s));
  }
  if (p.ak) {
    ExpandArgs e;
    e.table = in->ak;
    e.row_stride = desc->ak_row_stride;
    e.head_stride = desc->ak_head_stride;
    e.beta = at_off<int32_t>(ws, p.ws_beta_k);
    e.out = at_off<char>(ws, p.ws_atk);
    e.Ht = p.Htk;
    e.S = p.S;
    RP_HIP(launch_expand(dt, e, s));
  }
  return RELPOS_OK;
}

int max_pitch(const SideLayout& L) {
  int m = 0;
  for (const auto& g : L.groups) m = std::max(m, g.pitch);
  return m;
}

// Projection into z: bias table, Z^Q, Z^K, boundary entries.  Needs the
// metadata and the expanded tables in ws.
int project_into(const Plan& p, const relpos_desc* desc, const relpos_tensors* in, void* z,
                 void* ws, hipStream_t s) {
  const int dt = p.dtype == RELPOS_DTYPE_F32 ? 0 : 1;
  ZView zv = z_view(p, z);
  BiasExpandArgs be;
  be.bias = p.bias ? in->bias : nullptr;
  be.row_stride = desc->bias_row_stride;
  be.head_stride = desc->bias_head_stride;
  be.beta_b = at_off<int32_t>(ws, p.ws_beta_b);
  be.vb = p.v ? in->vbias : nullptr;
  be.atq = p.aq ? atq_ptr(p, z, ws) : nullptr;
  be.htq_shared = p.aq_shared;
  be.bt = zv.bt;
  be.H = p.H;
  be.S = p.S;
  RP_HIP(launch_bias_expand(dt, be, s));
  if (p.aq && !p.in_tile) {
    ProjectArgs pa;
    pa.x = in->q;
    pa.at = atq_ptr(p, z, ws);
    pa.at_shared = p.aq_shared;
    pa.bt = zv.bt;
    pa.gi = at_off<GroupInfo>(z, p.z_gq);
    pa.z = zv.zq;
    pa.z_bh = p.zq.bh_elems;
    pa.N = p.N;
    pa.H = p.H;
    pa.D = p.delta;
    pa.S = p.S;
    pa.NG = p.NG;
    if (dt == 0)
      RP_HIP(launch_project_f32(pa, p.BH, max_pitch(p.zq), s));
    else
      RP_HIP(launch_project_bf16(pa, p.BH, max_pitch(p.zq), s));
  }
  if (p.ak) {
    ProjectArgs pa;
    pa.x = in->k;
    pa.at = at_off<char>(ws, p.ws_atk);
    pa.at_shared = p.ak_shared;
    pa.bt = nullptr;
    pa.gi = at_off<GroupInfo>(z, p.z_gk);
    pa.z = zv.zk;
    pa.z_bh = p.zk.bh_elems;
    pa.N = p.N;
    pa.H = p.H;
    pa.D = p.delta;
    pa.S = p.S;
    pa.NG = p.NG;
    if (dt == 0)
      RP_HIP(launch_project_f32(pa, p.BH, max_pitch(p.zk), s));
    else
      RP_HIP(launch_project_bf16(pa, p.BH, max_pitch(p.zk), s));
  }
  RowKeyArgs rk;
  rk.q = in->q;
  rk.k = in->k;
  rk.atq = p.aq ? atq_ptr(p, z, ws) : nullptr;
  rk.atk = p.ak ? at_off<char>(ws, p.ws_atk) : nullptr;
  rk.atq_shared = p.aq_shared;
  rk.atk_shared = p.ak_shared;
  rk.bt = zv.bt;
  rk.u = p.u ? in->u : nullptr;
  rk.rowlo = zv.rowlo;
  rk.rowhi = zv.rowhi;
  rk.keylo = zv.keylo;
  rk.keyhi = zv.keyhi;
  rk.keymid = zv.keymid;
  rk.N = p.N;
  rk.H = p.H;
  rk.S = p.S;
  RP_HIP(launch_rowkey(dt, rk, p.BH, s));
  return RELPOS_OK;
}

AttnArgs attn_args(const Plan& p, const relpos_tensors* in, void* z, void* ws) {
  ZView zv = z_view(p, z);
  AttnArgs a;
  std::memset(&a, 0, sizeof a);
  a.q = in->q;
  a.k = in->k;
  a.v = in->v;
  a.zq = zv.zq;
  a.zk = zv.zk;
  a.zq_bh = p.aq ? p.zq.bh_elems : 0;
  a.zk_bh = p.ak ? p.zk.bh_elems : 0;
  a.gq = p.need_qside ? at_off<GroupInfo>(z, p.z_gq) : nullptr;
  a.gk = p.ak ? at_off<GroupInfo>(z, p.z_gk) : nullptr;
  a.rowlo = zv.rowlo;
  a.rowhi = zv.rowhi;
  a.keylo = zv.keylo;
  a.keyhi = zv.keyhi;
  a.keymid = zv.keymid;
  a.bt = zv.bt;
  if (p.in_tile) {
    a.at = at_off<char>(z, p.z_atq);
    a.att = at_off<char>(z, p.z_atqt);
    a.at_shared = p.aq_shared;
    a.Sp = p.Sp;
  }
  a.N = p.N;
  a.H = p.H;
  a.D = p.delta;
  a.S = p.S;
  a.scale = p.scale;
  a.scale_log2 = p.scale * 1.4426950408889634f;
  a.out_f32 = p.out_dtype == RELPOS_DTYPE_F32;
  a.seg = p.segmented ? in->seg : nullptr;
  a.drop_p8 = p.drop_p8;
  a.drop_scale = 256.f / static_cast<float>(256 - p.drop_p8);
  return a;
}

int base_flags(const Plan& p) {
  int f = 0;
  if (p.segmented) f |= F_SEG;
  if (p.drop_p8 > 0) f |= F_DROP;
  if (p.aq) f |= p.in_tile ? F_IT : F_ZQ;
  if (p.ak) f |= F_ZK;
  if (p.bias && !p.aq) f |= F_BT;
  if (p.u) f |= F_U;
  if (p.causal) f |= F_CAUSAL;
  return f;
}

int run_project(const relpos_desc* desc, const relpos_shape* shape, const relpos_tensors* in,
                void* z, size_t z_bytes, void* ws, size_t ws_bytes, hipStream_t s) {
  int rc;
  const Plan* pp = get_plan(desc, shape, rc);
  if (pp == nullptr) return rc;
  const Plan& p = *pp;
  if ((rc = check_inputs(p, in)) != RELPOS_OK) return rc;
  if (z == nullptr || z_bytes < p.z_bytes) return fail(RELPOS_E_WORKSPACE_TOO_SMALL, "z too small");
  if (ws == nullptr || ws_bytes < p.ws_fwd_end)
    return fail(RELPOS_E_WORKSPACE_TOO_SMALL, "workspace too small");
  if (!aligned16(z) || !aligned16(ws)) return fail(RELPOS_E_MISALIGNED, "z / ws misaligned");
  if ((rc = build_groups(p, z, s)) != RELPOS_OK) return rc;
  if ((rc = build_maps(p, ws, s, false)) != RELPOS_OK) return rc;
  if ((rc = expand_tables(p, desc, in, z, ws, s)) != RELPOS_OK) return rc;
  return project_into(p, desc, in, z, ws, s);
}

// ---- allocation-free projection (relpos_project_noalloc)
//
// The workspace of relpos_project (row maps and expanded tables) lives in a
// file-scope device array of fixed size, one copy per GPU for the life of the
// process.  Host code never passes the array's name to a kernel: it is a
// host-side stand-in, not a device address.  The device address comes from
// hipGetSymbolAddress, taken once per device with that device current.
constexpr size_t kScratchBytes = static_cast<size_t>(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_address(void** out) {
  int dev = -1;
  RP_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(RELPOS_E_UNSUPPORTED, "device index above 63");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return fail(RELPOS_E_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return RELPOS_OK;
}

int run_project_noalloc(const relpos_desc* desc, const relpos_shape* shape,
                        const relpos_tensors* in, void* z, size_t z_bytes, hipStream_t s) {
  int rc;
  const Plan* pp = get_plan(desc, shape, rc);
  if (pp == nullptr) return rc;
  if (pp->ws_fwd_end > kScratchBytes)
    return fail(RELPOS_E_WORKSPACE_TOO_SMALL,
                "relpos_project_noalloc needs " + std::to_string(pp->ws_fwd_end) +
                    " bytes of workspace; its static scratch holds " +
                    std::to_string(kScratchBytes) + " (use relpos_project with a workspace)");
  void* ws = nullptr;
  if ((rc = scratch_address(&ws)) != RELPOS_OK) return rc;
  // every workspace entry the projection reads (row maps, expanded tables) is
  // written by it first, so the previous call's contents need no clearing
  return run_project(desc, shape, in, z, z_bytes, ws, kScratchBytes, s);
}

int run_fwd(const relpos_desc* desc, const relpos_shape* shape, const relpos_tensors* in,
            const void* zc, size_t z_bytes, void* o, float* lse, void* ws, size_t ws_bytes,
            hipStream_t s) {
  int rc;
  const Plan* pp = get_plan(desc, shape, rc);
  if (pp == nullptr) return rc;
  const Plan& p = *pp;
  if ((rc = check_inputs(p, in)) != RELPOS_OK) return rc;
  if (o == nullptr || lse == nullptr || !aligned16(o) || !aligned16(lse))
    return fail(o && lse ? RELPOS_E_MISALIGNED : RELPOS_E_INVALID_ARG, "o / lse");
  void* z = const_cast<void*>(zc);
  // with retained projections the forward is the attention kernel alone and
  // needs no workspace
  const size_t need = z ? 0 : p.ws_fwd_end + p.z_bytes;
  if (need > 0 && (ws == nullptr || ws_bytes < need))
    return fail(RELPOS_E_WORKSPACE_TOO_SMALL, "workspace too small");
  if (z && z_bytes < p.z_bytes) return fail(RELPOS_E_WORKSPACE_TOO_SMALL, "z too small");
  if ((need > 0 && !aligned16(ws)) || (z && !aligned16(z)))
    return fail(RELPOS_E_MISALIGNED, "z / ws misaligned");
  if (z == nullptr) {
    z = at_off<char>(ws, p.ws_fwd_end);
    if ((rc = build_groups(p, z, s)) != RELPOS_OK) return rc;
    if ((rc = build_maps(p, ws, s, false)) != RELPOS_OK) return rc;
    if ((rc = expand_tables(p, desc, in, z, ws, s)) != RELPOS_OK) return rc;
    if ((rc = project_into(p, desc, in, z, ws, s)) != RELPOS_OK) return rc;
  }
  AttnArgs a = attn_args(p, in, z, ws);
  a.o = o;
  a.lse = lse;
  a.seed_lo = static_cast<uint32_t>(desc->dropout_seed);
  a.seed_hi = static_cast<uint32_t>(desc->dropout_seed >> 32);
  const int ff = base_flags(p) | (p.split ? F_SPLIT : 0);
  RP_MARK(0);
  if (p.dtype == RELPOS_DTYPE_F32)
    RP_HIP(launch_attn_fwd_f32(ff, a, p.B, s));
  else
    RP_HIP(launch_attn_fwd_bf16(ff, a, p.B, s));
  RP_MARK(1);
  return RELPOS_OK;
}

int run_bwd(const relpos_desc* desc, const relpos_shape* shape, const relpos_tensors* in,
            const void* zc, size_t z_bytes, const void* o, const float* lse, const void* dout,
            relpos_grads* gr, void* ws, size_t ws_bytes, hipStream_t s) {
  int rc;
  const Plan* pp = get_plan(desc, shape, rc);
  if (pp == nullptr) return rc;
  const Plan& p = *pp;
  if ((rc = check_inputs(p, in)) != RELPOS_OK) return rc;
  if (!o || !lse || !dout || !gr) return fail(RELPOS_E_INVALID_ARG, "null o, lse, dout or grads");
  if (!aligned16(o) || !aligned16(dout)) return fail(RELPOS_E_MISALIGNED, "o / dout misaligned");
  if (!gr->dq || !gr->dk || !gr->dv) return fail(RELPOS_E_INVALID_ARG, "null dq, dk or dv");
  if (!aligned16(gr->dq) || !aligned16(gr->dk) || !aligned16(gr->dv))
    return fail(RELPOS_E_MISALIGNED, "dq, dk, dv misaligned");
  if ((p.aq && !gr->daq) || (p.ak && !gr->dak) || (p.bias && !gr->dbias) || (p.u && !gr->du) ||
      (p.v && !gr->dvbias))
    return fail(RELPOS_E_INVALID_ARG, "a table gradient pointer is null");
  void* z = const_cast<void*>(zc);
  const size_t need = z ? p.ws_bwd_end : p.ws_bwd_end + p.z_bytes;
  if (ws == nullptr || ws_bytes < need) return fail(RELPOS_E_WORKSPACE_TOO_SMALL, "workspace too small");
  if (z && z_bytes < p.z_bytes) return fail(RELPOS_E_WORKSPACE_TOO_SMALL, "z too small");
  if (!aligned16(ws) || (z && !aligned16(z))) return fail(RELPOS_E_MISALIGNED, "z / ws misaligned");

  const int dt = p.dtype == RELPOS_DTYPE_F32 ? 0 : 1;
  if ((rc = build_maps(p, ws, s, true)) != RELPOS_OK) return rc;
  const bool have_z = z != nullptr;
  if (!have_z) z = at_off<char>(ws, p.ws_bwd_end);
  // (in-tile products: the expanded tables are part of z, written with it)
  if (!p.in_tile || !have_z)
    if ((rc = expand_tables(p, desc, in, z, ws, s)) != RELPOS_OK) return rc;
  if (!have_z) {
    if ((rc = build_groups(p, z, s)) != RELPOS_OK) return rc;
    if ((rc = project_into(p, desc, in, z, ws, s)) != RELPOS_OK) return rc;
  }
  float* dvec = at_off<float>(ws, p.ws_D);
  float* dqacc = at_off<float>(ws, p.ws_dqacc);
  float* dkacc = at_off<float>(ws, p.ws_dkacc);
  void* dz = at_off<char>(ws, p.ws_dz);
  float* bndq = at_off<float>(ws, p.ws_bndq);
  float* bndk = at_off<float>(ws, p.ws_bndk);
  float* colsum = at_off<float>(ws, p.ws_colsum);
  float* p1 = at_off<float>(ws, p.ws_p1);
  float* p2 = at_off<float>(ws, p.ws_p2);
  float* db = at_off<float>(ws, p.ws_db);
  float* red = at_off<float>(ws, p.ws_red);
  const int64_t rows = static_cast<int64_t>(p.BH) * p.N;

  // Preprocessing: D = rowdot(dO, O)
  RP_MARK(0);
  RP_HIP(launch_rowdot(dt, p.out_dtype == RELPOS_DTYPE_F32, o, dout, dvec, rows, s));
  RP_MARK(1);

  AttnArgs a = attn_args(p, in, z, ws);
  a.seed_lo = static_cast<uint32_t>(desc->dropout_seed);
  a.seed_hi = static_cast<uint32_t>(desc->dropout_seed >> 32);
  a.dout = dout;
  a.o = const_cast<void*>(o);
  a.lse = const_cast<float*>(lse);
  a.dvec = dvec;
  a.dqacc = dqacc;
  a.dkacc = dkacc;
  a.dv = gr->dv;
  a.dz = dz;
  a.dz_bh = std::max(p.need_qside ? p.zq.bh_elems : 0, p.ak ? p.zk.bh_elems : 0);
  a.bndq = bndq;
  a.bndk = bndk;
  a.colsum = colsum;
  // A side without a table term (no A^Q; no A^K and no u) has nothing to add
  // to its pass's dQ (dK): with fp32 outputs the pass writes the output itself
  // and that side's finalize kernel is skipped
  const bool out32 = p.out_dtype == RELPOS_DTYPE_F32;
  const bool q_direct = out32 && !p.aq;
  const bool k_direct = out32 && !p.ak && !p.u;
  if (q_direct) a.dqacc = static_cast<float*>(gr->dq);
  if (k_direct) a.dkacc = static_cast<float*>(gr->dk);
  const int bf = base_flags(p) | (p.split ? F_SPLIT : 0);

  // With a segment mask the passes skip the tiles outside every segment of a
  // workgroup, leaving those pairs' offset-gradient entries unwritten; the
  // reductions read every entry a token's offsets reach, so the buffer is
  // cleared before each pass (a fill kernel; the passes write the rest)
  const size_t dz_bytes = static_cast<size_t>(p.BH) * a.dz_bh * p.dz_entry;
  if (p.segmented && !p.in_tile && (p.need_qside || p.ak)) RP_HIP(launch_zero(dz, dz_bytes, s));

  // Query-parallel pass, then the query reduction ([RPA] Table 9)
  // (in-tile products: the query pass adds the relation part of dQ itself and
  // writes no offset gradients; the offset-parallel pass below makes the
  // table sums)
  const bool qside_dz = p.need_qside && !p.in_tile;
  const int qflags = bf | (qside_dz ? F_DZQ | (p.dzq_f32 ? F_DZ32 : 0) | (p.dzq_f16 ? F_DZ16 : 0) : 0);
  if (dt == 0)
    RP_HIP(launch_attn_bwd_q_f32(qflags, a, p.B, s));
  else
    RP_HIP(launch_bwd_q_bf16(qflags, a, p.B, s));
  RP_MARK(2);
  if (!q_direct) {
    FinalizeArgs f;
    std::memset(&f, 0, sizeof f);
    f.acc = dqacc;
    const bool qtab = p.aq && !p.in_tile;
    f.dz = qtab ? dz : nullptr;
    f.dz_bh = a.dz_bh;
    f.gi = qside_dz ? at_off<GroupInfo>(z, p.z_gq) : nullptr;
    f.bnd = qtab ? bndq : nullptr;
    f.at = qtab ? at_off<char>(ws, p.ws_atq) : nullptr;
    f.at_shared = p.aq_shared;
    f.out = gr->dq;
    f.N = p.N;
    f.H = p.H;
    f.D = p.delta;
    f.S = p.S;
    f.key_side = 0;
    f.causal = p.causal;
    f.out_f32 = p.out_dtype == RELPOS_DTYPE_F32;
    f.dz_f32 = p.dzq_f32;
    f.dz_f16 = p.dzq_f16;
    if (dt == 0)
      RP_HIP(launch_finalize_f32(f, p.BH, s));
    else
      RP_HIP(launch_finalize_bf16(f, p.BH, s));
  }
  if (p.need_qside) {
    if (p.in_tile) {
      RP_HIP(launch_offset_pass_it(a, p.B, p.causal, p.u, p.segmented || p.drop_p8 > 0, p1, p2, s));
    } else {
      PartialArgs pa;
      pa.dz = dz;
      pa.dz_bh = a.dz_bh;
      pa.gi = at_off<GroupInfo>(z, p.z_gq);
      pa.bnd = bndq;
      pa.x = in->q;
      pa.p1 = p.aq ? p1 : nullptr;
      pa.p2 = (p.bias || p.v) ? p2 : nullptr;
      pa.B = p.B;
      pa.N = p.N;
      pa.H = p.H;
      pa.D = p.delta;
      pa.S = p.S;
      pa.nchunk = p.nchunk;
      pa.key_side = 0;
      pa.causal = p.causal;
      pa.dz_f32 = p.dzq_f32;
      pa.dz_f16 = p.dzq_f16;
      if (dt == 0)
        RP_HIP(launch_partials_f32(pa, s));
      else
        RP_HIP(launch_partials_bf16(pa, s));
    }
    if (p.aq) {
      FoldArgs fa;
      fa.p1 = p1;
      fa.p2 = p2;
      fa.fold = fold_ptr(p, ws, 0);
      fa.list = fold_list_ptr(p, ws, 0);
      fa.vb = p.v ? in->vbias : nullptr;
      fa.out = gr->daq;
      fa.row_stride = desc->aq_row_stride;
      fa.head_stride = desc->aq_head_stride;
      fa.H = p.H;
      fa.Ht = p.Htq;
      fa.R = p.R;
      fa.S = p.S;
      fa.nchunk = p.nchunk;
      fa.shared = p.aq_shared;
      RP_HIP(launch_fold_table(dt, fa, s));
    }
    if (p.bias || p.v) RP_HIP(launch_p2_sum(p2, db, p.H, p.S, p.nchunk, s));
    if (p.bias) {
      FoldBiasArgs fb;
      fb.db = db;
      fb.fold = fold_ptr(p, ws, 2);
      fb.list = fold_list_ptr(p, ws, 2);
      fb.out = gr->dbias;
      fb.row_stride = desc->bias_row_stride;
      fb.head_stride = desc->bias_head_stride;
      fb.H = p.H;
      fb.R = p.R;
      fb.S = p.S;
      RP_HIP(launch_fold_bias(fb, s));
    }
    if (p.v) {
      DvArgs dv;
      dv.db = db;
      dv.atq = atq_ptr(p, z, ws);
      dv.at_shared = p.aq_shared;
      dv.part = red;
      dv.out = gr->dvbias;
      dv.H = p.H;
      dv.S = p.S;
      RP_HIP(launch_dv(dt, dv, s));
    }
  }

  // Key-parallel pass, then the key reduction
  if (p.segmented && p.ak) RP_HIP(launch_zero(dz, dz_bytes, s));
  const int kflags = bf | (p.ak ? F_DZK : 0) | (p.u ? F_U : 0);
  RP_MARK(3);
  if (dt == 0)
    RP_HIP(launch_attn_bwd_k_f32(kflags, a, p.B, s));
  else
    RP_HIP(launch_bwd_k_bf16(kflags, a, p.B, s));
  RP_MARK(4);
  if (!k_direct) {
    FinalizeArgs f;
    std::memset(&f, 0, sizeof f);
    f.acc = dkacc;
    f.dz = p.ak ? dz : nullptr;
    f.dz_bh = a.dz_bh;
    f.gi = p.ak ? at_off<GroupInfo>(z, p.z_gk) : nullptr;
    f.bnd = p.ak ? bndk : nullptr;
    f.at = p.ak ? at_off<char>(ws, p.ws_atk) : nullptr;
    f.at_shared = p.ak_shared;
    f.colsum = p.u ? colsum : nullptr;
    f.u = p.u ? in->u : nullptr;
    f.out = gr->dk;
    f.N = p.N;
    f.H = p.H;
    f.D = p.delta;
    f.S = p.S;
    f.key_side = 1;
    f.causal = p.causal;
    f.out_f32 = p.out_dtype == RELPOS_DTYPE_F32;
    if (dt == 0)
      RP_HIP(launch_finalize_f32(f, p.BH, s));
    else
      RP_HIP(launch_finalize_bf16(f, p.BH, s));
  }
  if (p.ak) {
    PartialArgs pa;
    pa.dz = dz;
    pa.dz_bh = a.dz_bh;
    pa.gi = at_off<GroupInfo>(z, p.z_gk);
    pa.bnd = bndk;
    pa.x = in->k;
    pa.p1 = p1;
    pa.p2 = nullptr;
    pa.B = p.B;
    pa.N = p.N;
    pa.H = p.H;
    pa.D = p.delta;
    pa.S = p.S;
    pa.nchunk = p.nchunk;
    pa.key_side = 1;
    pa.causal = p.causal;
    pa.dz_f32 = 0;
    pa.dz_f16 = 0;
    if (dt == 0)
      RP_HIP(launch_partials_f32(pa, s));
    else
      RP_HIP(launch_partials_bf16(pa, s));
    FoldArgs fa;
    fa.p1 = p1;
    fa.p2 = nullptr;
    fa.fold = fold_ptr(p, ws, 1);
    fa.list = fold_list_ptr(p, ws, 1);
    fa.vb = nullptr;
    fa.out = gr->dak;
    fa.row_stride = desc->ak_row_stride;
    fa.head_stride = desc->ak_head_stride;
    fa.H = p.H;
    fa.Ht = p.Htk;
    fa.R = p.R;
    fa.S = p.S;
    fa.nchunk = p.nchunk;
    fa.shared = p.ak_shared;
    RP_HIP(launch_fold_table(dt, fa, s));
  }
  if (p.u) {
    DuArgs du;
    du.colsum = colsum;
    du.k = in->k;
    du.part = red;
    du.out = gr->du;
    du.B = p.B;
    du.H = p.H;
    du.N = p.N;
    RP_HIP(launch_du(dt, du, s));
  }
  RP_MARK(5);
  return RELPOS_OK;
}

}  // namespace
}  // namespace relpos

using namespace relpos;

extern "C" {

int relpos_plan_sizes(const relpos_desc* desc, const relpos_shape* shape, relpos_sizes* out) {
  try {
    if (out == nullptr) return fail(RELPOS_E_INVALID_ARG, "null output");
    int rc;
    const Plan* pp = get_plan(desc, shape, rc);
    if (pp == nullptr) return rc;
    const Plan& p = *pp;
    out->z_bytes = p.z_bytes;
    out->fwd_ws_bytes = p.ws_fwd_end;  // relpos_project; relpos_attn_fwd with z needs none
    out->fwd_ws_bytes_noz = p.ws_fwd_end + p.z_bytes;
    out->bwd_ws_bytes = p.ws_bwd_end;
    out->bwd_ws_bytes_noz = p.ws_bwd_end + p.z_bytes;
    out->delta = p.delta;
    out->expanded_rows = p.S;
    out->group_size = kGroup;
    out->num_groups = p.NG;
    return RELPOS_OK;
  } catch (const std::exception& e) {
    return fail(RELPOS_E_INVALID_ARG, e.what());
  } catch (...) {
    return fail(RELPOS_E_INVALID_ARG, "unknown host error");
  }
}

int relpos_plan_rows(const relpos_desc* desc, const relpos_shape* shape, int32_t which,
                     int32_t* rows_out, int32_t cap) {
  try {
    int rc;
    const Plan* pp = get_plan(desc, shape, rc);
    if (pp == nullptr) return rc;
    const Plan& p = *pp;
    const std::vector<int32_t>* b = which == 0 ? &p.beta_q : which == 1 ? &p.beta_k
                                     : which == 2 ? &p.beta_b : nullptr;
    if (b == nullptr || rows_out == nullptr) return fail(RELPOS_E_INVALID_ARG, "bad table index");
    if (cap < p.S) return fail(RELPOS_E_INVALID_ARG, "capacity too small");
    for (int s = 0; s < p.S; ++s) rows_out[s] = (*b)[s];
    return p.S;
  } catch (...) {
    return fail(RELPOS_E_INVALID_ARG, "host error");
  }
}

int relpos_project(const relpos_desc* desc, const relpos_shape* shape, const relpos_tensors* in,
                   void* z, size_t z_bytes, void* ws, size_t ws_bytes, void* stream) {
  try {
    return run_project(desc, shape, in, z, z_bytes, ws, ws_bytes, static_cast<hipStream_t>(stream));
  } catch (...) {
    return fail(RELPOS_E_INVALID_ARG, "host error");
  }
}

int relpos_project_noalloc(const relpos_desc* desc, const relpos_shape* shape,
                           const relpos_tensors* in, void* z, size_t z_bytes, void* stream) {
  try {
    return run_project_noalloc(desc, shape, in, z, z_bytes, static_cast<hipStream_t>(stream));
  } catch (...) {
    return fail(RELPOS_E_INVALID_ARG, "host error");
  }
}

int relpos_attn_fwd(const relpos_desc* desc, const relpos_shape* shape, const relpos_tensors* in,
                    const void* z, size_t z_bytes, void* o, float* lse, void* ws, size_t ws_bytes,
                    void* stream) {
  try {
    return run_fwd(desc, shape, in, z, z_bytes, o, lse, ws, ws_bytes,
                   static_cast<hipStream_t>(stream));
  } catch (...) {
    return fail(RELPOS_E_INVALID_ARG, "host error");
  }
}

int relpos_attn_bwd(const relpos_desc* desc, const relpos_shape* shape, const relpos_tensors* in,
                    const void* z, size_t z_bytes, const void* o, const float* lse,
                    const void* dout, relpos_grads* grads, void* ws, size_t ws_bytes,
                    void* stream) {
  try {
    return run_bwd(desc, shape, in, z, z_bytes, o, lse, dout, grads, ws, ws_bytes,
                   static_cast<hipStream_t>(stream));
  } catch (...) {
    return fail(RELPOS_E_INVALID_ARG, "host error");
  }
}

const char* relpos_strerror(int code) {
  switch (code) {
    case RELPOS_OK:
      return "success";
    case RELPOS_E_INVALID_ARG:
      return "invalid argument";
    case RELPOS_E_UNSUPPORTED:
      return "unsupported configuration";
    case RELPOS_E_UNSUPPORTED_MAP:
      return "unsupported relation map";
    case RELPOS_E_MISALIGNED:
      return "misaligned pointer or stride";
    case RELPOS_E_WORKSPACE_TOO_SMALL:
      return "buffer too small";
    case RELPOS_E_HIP:
      return "HIP error";
    case RELPOS_E_ABI:
      return "ABI version mismatch";
    default:
      return "unknown error";
  }
}

const char* relpos_last_error(void) { return g_last_error.c_str(); }

int relpos_set_stage_events(void* const* events, int32_t count) {
  if (count < 0 || count > kMaxStageEvents || (count > 0 && events == nullptr)) {
    g_last_error = "stage event count must be in [0, 8]";
    return RELPOS_E_INVALID_ARG;
  }
  for (int k = 0; k < kMaxStageEvents; ++k) g_stage_events[k] = k < count ? events[k] : nullptr;
  g_stage_event_count = count;
  return RELPOS_OK;
}

int relpos_abi_version(void) { return RELPOS_ABI_VERSION; }

}  // extern "C"
