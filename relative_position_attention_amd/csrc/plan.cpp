// Host plan: descriptor validation, map expansion and buffer layout.
// [RPA] = "Fast and Exact Relative-Position Attention via Structure-Aware
// Kernels" (arXiv 2611.01182).
#include "plan.hpp"

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>

namespace relpos {

namespace {

// ---- a minimal unsigned big integer: exact tie-breaking of the bucket logs

struct Big {
  std::vector<uint32_t> w;  // little-endian limbs
  explicit Big(uint64_t v = 0) {
    while (v) {
      w.push_back(static_cast<uint32_t>(v));
      v >>= 32;
    }
  }
  void mul(uint32_t m) {
    uint64_t carry = 0;
    for (auto& x : w) {
      uint64_t t = static_cast<uint64_t>(x) * m + carry;
      x = static_cast<uint32_t>(t);
      carry = t >> 32;
    }
    if (carry) w.push_back(static_cast<uint32_t>(carry));
  }
};

Big pow_big(uint32_t base, int e) {
  Big r(1);
  for (int k = 0; k < e; ++k) r.mul(base);
  return r;
}

Big mul_big(Big a, uint32_t base, int e) {
  for (int k = 0; k < e; ++k) a.mul(base);
  return a;
}

int cmp_big(const Big& a, const Big& b) {
  size_t na = a.w.size(), nb = b.w.size();
  while (na && a.w[na - 1] == 0) --na;
  while (nb && b.w[nb - 1] == 0) --nb;
  if (na != nb) return na < nb ? -1 : 1;
  for (size_t k = na; k-- > 0;) {
    if (a.w[k] != b.w[k]) return a.w[k] < b.w[k] ? -1 : 1;
  }
  return 0;
}

// floor(span * ln(n/me) / ln(md/me)) for n >= me >= 1, md > me: evaluated in
// long double, and exactly (big integers) when the value is near an integer.
int64_t t5_log_floor(int64_t n, int64_t me, int64_t md, int span) {
  long double v = span * std::log(static_cast<long double>(n) / me) /
                  std::log(static_cast<long double>(md) / me);
  long double r = std::nearbyint(v);
  if (std::fabs(v - r) > 1e-9L) return static_cast<int64_t>(std::floor(v));
  int k = static_cast<int>(r);
  if (k < 0) return static_cast<int64_t>(std::floor(v));
  // k <= v  <=>  md^k * me^span <= n^span * me^k
  Big lhs = mul_big(pow_big(static_cast<uint32_t>(md), k), static_cast<uint32_t>(me), span);
  Big rhs = mul_big(pow_big(static_cast<uint32_t>(n), span), static_cast<uint32_t>(me), k);
  return cmp_big(lhs, rhs) <= 0 ? k : k - 1;
}

// ceil((mid-1) * ln(n/mid) / ln(top/mid)) for n > mid, same scheme.
int64_t deberta_log_ceil(int64_t n, int64_t mid, int64_t top) {
  long double v = (mid - 1) * std::log(static_cast<long double>(n) / mid) /
                  std::log(static_cast<long double>(top) / mid);
  long double r = std::nearbyint(v);
  if (std::fabs(v - r) > 1e-9L) return static_cast<int64_t>(std::ceil(v));
  int k = static_cast<int>(r);
  // k >= v  <=>  top^k * mid^(mid-1) >= n^(mid-1) * mid^k
  Big lhs = mul_big(pow_big(static_cast<uint32_t>(top), k), static_cast<uint32_t>(mid),
                    static_cast<int>(mid - 1));
  Big rhs = mul_big(pow_big(static_cast<uint32_t>(n), static_cast<int>(mid - 1)),
                    static_cast<uint32_t>(mid), k);
  return cmp_big(lhs, rhs) >= 0 ? k : k + 1;
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

}  // namespace

bool map_row(const relpos_map& mp, int64_t x, int64_t& row) {
  switch (mp.kind) {
    case RELPOS_MAP_IDENTITY:
      row = x + mp.identity_offset;
      return true;
    case RELPOS_MAP_CLIPPED: {
      if (mp.clip < 0) return false;
      int64_t c = mp.clip;
      row = std::min(std::max(x, -c), c) + c;
      return true;
    }
    case RELPOS_MAP_T5_BUCKET: {
      // T5 relative-position buckets ([RPA] §5.1 "Mechanisms" names the
      // original T5 scheme); x is T5's argument (key position minus query
      // position).
      int64_t nb = mp.num_buckets;
      if (nb < 2 || mp.max_distance < 1) return false;
      int64_t ret = 0, n;
      if (mp.bidirectional) {
        nb /= 2;
        if (x > 0) ret = nb;
        n = x < 0 ? -x : x;
      } else {
        n = x < 0 ? -x : 0;
      }
      int64_t me = nb / 2;
      if (me < 1 || mp.max_distance <= me) return false;
      if (n < me) {
        row = ret + n;
      } else {
        int64_t big = me + t5_log_floor(n, me, mp.max_distance, static_cast<int>(nb - me));
        row = ret + std::min(big, nb - 1);
      }
      return true;
    }
    case RELPOS_MAP_LOG_BUCKET: {
      // DeBERTa-v3 logarithmic buckets ([RPA] §5.1 "Mechanisms").
      int64_t bs = mp.bucket_size;
      int64_t mid = bs / 2;
      if (bs < 4 || mp.max_position <= mid + 1) return false;
      int64_t a = x < 0 ? -x : x;
      int64_t bkt;
      if (a <= mid) {
        bkt = x;
      } else {
        int64_t mag = mid + deberta_log_ceil(a, mid, mp.max_position - 1);
        bkt = x < 0 ? -mag : mag;
      }
      row = std::min(std::max(bkt + bs, static_cast<int64_t>(0)), 2 * bs - 1);
      return true;
    }
    case RELPOS_MAP_EXPLICIT: {
      if (mp.clip < 0 || mp.explicit_rows == nullptr) return false;
      int64_t c = mp.clip;
      row = mp.explicit_rows[std::min(std::max(x, -c), c) + c];
      return true;
    }
    default:
      return false;
  }
}

namespace {

// Smallest D such that the table's row is constant over delta in [D, N-1]
// (and, non-causal, over delta in [-(N-1), -D]) -- the saturation of [RPA]
// §4.1 "Constant-Range Reuse", restricted to reachable offsets.
bool saturation(const relpos_map& mp, int sign, int N, bool causal, int& D) {
  int64_t end_row, r;
  int hi = N - 1;
  if (!map_row(mp, static_cast<int64_t>(sign) * (N - 1), end_row)) return false;
  while (hi > 0) {
    if (!map_row(mp, static_cast<int64_t>(sign) * (hi - 1), r)) return false;
    if (r != end_row) break;
    --hi;
  }
  int lo = 0;
  if (!causal) {
    lo = N - 1;
    if (!map_row(mp, -static_cast<int64_t>(sign) * (N - 1), end_row)) return false;
    while (lo > 0) {
      if (!map_row(mp, -static_cast<int64_t>(sign) * (lo - 1), r)) return false;
      if (r != end_row) break;
      --lo;
    }
  }
  D = std::max(hi, lo);
  return true;
}

// Whether every table row covers one interval of expanded rows.  The
// bucket-copy expansion gives each offset its own expanded row, so the
// backward never needs this ([RPA] "Atomic fallback" accumulates such maps
// with atomics instead): a row's gradient is the fixed-order sum over its
// copies, read through an index list when they are not one interval.
bool contiguous(const std::vector<int32_t>& beta, int R) {
  std::vector<int> last(std::max(R, 1), -2);
  for (size_t s = 0; s < beta.size(); ++s) {
    int r = beta[s];
    if (r < 0) continue;
    if (last[r] != -2 && last[r] != static_cast<int>(s) - 1) return false;
    last[r] = static_cast<int>(s);
  }
  return true;
}

// Fold index of a table whose rows are not intervals: list = the reachable
// expanded rows s grouped by table row (ascending r, then ascending s), and
// fold[2r], fold[2r+1] = first and last position of row r in list ([1, 0]
// for a row no offset reaches).
void fold_index(const std::vector<int32_t>& beta, int R, std::vector<int32_t>& fold,
                std::vector<int32_t>& list) {
  const int Rm = std::max(R, 1);
  std::vector<int32_t> count(Rm, 0);
  for (int32_t r : beta)
    if (r >= 0) ++count[r];
  fold.assign(2 * static_cast<size_t>(Rm), 0);
  int pos = 0;
  for (int r = 0; r < Rm; ++r) {
    fold[2 * r] = count[r] ? pos : 1;
    fold[2 * r + 1] = count[r] ? pos + count[r] - 1 : 0;
    pos += count[r];
  }
  list.assign(pos, 0);
  std::vector<int32_t> fill(Rm, 0);
  for (size_t s = 0; s < beta.size(); ++s) {
    const int r = beta[s];
    if (r < 0) continue;
    list[fold[2 * r] + fill[r]++] = static_cast<int32_t>(s);
  }
}

bool build_side(Plan& p, bool query_side, std::string& detail) {
  SideLayout& L = query_side ? p.zq : p.zk;
  L.present = true;
  L.groups.resize(p.NG);
  int64_t base = 0;
  for (int g = 0; g < p.NG; ++g) {
    int slo, shi;
    if (query_side)
      query_group_window(g, p.N, p.delta, p.causal, slo, shi);
    else
      key_group_window(g, p.N, p.delta, p.causal, slo, shi);
    int width = shi - slo + 1;
    int pad = query_side ? query_pad(slo, p.delta) : key_pad(slo, p.delta);
    int pitch = pitch_mod8(pad + width + 4, query_side ? 7 : 1);
    int rows = std::min(kGroup, p.N - g * kGroup);
    GroupInfo gi;
    gi.slo = slo;
    gi.pad = pad;
    gi.pitch = pitch;
    gi.base = static_cast<int32_t>(base);
    L.groups[g] = gi;
    base += static_cast<int64_t>(rows) * pitch;
    base = (base + 7) & ~static_cast<int64_t>(7);
    if (base >= (static_cast<int64_t>(1) << 31) - 64) {  // group bases are int32
      detail = "projection slice exceeds 2^31 elements (N too large for this map)";
      return false;
    }
  }
  L.bh_elems = base + 8;
  return true;
}

// The kernels address one (batch, head) slice of Z and of the offset
// gradients through a buffer resource: 32-bit byte offsets, a range of at
// most 2^31 - 1 bytes, and offset 2^31 as "no access".  A slice must
// therefore stay below 2^31 bytes at its widest entry.
constexpr int64_t kSliceByteLimit = (static_cast<int64_t>(1) << 31) - 256;

}  // namespace

int make_plan(const relpos_desc* desc, const relpos_shape* shape, Plan& p,
              std::string& detail) {
  if (desc == nullptr || shape == nullptr) {
    detail = "null descriptor or shape";
    return RELPOS_E_INVALID_ARG;
  }
  if (desc->abi_version != RELPOS_ABI_VERSION) {
    detail = "abi_version mismatch";
    return RELPOS_E_ABI;
  }
  if (shape->d != kHeadDim) {
    detail = "only head dimension 64 is supported";
    return RELPOS_E_UNSUPPORTED;
  }
  if (shape->B < 1 || shape->H < 1 || shape->N < 1) {
    detail = "B, H, N must be >= 1";
    return RELPOS_E_INVALID_ARG;
  }
  if (shape->N > (1 << 22)) {
    detail = "N > 2^22 is not supported";
    return RELPOS_E_UNSUPPORTED;
  }
  const int known = RELPOS_TERM_AQ | RELPOS_TERM_AK | RELPOS_TERM_BIAS | RELPOS_TERM_U |
                    RELPOS_TERM_V;
  if (desc->terms & ~known) {
    detail = "unknown term bits";
    return RELPOS_E_INVALID_ARG;
  }
  if ((desc->terms & RELPOS_TERM_V) && !(desc->terms & RELPOS_TERM_AQ)) {
    detail = "term V needs term AQ";
    return RELPOS_E_INVALID_ARG;
  }
  if (desc->dtype != RELPOS_DTYPE_F32 && desc->dtype != RELPOS_DTYPE_BF16) {
    detail = "dtype must be F32 or BF16";
    return RELPOS_E_INVALID_ARG;
  }
  if (desc->out_dtype != RELPOS_DTYPE_F32 && desc->out_dtype != RELPOS_DTYPE_BF16) {
    detail = "out_dtype must be F32 or BF16";
    return RELPOS_E_INVALID_ARG;
  }
  if (desc->split_operands != 0 && desc->split_operands != 1) {
    detail = "split_operands must be 0 or 1";
    return RELPOS_E_INVALID_ARG;
  }
  if (desc->segmented != 0 && desc->segmented != 1) {
    detail = "segmented must be 0 or 1";
    return RELPOS_E_INVALID_ARG;
  }
  if (desc->dropout_p8 < 0 || desc->dropout_p8 > 255) {
    detail = "dropout_p8 must be in 0..255";
    return RELPOS_E_INVALID_ARG;
  }
  if ((desc->in_tile != 0 && desc->in_tile != 1) || desc->reserved0 != 0) {
    detail = "in_tile must be 0 or 1 and reserved0 0";
    return RELPOS_E_INVALID_ARG;
  }
  if (desc->in_tile) {
    // the in-tile kernels compute q . A~^Q per tile (bf16 MFMA) and take the
    // table gradient from the offset-parallel pass
    const char* why = nullptr;
    if (desc->dtype != RELPOS_DTYPE_BF16)
      why = "in_tile needs bf16 inputs";
    else if (!(desc->terms & RELPOS_TERM_AQ))
      why = "in_tile needs the A^Q term (a scalar bias alone has no projections)";
    else if (desc->terms & RELPOS_TERM_AK)
      why = "in_tile does not support the A^K term";
    else if (desc->split_operands && (desc->segmented || desc->dropout_p8 > 0))
      why = "in_tile with segment masks or dropout does not support split_operands";
    if (why != nullptr) {
      detail = why;
      return RELPOS_E_UNSUPPORTED;
    }
  }
  if (!std::isfinite(desc->scale) || !(desc->scale > 0.f)) {
    detail = "scale must be finite and positive";
    return RELPOS_E_INVALID_ARG;
  }
  p = Plan();
  p.B = shape->B;
  p.H = shape->H;
  p.N = shape->N;
  p.BH = p.B * p.H;
  p.causal = desc->causal != 0;
  p.scale = desc->scale;
  p.dtype = desc->dtype;
  p.out_dtype = desc->out_dtype;
  p.aq = desc->terms & RELPOS_TERM_AQ;
  p.ak = desc->terms & RELPOS_TERM_AK;
  p.bias = desc->terms & RELPOS_TERM_BIAS;
  p.u = desc->terms & RELPOS_TERM_U;
  p.v = desc->terms & RELPOS_TERM_V;
  p.R = desc->num_rows;
  p.t_size = desc->dtype == RELPOS_DTYPE_F32 ? 4 : 2;
  p.z_size = p.t_size;  // fp16 projections for bf16 inputs ([RPA] "Half-precision numerics")
  p.g_size = p.t_size;  // offset gradients in the input precision
  // ... except where their plain sums are needed (a bias, or the v term):
  // fp32, since those sums cancel
  // Precision of the query offset gradients: their per-offset sums over all
  // queries feed db and dv, and every row of dS sums to zero, so these sums
  // cancel.  A scalar bias (T5) keeps fp32 entries; the v term alone (TXL)
  // needs 11 mantissa bits (fp16) rather than bf16's 8.
  const bool f32in = p.dtype == RELPOS_DTYPE_F32;
  p.dzq_f32 = p.bias || (p.v && f32in);
  p.dzq_f16 = p.v && !p.bias && !f32in;
  p.split = desc->split_operands != 0 && p.dtype == RELPOS_DTYPE_BF16;
  p.segmented = desc->segmented != 0;
  p.drop_p8 = desc->dropout_p8;
  p.in_tile = desc->in_tile != 0;
  bool any_table = p.aq || p.ak || p.bias;
  if (any_table && p.R < 1) {
    detail = "num_rows must be >= 1";
    return RELPOS_E_INVALID_ARG;
  }
  auto sign_ok = [](int s) { return s == 1 || s == -1; };
  if ((p.aq && !sign_ok(desc->sign_q)) || (p.ak && !sign_ok(desc->sign_k)) ||
      (p.bias && !sign_ok(desc->sign_b))) {
    detail = "table signs must be +1 or -1";
    return RELPOS_E_INVALID_ARG;
  }
  const int64_t align_elems = 16 / static_cast<int64_t>(p.t_size);
  if (p.aq) {
    if (desc->aq_row_stride < kHeadDim || desc->aq_head_stride < 0 ||
        desc->aq_row_stride % align_elems || desc->aq_head_stride % align_elems) {
      detail = "A^Q strides must be >= 64 (rows), >= 0 (heads) and keep 16-byte rows";
      return desc->aq_row_stride % align_elems || desc->aq_head_stride % align_elems
                 ? RELPOS_E_MISALIGNED
                 : RELPOS_E_INVALID_ARG;
    }
    p.aq_shared = desc->aq_head_stride == 0;
  }
  if (p.ak) {
    if (desc->ak_row_stride < kHeadDim || desc->ak_head_stride < 0 ||
        desc->ak_row_stride % align_elems || desc->ak_head_stride % align_elems) {
      detail = "A^K strides must be >= 64 (rows), >= 0 (heads) and keep 16-byte rows";
      return desc->ak_row_stride % align_elems || desc->ak_head_stride % align_elems
                 ? RELPOS_E_MISALIGNED
                 : RELPOS_E_INVALID_ARG;
    }
    p.ak_shared = desc->ak_head_stride == 0;
  }
  if (p.bias && (desc->bias_row_stride < 0 || desc->bias_head_stride < 0)) {
    detail = "bias strides must be >= 0";
    return RELPOS_E_INVALID_ARG;
  }
  if (any_table && desc->map.kind == RELPOS_MAP_EXPLICIT && desc->map.explicit_rows == nullptr) {
    detail = "explicit map without rows";
    return RELPOS_E_INVALID_ARG;
  }

  // Saturation radius over every table ([RPA] §4.1 "Constant-Range Reuse").
  int D = 0;
  struct T {
    bool on;
    int sign;
  } tabs[3] = {{p.aq, desc->sign_q}, {p.ak, desc->sign_k}, {p.bias, desc->sign_b}};
  for (auto& t : tabs) {
    if (!t.on) continue;
    int d = 0;
    if (!saturation(desc->map, t.sign, p.N, p.causal, d)) {
      detail = "malformed map parameters";
      return RELPOS_E_INVALID_ARG;
    }
    D = std::max(D, d);
  }
  // In-tile products: every pair is a band pair (D > N - 1, so no saturated
  // tiles and no boundary entries), and D = 15 mod 16 with D >= N + 3, so a
  // 16-query block's row window against a 64-key tile starts on a multiple of
  // 16 (aligned table loads) and the last four expanded rows are unreachable.
  if (p.in_tile) D = (p.N + 3) + ((15 - (p.N + 3) % 16) + 16) % 16;
  p.delta = D;
  p.S = 2 * D + 1;
  p.NG = (p.N + kGroup - 1) / kGroup;

  // Bucket copies ([RPA] App. B.1 bucket-copy lemma): beta(s) = phi(s - D).
  auto expand = [&](bool on, int sign, std::vector<int32_t>& beta) -> int {
    beta.assign(p.S, -1);
    if (!on) return RELPOS_OK;
    for (int s = 0; s < p.S; ++s) {
      int delta = s - D;
      if (p.causal && delta < 0) continue;  // unreachable under the mask
      if (delta > p.N - 1 || delta < -(p.N - 1)) continue;  // no pair has this offset
      int64_t r;
      if (!map_row(desc->map, static_cast<int64_t>(sign) * delta, r)) {
        detail = "malformed map parameters";
        return RELPOS_E_INVALID_ARG;
      }
      if (r < 0 || r >= p.R) {
        char buf[160];
        std::snprintf(buf, sizeof buf,
                      "map sends offset %d to row %lld outside the %d-row table", delta,
                      static_cast<long long>(r), p.R);
        detail = buf;
        return RELPOS_E_UNSUPPORTED_MAP;
      }
      beta[s] = static_cast<int32_t>(r);
    }
    return RELPOS_OK;
  };
  int rc;
  if ((rc = expand(p.aq, desc->sign_q, p.beta_q)) != RELPOS_OK) return rc;
  if ((rc = expand(p.ak, desc->sign_k, p.beta_k)) != RELPOS_OK) return rc;
  if ((rc = expand(p.bias, desc->sign_b, p.beta_b)) != RELPOS_OK) return rc;
  // rows that are not one interval of offsets (e.g. delta and -delta sharing a
  // row): their gradient folds read an index list built here
  {
    const std::vector<int32_t>* betas[3] = {&p.beta_q, &p.beta_k, &p.beta_b};
    const bool on[3] = {p.aq, p.ak, p.bias};
    for (int t = 0; t < 3; ++t) {
      p.fold_listed[t] = on[t] && !contiguous(*betas[t], p.R);
      if (p.fold_listed[t]) fold_index(*betas[t], p.R, p.fold_rows[t], p.fold_list[t]);
    }
  }
  p.map_kind = desc->map.kind;
  p.affine_map = desc->map.kind == RELPOS_MAP_IDENTITY || desc->map.kind == RELPOS_MAP_CLIPPED;
  p.map_offset = desc->map.identity_offset;
  p.map_clip = desc->map.clip;
  p.sign_q = desc->sign_q;
  p.sign_k = desc->sign_k;
  p.sign_b = desc->sign_b;

  p.Htq = p.aq ? (p.aq_shared ? 1 : p.H) : 0;
  p.Htk = p.ak ? (p.ak_shared ? 1 : p.H) : 0;
  p.need_qside = p.aq || p.bias || p.v;
  // (in-tile: no stored projections, hence no group layouts)
  if (p.need_qside && !p.in_tile && !build_side(p, true, detail)) return RELPOS_E_UNSUPPORTED;
  if (p.ak && !build_side(p, false, detail)) return RELPOS_E_UNSUPPORTED;
  // per-slice bytes at the entry widths: Z (z_size) on either side, and the
  // one offset-gradient buffer (the larger side's elements at the wider
  // entry) that both passes share
  p.dz_entry = p.dzq_f32 ? 4 : (p.dzq_f16 ? 2 : p.g_size);
  {
    const int64_t zq = p.need_qside ? p.zq.bh_elems : 0, zk = p.ak ? p.zk.bh_elems : 0;
    const int64_t zmax = std::max(zq, zk);
    const int64_t zbytes = zmax * static_cast<int64_t>(p.z_size);
    const int64_t gbytes = zmax * static_cast<int64_t>(p.dz_entry);
    if (zbytes > kSliceByteLimit || gbytes > kSliceByteLimit) {
      char buf[200];
      std::snprintf(buf, sizeof buf,
                    "a (batch, head) slice of the projections or offset gradients needs %lld "
                    "bytes; the kernels address at most 2^31 - 256 per slice (N too large for "
                    "this map)",
                    static_cast<long long>(std::max(zbytes, gbytes)));
      detail = buf;
      return RELPOS_E_UNSUPPORTED;
    }
  }

  // Token chunks for the two-phase table-gradient sums ([RPA] "Deterministic
  // table gradients"): enough blocks to fill the chip.
  int sblocks = (p.S + 63) / 64;
  int subs = p.B * ((p.N + 63) / 64);
  int want = (2048 + sblocks * p.H - 1) / std::max(1, sblocks * p.H);
  // causal: the offsets near 0 reach every token and the far ones few, so
  // the longest blocks are split four ways
  if (p.causal) want = std::max(want, 4);
  p.nchunk = std::max(1, std::min(want, subs));
  // in-tile: the offset-parallel pass writes one partial per batch row
  if (p.in_tile) p.nchunk = p.B;
  p.Sp = (p.S + 7) & ~7;

  // ---- z layout (group tables first)
  size_t off = 0;
  p.z_gq = off;
  off = align256(off + sizeof(GroupInfo) * p.NG);
  p.z_gk = off;
  off = align256(off + sizeof(GroupInfo) * p.NG);
  const size_t bhn4 = static_cast<size_t>(p.BH) * p.N * 4;
  if (p.aq && !p.in_tile) {
    p.z_zq = off;
    off = align256(off + static_cast<size_t>(p.BH) * p.zq.bh_elems * p.z_size);
  }
  if (p.ak) {
    p.z_zk = off;
    off = align256(off + static_cast<size_t>(p.BH) * p.zk.bh_elems * p.z_size);
  }
  p.z_rowlo = off;
  off = align256(off + bhn4);
  p.z_rowhi = off;
  off = align256(off + bhn4);
  p.z_keylo = off;
  off = align256(off + bhn4);
  p.z_keyhi = off;
  off = align256(off + bhn4);
  p.z_keymid = off;
  off = align256(off + bhn4);
  p.z_bt = off;
  off = align256(off + static_cast<size_t>(p.H) * p.S * 4);
  if (p.in_tile) {
    // the expanded table A~^Q ([Htq, S, 64]) and its transpose ([Htq, 64, Sp],
    // columns past S zero) travel with the per-token entries: the in-tile
    // passes read them instead of projections
    p.z_atq = off;
    off = align256(off + static_cast<size_t>(p.Htq) * p.S * kHeadDim * p.t_size);
    p.z_atqt = off;
    off = align256(off + static_cast<size_t>(p.Htq) * kHeadDim * p.Sp * p.t_size);
  }
  p.z_bytes = off;

  // ---- workspace, forward part
  off = 0;
  p.ws_beta_q = off;
  off = align256(off + 4 * p.S);
  p.ws_beta_k = off;
  off = align256(off + 4 * p.S);
  p.ws_beta_b = off;
  off = align256(off + 4 * p.S);
  p.ws_fold = off;  // three [R, 2] interval tables (A^Q, A^K, b)
  off = align256(off + 3 * static_cast<size_t>(std::max(p.R, 1)) * 2 * 4);
  p.ws_fold_list = off;  // three [S] index lists (tables with listed folds)
  off = align256(off + 3 * static_cast<size_t>(p.S) * 4);
  if (p.aq && !p.in_tile) {
    p.ws_atq = off;
    off = align256(off + static_cast<size_t>(p.Htq) * p.S * kHeadDim * p.t_size);
  }
  if (p.ak) {
    p.ws_atk = off;
    off = align256(off + static_cast<size_t>(p.Htk) * p.S * kHeadDim * p.t_size);
  }
  p.ws_fwd_end = off;

  // ---- workspace, backward part
  p.ws_D = off;
  off = align256(off + bhn4);
  p.ws_dqacc = off;
  off = align256(off + bhn4 * kHeadDim);
  p.ws_dkacc = off;
  off = align256(off + bhn4 * kHeadDim);
  // one buffer holds the query side's entries, then the key side's ([RPA]
  // Table 9: the query reduction finishes before the key pass starts)
  // (slice stride: the larger side's element count; entry size: the wider type)
  int64_t dz_elems = 0;
  if (p.need_qside) dz_elems = std::max(dz_elems, p.zq.bh_elems);
  if (p.ak) dz_elems = std::max(dz_elems, p.zk.bh_elems);
  p.ws_dz = off;
  off = align256(off + static_cast<size_t>(p.BH) * dz_elems * p.dz_entry);
  p.ws_bndq = off;
  off = align256(off + 2 * bhn4);
  p.ws_bndk = off;
  off = align256(off + 2 * bhn4);
  p.ws_colsum = off;
  off = align256(off + bhn4);
  p.ws_p1 = off;
  if (p.aq || p.ak)
    off = align256(off + static_cast<size_t>(p.H) * p.nchunk * p.S * kHeadDim * 4);
  p.ws_p2 = off;
  off = align256(off + static_cast<size_t>(p.H) * p.nchunk * p.S * 4);
  p.ws_db = off;  // [H, S] chunk-summed P2
  off = align256(off + static_cast<size_t>(p.H) * p.S * 4);
  p.ws_red = off;  // [H, 64, 64] two-phase row-sum partials (dv, du)
  off = align256(off + static_cast<size_t>(p.H) * 64 * 64 * 4);
  p.ws_bwd_end = off;
  return RELPOS_OK;
}

}  // namespace relpos
