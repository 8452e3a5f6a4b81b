// Host side of the C ABI declared in include/mla.h: argument validation (always
// before any launch), the split-KV plan, workspace layout and launches.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/mla.h"
#include "mla_common.h"

namespace {

thread_local std::string g_last_error;

mla_status fail(mla_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
mla_status fail(mla_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

mla_status hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return MLA_OK;
  return fail(MLA_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

constexpr int kNumCUs = 256;     // MI355X compute units (the plan is device independent)
constexpr int kMinSplitRows = 256;
// rows per split at most (MFMA paths, fewer than four rounds of queries): a
// sweep of the ragged 16-head batch (128 sequences of U[1, 32768] rows) gave
// its attention 496 / 472 / 480 / 469 / 492 us at 8 / 10 / 12 / 14 / 16
// splits (Infinity Cache flushed), the combine 17.5 / 19.8 / 20.4 / 22.0 /
// 25.5 us; 3,328 rows give it 10
constexpr int kMaxSplitRows = 3328;
constexpr int kMaxSplits = 65535;
// unabsorbed prefill: a workgroup whose first query sees fewer keys than this
// takes the hi + lo products
constexpr int kPreciseBelow = 2048;
// absorbed path, 32 to 128 heads: a query that attends fewer rows than this
// scores with hi + lo and carries its softmax weights as hi + lo (the
// 16-head-group body); longer ones take the wide kernels' single bf16 operands
constexpr int kPreciseRows = 4096;
constexpr int32_t kAllPrecise = 0x7fffffff;

mla_status check_dims(const mla_dims* d, mla_dtype dt) {
  if (!d) return fail(MLA_ERR_INVALID_ARGUMENT, "dims is NULL");
  if (dt != MLA_F32 && dt != MLA_BF16) return fail(MLA_ERR_INVALID_ARGUMENT, "unknown dtype %d", (int)dt);
  if (d->n_h < 1 || d->n_h > 4096) return fail(MLA_ERR_INVALID_ARGUMENT, "n_h=%d out of range [1,4096]", d->n_h);
  if (d->d_hR <= 0 || (d->d_hR & 1)) return fail(MLA_ERR_INVALID_ARGUMENT, "d_hR=%d must be positive and even", d->d_hR);
  if (d->d_c <= 0 || d->d_h <= 0) return fail(MLA_ERR_INVALID_ARGUMENT, "d_c=%d, d_h=%d must be positive", d->d_c, d->d_h);
  if (d->d_c != mla::D_C || d->d_h != mla::D_H || d->d_hR != mla::D_R)
    return fail(MLA_ERR_UNSUPPORTED, "only d_c=512, d_h=128, d_hR=64 are built (got %d, %d, %d)", d->d_c, d->d_h, d->d_hR);
  if (!(d->rope_base > 0.0) || !std::isfinite(d->rope_base))
    return fail(MLA_ERR_INVALID_ARGUMENT, "rope_base must be finite and > 0");
  if (!(d->softmax_scale >= 0.0) || !std::isfinite(d->softmax_scale))
    return fail(MLA_ERR_INVALID_ARGUMENT, "softmax_scale must be finite and >= 0");
  if (!(d->yarn_factor >= 0.0) || !std::isfinite(d->yarn_factor))
    return fail(MLA_ERR_INVALID_ARGUMENT, "yarn_factor must be finite and >= 0");
  if (d->yarn_factor > 1.0) {
    if (!(d->yarn_orig_ctx > 0.0) || !std::isfinite(d->yarn_orig_ctx))
      return fail(MLA_ERR_INVALID_ARGUMENT, "yarn_orig_ctx must be finite and > 0");
    if (!(d->yarn_alpha > 0.0) || !(d->yarn_beta > d->yarn_alpha) || !std::isfinite(d->yarn_beta))
      return fail(MLA_ERR_INVALID_ARGUMENT, "YaRN needs 0 < yarn_alpha < yarn_beta (finite)");
  }
  return MLA_OK;
}

// Long-context scaling in force: yarn_factor > 1.
static bool yarn_on(const mla_dims* d) { return d->yarn_factor > 1.0; }

double scale_of(const mla_dims* d) {
  if (d->softmax_scale > 0.0) return d->softmax_scale;
  double s = 1.0 / std::sqrt(static_cast<double>(d->d_h + d->d_hR));
  if (yarn_on(d)) {  // YaRN's temperature on the whole logit: (0.1 ln s + 1)^2
    const double m = 0.1 * std::log(d->yarn_factor) + 1.0;
    s *= m * m;
  }
  return s;
}

// Pair frequencies in fp64: plain base^(-2k/d_hR), or YaRN's blend between
// theta / s (wavelengths longer than the pretraining context) and theta
// (wavelengths that fit yarn_beta times or more), linear in the count of
// wavelengths that fit.
void fill_rope(const mla_dims* d, mla::RopeTable& t) {
  std::memset(&t, 0, sizeof(t));
  constexpr double TWO_PI = 6.283185307179586476925;
  for (int k = 0; k < d->d_hR / 2; ++k) {
    const double th = std::pow(d->rope_base, -2.0 * k / d->d_hR);
    if (!yarn_on(d)) {
      t.theta[k] = th;
      continue;
    }
    const double fits = d->yarn_orig_ctx * th / TWO_PI;
    const double g = std::min(1.0, std::max(0.0, (fits - d->yarn_alpha) / (d->yarn_beta - d->yarn_alpha)));
    t.theta[k] = (1.0 - g) * (th / d->yarn_factor) + g * th;
  }
}


int64_t split_rows(int32_t max_seq_len, int32_t num_splits) {
  if (max_seq_len <= 0 || num_splits <= 0) return 0;
  int64_t r = (static_cast<int64_t>(max_seq_len) + num_splits - 1) / num_splits;
  return (r + mla::TILE - 1) / mla::TILE * mla::TILE;
}

// Attended length below which a query reads the lo plane (mla_precise_rows).
// bf16 only: 16 heads, the generic kernels and the long-context temperature
// (which sharpens the softmax so that single bf16 operands show at every
// length) always use hi + lo.
int32_t precise_rows_of(const mla_dims* d, mla_dtype dt) {
  if (dt != MLA_BF16) return 0;
  if (yarn_on(d) || d->n_h == 16 || !mla::splitkv_has_fast_path(d->n_h, 1, d->d_c, d->d_hR)) return kAllPrecise;
  return kPreciseRows;
}

// Split plan.  The MFMA kernels hold one workgroup per CU (their LDS ring),
// so the plan aims at one round of kNumCUs workgroups and, for batches of
// fewer than four rounds of queries, caps a split at kMaxSplitRows rows, which
// keeps ragged batches balanced (a long sequence is cut into several
// workgroups; splits past a short one's length exit at once).
// The generic kernels run several workgroups per CU and aim at two rounds.
int32_t plan_splits(const mla_dims* d, mla_dtype dt, int64_t n_q, int64_t max_len) {
  if (n_q <= 0 || max_len <= 0) return 1;
  const bool fast = mla::splitkv_has_fast_path(d->n_h, dt == MLA_BF16, d->d_c, d->d_hR);
  const int64_t target = static_cast<int64_t>(kNumCUs) * (fast ? 1 : 2);
  // when every query takes the 16-head-group path, each (query, split) is
  // n_h / 16 workgroups
  const int64_t units =
      (fast && mla::splitkv_all_precise(d->n_h, static_cast<int32_t>(std::min<int64_t>(max_len, kAllPrecise)),
                                        precise_rows_of(d, dt)))
          ? n_q * (d->n_h / 16)
          : n_q;
  int64_t s = (target + units - 1) / units;
  // (with four or more rounds of queries, e.g. a prefill chunk, the hardware
  // scheduler already balances whole queries and splitting only adds partials)
  if (fast && units < 4 * static_cast<int64_t>(kNumCUs))
    s = std::max<int64_t>(s, (max_len + kMaxSplitRows - 1) / kMaxSplitRows);
  const int64_t max_s = std::max<int64_t>(1, (max_len + kMinSplitRows - 1) / kMinSplitRows);
  s = std::min(std::max<int64_t>(s, 1), max_s);
  return static_cast<int32_t>(std::min<int64_t>(s, kMaxSplits));
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// The lo plane of the absorbed queries exists for bf16 storage only.
mla_status check_lo(mla_dtype dt, const void* q_lat_lo) {
  if (q_lat_lo && dt != MLA_BF16)
    return fail(MLA_ERR_INVALID_ARGUMENT, "q_lat_lo is for bf16 storage only (pass NULL with MLA_F32)");
  return MLA_OK;
}

int32_t page_shift_of(int32_t page_rows) {
  int32_t k = 0;
  while ((int64_t{1} << k) < page_rows) ++k;
  return k;
}

// Paged-cache descriptor: pool and table present, page_rows a power of two in
// [32, 65536], and room in the table for `max_len` rows.  Returns the row
// capacity per sequence (the stride the kernels clamp lengths to).
mla_status check_paged(const mla_paged_cache* c, int64_t max_len, int64_t& cap) {
  if (!c) return fail(MLA_ERR_INVALID_ARGUMENT, "paged cache descriptor is NULL");
  if (!c->pool || !c->block_table) return fail(MLA_ERR_INVALID_ARGUMENT, "paged cache: NULL pool or block_table");
  if (c->page_rows < 32 || c->page_rows > 65536 || (c->page_rows & (c->page_rows - 1)))
    return fail(MLA_ERR_INVALID_ARGUMENT, "page_rows=%d must be a power of two in [32, 65536]", c->page_rows);
  if (c->max_pages < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "max_pages=%d < 1", c->max_pages);
  if (c->num_pages < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "num_pages=%lld < 1", (long long)c->num_pages);
  if (c->num_pages > (int64_t{1} << 31) - 1)
    return fail(MLA_ERR_INVALID_ARGUMENT, "num_pages=%lld exceeds the int32 page index", (long long)c->num_pages);
  cap = static_cast<int64_t>(c->max_pages) * c->page_rows;
  if (max_len > cap)
    return fail(MLA_ERR_INVALID_ARGUMENT, "attended length bound %lld > max_pages * page_rows = %lld",
                (long long)max_len, (long long)cap);
  return MLA_OK;
}

size_t partial_bytes(const mla_dims* d, int64_t n_q, int32_t S) {
  return align256(static_cast<size_t>(n_q) * S * d->n_h * d->d_c * sizeof(float)) +
         align256(static_cast<size_t>(n_q) * S * d->n_h * sizeof(float));
}

}  // namespace

extern "C" {

int32_t mla_abi_version(void) { return MLA_ABI_VERSION; }

const char* mla_status_string(mla_status s) {
  switch (s) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARGUMENT: return "MLA_ERR_INVALID_ARGUMENT";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED";
    case MLA_ERR_WORKSPACE_TOO_SMALL: return "MLA_ERR_WORKSPACE_TOO_SMALL";
    case MLA_ERR_HIP: return "MLA_ERR_HIP";
  }
  return "MLA_ERR_UNKNOWN";
}

const char* mla_last_error(void) { return g_last_error.c_str(); }

mla_status mla_append_kv(const mla_dims* dims, mla_dtype dtype, int32_t n_tok, const void* c_kv,
                         const void* k_r, const int32_t* pos, const int64_t* row, void* cache,
                         void* stream) {
  mla_status st = check_dims(dims, dtype);
  if (st != MLA_OK) return st;
  if (n_tok < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "n_tok=%d < 0", n_tok);
  if (n_tok == 0) return MLA_OK;
  if (!c_kv || !k_r || !pos || !row || !cache) return fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  mla::AppendArgs a{};
  a.c_kv = c_kv;
  a.k_r = k_r;
  a.pos = pos;
  a.row = row;
  a.cache = cache;
  a.n_tok = n_tok;
  a.d_c = dims->d_c;
  a.d_r = dims->d_hR;
  fill_rope(dims, a.rope);
  return hip_status(mla::launch_append(a, dtype == MLA_BF16, static_cast<hipStream_t>(stream)), "mla_append_kv");
}

size_t mla_append_kv_from_hidden_workspace_bytes(const mla_dims* dims, mla_dtype dtype, int32_t n_tok,
                                                 int32_t d_model) {
  if (check_dims(dims, dtype) != MLA_OK || n_tok < 1 || d_model < 1) return 0;
  int32_t slices = 1, kr = 0;
  mla::kv_project_plan(n_tok, d_model, dtype == MLA_BF16, slices, kr);
  return static_cast<size_t>(slices) * n_tok * mla::ROWE * sizeof(float);
}

mla_status mla_append_kv_from_hidden(const mla_dims* dims, mla_dtype dtype, int32_t n_tok, int32_t d_model,
                                     const void* h, const void* w_dkv, const void* w_kr, const void* norm_weight,
                                     double eps, const int32_t* pos, const int64_t* row, void* cache,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  mla_status st = check_dims(dims, dtype);
  if (st != MLA_OK) return st;
  if (n_tok < 0 || n_tok > 65535) return fail(MLA_ERR_INVALID_ARGUMENT, "n_tok=%d out of range [0,65535]", n_tok);
  if (n_tok == 0) return MLA_OK;
  if (d_model < 1 || d_model > (1 << 20))
    return fail(MLA_ERR_INVALID_ARGUMENT, "d_model=%d out of range [1,%d]", d_model, 1 << 20);
  if (!(eps >= 0.0) || !std::isfinite(eps)) return fail(MLA_ERR_INVALID_ARGUMENT, "eps must be finite and >= 0");
  if (!h || !w_dkv || !w_kr || !pos || !row || !cache || !workspace)
    return fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  const size_t need = mla_append_kv_from_hidden_workspace_bytes(dims, dtype, n_tok, d_model);
  if (workspace_bytes < need)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu B < %zu B needed", workspace_bytes, need);
  mla::KvProjArgs a{};
  a.h = h;
  a.w_dkv = w_dkv;
  a.w_kr = w_kr;
  a.norm_w = norm_weight;
  a.pos = pos;
  a.row = row;
  a.cache = cache;
  a.part = static_cast<float*>(workspace);
  a.n_tok = n_tok;
  a.d_model = d_model;
  mla::kv_project_plan(n_tok, d_model, dtype == MLA_BF16, a.k_slices, a.k_per_slice);
  a.eps = static_cast<float>(eps);
  fill_rope(dims, a.rope);
  return hip_status(mla::launch_kv_project_append(a, dtype == MLA_BF16, static_cast<hipStream_t>(stream)),
                    "mla_append_kv_from_hidden");
}

static mla_status absorb_launch(const mla_dims* dims, int bf, int32_t n_q, const void* q_c, const void* q_r,
                                const int32_t* q_pos, const void* w_uk, void* q_lat, void* q_lat_lo, hipStream_t s,
                                const char* who, int q_r_f32 = 0, const mla::AppendArgs* fused_append = nullptr) {
  mla::AbsorbArgs a{};
  if (fused_append) {  // the caller checked that the fused bf16 kernel runs
    a.app_c = fused_append->c_kv;
    a.app_k = fused_append->k_r;
    a.app_pos = fused_append->pos;
    a.app_row = fused_append->row;
    a.app_cache = fused_append->cache;
    a.app_n = fused_append->n_tok;
  }
  a.q_r_f32 = q_r_f32;
  a.q_c = q_c;
  a.w_uk = w_uk;
  a.q_lat = q_lat;
  a.q_lat_lo = q_lat_lo;
  a.n_q = n_q;
  a.n_h = dims->n_h;
  a.d_c = dims->d_c;
  a.d_h = dims->d_h;
  a.d_r = dims->d_hR;
  a.q_r = q_r;
  a.q_pos = q_pos;
  fill_rope(dims, a.rope);
  mla_status r = hip_status(mla::launch_absorb(a, bf, s), who);
  if (r != MLA_OK || mla::absorb_fuses_rope(bf, dims->d_c, dims->d_h, dims->d_hR)) return r;
  mla::RopeQArgs ra{};
  ra.q_r = q_r;
  ra.q_pos = q_pos;
  ra.q_lat = q_lat;
  ra.q_lat_lo = q_lat_lo;
  ra.n_q = n_q;
  ra.n_h = dims->n_h;
  ra.d_c = dims->d_c;
  ra.d_r = dims->d_hR;
  fill_rope(dims, ra.rope);
  return hip_status(mla::launch_rope_q(ra, bf, s), who);
}

mla_status mla_absorb_q(const mla_dims* dims, mla_dtype dtype, int32_t n_q, const void* q_c, const void* q_r,
                        const int32_t* q_pos, const void* w_uk, void* q_lat, void* q_lat_lo, void* stream) {
  mla_status st = check_dims(dims, dtype);
  if (st != MLA_OK) return st;
  st = check_lo(dtype, q_lat_lo);
  if (st != MLA_OK) return st;
  if (n_q < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "n_q=%d < 0", n_q);
  if (n_q == 0) return MLA_OK;
  if (n_q > 65535 * 256) return fail(MLA_ERR_INVALID_ARGUMENT, "n_q=%d too large", n_q);
  if (!q_c || !q_r || !q_pos || !w_uk || !q_lat) return fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  return absorb_launch(dims, dtype == MLA_BF16, n_q, q_c, q_r, q_pos, w_uk, q_lat, q_lat_lo,
                       static_cast<hipStream_t>(stream), "mla_absorb_q");
}

mla_status mla_append_absorb(const mla_dims* dims, mla_dtype dtype, int32_t n_tok, const void* c_kv,
                             const void* k_r, const int32_t* pos, const int64_t* row, void* cache, int32_t n_q,
                             const void* q_c, const void* q_r, const int32_t* q_pos, const void* w_uk, void* q_lat,
                             void* q_lat_lo, void* stream) {
  mla_status st = check_dims(dims, dtype);
  if (st != MLA_OK) return st;
  st = check_lo(dtype, q_lat_lo);
  if (st != MLA_OK) return st;
  if (n_tok < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "n_tok=%d < 0", n_tok);
  if (n_q < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "n_q=%d < 0", n_q);
  if (n_q > 65535 * 256) return fail(MLA_ERR_INVALID_ARGUMENT, "n_q=%d too large", n_q);
  if (n_tok > 0 && (!c_kv || !k_r || !pos || !row || !cache))
    return fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  if (n_q > 0 && (!q_c || !q_r || !q_pos || !w_uk || !q_lat))
    return fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int bf = dtype == MLA_BF16;
  mla::AppendArgs ap{};
  ap.c_kv = c_kv;
  ap.k_r = k_r;
  ap.pos = pos;
  ap.row = row;
  ap.cache = cache;
  ap.n_tok = n_tok;
  ap.d_c = dims->d_c;
  ap.d_r = dims->d_hR;
  fill_rope(dims, ap.rope);
  if (n_q > 0 && n_tok > 0 && mla::absorb_fuses_rope(bf, dims->d_c, dims->d_h, dims->d_hR))
    return absorb_launch(dims, bf, n_q, q_c, q_r, q_pos, w_uk, q_lat, q_lat_lo, s, "mla_append_absorb", 0, &ap);
  // other shapes: the two launches of mla_append_kv and mla_absorb_q
  if (n_tok > 0) {
    st = hip_status(mla::launch_append(ap, bf, s), "mla_append_absorb");
    if (st != MLA_OK) return st;
  }
  if (n_q == 0) return MLA_OK;
  return absorb_launch(dims, bf, n_q, q_c, q_r, q_pos, w_uk, q_lat, q_lat_lo, s, "mla_append_absorb");
}

// ---- the query path from hidden states: c^Q = RMSNorm(W^DQ h), [q^C ; q^R] =
// [W^UQ ; W^QR] c^Q, then A2.  Workspace: slices of W^DQ h (fp32), c^Q and q^C
// (bf16: matrix-core operands), q^R (fp32: only rotated).
struct QPathLayout {
  int32_t slices, kps, slices2, kps2;
  size_t part, cq, qc, qr, total;
};
static QPathLayout qpath_layout(const mla_dims* d, int32_t n_q, int32_t d_model, int32_t d_cq) {
  QPathLayout L{};
  const int32_t d_out2 = d->n_h * (d->d_h + d->d_hR);
  mla::gemm_plan(n_q, d_model, d_cq, d_cq, L.slices, L.kps);
  mla::gemm_plan(n_q, d_cq, d_out2, d->n_h * d->d_h, L.slices2, L.kps2);
  L.part = 0;   // partials of W^DQ h, then (reused) of [W^UQ ; W^QR] c^Q
  L.cq = align256(std::max(static_cast<size_t>(L.slices) * n_q * d_cq,
                           L.slices2 > 1 ? static_cast<size_t>(L.slices2) * n_q * d_out2 : size_t{0}) *
                  sizeof(float));
  L.qc = L.cq + align256(static_cast<size_t>(n_q) * d_cq * 2);
  L.qr = L.qc + align256(static_cast<size_t>(n_q) * d->n_h * d->d_h * 2);
  L.total = L.qr + align256(static_cast<size_t>(n_q) * d->n_h * d->d_hR * sizeof(float));
  return L;
}

size_t mla_absorb_q_from_hidden_workspace_bytes(const mla_dims* dims, int32_t n_q, int32_t d_model, int32_t d_cq) {
  if (check_dims(dims, MLA_BF16) != MLA_OK || n_q < 1 || d_model < 1 || d_cq < 1) return 0;
  return qpath_layout(dims, n_q, d_model, d_cq).total;
}

mla_status mla_absorb_q_from_hidden(const mla_dims* dims, int32_t n_q, int32_t d_model, int32_t d_cq, const void* h,
                                    const void* w_dq, const void* norm_weight, double eps, const void* w_uq,
                                    const void* w_qr, const int32_t* q_pos, const void* w_uk, void* q_lat,
                                    void* q_lat_lo, void* workspace, size_t workspace_bytes, void* stream) {
  mla_status st = check_dims(dims, MLA_BF16);
  if (st != MLA_OK) return st;
  if (n_q < 0 || n_q > 65535) return fail(MLA_ERR_INVALID_ARGUMENT, "n_q=%d out of range [0,65535]", n_q);
  if (n_q == 0) return MLA_OK;
  if (d_model < 1 || d_model > (1 << 20)) return fail(MLA_ERR_INVALID_ARGUMENT, "d_model=%d out of range", d_model);
  if (d_cq < 1 || d_cq > 4096) return fail(MLA_ERR_INVALID_ARGUMENT, "d_cq=%d out of range [1,4096]", d_cq);
  if (!(eps >= 0.0) || !std::isfinite(eps)) return fail(MLA_ERR_INVALID_ARGUMENT, "eps must be finite and >= 0");
  if (!h || !w_dq || !w_uq || !w_qr || !q_pos || !w_uk || !q_lat || !workspace)
    return fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  const QPathLayout L = qpath_layout(dims, n_q, d_model, d_cq);
  if (workspace_bytes < L.total)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu B < %zu B needed", workspace_bytes, L.total);
  char* ws = static_cast<char*>(workspace);
  float* part = reinterpret_cast<float*>(ws + L.part);
  uint16_t* cq = reinterpret_cast<uint16_t*>(ws + L.cq);
  uint16_t* qc = reinterpret_cast<uint16_t*>(ws + L.qc);
  float* qr = reinterpret_cast<float*>(ws + L.qr);   // q^R stays fp32 up to its rotation
  hipStream_t s = static_cast<hipStream_t>(stream);
  mla::GemmArgs g1{};
  g1.x = h;
  g1.w0 = w_dq;
  g1.part = part;
  g1.n = n_q;
  g1.d_in = d_model;
  g1.d_out = d_cq;
  g1.split = d_cq;
  g1.k_slices = L.slices;
  g1.k_per_slice = L.kps;
  st = hip_status(mla::launch_gemm_partial(g1, 1, s), "mla_absorb_q_from_hidden (W^DQ)");
  if (st != MLA_OK) return st;
  st = hip_status(mla::launch_rmsnorm_rows(part, L.slices, n_q, d_cq, norm_weight, static_cast<float>(eps), cq, s),
                  "mla_absorb_q_from_hidden (RMSNorm)");
  if (st != MLA_OK) return st;
  mla::GemmArgs g2{};
  g2.x = cq;
  g2.w0 = w_uq;
  g2.w1 = w_qr;
  if (L.slices2 == 1) {   // one slice: q^C (bf16) and q^R (fp32) straight from the product
    g2.out0 = qc;
    g2.out1_f32 = qr;
  } else {
    g2.part = part;
  }
  g2.n = n_q;
  g2.d_in = d_cq;
  g2.d_out = dims->n_h * (dims->d_h + dims->d_hR);
  g2.split = dims->n_h * dims->d_h;
  g2.k_slices = L.slices2;
  g2.k_per_slice = L.kps2;
  st = hip_status(mla::launch_gemm_partial(g2, 1, s), "mla_absorb_q_from_hidden (W^UQ, W^QR)");
  if (st != MLA_OK) return st;
  if (L.slices2 > 1) {
    st = hip_status(mla::launch_slices_to_outputs(part, L.slices2, n_q, g2.d_out, g2.split, qc, qr, s),
                    "mla_absorb_q_from_hidden (q^C, q^R)");
    if (st != MLA_OK) return st;
  }
  return absorb_launch(dims, 1, n_q, qc, qr, q_pos, w_uk, q_lat, q_lat_lo, s, "mla_absorb_q_from_hidden (absorb)", 1);
}

// ---- the output projection: u = W^O o (o rounded once to bf16 for the matrix cores)
struct OutLayout {
  int32_t slices, kps;
  size_t o16, part, total;
};
static OutLayout out_layout(const mla_dims* d, int32_t n_q, int32_t d_model) {
  OutLayout L{};
  const int32_t d_in = d->n_h * d->d_h;
  mla::gemm_plan(n_q, d_in, d_model, d_model, L.slices, L.kps);
  L.o16 = 0;
  L.part = align256(static_cast<size_t>(n_q) * d_in * 2);
  L.total = L.part + (L.slices > 1 ? align256(static_cast<size_t>(L.slices) * n_q * d_model * sizeof(float)) : 0);
  return L;
}

size_t mla_output_projection_workspace_bytes(const mla_dims* dims, int32_t n_q, int32_t d_model) {
  if (check_dims(dims, MLA_BF16) != MLA_OK || n_q < 1 || d_model < 1) return 0;
  return out_layout(dims, n_q, d_model).total;
}

mla_status mla_output_projection(const mla_dims* dims, int32_t n_q, int32_t d_model, const float* o, const void* w_o,
                                 float* out, void* workspace, size_t workspace_bytes, void* stream) {
  mla_status st = check_dims(dims, MLA_BF16);
  if (st != MLA_OK) return st;
  if (n_q < 0 || n_q > 65535) return fail(MLA_ERR_INVALID_ARGUMENT, "n_q=%d out of range [0,65535]", n_q);
  if (n_q == 0) return MLA_OK;
  if (d_model < 1 || d_model > (1 << 20)) return fail(MLA_ERR_INVALID_ARGUMENT, "d_model=%d out of range", d_model);
  if (!o || !w_o || !out || !workspace) return fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  const OutLayout L = out_layout(dims, n_q, d_model);
  if (workspace_bytes < L.total)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu B < %zu B needed", workspace_bytes, L.total);
  char* ws = static_cast<char*>(workspace);
  uint16_t* o16 = reinterpret_cast<uint16_t*>(ws + L.o16);
  float* part = (L.slices > 1) ? reinterpret_cast<float*>(ws + L.part) : out;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t n_in = static_cast<int64_t>(n_q) * dims->n_h * dims->d_h;
  st = hip_status(mla::launch_to_bf16(o, n_in, o16, s), "mla_output_projection (bf16)");
  if (st != MLA_OK) return st;
  mla::GemmArgs g{};
  g.x = o16;
  g.w0 = w_o;
  g.part = part;
  g.n = n_q;
  g.d_in = dims->n_h * dims->d_h;
  g.d_out = d_model;
  g.split = d_model;
  g.k_slices = L.slices;
  g.k_per_slice = L.kps;
  st = hip_status(mla::launch_gemm_partial(g, 1, s), "mla_output_projection (W^O)");
  if (st != MLA_OK || L.slices == 1) return st;
  return hip_status(mla::launch_sum_slices(part, L.slices, static_cast<int64_t>(n_q) * d_model, out, s),
                    "mla_output_projection (slices)");
}

int32_t mla_decode_num_splits(const mla_dims* dims, mla_dtype dtype, int32_t batch, int32_t max_seq_len) {
  if (check_dims(dims, dtype) != MLA_OK) return 1;
  return plan_splits(dims, dtype, batch, max_seq_len);
}

int64_t mla_split_rows(int32_t max_seq_len, int32_t num_splits) { return split_rows(max_seq_len, num_splits); }

int32_t mla_precise_rows(const mla_dims* dims, mla_dtype dtype) {
  if (check_dims(dims, dtype) != MLA_OK) return 0;
  return precise_rows_of(dims, dtype);
}

static mla_status run_partials(const mla_dims* dims, mla_dtype dtype, int64_t n_q, const void* q_lat,
                               const void* q_lat_lo, const void* cache, int64_t stride, const int32_t* lens, int32_t max_len,
                               int32_t q_per_seq, int prefill, int32_t num_splits, float* z_part,
                               float* lse_part, hipStream_t s, const char* who,
                               const mla_paged_cache* paged = nullptr) {
  mla::SplitArgs a{};
  if (paged) {
    a.block_table = paged->block_table;
    a.num_pages = paged->num_pages;
    a.bt_stride = paged->max_pages;
    a.page_shift = page_shift_of(paged->page_rows);
  }
  a.q_lat = q_lat;
  a.q_lat_lo = q_lat_lo;
  a.cache = cache;
  a.lens = lens;
  a.z_part = z_part;
  a.lse_part = lse_part;
  a.stride = stride;
  a.split_rows = split_rows(max_len, num_splits);
  a.n_q = static_cast<int32_t>(n_q);
  a.n_h = dims->n_h;
  a.d_c = dims->d_c;
  a.d_r = dims->d_hR;
  a.num_splits = num_splits;
  a.max_len = max_len;
  a.q_per_seq = q_per_seq;
  a.prefill = prefill;
  a.qscale = static_cast<float>(scale_of(dims) * 1.4426950408889634);
  a.precise_below = precise_rows_of(dims, dtype);
  return hip_status(mla::launch_splitkv(a, dtype == MLA_BF16, s), who);
}

mla_status mla_decode_partials(const mla_dims* dims, mla_dtype dtype, int32_t batch, const void* q_lat,
                               const void* q_lat_lo, const void* cache, int64_t cache_seq_stride,
                               const int32_t* seq_lens, int32_t max_seq_len, int32_t num_splits, float* z_part,
                               float* lse_part, void* stream) {
  mla_status st = check_dims(dims, dtype);
  if (st != MLA_OK) return st;
  st = check_lo(dtype, q_lat_lo);
  if (st != MLA_OK) return st;
  if (batch < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "batch=%d < 1", batch);
  if (max_seq_len < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "max_seq_len=%d < 1", max_seq_len);
  if (cache_seq_stride < max_seq_len)
    return fail(MLA_ERR_INVALID_ARGUMENT, "cache_seq_stride=%lld < max_seq_len=%d", (long long)cache_seq_stride, max_seq_len);
  if (num_splits < 1 || num_splits > kMaxSplits)
    return fail(MLA_ERR_INVALID_ARGUMENT, "num_splits=%d out of range [1,%d]", num_splits, kMaxSplits);
  if (!q_lat || !cache || !seq_lens || !z_part || !lse_part) return fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  return run_partials(dims, dtype, batch, q_lat, q_lat_lo, cache, cache_seq_stride, seq_lens, max_seq_len, 1, 0,
                      num_splits, z_part, lse_part, static_cast<hipStream_t>(stream), "mla_decode_partials");
}

mla_status mla_decode_partials_paged(const mla_dims* dims, mla_dtype dtype, int32_t batch, const void* q_lat,
                                     const void* q_lat_lo, const mla_paged_cache* cache, const int32_t* seq_lens,
                                     int32_t max_seq_len, int32_t num_splits, float* z_part, float* lse_part,
                                     void* stream) {
  mla_status st = check_dims(dims, dtype);
  if (st != MLA_OK) return st;
  st = check_lo(dtype, q_lat_lo);
  if (st != MLA_OK) return st;
  if (batch < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "batch=%d < 1", batch);
  if (max_seq_len < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "max_seq_len=%d < 1", max_seq_len);
  int64_t cap = 0;
  st = check_paged(cache, max_seq_len, cap);
  if (st != MLA_OK) return st;
  if (num_splits < 1 || num_splits > kMaxSplits)
    return fail(MLA_ERR_INVALID_ARGUMENT, "num_splits=%d out of range [1,%d]", num_splits, kMaxSplits);
  if (!q_lat || !seq_lens || !z_part || !lse_part) return fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  return run_partials(dims, dtype, batch, q_lat, q_lat_lo, cache->pool, cap, seq_lens, max_seq_len, 1, 0, num_splits,
                      z_part, lse_part, static_cast<hipStream_t>(stream), "mla_decode_partials_paged", cache);
}

mla_status mla_combine_project(const mla_dims* dims, mla_dtype dtype, int32_t n_q, int32_t num_splits,
                               const float* z_part, const float* lse_part, const void* w_uv, float* out,
                               float* out_latent, void* stream) {
  mla_status st = check_dims(dims, dtype);
  if (st != MLA_OK) return st;
  if (n_q < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "n_q=%d < 1", n_q);
  if (num_splits < 1 || num_splits > kMaxSplits)
    return fail(MLA_ERR_INVALID_ARGUMENT, "num_splits=%d out of range [1,%d]", num_splits, kMaxSplits);
  if (!z_part || !lse_part || !w_uv || !out) return fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  mla::CombineArgs a{z_part, lse_part, w_uv, out, out_latent, n_q, dims->n_h, dims->d_c, dims->d_h, num_splits};
  return hip_status(mla::launch_combine(a, dtype == MLA_BF16, static_cast<hipStream_t>(stream)), "mla_combine_project");
}

size_t mla_decode_workspace_bytes(const mla_dims* dims, mla_dtype dtype, int32_t batch, int32_t max_seq_len) {
  if (check_dims(dims, dtype) != MLA_OK || batch < 1 || max_seq_len < 1) return 0;
  return partial_bytes(dims, batch, plan_splits(dims, dtype, batch, max_seq_len));
}

static mla_status decode_impl(const mla_dims* dims, mla_dtype dtype, int32_t batch, const void* q_lat,
                              const void* q_lat_lo, const void* cache, int64_t cache_seq_stride, const mla_paged_cache* paged,
                              const int32_t* seq_lens, int32_t max_seq_len, const void* w_uv, float* out,
                              float* out_latent, void* workspace, size_t workspace_bytes, void* stream) {
  mla_status st = check_dims(dims, dtype);
  if (st != MLA_OK) return st;
  st = check_lo(dtype, q_lat_lo);
  if (st != MLA_OK) return st;
  if (batch < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "batch=%d < 1", batch);
  if (max_seq_len < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "max_seq_len=%d < 1", max_seq_len);
  if (paged) {
    st = check_paged(paged, max_seq_len, cache_seq_stride);
    if (st != MLA_OK) return st;
    cache = paged->pool;
  }
  if (cache_seq_stride < max_seq_len)
    return fail(MLA_ERR_INVALID_ARGUMENT, "cache_seq_stride=%lld < max_seq_len=%d", (long long)cache_seq_stride, max_seq_len);
  if (!q_lat || !cache || !seq_lens || !w_uv || !out || !workspace)
    return fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  const int32_t S = plan_splits(dims, dtype, batch, max_seq_len);
  const size_t need = partial_bytes(dims, batch, S);
  if (workspace_bytes < need)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu B < %zu B needed", workspace_bytes, need);
  float* z = static_cast<float*>(workspace);
  float* lse = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                        align256(static_cast<size_t>(batch) * S * dims->n_h * dims->d_c * sizeof(float)));
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = run_partials(dims, dtype, batch, q_lat, q_lat_lo, cache, cache_seq_stride, seq_lens, max_seq_len, 1, 0, S, z,
                    lse, s, "mla_decode (partials)", paged);
  if (st != MLA_OK) return st;
  mla::CombineArgs a{z, lse, w_uv, out, out_latent, batch, dims->n_h, dims->d_c, dims->d_h, S};
  return hip_status(mla::launch_combine(a, dtype == MLA_BF16, s), "mla_decode (combine)");
}

mla_status mla_decode(const mla_dims* dims, mla_dtype dtype, int32_t batch, const void* q_lat, const void* q_lat_lo,
                      const void* cache, int64_t cache_seq_stride, const int32_t* seq_lens, int32_t max_seq_len,
                      const void* w_uv, float* out, float* out_latent, void* workspace, size_t workspace_bytes,
                      void* stream) {
  return decode_impl(dims, dtype, batch, q_lat, q_lat_lo, cache, cache_seq_stride, nullptr, seq_lens, max_seq_len,
                     w_uv, out, out_latent, workspace, workspace_bytes, stream);
}

mla_status mla_decode_paged(const mla_dims* dims, mla_dtype dtype, int32_t batch, const void* q_lat,
                            const void* q_lat_lo, const mla_paged_cache* cache, const int32_t* seq_lens,
                            int32_t max_seq_len, const void* w_uv, float* out, float* out_latent, void* workspace,
                            size_t workspace_bytes, void* stream) {
  if (!cache) return fail(MLA_ERR_INVALID_ARGUMENT, "paged cache descriptor is NULL");
  return decode_impl(dims, dtype, batch, q_lat, q_lat_lo, nullptr, 0, cache, seq_lens, max_seq_len, w_uv, out,
                     out_latent, workspace, workspace_bytes, stream);
}

size_t mla_prefill_workspace_bytes(const mla_dims* dims, mla_dtype dtype, int32_t batch, int32_t chunk,
                                   int32_t max_prefix_len) {
  if (check_dims(dims, dtype) != MLA_OK || batch < 1 || chunk < 1 || max_prefix_len < 0) return 0;
  const int64_t n_q = static_cast<int64_t>(batch) * chunk;
  const int64_t max_len = static_cast<int64_t>(max_prefix_len) + chunk;
  return partial_bytes(dims, n_q, plan_splits(dims, dtype, n_q, max_len));
}

static mla_status prefill_impl(const mla_dims* dims, mla_dtype dtype, int32_t batch, int32_t chunk,
                               const void* q_lat, const void* q_lat_lo, const void* cache, int64_t cache_seq_stride,
                               const mla_paged_cache* paged, const int32_t* prefix_lens, int32_t max_prefix_len,
                               const void* w_uv, float* out, void* workspace, size_t workspace_bytes,
                               void* stream) {
  mla_status st = check_dims(dims, dtype);
  if (st != MLA_OK) return st;
  st = check_lo(dtype, q_lat_lo);
  if (st != MLA_OK) return st;
  if (batch < 1 || chunk < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "batch=%d, chunk=%d must be >= 1", batch, chunk);
  if (max_prefix_len < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "max_prefix_len=%d < 0", max_prefix_len);
  const int64_t max_len = static_cast<int64_t>(max_prefix_len) + chunk;
  if (paged) {
    st = check_paged(paged, max_len, cache_seq_stride);
    if (st != MLA_OK) return st;
    cache = paged->pool;
  }
  if (max_len > cache_seq_stride)
    return fail(MLA_ERR_INVALID_ARGUMENT, "max_prefix_len + chunk = %lld > cache_seq_stride=%lld",
                (long long)max_len, (long long)cache_seq_stride);
  if (max_len > 0x7fffffff) return fail(MLA_ERR_INVALID_ARGUMENT, "prefix + chunk too large");
  const int64_t n_q = static_cast<int64_t>(batch) * chunk;
  if (n_q > 0x7fffffff / 2) return fail(MLA_ERR_INVALID_ARGUMENT, "batch*chunk too large");
  if (!q_lat || !cache || !prefix_lens || !w_uv || !out || !workspace)
    return fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  const int32_t S = plan_splits(dims, dtype, n_q, max_len);
  const size_t need = partial_bytes(dims, n_q, S);
  if (workspace_bytes < need)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu B < %zu B needed", workspace_bytes, need);
  float* z = static_cast<float*>(workspace);
  float* lse = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                        align256(static_cast<size_t>(n_q) * S * dims->n_h * dims->d_c * sizeof(float)));
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = run_partials(dims, dtype, n_q, q_lat, q_lat_lo, cache, cache_seq_stride, prefix_lens,
                    static_cast<int32_t>(max_len), chunk, 1, S, z, lse, s, "mla_prefill (partials)", paged);
  if (st != MLA_OK) return st;
  mla::CombineArgs a{z, lse, w_uv, out, nullptr, static_cast<int32_t>(n_q), dims->n_h, dims->d_c, dims->d_h, S};
  return hip_status(mla::launch_combine(a, dtype == MLA_BF16, s), "mla_prefill (combine)");
}

mla_status mla_prefill(const mla_dims* dims, mla_dtype dtype, int32_t batch, int32_t chunk, const void* q_lat,
                       const void* q_lat_lo, const void* cache, int64_t cache_seq_stride, const int32_t* prefix_lens,
                       int32_t max_prefix_len, const void* w_uv, float* out, void* workspace,
                       size_t workspace_bytes, void* stream) {
  return prefill_impl(dims, dtype, batch, chunk, q_lat, q_lat_lo, cache, cache_seq_stride, nullptr, prefix_lens,
                      max_prefix_len, w_uv, out, workspace, workspace_bytes, stream);
}

mla_status mla_prefill_paged(const mla_dims* dims, mla_dtype dtype, int32_t batch, int32_t chunk, const void* q_lat,
                             const void* q_lat_lo, const mla_paged_cache* cache, const int32_t* prefix_lens,
                             int32_t max_prefix_len, const void* w_uv, float* out, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if (!cache) return fail(MLA_ERR_INVALID_ARGUMENT, "paged cache descriptor is NULL");
  return prefill_impl(dims, dtype, batch, chunk, q_lat, q_lat_lo, nullptr, 0, cache, prefix_lens, max_prefix_len, w_uv,
                      out, workspace, workspace_bytes, stream);
}


size_t mla_prefill_unabsorbed_workspace_bytes(const mla_dims* dims, mla_dtype dtype, int32_t batch,
                                              int32_t chunk, int32_t max_prefix_len) {
  if (check_dims(dims, dtype) != MLA_OK || dtype != MLA_BF16 || batch < 1 || chunk < 1 || max_prefix_len < 0)
    return 0;
  const int64_t rows = static_cast<int64_t>(max_prefix_len) + chunk;
  const int64_t rows_cap = (rows + mla::XROWS_ALIGN - 1) / mla::XROWS_ALIGN * mla::XROWS_ALIGN;
  return static_cast<size_t>(batch) * dims->n_h * rows_cap * mla::ROWB;
}

static mla_status prefill_unabsorbed_impl(const mla_dims* dims, mla_dtype dtype, int32_t batch, int32_t chunk,
                                          const void* q_c, const void* q_r, const void* cache,
                                          int64_t cache_seq_stride, const mla_paged_cache* paged,
                                          const int32_t* prefix_lens, int32_t max_prefix_len, const void* w_uk,
                                          const void* w_uv, float* out, void* workspace, size_t workspace_bytes,
                                          void* stream) {
  mla_status st = check_dims(dims, dtype);
  if (st != MLA_OK) return st;
  if (dtype != MLA_BF16) return fail(MLA_ERR_UNSUPPORTED, "mla_prefill_unabsorbed: bf16 storage only");
  if (dims->n_h % 8) return fail(MLA_ERR_UNSUPPORTED, "mla_prefill_unabsorbed: n_h=%d must be a multiple of 8", dims->n_h);
  if (batch < 1 || chunk < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "batch=%d, chunk=%d must be >= 1", batch, chunk);
  if (batch > 65535) return fail(MLA_ERR_INVALID_ARGUMENT, "batch=%d > 65535", batch);
  if (max_prefix_len < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "max_prefix_len=%d < 0", max_prefix_len);
  const int64_t max_len = static_cast<int64_t>(max_prefix_len) + chunk;
  if (paged) {
    st = check_paged(paged, max_len, cache_seq_stride);
    if (st != MLA_OK) return st;
    cache = paged->pool;
  }
  if (max_len > cache_seq_stride)
    return fail(MLA_ERR_INVALID_ARGUMENT, "max_prefix_len + chunk = %lld > cache_seq_stride=%lld",
                (long long)max_len, (long long)cache_seq_stride);
  if (max_len > 0x7fffffff - mla::XROWS_ALIGN) return fail(MLA_ERR_INVALID_ARGUMENT, "prefix + chunk too large");
  if (!q_c || !q_r || !cache || !prefix_lens || !w_uk || !w_uv || !out || !workspace)
    return fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  const size_t need = mla_prefill_unabsorbed_workspace_bytes(dims, dtype, batch, chunk, max_prefix_len);
  if (workspace_bytes < need)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu B < %zu B needed", workspace_bytes, need);
  const int64_t rows_cap = (max_len + mla::XROWS_ALIGN - 1) / mla::XROWS_ALIGN * mla::XROWS_ALIGN;
  mla::ExpandArgs e{};
  e.cache = cache;
  e.prefix_lens = prefix_lens;
  e.w_uk = w_uk;
  e.w_uv = w_uv;
  e.x = workspace;
  e.stride = cache_seq_stride;
  e.rows_cap = rows_cap;
  e.batch = batch;
  e.n_h = dims->n_h;
  e.chunk = chunk;
  e.max_len = static_cast<int32_t>(max_len);
  if (paged) {
    e.block_table = paged->block_table;
    e.num_pages = paged->num_pages;
    e.bt_stride = paged->max_pages;
    e.page_shift = page_shift_of(paged->page_rows);
  }
  mla::PrefillArgs p{};
  p.q_c = q_c;
  p.q_r = q_r;
  p.x = workspace;
  p.prefix_lens = prefix_lens;
  p.out = out;
  p.rows_cap = rows_cap;
  p.batch = batch;
  p.n_h = dims->n_h;
  p.chunk = chunk;
  p.max_len = static_cast<int32_t>(max_len);
  p.precise_below = yarn_on(dims) ? kAllPrecise : kPreciseBelow;   // YaRN: hi + lo everywhere
  p.qscale = static_cast<float>(scale_of(dims) * 1.4426950408889634);
  fill_rope(dims, p.rope);
  return hip_status(mla::launch_prefill_unabsorbed(e, p, static_cast<hipStream_t>(stream)), "mla_prefill_unabsorbed");
}

mla_status mla_prefill_unabsorbed(const mla_dims* dims, mla_dtype dtype, int32_t batch, int32_t chunk,
                                  const void* q_c, const void* q_r, const void* cache, int64_t cache_seq_stride,
                                  const int32_t* prefix_lens, int32_t max_prefix_len, const void* w_uk,
                                  const void* w_uv, float* out, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  return prefill_unabsorbed_impl(dims, dtype, batch, chunk, q_c, q_r, cache, cache_seq_stride, nullptr, prefix_lens,
                                 max_prefix_len, w_uk, w_uv, out, workspace, workspace_bytes, stream);
}

mla_status mla_prefill_unabsorbed_paged(const mla_dims* dims, mla_dtype dtype, int32_t batch, int32_t chunk,
                                        const void* q_c, const void* q_r, const mla_paged_cache* cache,
                                        const int32_t* prefix_lens, int32_t max_prefix_len, const void* w_uk,
                                        const void* w_uv, float* out, void* workspace, size_t workspace_bytes,
                                        void* stream) {
  if (!cache) return fail(MLA_ERR_INVALID_ARGUMENT, "paged cache descriptor is NULL");
  return prefill_unabsorbed_impl(dims, dtype, batch, chunk, q_c, q_r, nullptr, 0, cache, prefix_lens, max_prefix_len,
                                 w_uk, w_uv, out, workspace, workspace_bytes, stream);
}
static mla_status check_fp8(const mla_fp8_cache* c) {
  if (!c) return fail(MLA_ERR_INVALID_ARGUMENT, "FP8 cache descriptor is NULL");
  if (!c->codes || !c->rope || !c->scale) return fail(MLA_ERR_INVALID_ARGUMENT, "FP8 cache: NULL array");
  return MLA_OK;
}

mla_status mla_append_kv_fp8(const mla_dims* dims, int32_t n_tok, const void* c_kv, const void* k_r,
                             const int32_t* pos, const int64_t* row, const mla_fp8_cache* cache, void* stream) {
  mla_status st = check_dims(dims, MLA_BF16);
  if (st != MLA_OK) return st;
  if (n_tok < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "n_tok=%d < 0", n_tok);
  if (n_tok == 0) return MLA_OK;
  st = check_fp8(cache);
  if (st != MLA_OK) return st;
  if (!c_kv || !k_r || !pos || !row) return fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  mla::AppendArgs a{};
  a.c_kv = c_kv;
  a.k_r = k_r;
  a.pos = pos;
  a.row = row;
  a.cache = cache->codes;
  a.fp8_rope = cache->rope;
  a.fp8_scale = cache->scale;
  a.n_tok = n_tok;
  a.d_c = dims->d_c;
  a.d_r = dims->d_hR;
  fill_rope(dims, a.rope);
  return hip_status(mla::launch_append_fp8(a, static_cast<hipStream_t>(stream)), "mla_append_kv_fp8");
}

static mla_status fp8_partials(const mla_dims* dims, int32_t batch, const void* q_lat, const void* q_lat_lo,
                               const mla_fp8_cache* cache,
                               int64_t stride, const int32_t* seq_lens, int32_t max_seq_len, int32_t S, float* z,
                               float* lse, hipStream_t s, const char* who, int32_t q_per_seq = 1, int prefill = 0) {
  mla::SplitArgs a{};
  a.q_lat = q_lat;
  a.q_lat_lo = q_lat_lo;
  a.cache = cache->codes;
  a.fp8_rope = cache->rope;
  a.fp8_scale = cache->scale;
  a.lens = seq_lens;
  a.z_part = z;
  a.lse_part = lse;
  a.stride = stride;
  a.split_rows = split_rows(max_seq_len, S);
  a.n_q = batch;   // queries (sequences x q_per_seq)
  a.n_h = dims->n_h;
  a.d_c = dims->d_c;
  a.d_r = dims->d_hR;
  a.num_splits = S;
  a.max_len = max_seq_len;
  a.q_per_seq = q_per_seq;
  a.prefill = prefill;
  a.qscale = static_cast<float>(scale_of(dims) * 1.4426950408889634);
  a.precise_below = precise_rows_of(dims, MLA_BF16);
  return hip_status(mla::launch_splitkv_fp8(a, s), who);
}

static mla_status check_fp8_decode(const mla_dims* dims, int32_t batch, const void* q_lat, const mla_fp8_cache* cache,
                                   int64_t stride, const int32_t* seq_lens, int32_t max_seq_len) {
  mla_status st = check_dims(dims, MLA_BF16);
  if (st != MLA_OK) return st;
  if (batch < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "batch=%d < 1", batch);
  if (max_seq_len < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "max_seq_len=%d < 1", max_seq_len);
  if (stride < max_seq_len)
    return fail(MLA_ERR_INVALID_ARGUMENT, "cache_seq_stride=%lld < max_seq_len=%d", (long long)stride, max_seq_len);
  st = check_fp8(cache);
  if (st != MLA_OK) return st;
  if (!q_lat || !seq_lens) return fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  return MLA_OK;
}

mla_status mla_decode_partials_fp8(const mla_dims* dims, int32_t batch, const void* q_lat, const void* q_lat_lo,
                                   const mla_fp8_cache* cache,
                                   int64_t cache_seq_stride, const int32_t* seq_lens, int32_t max_seq_len,
                                   int32_t num_splits, float* z_part, float* lse_part, void* stream) {
  mla_status st = check_fp8_decode(dims, batch, q_lat, cache, cache_seq_stride, seq_lens, max_seq_len);
  if (st != MLA_OK) return st;
  if (num_splits < 1 || num_splits > kMaxSplits)
    return fail(MLA_ERR_INVALID_ARGUMENT, "num_splits=%d out of range [1,%d]", num_splits, kMaxSplits);
  if (!z_part || !lse_part) return fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  return fp8_partials(dims, batch, q_lat, q_lat_lo, cache, cache_seq_stride, seq_lens, max_seq_len, num_splits, z_part,
                      lse_part, static_cast<hipStream_t>(stream), "mla_decode_partials_fp8");
}

mla_status mla_decode_fp8(const mla_dims* dims, int32_t batch, const void* q_lat, const void* q_lat_lo,
                          const mla_fp8_cache* cache,
                          int64_t cache_seq_stride, const int32_t* seq_lens, int32_t max_seq_len, const void* w_uv,
                          float* out, float* out_latent, void* workspace, size_t workspace_bytes, void* stream) {
  mla_status st = check_fp8_decode(dims, batch, q_lat, cache, cache_seq_stride, seq_lens, max_seq_len);
  if (st != MLA_OK) return st;
  if (!w_uv || !out || !workspace) return fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  const int32_t S = plan_splits(dims, MLA_BF16, batch, max_seq_len);
  const size_t need = partial_bytes(dims, batch, S);
  if (workspace_bytes < need)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu B < %zu B needed", workspace_bytes, need);
  float* z = static_cast<float*>(workspace);
  float* lse = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                        align256(static_cast<size_t>(batch) * S * dims->n_h * dims->d_c * sizeof(float)));
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = fp8_partials(dims, batch, q_lat, q_lat_lo, cache, cache_seq_stride, seq_lens, max_seq_len, S, z, lse, s,
                    "mla_decode_fp8 (partials)");
  if (st != MLA_OK) return st;
  mla::CombineArgs a{z, lse, w_uv, out, out_latent, batch, dims->n_h, dims->d_c, dims->d_h, S};
  return hip_status(mla::launch_combine(a, 1, s), "mla_decode_fp8 (combine)");
}
mla_status mla_prefill_fp8(const mla_dims* dims, int32_t batch, int32_t chunk, const void* q_lat,
                           const void* q_lat_lo, const mla_fp8_cache* cache, int64_t cache_seq_stride, const int32_t* prefix_lens,
                           int32_t max_prefix_len, const void* w_uv, float* out, void* workspace,
                           size_t workspace_bytes, void* stream) {
  mla_status st = check_dims(dims, MLA_BF16);
  if (st != MLA_OK) return st;
  if (batch < 1 || chunk < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "batch=%d, chunk=%d must be >= 1", batch, chunk);
  if (max_prefix_len < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "max_prefix_len=%d < 0", max_prefix_len);
  const int64_t max_len = static_cast<int64_t>(max_prefix_len) + chunk;
  if (max_len > cache_seq_stride)
    return fail(MLA_ERR_INVALID_ARGUMENT, "max_prefix_len + chunk = %lld > cache_seq_stride=%lld",
                (long long)max_len, (long long)cache_seq_stride);
  if (max_len > 0x7fffffff) return fail(MLA_ERR_INVALID_ARGUMENT, "prefix + chunk too large");
  const int64_t n_q = static_cast<int64_t>(batch) * chunk;
  if (n_q > 0x7fffffff / 2) return fail(MLA_ERR_INVALID_ARGUMENT, "batch*chunk too large");
  st = check_fp8(cache);
  if (st != MLA_OK) return st;
  if (!q_lat || !prefix_lens || !w_uv || !out || !workspace) return fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  const int32_t S = plan_splits(dims, MLA_BF16, n_q, max_len);
  const size_t need = partial_bytes(dims, n_q, S);
  if (workspace_bytes < need)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu B < %zu B needed", workspace_bytes, need);
  float* z = static_cast<float*>(workspace);
  float* lse = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                        align256(static_cast<size_t>(n_q) * S * dims->n_h * dims->d_c * sizeof(float)));
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = fp8_partials(dims, static_cast<int32_t>(n_q), q_lat, q_lat_lo, cache, cache_seq_stride, prefix_lens,
                    static_cast<int32_t>(max_len), S, z, lse, s, "mla_prefill_fp8 (partials)", chunk, 1);
  if (st != MLA_OK) return st;
  mla::CombineArgs a{z, lse, w_uv, out, nullptr, static_cast<int32_t>(n_q), dims->n_h, dims->d_c, dims->d_h, S};
  return hip_status(mla::launch_combine(a, 1, s), "mla_prefill_fp8 (combine)");
}
}  // extern "C"

// ---- allocation-free decode: the split partials live in this file-scope
// device array (one copy per GPU, held until the process ends).  Host code
// never uses the array's name as an address: the per-device pointer comes
// from hipGetSymbolAddress, taken once per device on its first call.
static __device__ __align__(256) uint8_t scratch[MLA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mutex;

mla_status scratch_of_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "mla_decode_noalloc (hipGetDevice)");
  if (dev < 0 || dev >= kMaxDevices) return fail(MLA_ERR_UNSUPPORTED, "device %d beyond the %d supported", dev, kMaxDevices);
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return hip_status(e, "mla_decode_noalloc (hipGetSymbolAddress)");
      if (!p) return fail(MLA_ERR_HIP, "mla_decode_noalloc: no device address for the scratch array");
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return MLA_OK;
}
}  // namespace

extern "C" mla_status mla_decode_noalloc(const mla_dims* dims, mla_dtype dtype, int32_t batch, const void* q_lat,
                                         const void* q_lat_lo, const void* cache, int64_t cache_seq_stride,
                                         const int32_t* seq_lens, int32_t max_seq_len, const void* w_uv,
                                         float* out, float* out_latent, void* stream) {
  mla_status st = check_dims(dims, dtype);
  if (st != MLA_OK) return st;
  st = check_lo(dtype, q_lat_lo);
  if (st != MLA_OK) return st;
  if (batch < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "batch=%d < 1", batch);
  if (max_seq_len < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "max_seq_len=%d < 1", max_seq_len);
  if (cache_seq_stride < max_seq_len)
    return fail(MLA_ERR_INVALID_ARGUMENT, "cache_seq_stride=%lld < max_seq_len=%d", (long long)cache_seq_stride, max_seq_len);
  if (!q_lat || !cache || !seq_lens || !w_uv || !out) return fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  // every argument is checked before the device is touched
  const size_t need = partial_bytes(dims, batch, plan_splits(dims, dtype, batch, max_seq_len));
  if (need > MLA_NOALLOC_SCRATCH_BYTES)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL,
                "mla_decode_noalloc: the split partials of batch %d, max_seq_len %d take %zu B, beyond the "
                "library's %zu-B scratch array (use mla_decode with a workspace)",
                batch, max_seq_len, need, static_cast<size_t>(MLA_NOALLOC_SCRATCH_BYTES));
  void* ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st != MLA_OK) return st;
  return decode_impl(dims, dtype, batch, q_lat, q_lat_lo, cache, cache_seq_stride, nullptr, seq_lens, max_seq_len,
                     w_uv, out, out_latent, ws, MLA_NOALLOC_SCRATCH_BYTES, stream);
}
