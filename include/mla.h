/*
 * mla.h -- C ABI of the MI355X (gfx950) MLA latent-KV attention library.
 *
 * Multi-head Latent Attention keeps, per token and layer, one cache row
 *     row_t = [ c^KV_t (d_c) ; k^R_t (d_hR) ]
 * (jiphyeonjeon.kr DeepSeek-V2 review, sections 2-3; xyznot.com DeepSeek-V3
 * report, Metode 1: only c^KV and k^R are cached).  A head's query is folded
 * through W^UK into latent space, scored against whole rows, and the weighted
 * sum of c^KV is lifted by W^UV only at the end (review section 2, the
 * absorption identities).  The score of head i against row j is
 *     l_ij = (q~_i . c_j + q^R_i . k^R_j) * scale,   scale = 1/sqrt(d_h + d_hR)
 * (review section 3: the scale stays sqrt(128 + 64) after absorption).
 *
 * Conventions for every entry point
 *   - Pointers are DEVICE pointers unless marked (host).  The caller owns all
 *     buffers; the library never allocates, frees or retains device memory.
 *   - Every launch is asynchronous on `stream` (a hipStream_t; NULL = the
 *     null stream).  The return value only reports argument validation and
 *     launch errors; faults surface at the caller's next synchronisation.
 *   - Arguments are validated on the host BEFORE any launch.  On an error no
 *     kernel runs and no output is written.  mla_last_error() then returns a
 *     thread-local description.
 *   - Outputs must not alias inputs.
 *   - Storage dtype is MLA_BF16 (bfloat16 bits) or MLA_F32 for the cache,
 *     queries and weights; accumulation is always fp32; outputs marked
 *     "float" are fp32.
 *   - Identical inputs and launch arguments give bitwise-identical outputs.
 *   - RoPE (pages give no formula; the decoupled-RoPE section of the
 *     irregular6612 notes has no body): interleaved pairs (x[2k], x[2k+1])
 *     rotated by angle pos * rope_base^(-2k/d_hR); the angle and its sine and
 *     cosine are formed in fp64, the rotation in fp32.
 *   - Fast paths: d_c = 512, d_h = 128, d_hR = 64.  n_h in {16, 32, 64, 128}
 *     runs the MFMA kernels for MLA_BF16; any other n_h, and MLA_F32, run the
 *     generic fp32 kernels.  Other d_c / d_h / d_hR return MLA_ERR_UNSUPPORTED.
 */
#ifndef MLA_H
#define MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_ABI_VERSION 10

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARGUMENT = 1,
  MLA_ERR_UNSUPPORTED = 2,
  MLA_ERR_WORKSPACE_TOO_SMALL = 3,
  MLA_ERR_HIP = 4
} mla_status;

typedef enum { MLA_F32 = 0, MLA_BF16 = 1 } mla_dtype;

/* Model dimensions in the pages' notation (review sections 2-4):
 * d_c  latent width of c^KV (512 for V2 and V2-Lite)
 * d_h  per-head content dim of keys/values (128)
 * d_hR decoupled RoPE dim (64), even
 * n_h  number of query heads (V2: 128, V2-Lite: 16)
 * rope_base   RoPE frequency base (10000)
 * softmax_scale  0 selects the default: 1/sqrt(d_h + d_hR), times
 *             (0.1 ln s + 1)^2 when yarn_factor s > 1
 * Long-context RoPE (jiphyeonjeon.kr DeepSeek-V2 review, section 6: YaRN at
 * scale 40 over the 4K pretraining context; the formula is YaRN's published
 * frequency interpolation).  yarn_factor 0 or 1 keeps the plain frequencies
 * theta_k = rope_base^(-2k/d_hR).  For s = yarn_factor > 1, with
 * r_k = yarn_orig_ctx * theta_k / (2 pi) and
 * g_k = clamp((r_k - yarn_alpha) / (yarn_beta - yarn_alpha), 0, 1),
 * pair k rotates at (1 - g_k) theta_k / s + g_k theta_k.  Requires
 * yarn_orig_ctx > 0 and 0 < yarn_alpha < yarn_beta (the pages' setting is
 * s = 40 over 4,096 positions; alpha 1 and beta 32 are YaRN's published
 * values).  The frequencies act wherever RoPE does (A1, A2, the unabsorbed
 * prefill's query). */
typedef struct {
  int32_t d_c, d_h, d_hR, n_h;
  double rope_base;
  double softmax_scale;
  double yarn_factor;
  double yarn_orig_ctx;
  double yarn_alpha;
  double yarn_beta;
} mla_dims;

int32_t mla_abi_version(void);
const char* mla_status_string(mla_status s);
const char* mla_last_error(void);

/* A1 -- write cache rows of new tokens (review section 3; DeepSeek-V3 report,
 * Metode 1: k^R_t = RoPE(W^KR h_t), cached next to c^KV_t).
 *   c_kv [n_tok][d_c], k_r [n_tok][d_hR] (pre-RoPE), pos [n_tok] (int32 >= 0),
 *   row [n_tok] (int64, destination row index into `cache`, >= 0)
 *   cache [*][d_c + d_hR]: row[t] receives [c_kv[t] ; RoPE(k_r[t], pos[t])].
 * Rows must be distinct.  n_tok = 0 is a no-op.  Errors: null pointer with
 * n_tok > 0, n_tok < 0, bad dims. */
mla_status mla_append_kv(const mla_dims* dims, mla_dtype dtype, int32_t n_tok,
                         const void* c_kv, const void* k_r, const int32_t* pos,
                         const int64_t* row, void* cache, void* stream);

/* A1 from hidden states -- the cache rows of new tokens made from their
 * hidden states (irregular6612 notes, section 2.1.2, and DeepSeek-V3 report,
 * Metode 1: c^KV_t = W^DKV h_t, k^R_t = RoPE(W^KR h_t); review section 2: the
 * model normalises the compressed latent with an RMSNorm):
 *   x = W^DKV h_t (d_c), k = W^KR h_t (d_hR), fp32 sums;
 *   row[t] <- [ x / sqrt(mean(x^2) + eps) * norm_weight ; RoPE(k, pos[t]) ]
 * each half rounded once to the storage dtype (RoPE as mla_append_kv).
 *   h [n_tok][d_model], w_dkv [d_c][d_model], w_kr [d_hR][d_model] (row-major,
 *   one row per output), norm_weight [d_c] or NULL (weight 1; a model's extra
 *   latent scaling factor folds into it), eps >= 0 (1e-6 is the usual value),
 *   pos, row, cache: as mla_append_kv (rows must be distinct).
 *   workspace: at least mla_append_kv_from_hidden_workspace_bytes() (fp32
 *   partial sums; device).
 * n_tok in [0, 65535] (0 is a no-op); d_model in [1, 2^20].  The bf16 matrix-core
 * kernel needs d_model to be a multiple of 128; other shapes and MLA_F32 run
 * a generic fp32 kernel. */
size_t mla_append_kv_from_hidden_workspace_bytes(const mla_dims* dims, mla_dtype dtype,
                                                 int32_t n_tok, int32_t d_model);
mla_status mla_append_kv_from_hidden(const mla_dims* dims, mla_dtype dtype, int32_t n_tok,
                                     int32_t d_model, const void* h, const void* w_dkv,
                                     const void* w_kr, const void* norm_weight, double eps,
                                     const int32_t* pos, const int64_t* row, void* cache,
                                     void* workspace, size_t workspace_bytes, void* stream);

/* A2 -- absorbed query (review section 2: (U^K_i)^T q^C folded into the
 * query; section 3: per-head RoPE query).
 *   q_c [n_q][n_h][d_h], q_r [n_q][n_h][d_hR] (pre-RoPE), q_pos [n_q],
 *   w_uk [n_h][d_h][d_c] (U^K_i = w_uk[i], so k^C = U^K_i c)
 * Each absorbed query row v (d_c + d_hR values) is formed in fp32:
 *     v[0:d_c] = sum_d q_c[n][i][d] * w_uk[i][d][:]   (fp32 sum)
 *     v[d_c:]  = RoPE(q_r[n][i], q_pos[n])
 * and stored as one row per (query, head) in the storage dtype:
 *   q_lat    [n_q][n_h][d_c + d_hR]  v (MLA_F32), or hi = bf16(v) (MLA_BF16)
 *   q_lat_lo [n_q][n_h][d_c + d_hR]  optional, MLA_BF16 only (NULL otherwise):
 *            lo = bf16(v - hi); both rounded to nearest even, so hi + lo
 *            carries v to ~2^-17 relative.  NULL: lo is not written.
 * q_c, q_r and w_uk have the storage dtype.
 * Why a second plane: the matrix cores take bf16 operands, and a score from
 * the rounded query alone is off by a relative ~2^-9 per row; the attention
 * entry points below refine the score with lo wherever that would show (see
 * mla_precise_rows), and read nothing else of it. */
mla_status mla_absorb_q(const mla_dims* dims, mla_dtype dtype, int32_t n_q,
                        const void* q_c, const void* q_r, const int32_t* q_pos,
                        const void* w_uk, void* q_lat, void* q_lat_lo, void* stream);

/* A1 + A2 of one decode step in one call (the review's section 3: the step's
 * new token is cached as [c^KV ; RoPE(k^R)] and its query absorbed; the two
 * are independent, both precede the attention).  Exactly
 *     mla_append_kv(dims, dtype, n_tok, c_kv, k_r, pos, row, cache, stream);
 *     mla_absorb_q(dims, dtype, n_q, q_c, q_r, q_pos, w_uk, q_lat, q_lat_lo, stream);
 * with the same arguments, layouts, results (bit for bit) and errors, except
 * that n_tok = 0 or n_q = 0 skips that half only, and its pointers may then be
 * NULL.  Where the absorbed query has its bf16 matrix-core kernel (MLA_BF16,
 * d_c = 512, d_h = 128, d_hR = 64) both run in that kernel's one launch: its
 * workgroups also write the cache rows, whose loads overlap the W^UK stream;
 * otherwise the two calls' launches run in order.  The cache rows must not
 * overlap q_c, q_r, w_uk, q_lat or q_lat_lo. */
mla_status mla_append_absorb(const mla_dims* dims, mla_dtype dtype, int32_t n_tok,
                             const void* c_kv, const void* k_r, const int32_t* pos,
                             const int64_t* row, void* cache, int32_t n_q, const void* q_c,
                             const void* q_r, const int32_t* q_pos, const void* w_uk,
                             void* q_lat, void* q_lat_lo, void* stream);

/* The query path from hidden states into A2 (review section 2: queries pass
 * through a 1,536-wide latent; DeepSeek-V3 report, Metode 1: c^Q; the latent
 * normalised as c^KV is):
 *   c^Q = RMSNorm(W^DQ h) * norm_weight,  q^C = W^UQ c^Q,  q^R = W^QR c^Q,
 *   then q_lat = A2(q^C, q^R, q_pos, w_uk) exactly as mla_absorb_q.
 *   h [n_q][d_model], w_dq [d_cq][d_model], norm_weight [d_cq] or NULL,
 *   w_uq [n_h * d_h][d_cq] (head i = rows i*d_h ..), w_qr [n_h * d_hR][d_cq],
 *   all bf16; q_pos, w_uk, q_lat, q_lat_lo as mla_absorb_q (bf16).
 * c^Q and q^C pass between the launches as bf16 (fp32 sums, one rounding
 * each: they are matrix-core operands), q^R as fp32, in `workspace`
 * (mla_absorb_q_from_hidden_workspace_bytes).
 * n_q in [0, 65535] (0: no-op), d_cq <= 4096; the matrix-core kernels need
 * d_model and d_cq to be multiples of 128, other shapes run generic kernels.
 * W^UQ and W^UK are applied in turn, not composed: a composed per-head
 * [d_cq][d_c] matrix would hold three times the bytes of the two factors. */
size_t mla_absorb_q_from_hidden_workspace_bytes(const mla_dims* dims, int32_t n_q,
                                                int32_t d_model, int32_t d_cq);
mla_status mla_absorb_q_from_hidden(const mla_dims* dims, int32_t n_q, int32_t d_model,
                                    int32_t d_cq, const void* h, const void* w_dq,
                                    const void* norm_weight, double eps, const void* w_uq,
                                    const void* w_qr, const int32_t* q_pos, const void* w_uk,
                                    void* q_lat, void* q_lat_lo, void* workspace,
                                    size_t workspace_bytes, void* stream);

/* The output projection after A5 (review section 2: u_t = sum_i O_i U^V_i
 * sum_j a_ij c_j):  out[t] = W^O o_t, o [n_q][n_h][d_h] fp32 (A5's output),
 * w_o [d_model][n_h * d_h] bf16 (O_i = columns i*d_h ..), out [n_q][d_model]
 * fp32.  o is rounded once to bf16 for the matrix cores; the sums are fp32.
 * workspace: mla_output_projection_workspace_bytes().  n_q in [0, 65535].
 * W^O is applied after the lift, not folded into W^UV: O_i U^V_i would be a
 * [d_model][d_c] matrix per head, four times the bytes of the two factors. */
size_t mla_output_projection_workspace_bytes(const mla_dims* dims, int32_t n_q, int32_t d_model);
mla_status mla_output_projection(const mla_dims* dims, int32_t n_q, int32_t d_model,
                                 const float* o, const void* w_o, float* out, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* Split-KV plan.  Sequence rows [0, len) are cut into `num_splits` ranges of
 * mla_split_rows(max_seq_len, num_splits) rows each (split s covers
 * [s*R, min((s+1)*R, len)); trailing splits may be empty).
 * mla_decode_num_splits() is the split count mla_decode() uses. */
int32_t mla_decode_num_splits(const mla_dims* dims, mla_dtype dtype, int32_t batch,
                              int32_t max_seq_len);
int64_t mla_split_rows(int32_t max_seq_len, int32_t num_splits);

/* Precision of the bf16 attention (review section 3: l_ij and a_ij per head).
 * A query that attends fewer rows than mla_precise_rows() is scored with
 * hi + lo of its absorbed query and its softmax weights enter the value
 * product as a bf16 hi + lo pair: the result then matches the exact
 * attention of the stored values to ~1e-5 of the output rms.  Longer queries
 * (32 to 128 heads, plain RoPE) score with hi alone and round each weight to
 * bf16 once (a relative ~2^-9 on each score and weight, which averages out
 * over thousands of rows).  Returns 0 for MLA_F32 (exact fp32, no lo plane),
 * INT32_MAX where every query takes hi + lo (16 heads, n_h without a
 * matrix-core kernel, and yarn_factor > 1, whose temperature sharpens the
 * softmax so that single bf16 operands show at every length).  Callers pass
 * q_lat_lo to the calls below whenever some query attends fewer rows; without
 * it, lo reads as zero (the hi-only score). */
int32_t mla_precise_rows(const mla_dims* dims, mla_dtype dtype);

/* A3 -- split-KV latent attention.  For query n (one per sequence), split s
 * and head i, over rows j of split s (review section 3, softmax_j restricted
 * to a range of j and re-associated):
 *   lse_part[n][s][i]      = log sum_j exp(l_ij)                (natural log)
 *   z_part[n][s][i][0:d_c] = sum_j exp(l_ij - lse) * c_j        (fp32)
 * An empty split stores lse = -inf and z = 0.
 *   q_lat, q_lat_lo: the batch's absorbed queries (A2; q_lat_lo optional,
 *   bf16 only, read by the queries that mla_precise_rows() names).  The cache
 *   has the storage dtype.
 *   cache rows of sequence b start at row b * cache_seq_stride
 *   seq_lens [batch]: 1 <= len <= min(max_seq_len, cache_seq_stride)
 *   max_seq_len (host) bounds every len; it fixes the split rows.
 *   z_part [batch][num_splits][n_h][d_c], lse_part [batch][num_splits][n_h]
 * The query of sequence b attends to rows 0..len_b-1 (the new token's row is
 * appended first, so the query at position len_b-1 sees itself).
 * A device-side length outside [1, stride] is clamped for memory safety
 * (len < 1 behaves as an empty sequence: lse = -inf for every split). */
mla_status mla_decode_partials(const mla_dims* dims, mla_dtype dtype, int32_t batch,
                               const void* q_lat, const void* q_lat_lo, const void* cache,
                               int64_t cache_seq_stride, const int32_t* seq_lens,
                               int32_t max_seq_len, int32_t num_splits,
                               float* z_part, float* lse_part, void* stream);

/* A4 + A5 -- combine split partials and lift by W^UV (review section 2:
 * sum_j a_ij U^V_i c_j = U^V_i sum_j a_ij c_j).
 *   LSE = log sum_s exp(lse_s);  z = sum_s exp(lse_s - LSE) z_s
 *   out[n][i][:] = w_uv[i] @ z      (w_uv [n_h][d_h][d_c]; out fp32 [n_q][n_h][d_h])
 *   out_latent (optional, may be NULL): z, fp32 [n_q][n_h][d_c]
 * n_q queries, each with num_splits partials laid out as in A3.  A query
 * whose every split is empty (lse = -inf: a sequence of length 0) gets
 * z = 0 and out = 0. */
mla_status mla_combine_project(const mla_dims* dims, mla_dtype dtype, int32_t n_q,
                               int32_t num_splits, const float* z_part,
                               const float* lse_part, const void* w_uv, float* out,
                               float* out_latent, void* stream);

/* A3 + A4 + A5 in one call with the automatic split plan.  `workspace` holds
 * the partials; its size must be at least mla_decode_workspace_bytes(). */
size_t mla_decode_workspace_bytes(const mla_dims* dims, mla_dtype dtype, int32_t batch,
                                  int32_t max_seq_len);
mla_status mla_decode(const mla_dims* dims, mla_dtype dtype, int32_t batch,
                      const void* q_lat, const void* q_lat_lo, const void* cache,
                      int64_t cache_seq_stride,
                      const int32_t* seq_lens, int32_t max_seq_len, const void* w_uv,
                      float* out, float* out_latent, void* workspace,
                      size_t workspace_bytes, void* stream);

/* mla_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation, split plan and kernels as mla_decode, bitwise the same
 * output, with the split partials kept in a library-owned device array of
 * MLA_NOALLOC_SCRATCH_BYTES per GPU instead of a caller workspace.  The array
 * is reserved on every GPU the library runs on and held until the process
 * ends; nothing in it needs clearing (every split writes its own partials).
 * Calls that overlap on one GPU (concurrent streams, threads) share the array
 * and race: serialise them.  A batch whose partials
 * (mla_decode_workspace_bytes) exceed the array returns
 * MLA_ERR_WORKSPACE_TOO_SMALL before any launch; other errors as mla_decode.
 * Makes no hipMalloc / hipFree call. */
#define MLA_NOALLOC_SCRATCH_BYTES (128u << 20)
mla_status mla_decode_noalloc(const mla_dims* dims, mla_dtype dtype, int32_t batch,
                              const void* q_lat, const void* q_lat_lo, const void* cache,
                              int64_t cache_seq_stride, const int32_t* seq_lens,
                              int32_t max_seq_len, const void* w_uv, float* out,
                              float* out_latent, void* stream);

/* A6 -- causal prefill of a chunk of `chunk` new tokens per sequence.  Their
 * rows must already be in the cache (mla_append_kv).  Query i of sequence b
 * sits at position prefix_lens[b] + i and attends to rows 0..prefix_lens[b]+i
 * (inclusive causal mask), with the same score, softmax and W^UV lift as
 * decode (review section 3).
 *   q_lat, q_lat_lo: batch * chunk absorbed queries (A2; query index
 *   b * chunk + i; q_lat_lo as in mla_decode_partials), prefix_lens [batch] (device,
 *   0 <= prefix <= max_prefix_len), max_prefix_len (host) with
 *   max_prefix_len + chunk <= cache_seq_stride,
 *   out fp32 [batch][chunk][n_h][d_h]. */
size_t mla_prefill_workspace_bytes(const mla_dims* dims, mla_dtype dtype, int32_t batch,
                                   int32_t chunk, int32_t max_prefix_len);
mla_status mla_prefill(const mla_dims* dims, mla_dtype dtype, int32_t batch, int32_t chunk,
                       const void* q_lat, const void* q_lat_lo, const void* cache,
                       int64_t cache_seq_stride,
                       const int32_t* prefix_lens, int32_t max_prefix_len,
                       const void* w_uv, float* out, void* workspace,
                       size_t workspace_bytes, void* stream);

/* A6, unabsorbed form -- the causal prefill of mla_prefill computed from
 * per-head keys and values made explicit (review section 2: k^C_{j,i} =
 * U^K_i c_j, v^C_{j,i} = U^V_i c_j; section 3: k_{j,i} = [k^C_{j,i}; k^R_j],
 * l_ij = [q^C_i; RoPE(q^R_i)] . k_{j,i} / sqrt(d_h + d_hR),
 * o_i = sum_j softmax_j(l_ij) v^C_{j,i}).  Per (key, query, head) this is
 * 640 multiply-adds against the absorbed form's 1,088, at the price of one
 * pass that writes the explicit keys and values into the workspace.
 *   q_c [batch][chunk][n_h][d_h] and q_r [batch][chunk][n_h][d_hR] (before
 *   RoPE; query i of sequence b sits at position prefix_lens[b] + i and is
 *   rotated there), bf16.
 *   cache, cache_seq_stride, prefix_lens, max_prefix_len: as mla_prefill.
 *   w_uk, w_uv [n_h][d_h][d_c] bf16; out fp32 [batch][chunk][n_h][d_h].
 *   workspace: at least mla_prefill_unabsorbed_workspace_bytes() (device;
 *   batch * n_h * round_up(max_prefix_len + chunk, 128) rows of 1,152 B).
 * bf16 storage and n_h a multiple of 8 only (else MLA_ERR_UNSUPPORTED).
 * Precision: queries that see few keys (a workgroup of 256 queries whose
 * first one sees fewer than 2,048), and every query when yarn_factor > 1,
 * take every operand as a bf16 hi + lo pair; longer ones round k^C, v^C,
 * RoPE(q^R) and the softmax weights to bf16 once.
 * A device-side prefix outside [0, max_prefix_len] is clamped into it. */
size_t mla_prefill_unabsorbed_workspace_bytes(const mla_dims* dims, mla_dtype dtype,
                                              int32_t batch, int32_t chunk,
                                              int32_t max_prefix_len);
mla_status mla_prefill_unabsorbed(const mla_dims* dims, mla_dtype dtype, int32_t batch,
                                  int32_t chunk, const void* q_c, const void* q_r,
                                  const void* cache, int64_t cache_seq_stride,
                                  const int32_t* prefix_lens, int32_t max_prefix_len,
                                  const void* w_uk, const void* w_uv, float* out,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* Paged latent cache.  The pages serve the model through a dedicated vLLM
 * stack (axforge.ai DeepSeek-Lite page, section 3); what such a server needs
 * from the attention is a cache it can grow by fixed-size pages, so the
 * entry points below run the same computation as their contiguous
 * counterparts (review section 3) over this layout:
 *   pool [num_pages][page_rows][d_c + d_hR] in the storage dtype; row r of
 *   sequence b is row (r mod page_rows) of page block_table[b][r / page_rows];
 *   block_table [batch][max_pages] int32 (device).
 *   page_rows: a power of two in [32, 65536]; max_pages >= 1, num_pages >= 1.
 * Rows are written with mla_append_kv, whose `row` argument is then the pool
 * row page * page_rows + offset.  Only the table entries of pages that hold
 * attended rows are read.  An entry outside [0, num_pages) is never
 * dereferenced: its rows are not read, and the output of every query that
 * attends one of them is NaN (in the unabsorbed prefill, other queries of the
 * same sequence may be NaN too).
 * The partial sums follow the same split plan as the contiguous entry point
 * with the same batch and length bound, so a paged call returns bitwise the
 * output of the contiguous call on the same rows. */
typedef struct {
  const void* pool;
  const int32_t* block_table;
  int64_t num_pages;
  int32_t page_rows;
  int32_t max_pages;
} mla_paged_cache;

/* mla_decode_partials over a paged cache (max_seq_len <= max_pages *
 * page_rows); the split plan and the partials' layout are unchanged. */
mla_status mla_decode_partials_paged(const mla_dims* dims, mla_dtype dtype, int32_t batch,
                                     const void* q_lat, const void* q_lat_lo,
                                     const mla_paged_cache* cache,
                                     const int32_t* seq_lens, int32_t max_seq_len,
                                     int32_t num_splits, float* z_part, float* lse_part,
                                     void* stream);

/* mla_decode over a paged cache.  max_seq_len <= max_pages * page_rows takes
 * the place of cache_seq_stride; the workspace is mla_decode_workspace_bytes()
 * for the same dims, dtype, batch and max_seq_len. */
mla_status mla_decode_paged(const mla_dims* dims, mla_dtype dtype, int32_t batch,
                            const void* q_lat, const void* q_lat_lo,
                            const mla_paged_cache* cache,
                            const int32_t* seq_lens, int32_t max_seq_len,
                            const void* w_uv, float* out, float* out_latent,
                            void* workspace, size_t workspace_bytes, void* stream);

/* mla_prefill over a paged cache (max_prefix_len + chunk <= max_pages *
 * page_rows); the workspace is mla_prefill_workspace_bytes(). */
mla_status mla_prefill_paged(const mla_dims* dims, mla_dtype dtype, int32_t batch,
                             int32_t chunk, const void* q_lat, const void* q_lat_lo,
                             const mla_paged_cache* cache, const int32_t* prefix_lens,
                             int32_t max_prefix_len, const void* w_uv, float* out,
                             void* workspace, size_t workspace_bytes, void* stream);

/* mla_prefill_unabsorbed over a paged cache (bf16, n_h a multiple of 8;
 * max_prefix_len + chunk <= max_pages * page_rows); the workspace is
 * mla_prefill_unabsorbed_workspace_bytes(). */
mla_status mla_prefill_unabsorbed_paged(const mla_dims* dims, mla_dtype dtype, int32_t batch,
                                        int32_t chunk, const void* q_c, const void* q_r,
                                        const mla_paged_cache* cache,
                                        const int32_t* prefix_lens, int32_t max_prefix_len,
                                        const void* w_uk, const void* w_uv, float* out,
                                        void* workspace, size_t workspace_bytes,
                                        void* stream);

/* Quantised latent cache (the review's section 4 reports the served model's
 * cache at about 6 bits per element without giving a format; this is an 8-bit
 * one).  Row r holds
 *   codes[r][0:d_c]  uint8  FP8 E4M3 codes (OCP: 1 sign, 4 exponent bits of
 *                           bias 7, 3 mantissa bits; largest finite 448)
 *   rope[r][0:d_hR]  bf16   k^R after RoPE (as in the bf16 cache)
 *   scale[r]         float  per-row scale
 * and stands for the row [E4M3(codes) * scale ; rope]; the attention is that
 * of the bf16 entry points over these values.  Written by mla_append_kv_fp8:
 *   s = max_e |c^KV_e| / 448 (1 for a row of zeros), code_e = E4M3(c^KV_e / s)
 *   rounded to nearest even, both in fp32 with correctly rounded division.
 * 644 bytes per row against 1,152 for bf16.  Rows are indexed as in the
 * contiguous cache (sequence b at row b * cache_seq_stride). */
typedef struct {
  void* codes;
  void* rope;
  float* scale;
} mla_fp8_cache;

/* A1 into the FP8 cache: c_kv [n_tok][d_c] and k_r [n_tok][d_hR] (before RoPE)
 * in bf16, pos, row as mla_append_kv (rows distinct).  n_tok = 0 is a no-op. */
mla_status mla_append_kv_fp8(const mla_dims* dims, int32_t n_tok, const void* c_kv,
                             const void* k_r, const int32_t* pos, const int64_t* row,
                             const mla_fp8_cache* cache, void* stream);

/* A3 over the FP8 cache: as mla_decode_partials with bf16 absorbed queries
 * (q_lat, optional q_lat_lo, read as there) and the same split plan and
 * partials layout.  128 and 16 heads run matrix-core kernels, other head
 * counts a generic fp32 kernel. */
mla_status mla_decode_partials_fp8(const mla_dims* dims, int32_t batch, const void* q_lat,
                                   const void* q_lat_lo, const mla_fp8_cache* cache, int64_t cache_seq_stride,
                                   const int32_t* seq_lens, int32_t max_seq_len,
                                   int32_t num_splits, float* z_part, float* lse_part,
                                   void* stream);

/* A3 + A4 + A5 over the FP8 cache (w_uv bf16); the workspace is
 * mla_decode_workspace_bytes(dims, MLA_BF16, batch, max_seq_len). */
mla_status mla_decode_fp8(const mla_dims* dims, int32_t batch, const void* q_lat,
                          const void* q_lat_lo, const mla_fp8_cache* cache, int64_t cache_seq_stride,
                          const int32_t* seq_lens, int32_t max_seq_len, const void* w_uv,
                          float* out, float* out_latent, void* workspace,
                          size_t workspace_bytes, void* stream);

/* A6 over the FP8 cache: mla_prefill's causal chunk over rows
 * [E4M3(codes) * scale ; rope].  Query i of sequence b sits at position
 * prefix_lens[b] + i and attends rows 0..prefix_lens[b] + i, which must be
 * written (mla_append_kv_fp8) at rows b * cache_seq_stride + j.
 *   q_lat    bf16 absorbed queries [batch][chunk][n_h][d_c + d_hR] (A2), and
 *            q_lat_lo their optional lo plane (as mla_decode_partials)
 *   prefix_lens [batch] (device), each in [0, max_prefix_len]
 *   w_uv     bf16 [n_h][d_h][d_c];  out fp32 [batch][chunk][n_h][d_h]
 *   workspace at least mla_prefill_workspace_bytes(dims, MLA_BF16, batch,
 *            chunk, max_prefix_len) bytes (the split partials)
 * Errors: bf16 dims only (MLA_ERR_UNSUPPORTED otherwise), NULL pointers or
 * arrays in the descriptor, chunk < 1, max_prefix_len + chunk beyond
 * cache_seq_stride (MLA_ERR_INVALID_ARGUMENT), a short workspace
 * (MLA_ERR_WORKSPACE_TOO_SMALL). */
mla_status mla_prefill_fp8(const mla_dims* dims, int32_t batch, int32_t chunk, const void* q_lat,
                           const void* q_lat_lo, const mla_fp8_cache* cache, int64_t cache_seq_stride,
                           const int32_t* prefix_lens, int32_t max_prefix_len, const void* w_uv,
                           float* out, void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MLA_H */
