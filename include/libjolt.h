/*
 * libjolt -- JoLT per-layer-group KV-cache compressor for MI355X (gfx950).
 *
 * What it computes ("A JoLT for the KV cache", Krishnan & Schulz; paper landing
 * page, abstract; author page, abstract):
 *   - a grouped prefill cache item X[L][H][T][d] (one layer group's K or V) is
 *     factored by a partial Tucker decomposition along the token and feature
 *     modes only; heads and layers stay intact, so the core is per (layer, head);
 *   - the token factor comes from an exact eigensolve of A A^T (A = token
 *     unfolding, "exact token-mode SVD") or from the FlashJoLT randomized range
 *     finder; the feature factor from the d x d feature Gram;
 *   - the truncation residual is rotated by a seeded randomized Hadamard (JL)
 *     transform and quantized to b bits per element with one bf16 scale per 64;
 *   - one Lagrangian dual picks (token rank, feature rank, bits) for every item,
 *     K and V separately, under one global byte budget;
 *   - decompression rebuilds the dense cache.
 *
 * Conventions (all entry points):
 *   - Device pointers are caller-owned device memory; host pointers are
 *     caller-owned host memory.  libjolt never allocates device memory; the
 *     workspace sizes come from jolt_workspace_size() (jolt_eigh_workspace_size
 *     for jolt_eigh).  A handle holds one small pinned host buffer (at least
 *     64 KiB, grown as the plan's readback needs) from its first plan on.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls are
 *     stream-ordered and asynchronous, except jolt_plan(), which synchronises
 *     `stream` once to read the energy tables back.  Two cases add
 *     synchronisations: exact token mode with T > 272, whose T x T
 *     eigenproblem runs block Jacobi with one convergence readback per sweep,
 *     and a sketch whose order 141..272 eigenproblem has numerically repeated
 *     eigenvalues, whose group of up to 16 items is then planned again with
 *     block Jacobi before a second readback.  jolt_plan() also forks
 *     the feature Gram onto a second stream owned by the handle (created on
 *     the first plan, default priority) and joins it back to `stream` before
 *     the work that reads it; everything it launched has finished when it
 *     returns.
 *   - Arguments are validated before any launch; an error leaves no partial
 *     work.  Device errors return JOLT_E_DEVICE with the HIP message in
 *     jolt_last_error().  No C++ exception crosses this interface.
 *   - A handle is used by one host thread at a time.
 *   - Tensors are dense row-major with the last index fastest.
 */
#ifndef LIBJOLT_H
#define LIBJOLT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    JOLT_OK = 0,
    JOLT_E_INVALID = 1,      /* bad argument, shape or config                     */
    JOLT_E_UNSUPPORTED = 2,  /* valid but not supported (e.g. d not 64 or 128)   */
    JOLT_E_WORKSPACE = 3,    /* workspace smaller than jolt_workspace_size()      */
    JOLT_E_INFEASIBLE = 4,   /* budget below the sum of minimum item bytes        */
    JOLT_E_NOCONV = 5,       /* an eigensolver hit its sweep cap (results written) */
    JOLT_E_DEVICE = 6,       /* HIP runtime error                                  */
    JOLT_E_CORRUPT = 7       /* payload header does not match item / allocation  */
} jolt_status;

typedef enum { JOLT_BF16 = 0, JOLT_F32 = 1 } jolt_dtype;
typedef enum { JOLT_TOKEN_EXACT = 0, JOLT_TOKEN_RANDOMIZED = 1 } jolt_token_mode;

/* One item = one layer group's K (or V) cache of one sequence, X[L][H][T][d].
 * d must be 64 or 128.  `dtype` is the dtype of X, of the stored Tucker
 * parameters and of the decompressed output.  (seed, item_id) select the
 * item's rotation signs and sketch matrix; item_id should be unique. */
typedef struct {
    int32_t L, H, T, d;
    int32_t dtype;
    uint32_t item_id;
    uint64_t seed;
} jolt_item;

/* Compressor settings (one per call, shared by all items).
 *   mode          exact eigensolve of A A^T or FlashJoLT randomized range finder
 *   oversample    p: sketch width k = rt_max + p (randomized mode)
 *   power_iters   q: subspace iterations (randomized mode)
 *   rank_step     candidate ranks are multiples of rank_step (8)
 *   rt_max        largest token rank considered (<= T; <= 256)
 *   rf_max        largest feature rank considered, 0 = d
 *   bits_mask     bit b set = residual width b allowed; b in {0, 2..8};
 *                 {0,2,3,4} = 0x1D
 *   group_size    quantization group, must be 64
 *   budget_bytes  global byte budget over all items; < 0 = fixed ranks below
 *   fixed_*       (r_t, r_f, b) for every item when budget_bytes < 0
 *   max_sweeps    eigensolver sweep cap, 0 = default (30)
 *   delta_b[b]    distortion model: relative MSE of the b-bit residual
 *                 quantizer; delta_b[0] must be 1 (caller supplied)          */
typedef struct {
    int32_t mode;
    int32_t oversample;
    int32_t power_iters;
    int32_t rank_step;
    int32_t rt_max;
    int32_t rf_max;
    uint32_t bits_mask;
    int32_t group_size;
    int64_t budget_bytes;
    int32_t fixed_rt, fixed_rf, fixed_bits;
    int32_t max_sweeps;
    double delta_b[9];
} jolt_config;

/* Allocation of one item: ranks, residual bits, accounted bytes
 * e (T r_t + d r_f + L H r_t r_f) + [b > 0] (N b / 8 + 2 N / 64) with
 * e = 2 (bf16) or 4 (fp32) and N = L H T d, and the modelled distortion
 * delta_b * max(0, ||X||^2 - captured energy). */
typedef struct {
    int32_t rt, rf, bits, reserved;
    int64_t bytes;
    double distortion;
} jolt_alloc;

typedef struct jolt_handle_s *jolt_handle;

/* ---- lifetime and errors ------------------------------------------------- */
/* Binds the calling thread's HIP device `hip_device`; no device memory is taken.
 * jolt_destroy() waits for and releases the handle's second stream and its
 * pinned readback buffer, if any. */
jolt_status jolt_create(int hip_device, jolt_handle *out);
void jolt_destroy(jolt_handle h);
const char *jolt_status_str(jolt_status s);
/* Message of the last failing call on `h` (empty string if none). */
const char *jolt_last_error(jolt_handle h);

/* ---- sizes (pure host) --------------------------------------------------- */
/* Device workspace bytes for jolt_plan (plan_ws) and for jolt_compress /
 * jolt_decompress (codec_ws), for this config and item list. */
jolt_status jolt_workspace_size(const jolt_config *cfg, const jolt_item *items, int32_t n,
                                size_t *plan_ws_bytes, size_t *codec_ws_bytes);
/* Accounted bytes of one item at (rt, rf, bits) -- the formula above. */
int64_t jolt_item_bytes(const jolt_item *item, int32_t rt, int32_t rf, int32_t bits);
/* Payload buffer bytes for one item: 256-B aligned sections
 * [header 64 B | U_t T x r_t | U_f d x r_f | core L H r_t r_f | scales N/64 bf16 |
 *  codes N b / 8], parameter sections in the item dtype. */
jolt_status jolt_payload_size(const jolt_item *item, const jolt_alloc *a, size_t *bytes);
/* Byte offsets of the five sections (ut, uf, core, scales, codes) and the total. */
jolt_status jolt_payload_layout(const jolt_item *item, const jolt_alloc *a, size_t offsets[5],
                                size_t *total);
/* Fill a 64-byte header (host memory) for (item, alloc). */
jolt_status jolt_payload_header(const jolt_item *item, const jolt_alloc *a, void *header64);
/* Check a header copy (host memory) against (item, alloc): JOLT_E_CORRUPT if
 * the magic, version, shape, ranks, bits, seed or checksum disagree. */
jolt_status jolt_payload_validate(const void *header64, const jolt_item *item, const jolt_alloc *a);

/* ---- the three calls ----------------------------------------------------- */
/* Factor every item and allocate.  The method factors a grouped prefill cache
 * by a partial Tucker decomposition along the token and feature modes, the
 * token factor by an exact SVD or by FlashJoLT's randomized approximation, and
 * picks Tucker ranks and residual bits with a single Lagrangian dual per layer
 * group, K and V separately, under one global byte budget ("A JoLT for the KV
 * cache", paper landing page, abstract; author page, abstract).  Here: feature
 * Gram + eigensolve; exact or randomized token factor; core and energy table;
 * one synchronisation; the distortion and byte tables and the single-dual
 * allocation (the breakpoints of lambda).  x_dev[i] points to item i's X.  On return
 * alloc_host[i] holds item i's allocation and *lambda_out the dual (0 when the
 * unconstrained optimum fits, -1 in fixed-rank mode).  The factors stay in
 * plan_ws for jolt_compress.  JOLT_E_INFEASIBLE: alloc_host holds the
 * minimum-byte choices. */
jolt_status jolt_plan(jolt_handle h, const jolt_config *cfg, const jolt_item *items, int32_t n,
                      const void *const *x_dev, void *plan_ws, size_t plan_ws_bytes,
                      void *stream, jolt_alloc *alloc_host, double *lambda_out);

/* The allocation alone, under a new budget: reads back the energy tables that
 * jolt_plan left in plan_ws for the same items (one device-to-host copy;
 * synchronises `stream` once) and runs the single dual again.  The method
 * picks ranks and residual bits per item under one byte budget from per-item
 * distortion tables ("A JoLT for the KV cache", landing page abstract), so a
 * new budget needs no new factorization.  cfg must be the configuration
 * jolt_plan ran with, except budget_bytes (>= 0 here) and delta_b; the
 * factors in plan_ws stay valid for jolt_compress with the new allocation.
 * Errors as jolt_plan (JOLT_E_INFEASIBLE: alloc_host holds the minimum-byte
 * choices; JOLT_E_NOCONV: the plan's eigensolver status). */
jolt_status jolt_replan(jolt_handle h, const jolt_config *cfg, const jolt_item *items, int32_t n,
                        const void *plan_ws, size_t plan_ws_bytes, void *stream, jolt_alloc *alloc_host,
                        double *lambda_out);

/* Write each item's payload: header, stored Tucker parameters (rounded to the
 * item dtype) and the quantized rotated residual against the reconstruction
 * the decoder will form from those stored parameters.  The method captures
 * the truncation residual with a rotated low-bit quantizer, the rotation a
 * Johnson-Lindenstrauss one (paper landing page, abstract; author page,
 * abstract).  plan_ws must hold the
 * jolt_plan results for the same (cfg, items).  payload_dev[i] must have
 * jolt_payload_size() bytes. */
jolt_status jolt_compress(jolt_handle h, const jolt_config *cfg, const jolt_item *items, int32_t n,
                          const void *const *x_dev, const jolt_alloc *alloc, const void *plan_ws,
                          size_t plan_ws_bytes, void *codec_ws, size_t codec_ws_bytes,
                          void *const *payload_dev, void *stream);

/* The residual half of jolt_compress alone: payload_dev[i] already holds the
 * header and the stored parameters (written by the caller, or by an earlier
 * jolt_compress); computes and writes the scales and codes. */
jolt_status jolt_encode_residual(jolt_handle h, const jolt_item *items, int32_t n,
                                 const void *const *x_dev, const jolt_alloc *alloc,
                                 void *codec_ws, size_t codec_ws_bytes, void *const *payload_dev,
                                 void *stream);

/* Rebuild every item's dense X~ = U_t (C U_f^T) + rotate^T(dequant(codes))
 * into out_dev[i] (item dtype, [L][H][T][d]); the method's errors are those of
 * this reconstruction (author page, abstract: relative Frobenius error).
 * C U_f^T is held as a bf16 hi + lo pair (about 2^-16 relative) for bf16
 * items, in fp32 for fp32 items.  Reads only the payloads; the
 * device header is not read (validate a host copy with jolt_payload_validate). */
jolt_status jolt_decompress(jolt_handle h, const jolt_item *items, int32_t n, const jolt_alloc *alloc,
                            const void *const *payload_dev, void *codec_ws, size_t codec_ws_bytes,
                            void *const *out_dev, void *stream);

/* jolt_decompress without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The W~ workspace is a fixed scratch
 * array of 64 MiB that the library holds on every GPU it runs on until the
 * process ends; this call allocates nothing.  The items of one call may need
 * at most 64 MiB of it (L H d r_t' 4 bytes per item, r_t' = r_t rounded up to
 * 16; 4 MiB for a 4 x 8 x T x 128 item at r_t = 256), else JOLT_E_WORKSPACE
 * before any launch.  Every call on one GPU uses the same array: calls that
 * overlap on one GPU (different streams, or different host threads) race.
 * Nothing in the array needs to start zeroed (each call writes all of what it
 * reads).  Results are those of jolt_decompress. */
jolt_status jolt_decompress_noalloc(jolt_handle h, const jolt_item *items, int32_t n, const jolt_alloc *alloc,
                                    const void *const *payload_dev, void *const *out_dev, void *stream);

/* ---- decode attention over the stored factors --------------------------- */
/* The method's decode kernel evaluates attention directly over the stored
 * factors, without materializing dense K and V ("A JoLT for the KV cache",
 * paper landing page, abstract).  For one decode step, every query head j of
 * layer l (q_heads per layer, grouped-query: KV head j / (q_heads / H))
 * attends to the cached tokens of its layer group:
 *   out = sum_t p_t v_t,  p = softmax(scale * q . k_t),  lse = log sum_t exp(scale * q . k_t)
 * where k_t, v_t are the rows the K and V payloads represent (Tucker part plus
 * rotated residual, unrounded).  Scores come from U_t and the K codes with a
 * per-head z = scale C (U_f^T q) and rotated query; values are summed in the
 * factor and rotated domains and mapped to features once per head.  lse lets
 * a caller merge attention over tokens kept outside the payloads.
 *   k_item / v_item   the group's K and V items (same L, H, T, d, dtype)
 *   k_alloc / v_alloc their allocations; k_payload / v_payload (device)
 *   q    device fp32 [L][q_heads][d];  out device fp32 [L][q_heads][d];
 *   lse  device fp32 [L][q_heads]
 * All groups of a call share dtype, d and H; q_heads / H must be 1, 2, 4 or
 * 8; workspace (device) of jolt_attention_workspace_size() bytes. */
typedef struct {
    jolt_item k_item, v_item;
    jolt_alloc k_alloc, v_alloc;
    const void *k_payload, *v_payload;
    const float *q;
    float *out;
    float *lse;
} jolt_attn_group;
jolt_status jolt_attention_workspace_size(const jolt_attn_group *groups, int32_t n, int32_t q_heads, size_t *bytes);
jolt_status jolt_decode_attention(jolt_handle h, const jolt_attn_group *groups, int32_t n, int32_t q_heads,
                                  float scale, void *workspace, size_t workspace_bytes, void *stream);

/* ---- factor export (device pointers into plan_ws) ------------------------ */
/* After jolt_plan: where item i's factors live in plan_ws (fp32, device):
 *   ut    rt_max x T   row r = token-factor column r (descending eigenvalue)
 *   uf    d x d        feature factor, row-major, column j = eigenvector j
 *   lam_t rt_max, lam_f d   eigenvalues (Ritz values in randomized mode)
 *   core  L H x rt_max x d   full core C = U_t^T X U_f per (layer, head)
 *   energy rt_max x d       E[i][j] = sum over (l,h) of core^2
 *   normx2 (double, 1)      ||X||^2                                          */
typedef struct {
    const float *ut, *uf, *lam_t, *lam_f, *core, *energy;
    const double *normx2;
    int32_t rt_max, rf_max;
} jolt_factor_view;
jolt_status jolt_plan_factors(const jolt_config *cfg, const jolt_item *items, int32_t n,
                              const void *plan_ws, int32_t i, jolt_factor_view *out);

/* ---- test hooks (exported and documented as such) ----------------------- */
/* The allocation alone from given tables (pure host, no device):
 * n_cand[i] candidates for item i, cand[i] = (rt, rf, bits) triples, D[i] the
 * distortions, B[i] the byte counts.  Same rule as jolt_plan: per item the
 * argmin of D + lambda B (ties: fewer bytes, then smaller rt, rf, bits), and
 * lambda* the least lambda >= 0 whose total bytes fit the budget. */
jolt_status jolt_plan_from_tables(int32_t n, const int32_t *n_cand, const int32_t *const *cand,
                                  const double *const *D, const int64_t *const *B, int64_t budget,
                                  jolt_alloc *out, double *lambda_out);
/* Randomized Hadamard rotation of fp32 rows (device): out = (1/sqrt d) H (s o in)
 * or, with inverse != 0, out = s o ((1/sqrt d) H in). */
jolt_status jolt_rotate(jolt_handle h, const float *in, float *out, int64_t rows, int32_t d,
                        uint64_t seed, uint32_t item_id, int32_t inverse, void *stream);
/* Quantize and pack fp32 rotated rows (device; rows x d, d = 64 or 128):
 * codes = (rows d / 64) groups x bits uint64 words, scales = bf16 per group.
 * Runs the fused encoder's own quantize / pack / store code on rows read from
 * memory, so its output is the encoder's for the same rotated residual. */
jolt_status jolt_quantize_pack(jolt_handle h, const float *rot, int64_t rows, int32_t d, int32_t bits,
                               uint64_t *codes, uint16_t *scales, void *stream);
/* Inverse of jolt_quantize_pack: q * scale per element (fp32, device), with
 * the fused decoder's own code loading and unpacking. */
jolt_status jolt_unpack_dequant(jolt_handle h, const uint64_t *codes, const uint16_t *scales,
                                int64_t rows, int32_t d, int32_t bits, float *out, void *stream);
/* +-1 values of the counter stream (device, fp32): out[i] for counters
 * first..first+count-1 of stream `stream_id` (0 = rotation signs,
 * 1 = sketch matrix). */
jolt_status jolt_rademacher(jolt_handle h, uint64_t seed, uint32_t item_id, uint32_t stream_id,
                            uint64_t first, int64_t count, float *out, void *stream);

/* The plan's symmetric eigensolver on caller matrices (device).  count
 * matrices of order n <= 272: matrix i starts at a + i * mat_stride, row
 * stride lda, and only its symmetric part (A + A^T) / 2 is used.  Matrix i's
 * eigenvalues go to lam + i n in descending order and its eigenvectors to the
 * columns of vec + i n n (row stride n), each column's entry of largest
 * magnitude (first such row) positive.  info (count int32, device) receives
 * 0 when the Householder-tridiagonal solver produced the result, the sweep
 * count when the Jacobi solver did (force_jacobi != 0, for n <= 142, or
 * numerically repeated eigenvalues at n <= 140), -1 when Jacobi
 * hit its sweep cap, -3 when, for n > 140, the tridiagonal solver could not
 * make the eigenvectors orthonormal (results written as they stand).
 * workspace (device, 16-byte aligned) of at least
 * jolt_eigh_workspace_size(n, count, force_jacobi) bytes carries the
 * tridiagonal solver's intermediates from launch to launch; calls that
 * overlap on one workspace race. */
jolt_status jolt_eigh(jolt_handle h, int32_t n, int32_t count, const float *a, int32_t lda, int64_t mat_stride,
                      float *vec, float *lam, int32_t *info, int32_t force_jacobi, void *workspace,
                      size_t workspace_bytes, void *stream);
/* Bytes of workspace that jolt_eigh needs for these arguments (0 when the
 * Jacobi solver does all of it). */
size_t jolt_eigh_workspace_size(int32_t n, int32_t count, int32_t force_jacobi);

/* ---- measurement hooks -------------------------------------------------- */
/* Launch timing of one of the library's kernels, named as in its source
 * ("k_decode", "k_encode", "k_xm", "k_xtq", "k_eig_tridiag", "k_eig_trivec",
 * "k_eig_backtr", "k_eig_polish", "k_chol_inv",
 * "k_apply_linv", "k_gemm", "k_gram_rows", "k_reduce", "k_build_wt",
 * "k_jacobi_lds").  While a kernel's timer is on, each of its launches is
 * bracketed by a HIP event pair on its launch stream.  enable != 0 turns the
 * timer on and resets it; enable == 0 turns it off (the totals are kept).
 * Process-wide; h is used for error reporting only. */
jolt_status jolt_kernel_timer(jolt_handle h, const char *kernel, int32_t enable);
/* Total device time (ms) and number of timed launches of a kernel since its
 * timer was last turned on.  Waits for the recorded events. */
jolt_status jolt_kernel_time(jolt_handle h, const char *kernel, double *total_ms, int64_t *launches);

#ifdef __cplusplus
}
#endif
#endif /* LIBJOLT_H */
