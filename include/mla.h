/*
 * mla.h -- C ABI of libmla: Multi-head Latent Attention (MLA) for a block of
 * L query rows (a speculative-decoding verify step) against a long
 * compressed latent KV cache, on AMD Instinct MI355X (gfx950).
 *
 * Method (pages: "One guard, 110x off the verify step", sections "The
 * defect", "The threshold is not a constant" and "The change"; mlx-lm PR
 * #1817 "fix: Speed up multi-token decode by computing the absorbed MLA
 * threshold", opening paragraphs).  MLA caches per token t a latent c_kv[t]
 * of width r (kv_lora_rank) and a rope key k_pe[t] of width `rope` shared by
 * every head.  Attention of the L new rows can be taken two ways that agree
 * up to rounding:
 *   absorbed      fold W_UK into the query (mla_fold_query), score against
 *                 the latent plus the rope key, softmax, accumulate in latent
 *                 space, up-project through W_UV (mla_absorbed_attention);
 *                 cost grows with the number of new rows;
 *   materialised  expand the cache into per-head K and V
 *                 (mla_materialize_kv), then ordinary attention
 *                 (mla_materialized_attention); cost grows with the cache.
 * mla_select_path picks between them with the integer query-count threshold.
 *
 * Symbols: r = kv_lora_rank, n = qk_nope_head_dim, v = v_head_dim,
 * rope = rope width, H = heads, B = sequences, L = query rows per sequence,
 * Kv_b = positions sequence b attends over (its L new rows included).
 *
 * Conventions for every entry point:
 *   - All functions are extern "C", never throw, and return an int status:
 *     MLA_OK or a negative MLA_E_* code.  mla_status_string() names it.
 *   - Arguments are validated on the host before anything is enqueued; on
 *     any error nothing is launched and output buffers are untouched.
 *   - The caller owns every buffer.  The library never allocates, frees,
 *     copies between host and device, or synchronises.  Device pointers
 *     must stay valid until the work enqueued on `stream` has finished.
 *   - `stream` is a hipStream_t (NULL = the default stream); all launches
 *     are asynchronous on it.  Calls that share a workspace must not run
 *     concurrently.
 *   - All tensors are dense, row-major and contiguous.  Element type is
 *     given by mla_dtype: MLA_BF16 = bfloat16 storage, MLA_F32 = float.
 *     Outputs of the attention entry points are always float32.
 *   - Causal rule of a verify block: the L new rows of sequence b are its
 *     last L positions, so row i (0-based) sees the first Kv_b - L + i + 1
 *     positions of the sequence.  Kv_b >= L is required.
 *   - Packed variable-length caches: sequence b owns cache positions
 *     kv_offsets[b] .. kv_offsets[b+1]-1 of c_kv / k_pe (or of K / V).
 *     Offsets are int32, non-decreasing, kv_offsets[0] >= 0.  The same
 *     offsets are passed twice: a host copy (validation and launch
 *     planning) and a device copy (read by the kernels); they must hold the
 *     same values.
 *   - Supported geometry is listed per entry point; anything else returns
 *     MLA_E_UNSUPPORTED.
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Head geometry of one MLA attention layer. */
typedef struct mla_geom {
  int32_t r;     /* kv_lora_rank: width of the latent c_kv                 */
  int32_t n;     /* qk_nope_head_dim: per-head query/key width without rope */
  int32_t v;     /* v_head_dim: per-head value width                        */
  int32_t rope;  /* width of q_pe and of the shared rope key k_pe (may be 0) */
  int32_t heads; /* H: query heads                                           */
} mla_geom;

typedef enum mla_dtype { MLA_F32 = 0, MLA_BF16 = 1 } mla_dtype;
typedef enum mla_path { MLA_ABSORBED = 0, MLA_MATERIALIZED = 1 } mla_path;

enum {
  MLA_OK = 0,
  MLA_E_NULL = -1,        /* a required pointer is NULL                       */
  MLA_E_SHAPE = -2,       /* a size or offset is out of range / inconsistent */
  MLA_E_UNSUPPORTED = -3, /* geometry or dtype not compiled in               */
  MLA_E_WORKSPACE = -4,   /* workspace missing or too small                  */
  MLA_E_HIP = -5          /* a HIP launch or runtime call failed             */
};

/* Static text for a status code ("ok", "null pointer", ...). */
const char* mla_status_string(int status);

/* Library ABI version (this header: 1). */
int mla_version(void);

/*
 * mla_select_path -- choose the absorbed or the materialised path for a
 * block of L query rows attending over T cached positions (host only, no
 * device call, integer arithmetic, exact).
 *
 * Defined by the query-count threshold of "One guard, 110x off the verify
 * step", sections "The threshold is not a constant" (cost model) and "The
 * change" (helper and guard), and the finite-cache form of mlx-lm PR #1817
 * (opening paragraphs).  With d = n + v:
 *   if 2r - d <= 0:   max_absorbed = 1
 *   elif T == 0:      max_absorbed = max(1, floor(r d / (2r - d)))            (long-cache limit)
 *   else:             max_absorbed = max(1, floor(T r d / (r d + T (2r - d)))) (cache of T)
 * The path is MLA_ABSORBED iff L <= max_absorbed (ties go to absorbed, as
 * the guard is `L <= max_absorbed`).  T counts the block's own L rows;
 * T == 0 asks for the limit form.  Products are formed in 128-bit integers,
 * so the result is exact for every non-negative int32 geometry and int64 T.
 *
 * Arguments: g (host pointer; r >= 1, n >= 0, v >= 0), L >= 1, T >= 0
 * (T >= L when T > 0).  path_out receives an mla_path value; max_absorbed_out
 * may be NULL.  Errors: MLA_E_NULL (g or path_out NULL), MLA_E_SHAPE.
 */
int mla_select_path(const mla_geom* g, int64_t L, int64_t T, int32_t* path_out,
                    int64_t* max_absorbed_out);

/*
 * mla_draft_cap -- the draft cap a speculative decoder derives from a measured
 * verify-cost curve ("Draft caps and calibration", sections "Play with it"
 * and "How mlx-dspark picks it").  For caps C = 1 .. n_widths - 1:
 *   speedup(C) = (1 + p + p^2 + ... + p^C) / (drafter + verify_cost[C] / verify_cost[0])
 *   verify_cost[w - 1]  measured cost of one verify pass over w rows, any unit
 *                       (dividing by the one-row cost gives single-token steps)
 *   p                   probability that each drafted token survives, in [0, 1]
 *   drafter             the drafter's cost per round, in single-token steps (>= 0)
 * Writes the cap with the largest speedup (ties: the smaller cap) and its
 * speedup, or cap 0 with speedup 1 when no cap beats plain decoding.  If
 * speedup_by_cap is not null it receives n_widths values: 1 for C = 0 (no
 * drafting), then speedup(C).  Host only; every pointer is host memory owned by
 * the caller.  Returns MLA_E_NULL if verify_cost, cap_out or speedup_out is
 * null; MLA_E_SHAPE if n_widths < 1, p is outside [0, 1], drafter is negative or
 * not finite, or a cost is not finite and positive.
 */
int mla_draft_cap(const double* verify_cost, int32_t n_widths, double p, double drafter,
                  int32_t* cap_out, double* speedup_out, double* speedup_by_cap);

/*
 * mla_fold_query -- fold the key up-projection into the query ("One
 * guard...", section "The defect": the absorbed path folds the
 * up-projection into the query):
 *   q_lat[m, h, c] = sum_j q_nope[m, h, j] * w_uk[h, j, c]
 * for m < rows (rows = B*L), h < H, c < r.
 *
 *   q_nope  device, [rows, H, n], dtype dt
 *   w_uk    device, [H, n, r],   dtype dt
 *   q_lat   device, [rows, H, r], dtype dt (bf16: accumulated in float32,
 *           rounded to nearest-even once)
 * Supported: n % 32 == 0, n <= 512, r % 64 == 0 (bf16); any n, r >= 1 (f32).
 */
int mla_fold_query(const mla_geom* g, mla_dtype dt, int64_t rows, const void* q_nope,
                   const void* w_uk, void* q_lat, void* stream);

/*
 * mla_absorbed_workspace_size -- bytes of device workspace that
 * mla_absorbed_attention needs for these sizes (the split-KV partial
 * results).  kv_offsets_host: host, [B+1].  Same validation as the
 * attention call.
 */
int mla_absorbed_workspace_size(const mla_geom* g, mla_dtype dt, int32_t B, int32_t L,
                                const int32_t* kv_offsets_host, size_t* bytes_out);

/*
 * mla_absorbed_attention -- the absorbed path after the fold ("One
 * guard...", section "The defect": attend directly against the compressed
 * latent, then up-project).  For sequence b, row i, head h, with
 * vis = Kv_b - L + i + 1 and t running over the sequence's first vis
 * positions:
 *   s_t        = scale * (q_lat[b,i,h,:] . c_kv[t,:] + q_pe[b,i,h,:] . k_pe[t,:])
 *   o_lat      = sum_t softmax(s)_t * c_kv[t,:]
 *   out[b,i,h,:] = o_lat . w_uv[h]
 * Each latent tile is read once for all L*H (row, head) pairs of a
 * sequence; positions are split across compute units and the splits are
 * merged with a log-sum-exp combine that also applies w_uv.
 *
 *   q_lat   device, [B, L, H, r], dtype dt
 *   q_pe    device, [B, L, H, rope], dtype dt (NULL allowed when rope == 0)
 *   c_kv    device, [sum Kv, r], dtype dt
 *   k_pe    device, [sum Kv, rope], dtype dt (NULL allowed when rope == 0)
 *   kv_offsets_host / kv_offsets_dev   [B+1] int32 (see conventions)
 *   w_uv    device, [H, r, v], dtype dt
 *   scale   softmax scale (usually 1/sqrt(n + rope))
 *   out     device, [B, L, H, v], float32
 *   workspace / workspace_bytes   device scratch of at least
 *           mla_absorbed_workspace_size() bytes, 256-byte aligned
 * Supported (bf16): r == 512, rope in {0, 64}, v % 64 == 0.
 * Supported (f32): r <= 1024, r + rope <= 1152, v <= 1024.
 * The result is deterministic: no floating-point atomics are used.
 */
int mla_absorbed_attention(const mla_geom* g, mla_dtype dt, int32_t B, int32_t L,
                           const void* q_lat, const void* q_pe, const void* c_kv,
                           const void* k_pe, const int32_t* kv_offsets_host,
                           const int32_t* kv_offsets_dev, const void* w_uv, float scale,
                           float* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * mla_absorbed_attention_noalloc -- mla_absorbed_attention for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the same arguments without the
 * workspace, the same kernels and the same result bits.  The split-KV partial
 * results go to a static device array of MLA_NOALLOC_SCRATCH_BYTES (32 MiB)
 * that the library holds on every GPU it runs on until the process ends; its
 * address is looked up on the first call on a device.  Nothing is allocated,
 * freed or copied, and no library routine that allocates is called.
 * Calls that would need more partial-result space than the array holds (the
 * size mla_absorbed_workspace_size reports) return MLA_E_WORKSPACE before
 * anything is enqueued: one-sequence verify steps fit (the 128-head, 8-row
 * step over 8192 positions needs about 16 MiB); large batches may not.
 * Every call on a GPU shares that GPU's array: calls that overlap on one GPU
 * (other streams, other host threads) race and must be serialised by the
 * caller.  Nothing in the array needs to start at zero; it keeps the last
 * call's contents.  Other errors as for mla_absorbed_attention, plus MLA_E_HIP
 * if the array's address cannot be looked up.
 */
#define MLA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int mla_absorbed_attention_noalloc(const mla_geom* g, mla_dtype dt, int32_t B, int32_t L,
                                   const void* q_lat, const void* q_pe, const void* c_kv,
                                   const void* k_pe, const int32_t* kv_offsets_host,
                                   const int32_t* kv_offsets_dev, const void* w_uv, float scale,
                                   float* out, void* stream);

/*
 * mla_absorbed_splits / mla_absorbed_merge -- the two launches that make up
 * mla_absorbed_attention, exposed separately so that each kernel can be
 * timed or overlapped on its own.  mla_absorbed_splits runs the split-KV
 * pass (scores, online softmax and the latent accumulation for every split
 * of every sequence) and leaves unnormalised partial results in the
 * workspace; mla_absorbed_merge combines the splits with a log-sum-exp
 * weighting and applies w_uv, writing out.  Calling splits then merge on
 * one stream with the same arguments and workspace equals
 * mla_absorbed_attention.  Arguments as for mla_absorbed_attention (merge
 * reads only the offsets, w_uv, out and the workspace; the other tensor
 * pointers are not used by it and may be NULL).
 */
int mla_absorbed_splits(const mla_geom* g, mla_dtype dt, int32_t B, int32_t L, const void* q_lat,
                        const void* q_pe, const void* c_kv, const void* k_pe,
                        const int32_t* kv_offsets_host, const int32_t* kv_offsets_dev, float scale,
                        void* workspace, size_t workspace_bytes, void* stream);
int mla_absorbed_merge(const mla_geom* g, mla_dtype dt, int32_t B, int32_t L,
                       const int32_t* kv_offsets_host, const int32_t* kv_offsets_dev, const void* w_uv,
                       float* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * mla_materialize_kv -- expand the cached latent into full per-head keys
 * and values ("One guard...", section "The defect": expand the entire
 * cached latent back into full K and V), for T positions:
 *   k[t, h, j]     = sum_c w_uk[h, j, c] * c_kv[t, c]     (j < n)
 *   k[t, h, n + p] = k_pe[t, p]                           (shared rope key)
 *   v[t, h, e]     = sum_c c_kv[t, c] * w_uv[h, c, e]      (e < v)
 *
 *   c_kv [T, r], k_pe [T, rope], w_uk [H, n, r], w_uv [H, r, v]: device, dtype dt
 *   k    device, [T, H, n + rope], dtype dt
 *   v    device, [T, H, v], dtype dt
 * Supported (bf16): r % 64 == 0, n % 64 == 0, v % 64 == 0, rope % 8 == 0.
 * Supported (f32): any sizes.
 */
int mla_materialize_kv(const mla_geom* g, mla_dtype dt, int64_t T, const void* c_kv,
                       const void* k_pe, const void* w_uk, const void* w_uv, void* k, void* v,
                       void* stream);

/*
 * fp8 latent cache.  The pages test a "quantised latent form" of the cache
 * without defining it (mlx-lm PR #1817, section "Tests"); the form built here:
 * each cached position's row [c_kv[t] | k_pe[t]] (r + rope values) is stored as
 * OCP E4M3 codes (1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits,
 * subnormals m x 2^-9, no infinities, largest finite value 448) with one scale
 * per position, the smallest power of two 2^k with max|row| <= 448 x 2^k
 * (k in [-126, 127]; 2^0 for an all-zero row).  Codes are the nearest E4M3
 * value of row / 2^k, ties to the even code (a negative value that rounds to
 * zero gets code 0x00).  Every dequantised value code x 2^k is exact in bf16,
 * and the fp8 attention computes the absorbed attention over exactly those values.
 *
 * mla_quantize_latent_fp8 -- c_kv [T, r], k_pe [T, rope] (device, bf16) ->
 *   codes [T, r + rope] (device, uint8; latent then rope per position) and
 *   scales [T] (device, float32, powers of two).  Buffers are the caller's.
 *   Errors: MLA_E_NULL, MLA_E_SHAPE (T < 1 or > INT32_MAX), MLA_E_UNSUPPORTED
 *   (r or rope not a multiple of 8, r + rope > 1024), MLA_E_HIP.
 */
int mla_quantize_latent_fp8(const mla_geom* g, int64_t T, const void* c_kv, const void* k_pe, void* codes,
                            float* scales, void* stream);

/*
 * mla_absorbed_attention_fp8 -- mla_absorbed_attention (bf16 queries q_lat, q_pe
 * and W_UV; float32 out) with the latent cache given as (codes, scales) from
 * mla_quantize_latent_fp8 instead of c_kv and k_pe.  The scores run on the fp8
 * matrix cores: each query row is quantised in the kernel to E4M3 with one
 * power-of-two scale per 32-wide block of its key dimension (blocks 32j ..
 * 32j + 31 of q_lat, then of q_pe), the smallest scale 2^e with every
 * |q| <= 448 x 2^e (e in [-126, 127]; 2^0 for an all-zero block), codes the
 * nearest E4M3 value of q / 2^e, ties to even; the score of a cached position is
 * the exact product of those values with its dequantised key, summed in float32.
 * The values are the dequantised cache, exact in bf16.  So the result is the
 * absorbed attention of the block-quantised queries over the dequantised cache
 * (within the bf16 path's rounding), and, against the unquantised inputs, within
 * the error that E4M3 rounding of queries and cache implies.
 * Workspace: mla_absorbed_workspace_size with MLA_BF16.  mla_absorbed_splits_fp8
 * is its split pass alone; mla_absorbed_merge (MLA_BF16) completes it.
 * Supported: r = 512, rope in {0, 64}; otherwise MLA_E_UNSUPPORTED.  Other
 * errors as for mla_absorbed_attention.
 */
int mla_absorbed_attention_fp8(const mla_geom* g, int32_t B, int32_t L, const void* q_lat, const void* q_pe,
                               const void* codes, const float* scales, const int32_t* kv_offsets_host,
                               const int32_t* kv_offsets_dev, const void* w_uv, float scale, float* out,
                               void* workspace, size_t workspace_bytes, void* stream);
int mla_absorbed_splits_fp8(const mla_geom* g, int32_t B, int32_t L, const void* q_lat, const void* q_pe,
                            const void* codes, const float* scales, const int32_t* kv_offsets_host,
                            const int32_t* kv_offsets_dev, float scale, void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * The fp8 route with the queries quantised once, by the fold, instead of in
 * every split of the attention kernel (each split of a row tile would quantise
 * the same rows again).
 *
 * mla_query_fp8_bytes -- bytes of the E4M3 query block for B sequences of L
 * query rows: B x ceil(L H / 32) x 19456 (32 rows a tile).
 *
 * mla_fold_query_fp8 -- mla_fold_query (bf16) for B sequences of L rows
 * (rows = B L), writing q_lat if it is not null and, into q8 (device,
 * mla_query_fp8_bytes), the E4M3 block quantisation that
 * mla_absorbed_attention_fp8 applies to q_lat and q_pe: per query row and
 * 32-wide block of its key dimension, the smallest power-of-two scale 2^e with
 * every |q| <= 448 x 2^e and the nearest E4M3 codes of q / 2^e, the latent
 * part taken from the bf16-rounded fold (the values q_lat holds).  q_pe: device,
 * [B, L, H, rope] bf16 (may be null when rope == 0).  The layout of q8 is the
 * attention kernel's and is not part of the ABI; it is valid only for these g,
 * B and L.  Supported: r = 512, rope in {0, 64}, n % 32 == 0, n <= 512;
 * otherwise MLA_E_UNSUPPORTED.  Errors: MLA_E_NULL, MLA_E_SHAPE (B, L < 1 or
 * B L H too large), MLA_E_HIP.
 *
 * mla_absorbed_attention_fp8q / mla_absorbed_splits_fp8q -- as
 * mla_absorbed_attention_fp8 / mla_absorbed_splits_fp8 with the queries given
 * as that block instead of q_lat and q_pe: the same kernels and, for the same
 * bf16 query values, the same result bits.  Same workspace, errors and support.
 */
int mla_query_fp8_bytes(const mla_geom* g, int32_t B, int32_t L, size_t* bytes_out);
int mla_fold_query_fp8(const mla_geom* g, int32_t B, int32_t L, const void* q_nope, const void* w_uk,
                       const void* q_pe, void* q_lat, void* q8, void* stream);
int mla_absorbed_attention_fp8q(const mla_geom* g, int32_t B, int32_t L, const void* q8, const void* codes,
                                const float* scales, const int32_t* kv_offsets_host, const int32_t* kv_offsets_dev,
                                const void* w_uv, float scale, float* out, void* workspace, size_t workspace_bytes,
                                void* stream);
int mla_absorbed_splits_fp8q(const mla_geom* g, int32_t B, int32_t L, const void* q8, const void* codes,
                             const float* scales, const int32_t* kv_offsets_host, const int32_t* kv_offsets_dev,
                             float scale, void* workspace, size_t workspace_bytes, void* stream);

/*
 * mla_absorbed_attention_sparse -- absorbed attention over selected cache
 * positions ("One guard, 110x off the verify step", section "The sparse model
 * is different": an indexer selects the top 2048 cached positions and attention
 * runs only over those).  Sequence b's selection is sel[sel_offsets[b] ..
 * sel_offsets[b+1]): positions relative to the sequence start, strictly
 * increasing, shared by the sequence's L rows and all heads; row i attends to
 * the selected positions p < Kv_b - L + i + 1 (the causal rule of the dense
 * call), and a row that sees none of them gets a zero output.  Everything else
 * as mla_absorbed_attention with MLA_BF16 (q_lat, q_pe, c_kv, k_pe, W_UV bf16;
 * out float32).  sel (int32) and sel_offsets_dev live on the device,
 * sel_offsets_host on the host.  Selection entries outside [0, Kv_b) are clamped
 * into it (no access leaves the cache).  Workspace:
 * mla_absorbed_sparse_workspace_size.  Errors: MLA_E_NULL, MLA_E_SHAPE (offsets
 * as for the dense call; 1 <= selection length <= Kv_b), MLA_E_UNSUPPORTED
 * (r != 512 or rope not in {0, 64}), MLA_E_WORKSPACE, MLA_E_HIP.
 */
int mla_absorbed_sparse_workspace_size(const mla_geom* g, int32_t B, int32_t L, const int32_t* kv_offsets_host,
                                       const int32_t* sel_offsets_host, size_t* bytes_out);
int mla_absorbed_attention_sparse(const mla_geom* g, int32_t B, int32_t L, const void* q_lat, const void* q_pe,
                                  const void* c_kv, const void* k_pe, const int32_t* kv_offsets_host,
                                  const int32_t* kv_offsets_dev, const int32_t* sel, const int32_t* sel_offsets_host,
                                  const int32_t* sel_offsets_dev, const void* w_uv, float scale, float* out,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * mla_absorbed_attention_sparse_fp8 -- mla_absorbed_attention_sparse over the
 * fp8 form of the latent cache (codes and scales of mla_quantize_latent_fp8
 * instead of c_kv and k_pe), with the scores on the fp8 matrix cores exactly as
 * in mla_absorbed_attention_fp8 (block-quantised queries): the attention of
 * those queries over the selected positions of the dequantised cache.
 * Workspace: mla_absorbed_sparse_workspace_size.
 * Errors as mla_absorbed_attention_sparse (MLA_E_NULL also for codes or scales).
 */
int mla_absorbed_attention_sparse_fp8(const mla_geom* g, int32_t B, int32_t L, const void* q_lat, const void* q_pe,
                                      const void* codes, const float* scales, const int32_t* kv_offsets_host,
                                      const int32_t* kv_offsets_dev, const int32_t* sel,
                                      const int32_t* sel_offsets_host, const int32_t* sel_offsets_dev,
                                      const void* w_uv, float scale, float* out, void* workspace,
                                      size_t workspace_bytes, void* stream);

/*
 * Pooled top-k indexer ("One guard, 110x off the verify step", sections "The
 * sparse model is different" and "The same bug, one layer over").  The indexer
 * pools the cached keys of each sequence into windows of four positions
 * (window w = positions 4w .. 4w+3, the last one possibly partial), scores the
 * windows, and picks the top `budget` positions for mla_absorbed_attention_sparse.
 *
 *   pooled key of window w = float32 mean of its bf16 key rows, summed in
 *                            position order (so a window pools to the same bits
 *                            however its positions arrived);
 *   score of window w      = q_b . pooled[w] in float32 (the pages do not define
 *                            the score; this is the library's reading);
 *   selection              = the first min(budget, Kv_b) positions in the order
 *                            (window score descending, position ascending),
 *                            written in increasing position order.
 *
 * The pool caches completed windows.  A step that appended S positions to
 * every sequence recomputes only the windows from floor((Kv_b - S) / 4) on if
 * all four guards hold: the pool holds keys, the cache has no padding, the
 * batch shape (sequence count, key width) is the one the pool was built for,
 * and every cache is exactly as long (minus S) as the pool remembers.
 * Otherwise every window is recomputed.  A wide step therefore pools exactly
 * as the same positions fed one at a time.  A cache cut back after a
 * speculative rejection either fails the last guard (full recompute) or is
 * announced with mla_indexer_pool_trim, after which the windows wholly before
 * the cut are kept.
 *
 * The pool's state lives in a caller-owned mla_pool on the host; its pooled
 * keys in a caller-owned device buffer [batch_max][capacity][d] float32.
 */
typedef struct mla_pool {
  float* pooled;        /* device [batch_max][capacity][d] float32 (caller-owned)        */
  int32_t capacity;     /* windows per sequence the buffer holds                          */
  int32_t batch_max;    /* sequences the buffer (and lengths) hold                        */
  int32_t batch;        /* sequences the pool was last built for                          */
  int32_t d;            /* key width the pool was last built for                          */
  int32_t valid;        /* 1 once a step has pooled keys; 0 after init or a failed step;  */
                        /* 2 after a trim that cut inside a window (a step must run       */
                        /* before the pool is scored; it still seeds an incremental step)  */
  int32_t* lengths;     /* host [batch_max]: cache length per sequence the pool covers    */
} mla_pool;

/* Initialise *pool over caller-owned storage (nothing is launched).  Errors:
 * MLA_E_NULL (pool, pooled or lengths NULL), MLA_E_SHAPE (capacity or
 * batch_max < 1). */
int mla_indexer_pool_init(mla_pool* pool, float* pooled, int32_t capacity, int32_t batch_max, int32_t* lengths);

/* The guard decision alone (host only, nothing launched): *incremental_out = 1
 * if a step of S new positions per sequence over caches with these offsets
 * would recompute only the tail, 0 if it would recompute every window.
 * padded != 0 declares that the cache rows of a sequence are not its positions
 * from 0 (padding).  Errors: MLA_E_NULL, MLA_E_SHAPE (B < 1, S < 1, a Kv_b < S). */
int mla_indexer_pool_plan(const mla_pool* pool, int32_t B, int32_t d, const int32_t* kv_offsets_host, int32_t S,
                          int32_t padded, int32_t* incremental_out);

/*
 * mla_indexer_pool_step -- bring the pool up to date after a step that
 * appended S positions to every sequence.
 *   keys: device bf16, row of position p of sequence b at
 *         keys + (kv_offsets[b] + p) * key_stride (elements), d columns used
 *   kv_offsets_host / kv_offsets_dev: the cache offsets as everywhere else
 *   incremental_out (may be NULL): which path ran (as mla_indexer_pool_plan)
 * On success pool->lengths[b] = Kv_b, batch = B, d = d, valid = 1.
 * Supported: d a multiple of 8, 8 <= d <= 1024.  Errors: MLA_E_NULL,
 * MLA_E_SHAPE (B outside [1, batch_max], S < 1, a Kv_b < S, key_stride < d,
 * ceil(Kv_b / 4) > capacity), MLA_E_UNSUPPORTED (d), MLA_E_HIP (the pool is then
 * marked invalid, so the next step recomputes everything).
 */
int mla_indexer_pool_step(mla_pool* pool, int32_t B, int32_t d, const void* keys, int64_t key_stride,
                          const int32_t* kv_offsets_host, const int32_t* kv_offsets_dev, int32_t S, int32_t padded,
                          int32_t* incremental_out, void* stream);

/*
 * Fixed-capacity update lists ("Over 107 tok/s Qwen3.8-Flash-Next on M3 Ultra",
 * section "Why doing eight rows can beat doing two", and its algorithm for
 * constructing a fixed-capacity update list), read for this indexer: a block is
 * a window of four positions and its destination the window's own slot in the
 * pooled array.  An incremental step's real updates are the windows from
 * floor((Kv - S) / 4) on, a count that varies with S and the alignment; padding
 * them to a fixed capacity P (8 or 16) with complete windows whose rows did not
 * change (each written back with the bits it already holds, at a destination not
 * otherwise in the list) gives every step one launch shape.
 *
 * mla_indexer_update_list -- the list for one sequence (host only): real updates
 * are the windows first .. windows - 1, the complete windows 0 .. complete - 1
 * (0 <= first <= complete <= windows), S the tokens of the step, target P in
 * {8, 16}.  The capacity is max(1, windows - first), raised to P when S <= 16,
 * that count is at most P and at least P windows are complete; an empty update
 * lists window 0 if complete, else window windows - 1 (-1 for an empty cache).
 * The real updates come first, in order, then fillers (complete windows in
 * increasing order whose destinations are not yet listed) up to the capacity.
 * list_out (host) must hold max(1, windows - first, target) entries; the list
 * length is *capacity_out.  Errors: MLA_E_NULL, MLA_E_SHAPE (bounds or target).
 */
int mla_indexer_update_list(int32_t first, int32_t windows, int32_t complete, int32_t S, int32_t target,
                            int32_t* list_out, int32_t* capacity_out);

/*
 * mla_indexer_pool_step_fixed -- mla_indexer_pool_step with the same arguments
 * plus target (8 or 16).  When the four guards hold, S <= 16, and every sequence
 * has at most target real updates and at least target complete windows, one
 * launch of fixed shape (target windows per sequence: the list of
 * mla_indexer_update_list) pools them, and *capacity_out = target; otherwise the
 * ordinary step runs (*capacity_out = 0).  Either way the pooled keys, lengths
 * and state after the call are those of mla_indexer_pool_step, bit for bit.
 * capacity_out and incremental_out may be NULL.  Errors: those of
 * mla_indexer_pool_step, and MLA_E_SHAPE for a target other than 8 or 16.
 */
int mla_indexer_pool_step_fixed(mla_pool* pool, int32_t B, int32_t d, const void* keys, int64_t key_stride,
                                const int32_t* kv_offsets_host, const int32_t* kv_offsets_dev, int32_t S,
                                int32_t padded, int32_t target, int32_t* incremental_out, int32_t* capacity_out,
                                void* stream);

/* A speculative rejection cut sequence b's cache back to new_lengths[b]
 * positions (host array [B]): the pool forgets what it covered past the cut
 * (host only; the next step recomputes from the window holding the cut).
 * Entries not below the remembered length change nothing.  A cut inside a
 * window (new length not a multiple of 4) leaves that window's pooled key
 * holding rows past the cut, so the pool is marked valid = 2 and
 * mla_indexer_scores refuses it until the next step has run.  Errors:
 * MLA_E_NULL, MLA_E_SHAPE (pool not valid, B != pool->batch, a negative length). */
int mla_indexer_pool_trim(mla_pool* pool, int32_t B, const int32_t* new_lengths);

/*
 * mla_indexer_scores -- scores[b * capacity + w] = q[b] . pooled key of window
 * w, for w < ceil(Kv_b / 4) (the rest untouched).  q: device float32 [B][d].
 * The pool must cover the caches as they are (pool->lengths[b] == Kv_b) and
 * hold no window cut by a trim (valid == 1).  Errors: MLA_E_NULL, MLA_E_SHAPE
 * (pool not valid or trimmed inside a window, B != pool->batch, a length not
 * covered), MLA_E_HIP.
 */
int mla_indexer_scores(const mla_pool* pool, int32_t B, const float* q, const int32_t* kv_offsets_host,
                       const int32_t* kv_offsets_dev, float* scores, void* stream);

/*
 * mla_indexer_pool_step_scores -- mla_indexer_pool_step followed by
 * mla_indexer_scores, with the same arguments, effects and results (the same
 * bits in pool->pooled and in scores), in fewer launches: when the guards hold
 * and every sequence's tail is at most 16 windows, the scoring launch pools the
 * tail windows itself (one launch instead of two); a longer tail is pooled by
 * the pooling kernel first; otherwise every window is pooled, then scored.  Errors: those of
 * mla_indexer_pool_step, and MLA_E_NULL for q or scores NULL; on MLA_E_HIP
 * the pool is marked invalid.
 */
int mla_indexer_pool_step_scores(mla_pool* pool, int32_t B, int32_t d, const void* keys, int64_t key_stride,
                                 const int32_t* kv_offsets_host, const int32_t* kv_offsets_dev, int32_t S,
                                 int32_t padded, const float* q, float* scores, int32_t* incremental_out,
                                 void* stream);

/* Offsets of the packed selection (host only): sel_offsets_out[0] = 0,
 * sel_offsets_out[b+1] = sel_offsets_out[b] + min(budget, Kv_b).  Errors:
 * MLA_E_NULL, MLA_E_SHAPE (B < 1, budget < 1, bad offsets). */
int mla_indexer_selection_offsets(int32_t B, const int32_t* kv_offsets_host, int32_t budget,
                                  int32_t* sel_offsets_out);

/*
 * mla_indexer_select -- the selection of sequence b into sel[sel_offsets[b] ..
 * sel_offsets[b+1]) (device int32, positions from the sequence start,
 * increasing), from window scores [B][capacity] (device float32, windows
 * w < ceil(Kv_b / 4) read).  Scores must not be NaN (their order is then
 * unspecified); -0 and +0 are equal.  sel_offsets_dev must hold what
 * mla_indexer_selection_offsets gives.  Errors: MLA_E_NULL, MLA_E_SHAPE (B < 1,
 * budget < 1, bad offsets, ceil(Kv_b / 4) > capacity), MLA_E_HIP.
 */
int mla_indexer_select(int32_t B, const float* scores, int32_t capacity, const int32_t* kv_offsets_host,
                       const int32_t* kv_offsets_dev, int32_t budget, const int32_t* sel_offsets_dev, int32_t* sel,
                       void* stream);

/* Bytes of workspace mla_materialized_attention needs (split-KV partials). */
int mla_materialized_workspace_size(const mla_geom* g, mla_dtype dt, int32_t B, int32_t L,
                                    const int32_t* kv_offsets_host, size_t* bytes_out);

/*
 * mla_materialized_attention -- ordinary causal attention over the
 * expanded per-head K and V ("One guard...", section "The defect": then
 * attend normally).  For sequence b, row i, head h, vis as above:
 *   s_t = scale * (q_nope[b,i,h,:] . k[t,h,:n] + q_pe[b,i,h,:] . k[t,h,n:])
 *   out[b,i,h,:] = sum_t softmax(s)_t * v[t,h,:]
 *
 *   q_nope [B, L, H, n], q_pe [B, L, H, rope]: device, dtype dt
 *   k [sum Kv, H, n + rope], v [sum Kv, H, v]: device, dtype dt
 *   out    device, [B, L, H, v], float32
 *   workspace: at least mla_materialized_workspace_size() bytes
 * Supported (bf16): n in {128, 192, 256}, rope in {0, 64}, v in {128, 256}.
 * Supported (f32): n + rope <= 1152, v <= 1024.
 */
int mla_materialized_attention(const mla_geom* g, mla_dtype dt, int32_t B, int32_t L,
                               const void* q_nope, const void* q_pe, const void* k,
                               const void* v, const int32_t* kv_offsets_host,
                               const int32_t* kv_offsets_dev, float scale, float* out,
                               void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
