/*
 * mla.h -- C ABI of the MI355X (gfx950) MLA latent-cache decode library.
 *
 * Multi-head latent attention (MLA) decode in the matrix-absorbed form over a
 * paged latent cache, as described on the page "DeepSeek MLA Architecture:
 * How Multi-Head Latent Attention Cuts KV Cache by 93%" (below: [MLA-93]),
 * sections "DeepSeek MLA Deep Dive: Core Mechanics" 1-3, "Total Cached
 * Scalars per Token" and "Production PyTorch Implementation: Single-Token MLA
 * Decoding" (below: [MLA-93] decoding section), and on "DeepSeek-V3 Architecture: Multi-Head
 * Latent Attention (MLA) & FP8 Mixed-Precision Training" (below: [V3-ARCH]),
 * sections 2, A and 3.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - All tensor pointers are DEVICE pointers owned by the caller; the library
 *    never allocates, frees or retains them, and keeps no per-call state.
 *  - Every call only validates its arguments on the host and enqueues work on
 *    `stream` (a hipStream_t; NULL = the default stream).  Nothing is
 *    synchronised; outputs are ready when the stream reaches that point.
 *  - Return value: MLA_OK (0) or a negative mla_status.  On error nothing has
 *    been enqueued (except MLA_ERR_HIP, where a launch itself failed) and
 *    mla_last_error() returns a description (thread-local).  No exception or
 *    abort crosses the ABI.
 *  - Row-major layouts; the last index is contiguous.
 *  - Cache layout (paged): `cache` is [num_blocks][block_size][D] with
 *    D = d_latent + d_rope; row = [c^KV (d_latent) ; k^R (d_rope)], the
 *    latent first.  Token at logical position p of sequence b lives in
 *    physical block page_table[b * max_blocks_per_seq + p / block_size], row
 *    p % block_size.  For the fp8 cache `cache_scales` is
 *    [num_blocks][block_size][n_tiles] fp32 with n_tiles = ceil(D / 128):
 *    element x of tile k (channels [128k, min(128k+128, D))) decodes to
 *    e4m3(x) * scale[k]  (tile-level scaling as in the FP8 paragraph of
 *    "DeepSeek Unveils DualPipe & Multi-Head Latent Attention").
 *  - Device-data preconditions (not checked unless noted): page-table entries
 *    that a call reads are in [0, num_blocks); n_q <= seq_lens[b] <=
 *    max_blocks_per_seq * block_size.  Entries that are never read may hold
 *    anything (e.g. -1).  Cache rows past seq_lens[b] are never used, whatever
 *    they hold (NaN included).
 */
#ifndef MLA_H
#define MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_ABI_VERSION 1

typedef void *mla_stream_t; /* a hipStream_t */

typedef enum mla_status {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARGUMENT = -1, /* null pointer, bad size, inconsistent dims */
  MLA_ERR_UNSUPPORTED = -2,      /* no kernel for this dims/dtype combination */
  MLA_ERR_WORKSPACE_TOO_SMALL = -3,
  MLA_ERR_HIP = -4               /* a HIP runtime call or launch failed */
} mla_status;

typedef enum mla_dtype {
  MLA_FP32 = 0,
  MLA_BF16 = 1,
  MLA_FP8_E4M3 = 2, /* OCP E4M3 (max 448, no infinities); cache only */
  /* The MLA_FP8_E4M3 layout (codes and one fp32 scale per (token, tile))
   * with every scale a power of two: the append picks the smallest 2^E with
   * max|tile| <= 448 * 2^E, and the matrix-core decode applies the scales
   * inside its fp8 score products.  Cache only. */
  MLA_FP8_E4M3_PO2 = 3
} mla_dtype;

/* Model dimensions, shared by every call.
 * [MLA-93] Core Mechanics 1 and 3: d_latent = d_c (512 for DeepSeek-V3),
 * d_rope = d_R (64), d_nope = per-head content width (128), d_v = per-head
 * value width (128), num_heads = H (128). */
typedef struct mla_dims {
  int32_t num_heads;
  int32_t d_latent;
  int32_t d_rope;      /* even */
  int32_t d_nope;      /* used only for the default softmax scale */
  int32_t d_v;
  int32_t block_size;  /* tokens per cache block, > 0 */
  int32_t cache_dtype; /* mla_dtype of the cache */
  int32_t act_dtype;   /* mla_dtype of q, h, weights, u, o: MLA_FP32 or MLA_BF16 */
  float softmax_scale; /* <= 0 selects 1/sqrt(d_nope + d_rope) */
  float rope_base;     /* <= 0 selects 10000 */
  int32_t flags;       /* bitwise OR of MLA_FLAG_*; 0 for defaults */
} mla_dims;

/* Use the generic VALU kernels (decode, query absorption) even where the
 * MFMA kernels apply (an independent second implementation, for
 * cross-checks). */
#define MLA_FLAG_GENERIC_DECODE 1

/* Validation mode: before its kernels run, a call checks the device-side
 * preconditions it relies on, with one small kernel and a synchronisation of
 * `stream`: n_q <= seq_lens[b] (and <= max_blocks_per_seq * block_size where
 * the call knows it), every page-table entry mla_decode would read >= 0,
 * positions[t] >= 0 (and < max_blocks_per_seq * block_size for
 * mla_cache_append), seq_ids[t] >= 0.  On a violation the call returns
 * MLA_ERR_INVALID_ARGUMENT, names the first offending element in
 * mla_last_error() and runs nothing.  Not detectable: entries past the
 * pool's end and sequence ids past the table's rows (neither size is an
 * argument).  Also on for every call when the environment variable
 * MLA_VALIDATE is 1.  Checked calls are serialised; meant for debugging. */
#define MLA_FLAG_VALIDATE 2

int mla_abi_version(void);

/* Description of the last error on the calling thread ("" if none). */
const char *mla_last_error(void);

/* Number of compute units of the current device (0 on failure). */
int mla_device_cu_count(void);

/*
 * mla_cache_append -- project, rotate and store new tokens' cache rows.
 * [MLA-93] Core Mechanics 1 (c = W^DKV h) and 3 (k^R = RoPE(W^KR h), shared
 * by all heads); in the [MLA-93] decoding section the new token's latent and
 * RoPE key are cached before attention.  RoPE is rotate-half: channel j of
 * k^R is paired with j + d_rope/2 and rotated by pos * base^(-j/(d_rope/2)).
 *
 *   h          [n_tokens][d_model]        act_dtype
 *   w_dkv      [d_latent][d_model]        act_dtype
 *   w_kr       [d_rope][d_model]          act_dtype
 *   seq_ids    [n_tokens] int32           sequence of each token
 *   positions  [n_tokens] int32           logical position of each token (>= 0)
 *   page_table [batch][max_blocks_per_seq] int32
 *   cache      pool (see conventions), written only at the tokens' slots
 *   cache_scales  fp8 only (else NULL): written for the same slots
 * Accumulation is fp32; the row is stored in cache_dtype (bf16: RNE; fp8:
 * per-tile amax scaling, scale = amax/448, code = e4m3_rne_sat(x * (448/amax)),
 * scale 1 and zero codes for an all-zero tile).  Two tokens mapping to the same
 * slot in one call is undefined.
 * workspace: device scratch of mla_cache_append_workspace_size() bytes
 * (4-byte aligned; may be NULL when that size is 0).  bf16 activations take
 * the matrix-core path (split-K partials in the workspace, then a per-token
 * finalize); fp32 activations take a VALU path that needs no workspace and
 * supports dims whose RoPE part lies in one 128-channel tile.
 * Errors: MLA_ERR_WORKSPACE_TOO_SMALL if workspace_bytes is below the size.
 */
size_t mla_cache_append_workspace_size(const mla_dims *dims, int32_t n_tokens, int32_t d_model);

int mla_cache_append(const mla_dims *dims, const void *h, int32_t n_tokens, int32_t d_model,
                     const void *w_dkv, const void *w_kr, const int32_t *seq_ids,
                     const int32_t *positions, const int32_t *page_table,
                     int32_t max_blocks_per_seq, void *cache, float *cache_scales,
                     void *workspace, size_t workspace_bytes, mla_stream_t stream);

/*
 * mla_query_absorb -- matrix-absorbed query of every (row, head).
 * [MLA-93] Core Mechanics 3 (decoupled RoPE and absorption of W^UK into the
 * query) and its decoding section: per head i,
 *   q~_i  = (W^UK_i)^T q^C_i                      in R^{d_latent}
 *   q^R_i = RoPE(q^R_i, position)                 (rotate-half, base rope_base)
 * written packed as [q~_i ; q^R_i], the query layout mla_decode reads.
 *   q_in      [rows][num_heads][d_nope + d_rope] act_dtype: per head the
 *             content part q^C then the un-rotated RoPE part (the head-major
 *             split of the query projection)
 *   positions [rows] int32 >= 0: the position each row's query sits at
 *   w_uk      [num_heads][d_nope][d_latent] act_dtype (k^C_i = W^UK_i c)
 *   q_out     [rows][num_heads][d_latent + d_rope] act_dtype; must not
 *             overlap q_in
 * rows = batch * n_q in mla_decode's order.  fp32 accumulation; RoPE angles in
 * fp64 with cos/sin rounded to fp32 (as in mla_cache_append); bf16 outputs
 * round to nearest even.  bf16 with d_nope = 128, d_latent = 512 and d_rope a
 * multiple of 8 up to 64 (16-byte aligned pointers) runs on the matrix cores;
 * other shapes on a VALU kernel.
 * Errors: MLA_ERR_INVALID_ARGUMENT (rows < 0, d_nope < 1, a NULL or misaligned
 * pointer, q_out overlapping q_in); rows = 0 does nothing.
 */
int mla_query_absorb(const mla_dims *dims, const void *q_in, const int32_t *positions,
                     const void *w_uk, void *q_out, int32_t rows, mla_stream_t stream);

/*
 * mla_cache_append_query_absorb -- mla_cache_append followed by
 * mla_query_absorb, in fewer launches.  The two operations of a decode step
 * before the attention ([MLA-93] Core Mechanics 1 and 3 and its decoding
 * section) do not depend on each other; when both take their matrix-core
 * forms the append's second step and the query absorption share one launch,
 * so each one's memory latency hides behind the other's work.
 * Arguments: those of mla_cache_append (h ... workspace_bytes), then those
 * of mla_query_absorb (q_in, q_positions = its positions, w_uk, q_out,
 * q_rows = its rows); each set has the meaning, layout and checks of its own
 * call, and n_tokens = 0 or q_rows = 0 skips that half.  Results are the
 * two calls' bit for bit, provided the query's buffers do not overlap the
 * cache, the scales or the workspace (not checked: the cache's extent is not
 * an argument).
 * Errors: those of either call; on an error neither operation runs.
 */
int mla_cache_append_query_absorb(const mla_dims *dims, const void *h, int32_t n_tokens,
                                  int32_t d_model, const void *w_dkv, const void *w_kr,
                                  const int32_t *seq_ids, const int32_t *positions,
                                  const int32_t *page_table, int32_t max_blocks_per_seq,
                                  void *cache, float *cache_scales, void *workspace,
                                  size_t workspace_bytes, const void *q_in,
                                  const int32_t *q_positions, const void *w_uk, void *q_out,
                                  int32_t q_rows, mla_stream_t stream);

/*
 * mla_linear -- y = x W^T, a bias-free linear layer with fp32 accumulation:
 * the query projections of the [MLA-93] decoding section (c^Q = W^DQ h, then
 * q^C = W^UQ c^Q and q^R = W^QR c^Q; placing the rows of W^UQ and W^QR head
 * by head, [W^UQ_i ; W^QR_i], gives mla_query_absorb's q_in in one call) and
 * its final output projection W^O.
 *   x  [rows][k] act_dtype
 *   w  [n][k]    act_dtype (a torch Linear weight)
 *   y  [rows][n] act_dtype; must not overlap x or w
 *   workspace: device scratch of mla_linear_workspace_size(dims, rows, n, k)
 *              bytes, 16-byte aligned (NULL when that size is 0)
 * bf16 outputs round to nearest even.  bf16 with k a multiple of 512 and n of
 * 32 (16-byte aligned x, w, y) runs on the matrix cores (the k range may be
 * split, the fp32 partials kept in the workspace and summed in a fixed order:
 * results are deterministic); other shapes on a VALU kernel.
 * Errors: MLA_ERR_INVALID_ARGUMENT (rows < 0, k < 1, n < 1, NULL, misaligned,
 * overlap), MLA_ERR_WORKSPACE_TOO_SMALL.
 */
size_t mla_linear_workspace_size(const mla_dims *dims, int32_t rows, int32_t n, int32_t k);

int mla_linear(const mla_dims *dims, const void *x, int32_t rows, int32_t k, const void *w, int32_t n,
               void *y, void *workspace, size_t workspace_bytes, mla_stream_t stream);

/*
 * Split-KV decode (mla_decode + mla_decode_combine).
 *
 * q [batch][n_q][num_heads][d_latent + d_rope] act_dtype: packed absorbed
 * queries [q~ ; q^R], q~_i = (W^UK_i)^T q^C_i, q^R already rotated at the
 * query position ([MLA-93] Core Mechanics 3).  Query j of sequence b sits at
 * position seq_lens[b] - n_q + j and attends to positions
 * 0 .. seq_lens[b] - n_q + j (itself included: the new tokens are appended
 * before attention, as in the [MLA-93] decoding section).  Per head i:
 *   s_t = scale * (q~_i . c_t + q^R_i . k^R_t),  p = softmax_t(s),
 *   u_i = sum_t p_t c_t  in R^{d_latent}   (attention and value aggregation in
 *                                          latent space, [MLA-93] decoding section).
 *
 * The cache blocks of all sequences are laid end to end and cut into
 * `num_partitions` near-equal ranges; one workgroup per (range, query token)
 * walks its range and writes, for every sequence piece it covers, a partial
 * (o = normalised latent output, lse = natural-log sum of exp of the scores)
 * into `workspace`, and records there, per sequence, the first slot and the
 * number of its pieces.  mla_decode_combine merges the pieces of each sequence
 * with a log-sum-exp weighting, reading that record (so it must follow an
 * mla_decode on the same workspace; the stream orders the two).  num_partitions <= 0 selects the default
 * (the device's compute-unit count divided by n_q, at least 1); values above
 * MLA_MAX_PARTITIONS are rejected with MLA_ERR_INVALID_ARGUMENT (and give a
 * workspace size of 0).  Results are deterministic for a fixed num_partitions.
 */
#define MLA_MAX_PARTITIONS (1 << 20)

size_t mla_decode_workspace_size(const mla_dims *dims, int32_t batch, int32_t n_q,
                                 int32_t num_partitions);

int mla_decode(const mla_dims *dims, const void *q, int32_t batch, int32_t n_q,
               const void *cache, const float *cache_scales, const int32_t *page_table,
               int32_t max_blocks_per_seq, const int32_t *seq_lens, int32_t num_partitions,
               void *workspace, size_t workspace_bytes, mla_stream_t stream);

/* Merge the partials written by the preceding mla_decode with the same
 * arguments: per (b, j, head) M = max_s lse_s, w_s = exp(lse_s - M),
 * u = sum_s w_s o_s / sum_s w_s, lse = M + ln sum_s w_s.
 *   u_out   [batch][n_q][num_heads][d_latent] act_dtype
 *   lse_out [batch][n_q][num_heads] fp32, may be NULL */
int mla_decode_combine(const mla_dims *dims, const void *workspace, size_t workspace_bytes,
                       int32_t batch, int32_t n_q, const int32_t *seq_lens,
                       int32_t num_partitions, void *u_out, float *lse_out,
                       mla_stream_t stream);

/*
 * mla_out_proj -- per-head value up-projection o_i = W^UV_i u_i.
 * [MLA-93] decoding section (W^UV applied to the latent output).
 *   u     [rows][num_heads][d_latent] act_dtype  (rows = batch * n_q)
 *   w_uv  [num_heads][d_v][d_latent]  act_dtype
 *   out   [rows][num_heads][d_v]      act_dtype
 * fp32 accumulation.
 */
int mla_out_proj(const mla_dims *dims, const void *u, int32_t rows, const void *w_uv, void *out,
                 mla_stream_t stream);

/*
 * mla_decode_combine_out_proj -- mla_decode_combine followed by mla_out_proj
 * in one pass, so the merged latent output u need not round-trip through
 * memory: per row r = b * n_q + j and head i,
 *   u = sum_s w_s o_s / sum_s w_s (as mla_decode_combine, rounded to the
 *   activation dtype), then out[r][i] = W^UV_i u ([MLA-93] decoding section).
 * Arguments as in the two calls it replaces:
 *   workspace / workspace_bytes / batch / n_q / seq_lens / num_partitions:
 *            exactly those of the preceding mla_decode;
 *   w_uv     [num_heads][d_v][d_latent] act_dtype;
 *   out      [batch * n_q][num_heads][d_v] act_dtype;
 *   u_out    [batch][n_q][num_heads][d_latent] act_dtype, or NULL (u is then
 *            not stored);
 *   lse_out  [batch][n_q][num_heads] fp32, or NULL.
 * The fused kernel covers bf16 activations with d_latent = 512 and d_v a
 * multiple of 32 up to 128; other shapes run the two separate kernels, which
 * needs u_out (else MLA_ERR_UNSUPPORTED).
 */
int mla_decode_combine_out_proj(const mla_dims *dims, const void *workspace,
                                size_t workspace_bytes, int32_t batch, int32_t n_q,
                                const int32_t *seq_lens, int32_t num_partitions,
                                const void *w_uv, void *out, void *u_out, float *lse_out,
                                mla_stream_t stream);

/*
 * mla_prefill -- one prefill chunk of a sequence over its latent cache, in
 * the un-absorbed form.  The prefill phase processes many prompt tokens at
 * once ([MLA-93], the prefill/decode contrast that opens the page); for a
 * long chunk the per-head keys and values are expanded from the cached
 * latents once per chunk (k_{t,i} = [W^UK_i c_t ; k^R_t], v_{t,i} = W^UV_i c_t,
 * [MLA-93] Core Mechanics 1 and 3) and attention runs in the usual form.
 * The chunk's own rows must already be in the cache (mla_cache_append): chunk
 * token j sits at position seq_len - n_tokens + j and attends to positions
 * 0 .. seq_len - n_tokens + j.  Per head i:
 *   o_i = sum_t softmax_t(scale * [q^C_i ; RoPE(q^R_i)] . k_{t,i}) v_{t,i}
 * (the rotation of q^R at the token's position is done here).
 *   q_in           [n_tokens][num_heads][d_nope + d_rope] bf16: per head q^C
 *                  then the not yet rotated q^R (mla_query_absorb's input layout)
 *   cache          the paged pool: bf16, or e4m3 codes (MLA_FP8_E4M3 or
 *                  MLA_FP8_E4M3_PO2) with cache_scales [num_blocks][block_size]
 *                  [5] fp32 as mla_decode reads them (NULL for bf16); e4m3 rows
 *                  are dequantised (code x tile scale in fp32, one bf16
 *                  rounding) when the chunk's sequence is gathered
 *   page_table_row [>= ceil(seq_len / block_size)] int32: the sequence's row
 *                  of the page table
 *   w_uk           [num_heads][d_nope][d_latent] bf16; w_uv [num_heads][d_v][d_latent]
 *   out            [n_tokens][num_heads][d_v] bf16 (the heads' outputs before W^O)
 *   workspace      mla_prefill_workspace_size(dims, n_tokens, seq_len) bytes,
 *                  256-byte aligned: the gathered latents and the expanded keys
 *                  and values ((d_latent + d_rope + 2 * 128 * num_heads) * 2
 *                  bytes per cached token) and the rotated queries
 *                  (n_tokens * num_heads * (d_nope + d_rope) * 2 bytes)
 * Supported: bf16 activations, a bf16 or e4m3 cache, the DeepSeek-V3
 * dimensions (H = 128, d_latent = 512, d_rope = 64, d_nope = d_v = 128);
 * other dims or dtypes return MLA_ERR_UNSUPPORTED (the workspace size is 0).  fp32 accumulation,
 * RoPE angles in fp64 with cos/sin rounded to fp32, bf16 outputs.
 * The page-table entries the chunk's sequence needs (ceil(seq_len /
 * block_size) of them) must lie in the pool; they are not checked, and
 * validation mode does not cover this call.
 * Errors: MLA_ERR_INVALID_ARGUMENT (n_tokens < 0, seq_len < n_tokens,
 * seq_len >= MLA_MAX_PREFILL_TOKENS, NULL or misaligned pointers: q, cache
 * and weights 16 bytes, out 8; cache_scales given for a bf16 cache or missing
 * for an e4m3 one), MLA_ERR_WORKSPACE_TOO_SMALL, MLA_ERR_UNSUPPORTED.
 * n_tokens = 0 does nothing.
 */
#define MLA_MAX_PREFILL_TOKENS (1 << 23) /* a head's expanded keys stay under 2 GiB */
size_t mla_prefill_workspace_size(const mla_dims *dims, int32_t n_tokens, int32_t seq_len);

int mla_prefill(const mla_dims *dims, const void *q_in, int32_t n_tokens, const void *cache,
                const float *cache_scales, const int32_t *page_table_row, int32_t seq_len,
                const void *w_uk, const void *w_uv, void *out, void *workspace, size_t workspace_bytes,
                mla_stream_t stream);

/*
 * mla_decode_noalloc -- mla_decode followed by mla_decode_combine, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  Instead of a
 * caller workspace, the partials live in a device array that the library
 * owns: MLA_NOALLOC_SCRATCH_BYTES (64 MiB) on every device the library runs
 * on, held until the process ends.  The call allocates and frees nothing.
 *   Arguments: those of mla_decode (without workspace / workspace_bytes),
 *   then u_out [batch][n_q][num_heads][d_latent] act_dtype (required) and
 *   lse_out [batch][n_q][num_heads] fp32 (may be NULL) as in
 *   mla_decode_combine.  Results equal the two calls' with the same
 *   num_partitions, bit for bit.
 * Limit: the call needs mla_decode_workspace_size(dims, batch, n_q,
 * num_partitions) <= MLA_NOALLOC_SCRATCH_BYTES; larger calls return
 * MLA_ERR_WORKSPACE_TOO_SMALL and run nothing (e.g. H = 128, d_latent = 512,
 * bf16: (batch + partitions) * n_q <= 509).
 * Every call on one device shares that device's array: calls that overlap
 * in time on one device (two streams, two threads) race and give undefined
 * results; calls ordered on one stream are safe.  The first call on each
 * device looks the array's address up (thread-safe).
 * Errors: those of mla_decode and mla_decode_combine, plus the above.
 */
#define MLA_NOALLOC_SCRATCH_BYTES (64u << 20)

int mla_decode_noalloc(const mla_dims *dims, const void *q, int32_t batch, int32_t n_q,
                       const void *cache, const float *cache_scales, const int32_t *page_table,
                       int32_t max_blocks_per_seq, const int32_t *seq_lens, int32_t num_partitions,
                       void *u_out, float *lse_out, mla_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H */
