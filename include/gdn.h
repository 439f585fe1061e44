/*
 * gdn.h -- libgdn: the gated delta rule recurrence on AMD MI355X (gfx950).
 *
 * One call runs a whole span of gated-delta-rule steps for every sequence and
 * head ("ggml attention kernels" model card, huggingface.co/marcsun13/
 * ggml-gated-delta-net, section "Ops": one dispatch for a whole run of steps,
 * signature (q, k, v, g, beta, state) -> (out, final_state), plus a supports
 * predicate on head_dim).
 *
 * Per sequence s and head h, with the state M stored [value][key] (row i is a
 * value channel, column j a key channel) and d = head_dim, each token t does
 *     M     <- exp(g_t) * M                      (gate; g is log-domain)
 *     delta  = beta_t * (v_t - M k_t)            (what the key now retrieves)
 *     M     <- M + delta k_t^T                   (delta-rule overwrite)
 *     out_t  = M q_t / sqrt(d)                   (readout after the write)
 * The gate and the overwrite are the two ideas described in "Gated Delta Net
 * on AMD: why ROCm stumbles on hybrid-attention LLMs" (velstech.net, section
 * "What Gated Delta Net is, in plain language"); the op exponentiates g itself
 * and applies the 1/sqrt(head_dim) output scaling itself (model card, the
 * paragraph after the contract bullets).  The retrieval uses the gated state
 * and the readout follows the write: the pages leave that order open and this
 * is the reading taken.
 *
 * All arrays are dense, row-major ("torch order", model card section "Shapes,
 * in torch order"):
 *     q, k, v, out : (n_seqs, n_tokens, n_heads, head_dim)   dtype gdn_dtype
 *     g, beta      : (n_seqs, n_tokens, n_heads)             fp32
 *     state_in/out : (n_seqs, n_heads, head_dim, head_dim)   fp32, [value][key]
 * For gdn_forward, q and k carry one head per value head, already expanded
 * (first contract bullet): head h of q and k pairs with head h of v, in the
 * caller's order.  gdn_forward_tiled takes fewer key heads instead.
 * q and k are used as given (no normalisation inside the op).
 *
 * Ownership and streams.  Every data pointer is a DEVICE pointer owned by the
 * caller.  The library keeps no pointer after a call returns and no call
 * allocates device memory: scratch space for the chunked algorithm is the
 * caller's workspace (gdn_forward_noalloc instead uses a fixed array that the
 * library holds on each GPU it runs on).  Work is enqueued on the caller's stream and the call
 * returns without synchronising; results are ready when that stream reaches
 * the end of the enqueued work (the model card, section "Where the kernels
 * come from", explains why kernels must join the caller's own queue).
 *
 * Errors.  Every entry point validates its arguments on the host first and
 * launches nothing when it returns an error.  Device faults, if any, surface
 * at the caller's next synchronisation of the stream.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage dtype of q, k, v and out.  g, beta and the state are always fp32. */
typedef enum {
    GDN_F32 = 0,
    GDN_BF16 = 1
} gdn_dtype;

/* Algorithm choice.  AUTO takes the chunked form (chunks of 64 tokens) from the
 * length at which it is faster than the token recurrence on MI355X, and the token
 * recurrence below that.  The crossover falls as the work per token grows: with
 * w = n_seqs * n_heads * (head_dim / 128)^2, bf16 switches at 20 tokens for
 * w <= 96, 18 for w <= 192, 16 for w <= 512 and 14 above; fp32 (whose chunked form
 * runs fp32 matrix products) at 48 tokens for w <= 40, 60 for w <= 96, 104 for
 * w <= 192 and 120 above.  The forced values exist so that tests can run either
 * algorithm on any input.
 *
 * The chunked form's chunk-to-chunk pass has two kernels for bf16 rows: one that
 * spreads each (seq, head)'s value rows over several workgroups (fewest steps in
 * sequence per compute unit: AUTO's choice while there are fewer (seq, head) pairs
 * than compute units), and one whole-head workgroup per (seq, head) that brings
 * each chunk's shared operands in once for all value rows (AUTO's choice from one
 * pair per compute unit on; 18-31% faster there on MI355X).  Both give the same
 * bits.  CHUNKED forces the first (and is the only chunked pass for fp32),
 * CHUNKED_HEAD (bf16 only) the second.
 *
 * CHUNKED_LAG (bf16 only; GDN_ERR_ALGO_UNAVAILABLE for fp32) is the chunked form
 * with the chunk-to-chunk pass rewritten so that a chunk's deltas depend on those of
 * the two chunks before it and on the state two chunks old, which takes the state
 * off the serial chain; its workspace is larger (gdn_workspace_size with this
 * value).  It computes the same quantities within the same tolerance, is never
 * chosen by AUTO, and on MI355X it is about twice as slow as CHUNKED at 4,096
 * tokens x 32 heads (each chunk step moves more operand bytes into every compute
 * unit); it is kept so that the comparison can be re-run. */
typedef enum {
    GDN_ALGO_AUTO = 0,
    GDN_ALGO_RECURRENT = 1,
    GDN_ALGO_CHUNKED = 2,
    GDN_ALGO_CHUNKED_LAG = 3,
    GDN_ALGO_CHUNKED_HEAD = 4
} gdn_algo;

/* Status codes: GDN_OK or a negative error. */
enum {
    GDN_OK = 0,
    GDN_ERR_UNSUPPORTED_HEAD_DIM = -1, /* head_dim not accepted by gdn_supports */
    GDN_ERR_BAD_SHAPE = -2,            /* a size is negative or too large     */
    GDN_ERR_NULL_POINTER = -3,         /* a needed pointer is NULL            */
    GDN_ERR_BAD_DTYPE = -4,            /* dtype is not a gdn_dtype value      */
    GDN_ERR_WORKSPACE_TOO_SMALL = -5,  /* workspace_bytes < gdn_workspace_size */
    GDN_ERR_ALGO_UNAVAILABLE = -6,     /* algo is not a gdn_algo value, or not
                                          one the dtype has (CHUNKED_LAG and
                                          CHUNKED_HEAD with fp32) */
    GDN_ERR_MISALIGNED = -7,           /* a pointer is not 16-byte aligned    */
    GDN_ERR_ALIASING = -8,             /* out overlaps an input, or state_out
                                          overlaps state_in without being equal */
    GDN_ERR_HIP = -9,                  /* the HIP runtime refused a launch     */
    GDN_ERR_BAD_FLAGS = -10,           /* unknown bits in gdn_forward_ex flags */
    GDN_ERR_SCRATCH_TOO_SMALL = -11    /* gdn_forward_noalloc: the call needs more
                                          scratch than the library's fixed array */
};

/* Input transforms gdn_forward_ex can apply inside the op (bit mask).  They are
 * the steps that come just before the recurrence in a model layer (the pages
 * count eager torch's version of a layer at ~200 ops: model card, section
 * "Ops", the sentence under the op list):
 *   GDN_PRE_L2NORM_QK  each q and k row (head_dim values) is divided by
 *                      sqrt(sum of its squares + 1e-6), in fp32, before use;
 *                      the epsilon keeps an all-zero row at zero
 *   GDN_PRE_RAW_GATES  g and beta are pre-activations: the op uses
 *                      g := -softplus(g) = -log(1 + exp(g)) as the log-domain
 *                      gate and beta := sigmoid(beta) = 1 / (1 + exp(-beta)) */
enum {
    GDN_PRE_NONE = 0,
    GDN_PRE_L2NORM_QK = 1,
    GDN_PRE_RAW_GATES = 2
};

/* 1 if head_dim is supported, else 0.  Supported widths are the multiples of 32
 * from 32 to 128 (32, 64, 96, 128): a state row is covered by 32 lanes holding
 * head_dim/32 values each, and widths above 128 are not built (model card, the
 * paragraph after the contract bullets, on asking rather than assuming). */
int gdn_supports(int head_dim);

/* Bytes of device workspace gdn_forward needs for these sizes, dtype and
 * algorithm (0 for the token recurrence).  Returns 0 for arguments
 * gdn_forward would reject.  The workspace's contents are internal and need no
 * initialisation; it may be reused by later calls on the same stream. */
size_t gdn_workspace_size(gdn_dtype dtype, int64_t n_seqs, int64_t n_tokens,
                          int64_t n_heads, int head_dim, gdn_algo algo);

/* Run n_tokens gated-delta-rule steps for every (sequence, head).
 *
 *   dtype        storage dtype of q, k, v, out
 *   q, k, v      (n_seqs, n_tokens, n_heads, head_dim), device, read only
 *   g, beta      (n_seqs, n_tokens, n_heads) fp32, device, read only; g is the
 *                log-domain gate and must be finite (exp(g) is the decay)
 *   state_in     (n_seqs, n_heads, head_dim, head_dim) fp32 [value][key],
 *                device, read only; NULL means a zero initial state
 *   out          like q, device, written; the output includes 1/sqrt(head_dim)
 *   state_out    like state_in, device, written with the state after the last
 *                token.  state_out == state_in is allowed (in-place update);
 *                any other overlap, and any overlap of out with an input, is
 *                rejected with GDN_ERR_ALIASING
 *   workspace    device scratch of at least gdn_workspace_size(...) bytes
 *                (may be NULL when that size is 0)
 *   algo         GDN_ALGO_AUTO, or a forced algorithm
 *   stream       a hipStream_t (NULL = the default stream)
 *
 * n_seqs == 0 or n_heads == 0 is a no-op.  n_tokens == 0 copies state_in to
 * state_out (or zero-fills it when state_in is NULL) and writes no output.
 * Every pointer must be 16-byte aligned.  Returns GDN_OK or a negative status;
 * on error nothing is launched.
 *
 * Size limits (a dispatch counts the work-items of its grid in 32 bits): at most
 * 2^27 state rows, n_seqs * n_heads * head_dim (a 64 GiB state at head_dim 128),
 * and, when the chunked form runs, fewer than 2^24 chunks,
 * n_seqs * n_heads * ceil(n_tokens / 64), and 64 token rows of all heads within
 * 4 GiB, 64 * n_heads * head_dim * (element size) < 2^32 (the kernels address a
 * row inside one 64-token chunk in 32 bits; at head_dim 128 this allows 131071
 * heads in fp32, 262143 in bf16).  Larger calls return GDN_ERR_BAD_SHAPE;
 * split the batch or the sequence over several calls (the state carries over). */
int gdn_forward(gdn_dtype dtype, const void *q, const void *k, const void *v,
                const float *g, const float *beta, const float *state_in,
                void *out, float *state_out, int64_t n_seqs, int64_t n_tokens,
                int64_t n_heads, int head_dim, void *workspace,
                size_t workspace_bytes, gdn_algo algo, void *stream);

/* gdn_forward for q and k that hold fewer heads than v: n_key_heads heads
 * shared by the n_heads value heads in the tiled order, value head h reading
 * key (and query) head h % n_key_heads.  That is the mapping the model card
 * names as upstream's ("ggml attention kernels" model card, first bullet
 * after the "Shapes, in torch order" table); with it the caller needs no
 * expanded copy of q and k.
 *
 *   q, k         (n_seqs, n_tokens, n_key_heads, head_dim), device, read only
 *   n_key_heads  >= 1 and a divisor of n_heads (else GDN_ERR_BAD_SHAPE); when
 *                n_heads == 0 the call is a no-op and n_key_heads only has to
 *                be >= 0
 *
 * Every other argument, the result, the workspace size (gdn_workspace_size
 * with the value-head count n_heads), alignment, aliasing and error rules are
 * those of gdn_forward; n_key_heads == n_heads is exactly gdn_forward. */
int gdn_forward_tiled(gdn_dtype dtype, const void *q, const void *k, const void *v,
                      const float *g, const float *beta, const float *state_in,
                      void *out, float *state_out, int64_t n_seqs, int64_t n_tokens,
                      int64_t n_heads, int64_t n_key_heads, int head_dim,
                      void *workspace, size_t workspace_bytes, gdn_algo algo,
                      void *stream);

/* The general form: gdn_forward_tiled plus input transforms.
 *
 *   n_key_heads  as in gdn_forward_tiled (n_heads for one key head per value
 *                head)
 *   flags        GDN_PRE_NONE or an OR of GDN_PRE_L2NORM_QK and
 *                GDN_PRE_RAW_GATES; other bits return GDN_ERR_BAD_FLAGS.  With
 *                GDN_PRE_RAW_GATES, g may hold any finite value.
 *
 * Everything else is as in gdn_forward; flags == GDN_PRE_NONE with
 * n_key_heads == n_heads is exactly gdn_forward. */
int gdn_forward_ex(gdn_dtype dtype, const void *q, const void *k, const void *v,
                   const float *g, const float *beta, const float *state_in,
                   void *out, float *state_out, int64_t n_seqs, int64_t n_tokens,
                   int64_t n_heads, int64_t n_key_heads, int head_dim,
                   unsigned int flags, void *workspace, size_t workspace_bytes,
                   gdn_algo algo, void *stream);

/* gdn_forward_ex for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  There is
 * no workspace argument: the chunked algorithm's scratch space is a fixed array
 * of gdn_noalloc_scratch_bytes() bytes (64 MiB) that the library holds on every
 * GPU it runs on until the process ends.  The call itself allocates nothing (no
 * hipMalloc, hipFree or allocating library routine); the caller still passes
 * inputs and outputs, with the meanings, rules and errors of gdn_forward_ex.
 *
 * A call whose gdn_workspace_size exceeds that array returns
 * GDN_ERR_SCRATCH_TOO_SMALL before any HIP call (nothing is launched); smaller
 * batches or shorter spans fit (the state carries over between calls).  The
 * array's contents need no initialisation and are overwritten by each call.
 * Every call on one GPU shares that GPU's array, so calls that overlap in time on
 * one GPU (on different streams, or from different threads without ordering)
 * race and may return wrong results: order them on one stream. */
int gdn_forward_noalloc(gdn_dtype dtype, const void *q, const void *k, const void *v,
                        const float *g, const float *beta, const float *state_in,
                        void *out, float *state_out, int64_t n_seqs, int64_t n_tokens,
                        int64_t n_heads, int64_t n_key_heads, int head_dim,
                        unsigned int flags, gdn_algo algo, void *stream);

/* Bytes of the fixed scratch array gdn_forward_noalloc uses on each GPU. */
size_t gdn_noalloc_scratch_bytes(void);

/* ---- decode flash attention ("ggml attention kernels" model card, section
 * "flash_attn": the vector variant, a few queries against a key/value cache) ----
 *
 * For sequence s, query head h and query i, with key/value head
 * j = h / (n_heads / n_heads_kv) (grouped-query attention, keys and values read
 * in place with no expanded copy; the card's second bullet under that section):
 *     score_t = scale * (q[s][h][i] . k[s][j][t]) + f16(mask[s][0][i][t])
 *     out[s][i][h] = sum_t softmax_t(score) v[s][j][t]
 * The additive mask is rounded to f16 before use, as the card says its kernel
 * does; all other arithmetic is fp32 (the card's kernel accumulates in f16).
 * A query row with no finite score (fully masked, or n_kv == 0) gives zeros.
 */

/* 1 if the decode attention runs these sizes: 1 <= n_q < 20 (the card's vector
 * variant; a caller falls back to its own attention otherwise) and
 * head_dim_k == head_dim_v in {64, 128, 256}. */
int gdn_flash_attn_supports(int n_q, int head_dim_k, int head_dim_v);

/* Bytes of device workspace gdn_flash_attn needs (0 when the cache is not split
 * across workgroups); 0 for sizes gdn_flash_attn would reject. */
size_t gdn_flash_attn_workspace_size(int64_t n_seqs, int64_t n_heads, int64_t n_heads_kv,
                                     int64_t n_q, int64_t n_kv, int head_dim);

/*   dtype        storage dtype of q, k, v, out
 *   q            (n_seqs, n_heads, n_q, head_dim), device, read only
 *   k, v         (n_seqs, n_heads_kv, n_kv, head_dim), device, read only
 *   mask         (n_seqs, 1, n_q, n_kv) fp32 additive, device, read only, or NULL
 *   out          (n_seqs, n_q, n_heads, head_dim): tokens before heads (the
 *                card's return layout), device, written
 *   n_heads_kv   >= 1 and a divisor of n_heads
 *   scale        multiplies q . k (callers usually pass 1/sqrt(head_dim))
 *   workspace    device scratch of at least gdn_flash_attn_workspace_size(...)
 *   stream       a hipStream_t (NULL = the default stream)
 * Rejects (nothing launched): unsupported sizes (GDN_ERR_UNSUPPORTED_HEAD_DIM
 * for the width, GDN_ERR_BAD_SHAPE for n_q, negative sizes or a non-dividing
 * n_heads_kv), a non-finite scale (GDN_ERR_BAD_SHAPE), null or misaligned
 * pointers, out overlapping an input, a too small workspace.  n_seqs == 0 or
 * n_heads == 0 is a no-op; n_kv == 0 writes zeros.  Size limits: at most 2^24
 * query rows (n_seqs * n_heads * n_q), fewer than 2^31 cached positions (n_kv),
 * and grids that fit one dispatch each (their work-items are counted in 32 bits);
 * else GDN_ERR_BAD_SHAPE. */
int gdn_flash_attn(gdn_dtype dtype, const void *q, const void *k, const void *v,
                   const float *mask, void *out, int64_t n_seqs, int64_t n_heads,
                   int64_t n_heads_kv, int64_t n_q, int64_t n_kv, int head_dim, float scale,
                   void *workspace, size_t workspace_bytes, void *stream);

/* Static, human-readable text for a status code (never NULL). */
const char *gdn_status_string(int status);

/* Library version as 10000*major + 100*minor + patch. */
int gdn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
