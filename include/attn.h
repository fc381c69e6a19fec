/*
 * attn.h -- C ABI of libattn.so: fused masked multi-head attention forward on AMD Instinct
 * MI355X (CDNA4, gfx950).
 *
 * Operation (what every entry point below computes). For batch b, query head hq and query
 * row i:
 *
 *     O[b,hq,i,:] = softmax_j( scale * Q[b,hq,i,:] . K[b,kv,j,:] + mask(b,i,j) ) V[b,kv,j,:]
 *     LSE[b,hq,i] = ln sum_{visible j} exp( scale * Q[b,hq,i,:] . K[b,kv,j,:] + add(b,hq,i,j) )
 *
 * where mask(b,i,j) is 0 for a visible key and -infinity for a hidden one (the causal and
 * valid_len masks below, and attn_fwd_masked's keep mask), and add(b,hq,i,j) is the additive
 * mask of attn_fwd_masked (0 everywhere else); the softmax is taken over the visible keys.
 *
 * - The formula softmax(Q K^T / sqrt(D) + Mask) V over [B,H,N,D] tensors is the one the masked
 *   multi-head attention CUDA article (wzjinhao.cn/news/73578) writes down in section 2.1; the
 *   scale is a caller argument here (the Triton file tiny_flash_attn_triton.py takes it as
 *   sm_scale), and 1/sqrt(D) is the usual value.
 * - The mask hides key j from query i when causal masking is on and j > i (article section 2.2,
 *   causal mask; "Triton Cuda Attention", section "Causal Attention"), or when valid_len is given
 *   and j >= valid_len[b] (article section 2.2, padding by per-sample valid length). Both may be
 *   on at once; a key must pass both (article sections 1.3 and 2.2).
 * - Grouped-query attention: query head hq reads key/value head kv = hq / (Hq / Hkv) (integer
 *   division: consecutive query heads share a KV head), as "Triton Cuda Attention" prescribes
 *   in section "GQA (Grouped-Query Attention)". Hkv = 1 is multi-query attention (section "MQA").
 * - A query row that sees no key (for instance every row of a batch with valid_len[b] = 0) is
 *   defined to output O = 0 exactly and LSE = -infinity, with no NaN (the article, section 3.2,
 *   on fully masked rows).
 * - LSE is the natural-log log-sum-exp of the row's visible scaled scores; a later backward pass
 *   or a merge of partial results over key shards uses it (tiny_flash_attn_triton.py stores the
 *   same quantity in base 2 for its backward pass).
 * - The computation is the tiled online softmax of "Triton Cuda Attention" (section on the
 *   online softmax core algorithm): the N x N score matrix never reaches memory.
 *
 * Numerics: 16-bit inputs with fp32 scores, softmax state and accumulation; the probabilities
 * are rounded to the input type before they multiply V; O is rounded to nearest-even in the
 * input type. With fp16 inputs the row's denominator (and so LSE) is the sum of those rounded
 * probabilities (within 2^-11 relative of the exact sum); with bf16 it is the fp32 sum of the
 * unrounded ones. fp32 inputs (ATTN_F32) stay fp32 throughout. Results are deterministic run to run
 * for the same inputs and shapes.
 *
 * Threading: every call is independent and the library keeps no state between calls except
 * compiled kernels and the static device workspace of attn_bwd_scratch; calls on different
 * streams may run concurrently (attn_bwd_scratch calls excepted, see there). The library
 * allocates no memory.
 */
#ifndef ATTN_H
#define ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of Q, K, V and O. */
typedef enum {
    ATTN_F16 = 0,  /* IEEE binary16 */
    ATTN_BF16 = 1, /* bfloat16 */
    ATTN_F32 = 2   /* IEEE binary32: every entry point */
} attn_dtype_t;

/* Return codes. Argument errors are detected on the host before anything is launched, so a
 * call either queues work or fails without touching memory: the launch-configuration failures
 * the masked multi-head attention CUDA article lists (section 5.2: an invalid configuration
 * from too many threads per block or too much shared memory; section 6.2, its symptom table:
 * launch failures, and wrong outputs from tensors indexed with the wrong layout) surface here as
 * ATTN_ERR_SHAPE, ATTN_ERR_HEAD_DIM and ATTN_ERR_LAYOUT before any launch, and a failure the
 * HIP runtime reports at launch as ATTN_ERR_LAUNCH. attn_status_string describes each code. */
typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_NULL = -1,     /* q, k, v or out is NULL */
    ATTN_ERR_SHAPE = -2,    /* B, Hq, Hkv or N < 1, Hq not a multiple of Hkv, or sizes beyond
                               the limits below */
    ATTN_ERR_HEAD_DIM = -3, /* D is not supported (see attn_fwd / attn_bwd) */
    ATTN_ERR_DTYPE = -4,    /* dtype is not one of attn_dtype_t */
    ATTN_ERR_SCALE = -5,    /* scale is NaN or infinite */
    ATTN_ERR_LAUNCH = -6,   /* the HIP runtime reported an error at launch; query HIP for it */
    ATTN_ERR_ALIAS = -7,    /* out or lse overlaps an input, or out overlaps lse */
    ATTN_ERR_LAYOUT = -8,   /* a pointer is not 16-byte aligned, a stride is negative or not a
                               multiple of 16 bytes, rows are less than D elements apart, or
                               two output rows share memory; for a mask see attn_fwd_masked */
    ATTN_ERR_MASK = -9,     /* mask_type is not one of attn_mask_t */
    ATTN_ERR_WORKSPACE = -10, /* attn_bwd_ws: ws_floats is below 2 * B * Hq * N; attn_fwd_ws:
                                 ws_floats is negative */
    ATTN_ERR_SCRATCH = -11  /* attn_bwd_scratch: 2 * B * Hq * N exceeds ATTN_SCRATCH_FLOATS */
} attn_status_t;

/* Explicit mask kinds of attn_fwd_masked. */
typedef enum {
    ATTN_MASK_NONE = 0,     /* no explicit mask (mask is ignored) */
    ATTN_MASK_KEEP_U8 = 1,  /* uint8 [.., N, N]: nonzero keeps key j for query i, zero hides it */
    ATTN_MASK_ADD = 2       /* [.., N, N] of the input dtype (fp16 or bf16; fp32 for ATTN_F32
                               inputs), added to the scaled score; -inf hides the key */
} attn_mask_t;

/* Size limits checked by attn_fwd_validate: N <= ATTN_MAX_N and
 * B * Hq * ceil(N / 128) <= ATTN_MAX_TILES (one workgroup of 256 work-items per 128-row tile,
 * and one launch holds fewer than 2^32 work-items); with strides, also ((N + 64) * (K or V row
 * stride) + D) * (element size) < 2^31 (the bytes the kernel may address inside one K or V
 * head). */
#define ATTN_MAX_N (1 << 22)
#define ATTN_MAX_TILES 16777215LL

/*
 * attn_fwd -- launch the attention forward described at the top of this file on `stream`.
 *
 *   q          device pointer, [B, Hq, N, D] elements of `dtype`, contiguous (row-major, D
 *              fastest), 16-byte aligned.
 *   k, v       device pointers, [B, Hkv, N, D] elements of `dtype`, contiguous, 16-byte aligned.
 *              With Hkv = 1 this is the same memory as a [B, N, D] tensor.
 *   out        device pointer, [B, Hq, N, D] elements of `dtype`, contiguous, 16-byte aligned;
 *              written completely (including rows with no visible key). Must not overlap q, k,
 *              v or lse.
 *   lse        device pointer to [B, Hq, N] float32, contiguous; NULL means "do not write".
 *   B, Hq, Hkv, N, D
 *              batch, query heads, key/value heads, sequence length (queries and keys share it),
 *              head dimension. Any N >= 1 is accepted; D must be 16, 32, 64, 128 or 256
 *              (attn_bwd too).
 *   scale      multiplier of the dot products (typically 1/sqrt(D)); any finite value.
 *   causal     nonzero hides key j from query i when j > i.
 *   valid_len  device pointer to int32[B], or NULL for no padding mask. Keys j >= valid_len[b]
 *              are hidden for every query of batch b; values are clamped into [0, N]. Only keys
 *              are masked: query rows at or beyond valid_len[b] are computed like any other row.
 *   dtype      ATTN_F16 or ATTN_BF16: 16-bit Q, K, V, O; scores, softmax and accumulation in
 *              fp32; P is rounded to the input type before P V (as the Triton pages do).
 *              ATTN_F32: fp32 Q, K, V, O and fp32 products throughout (the article's kernels
 *              work in fp32), on the fp32 matrix cores; nothing is rounded to 16 bits.
 *   stream     hipStream_t to launch on; NULL is the default stream.
 *
 * Ownership: the caller allocates and owns every buffer; the call is asynchronous and the
 * buffers must stay valid until the stream has finished it. Returns ATTN_OK once the work is
 * queued, an argument error (nothing launched, nothing written; a misaligned pointer is
 * ATTN_ERR_LAYOUT), or ATTN_ERR_LAUNCH.
 */
int attn_fwd(const void *q, const void *k, const void *v, void *out, float *lse, int B, int Hq,
             int Hkv, int N, int D, float scale, int causal, const int32_t *valid_len, int dtype,
             void *stream);

/*
 * attn_fwd_validate -- the argument check attn_fwd performs, on the host only: makes no HIP
 * call and touches no memory behind the pointers (they are compared, never dereferenced).
 * Same arguments and return codes as attn_fwd, except that it never returns ATTN_ERR_LAUNCH.
 */
int attn_fwd_validate(const void *q, const void *k, const void *v, const void *out,
                      const float *lse, int B, int Hq, int Hkv, int N, int D, float scale,
                      int causal, const int32_t *valid_len, int dtype);

/*
 * attn_fwd_strided -- attn_fwd on tensors given by strides, e.g. Q, K, V and O stored as
 * [B, N, H, D] (rows of all heads of one position together), rows padded past D, or K and V
 * shared by every batch (batch stride 0). The Triton kernel of "Triton Cuda Attention" (its
 * forward section) and tiny_flash_attn_triton.py take the same four tensors with full strides,
 * and the masked multi-head attention CUDA article (section 2.1) names both the [B, N, H, D]
 * and the [B, H, N, D] layouts.
 *
 *   q, k, v, out   device pointers as in attn_fwd, 16-byte aligned.
 *   q_strides, k_strides, v_strides, out_strides
 *                  host pointers to three int64 element strides each: batch, head, row (the
 *                  sequence position). The D elements of a row are contiguous. Element
 *                  (b, h, i, d) of a tensor is at ptr + b*s[0] + h*s[1] + i*s[2] + d. NULL means
 *                  the contiguous [B, H, N, D] strides {H*N*D, N*D, D}. The arrays are read
 *                  during the call only.
 *   lse            as in attn_fwd: contiguous [B, Hq, N] float32 or NULL.
 *   all else       as in attn_fwd.
 *
 * Every stride must be >= 0 and a multiple of 16 bytes (8 elements of a 16-bit type, 4 of fp32),
 * and row strides >= D (ATTN_ERR_LAYOUT otherwise). Inputs may share memory with each other
 * (for instance Q, K and V as views of one packed tensor, or a zero batch stride). The output's
 * rows must be distinct (its strides, ordered, must each step past the extent of the smaller
 * ones). For the alias check each tensor counts as the whole byte range from its pointer to the
 * end of its last row, so out must lie outside the ranges of q, k, v and lse. Returns as
 * attn_fwd.
 */
int attn_fwd_strided(const void *q, const int64_t *q_strides, const void *k,
                     const int64_t *k_strides, const void *v, const int64_t *v_strides,
                     void *out, const int64_t *out_strides, float *lse, int B, int Hq, int Hkv,
                     int N, int D, float scale, int causal, const int32_t *valid_len, int dtype,
                     void *stream);

/* attn_fwd_strided_validate -- the host-only argument check of attn_fwd_strided (no HIP call,
 * no pointer dereferenced except the three-element stride arrays). */
int attn_fwd_strided_validate(const void *q, const int64_t *q_strides, const void *k,
                              const int64_t *k_strides, const void *v,
                              const int64_t *v_strides, const void *out,
                              const int64_t *out_strides, const float *lse, int B, int Hq,
                              int Hkv, int N, int D, float scale, int causal,
                              const int32_t *valid_len, int dtype);

/*
 * attn_fwd_masked -- attn_fwd_strided with an explicit mask matrix as well. The masked multi-head
 * attention CUDA article (section 2.2) gives the mask as a [B, N, N] matrix, either a boolean
 * padding mask or, for combined masks, a float matrix that is 0 where the key is allowed and
 * -inf (or a large negative value) where it is not, added to the score before the softmax; the
 * article's formula (section 2.1) adds Mask to Q K^T / sqrt(D).
 *
 *   mask        device pointer, 16-byte aligned; element (b, hq, i, j) at
 *               mask + b*ms[0] + hq*ms[1] + i*ms[2] + j (elements of the mask type).
 *   mask_type   ATTN_MASK_KEEP_U8: key j is visible to query i only where the byte is nonzero.
 *               ATTN_MASK_ADD: the element (in the input dtype: fp16, bf16, or fp32 with
 *               ATTN_F32 inputs) is added to scale * q.k; values
 *               must be finite or -inf (a row whose visible keys all carry -inf, like an empty
 *               row, gives O = 0 and LSE = -inf; LSE includes the added values).
 *               ATTN_MASK_NONE: same as attn_fwd_strided.
 *   mask_strides host pointer to three int64 element strides: batch, query head, query row
 *               (the key index j is contiguous). NULL means a contiguous [B, N, N] mask shared
 *               by every head: {N*N, 0, N}. Use 0 to broadcast a dimension. Strides must be >= 0
 *               and multiples of 16 bytes, and the row stride >= N elements (a ragged N needs a
 *               row padded to a multiple of 16 bytes); otherwise ATTN_ERR_LAYOUT. Also
 *               (N + 128) * row stride bytes < 2^31 (else ATTN_ERR_SHAPE). Rows are read in
 *               16-byte units: the bytes after element N-1 of a row up to the next 16-byte
 *               boundary must be readable (they are inside the row stride) and are ignored.
 *   all else    as in attn_fwd_strided.
 *
 * The explicit mask combines with causal and valid_len: a key is used only if all of them allow
 * it (the article, section 1.3, on stacked masks). The mask may share memory with the inputs but
 * not with out or lse (ATTN_ERR_ALIAS, by byte range). Returns as attn_fwd, or ATTN_ERR_MASK.
 */
int attn_fwd_masked(const void *q, const int64_t *q_strides, const void *k,
                    const int64_t *k_strides, const void *v, const int64_t *v_strides, void *out,
                    const int64_t *out_strides, float *lse, int B, int Hq, int Hkv, int N, int D,
                    float scale, int causal, const int32_t *valid_len, const void *mask,
                    int mask_type, const int64_t *mask_strides, int dtype, void *stream);

/* attn_fwd_masked_validate -- the host-only argument check of attn_fwd_masked. */
int attn_fwd_masked_validate(const void *q, const int64_t *q_strides, const void *k,
                             const int64_t *k_strides, const void *v, const int64_t *v_strides,
                             const void *out, const int64_t *out_strides, const float *lse,
                             int B, int Hq, int Hkv, int N, int D, float scale, int causal,
                             const int32_t *valid_len, const void *mask, int mask_type,
                             const int64_t *mask_strides, int dtype);

/*
 * attn_fwd_ws -- attn_fwd_strided with a caller-owned workspace, for grids that leave the
 * device idle. With few (batch, query head, 128-row query tile) items over long key ranges, one
 * workgroup per query tile leaves CUs idle and the call lasts as long as its longest tile's key
 * loop. When the items fill at most a quarter of what the device runs at once (128 workgroups
 * up to D = 128, 64 at D = 256) and the longest key range holds at least 48 key tiles of 64
 * (3072 keys), the key range of every query tile is cut into chunks of equal numbers of key
 * tiles (the smallest chunk for which all chunks still run at once, 512 workgroups up to
 * D = 128 and 256 at D = 256, and whose partial results the workspace holds);
 * one workgroup per chunk writes the chunk's fp32 output, normalised by its own sum, and its
 * log-sum-exp, and a second kernel combines the chunks of every row:
 *
 *     M = max_c L_c,   O = sum_c 2^(L_c - M) O_c / sum_c 2^(L_c - M),
 *     L = M + log2 sum_c 2^(L_c - M)
 *
 * (L in base 2). Below those bounds a call's time is mostly fixed costs (launch, prologue,
 * epilogue) that a split only adds to, and the call runs as attn_fwd_strided. This is the
 * online-softmax update of "Triton Cuda Attention" (section on the
 * online softmax core algorithm) applied to whole chunks instead of single tiles, and the
 * reason tiny_flash_attn_triton.py keeps the per-row log-sum-exp L. The pages' own Triton
 * kernel fills the device with 64-row query blocks over a (cdiv(L, 64), B * H) grid
 * ("Triton Cuda Attention", complete example); splitting the key range instead keeps the
 * 128-row tiles and shortens the longest workgroup.
 *
 *   ws, ws_floats  device float32 workspace of ws_floats values, 16-byte aligned, owned by the
 *                  caller (scratch: nothing is left in it for the caller). NULL, too small for
 *                  any split, or a grid that fills the device: the call is attn_fwd_strided.
 *                  ws_floats < 0 is ATTN_ERR_WORKSPACE; a used part that overlaps an input or
 *                  output is ATTN_ERR_ALIAS.
 *   others         as in attn_fwd_strided (16-bit dtypes split; ATTN_F32 never splits and
 *                  ignores ws).
 *
 * Fully masked rows (valid_len 0) still give O = 0 and LSE = -inf; rows are combined in a fixed
 * order, so results are deterministic, but they differ from attn_fwd_strided's by rounding.
 */
int attn_fwd_ws(const void *q, const int64_t *q_strides, const void *k, const int64_t *k_strides,
                const void *v, const int64_t *v_strides, void *out, const int64_t *out_strides,
                float *lse, float *ws, int64_t ws_floats, int B, int Hq, int Hkv, int N, int D,
                float scale, int causal, const int32_t *valid_len, int dtype, void *stream);

/* attn_fwd_ws_validate -- the host-only argument check of attn_fwd_ws. */
int attn_fwd_ws_validate(const void *q, const int64_t *q_strides, const void *k,
                         const int64_t *k_strides, const void *v, const int64_t *v_strides,
                         const void *out, const int64_t *out_strides, const float *lse,
                         const float *ws, int64_t ws_floats, int B, int Hq, int Hkv, int N, int D,
                         float scale, int causal, const int32_t *valid_len, int dtype);

/*
 * attn_fwd_workspace_floats -- the workspace size (float32 values) with which attn_fwd_ws
 * splits the key ranges of these sizes as far as it would (B * Hq * ceil(N / 128) * nchunk
 * query tiles of 128 rows, D + 1 values each, plus 4); 0 when the grid fills the device and no
 * split helps; -1 when a size is below 1. Host only.
 */
int64_t attn_fwd_workspace_floats(int B, int Hq, int Hkv, int N, int D, int causal);

/*
 * attn_bwd -- gradients of the attn_fwd output with respect to Q, K and V (contiguous tensors,
 * no explicit mask), given the upstream gradient dO and the forward's own O and LSE.
 * tiny_flash_attn_triton.py stores the log-sum-exp for its backward pass; the pages stop at the
 * forward, and this is the derivative of the forward's definition: with
 * P = exp(scale * q.k - LSE) on the visible keys (the same causal / valid_len masks) and
 * Delta_i = sum_d dO[i,d] O[i,d],
 *
 *     dV = P^T dO,   dP = dO V^T,   dS = P o (dP - Delta),   dQ = scale dS K,   dK = scale dS^T Q,
 *
 * dK and dV summed over the query heads sharing a KV head. LSE is treated as an auxiliary
 * output (no gradient flows into it).
 *
 *   q, k, v      as in attn_fwd (device, [B,Hq,N,D] / [B,Hkv,N,D], contiguous, 16-byte aligned).
 *   out, dout    device, [B,Hq,N,D] of dtype: the forward's O and the gradient of the loss in O.
 *   lse          device float32 [B,Hq,N]: the forward's LSE (required).
 *   dq           device output [B,Hq,N,D] of dtype; dk, dv: device outputs [B,Hkv,N,D] of dtype.
 *                All written completely (rows with no visible key get dQ = 0; keys no query sees
 *                get dK = dV = 0).
 *   ws           device float32 workspace of 2 * B * Hq * N values owned by the caller (the
 *                library allocates nothing); on return ws[0 .. B*Hq*N) holds Delta [B,Hq,N] and
 *                the rest the LSE in base 2 (LSE * log2 e, 0 for rows with no visible key).
 *   dtype        ATTN_F16 / ATTN_BF16: P and dS are rounded to the input type before their
 *                products (as the forward rounds P), accumulation in fp32, gradients rounded to
 *                the input type. ATTN_F32: fp32 tensors and fp32 products throughout.
 *   others       as in attn_fwd.
 *
 * Kernels run on `stream` in order (dQ and Delta, then dK and dV; at D = 256 each in parts
 * over the head dimension: two halves for 16-bit tensors, for fp32 two (dQ) and four (dK, dV)).
 * Outputs must not overlap any input, each other or valid_len
 * (ATTN_ERR_ALIAS); misaligned pointers are ATTN_ERR_LAYOUT. Otherwise returns as attn_fwd.
 */
int attn_bwd(const void *q, const void *k, const void *v, const void *out, const void *dout,
             const float *lse, void *dq, void *dk, void *dv, float *ws, int B, int Hq,
             int Hkv, int N, int D, float scale, int causal, const int32_t *valid_len,
             int dtype, void *stream);

/* attn_bwd_validate -- the host-only argument check of attn_bwd. */
int attn_bwd_validate(const void *q, const void *k, const void *v, const void *out,
                      const void *dout, const float *lse, const void *dq, const void *dk,
                      const void *dv, const float *ws, int B, int Hq, int Hkv, int N, int D,
                      float scale, int causal, const int32_t *valid_len, int dtype);

/*
 * attn_bwd_strided -- attn_bwd on tensors given by (batch, head, row) element strides, as in
 * attn_fwd_strided (every stride a non-negative multiple of 8 elements, rows of D contiguous
 * elements, 16-byte aligned; NULL strides mean contiguous [B, H, N, D]; row strides up to
 * (2^31 - 2D) / (2 (N + 128)) elements). This covers the
 * [B, N, H, D] layout of "Triton Cuda Attention"'s host code and the article's §2.1 without
 * transposes. dq, dk and dv may use layouts of their own; each of their rows must be distinct
 * (ATTN_ERR_LAYOUT otherwise), and no output may overlap an input or another output
 * (ATTN_ERR_ALIAS). lse and ws stay contiguous [B, Hq, N] / [2, B, Hq, N] float32 arrays.
 */
int attn_bwd_strided(const void *q, const int64_t *q_strides, const void *k,
                     const int64_t *k_strides, const void *v, const int64_t *v_strides,
                     const void *out, const int64_t *out_strides, const void *dout,
                     const int64_t *dout_strides, const float *lse, void *dq,
                     const int64_t *dq_strides, void *dk, const int64_t *dk_strides, void *dv,
                     const int64_t *dv_strides, float *ws, int B, int Hq, int Hkv, int N, int D,
                     float scale, int causal, const int32_t *valid_len, int dtype, void *stream);

/* attn_bwd_strided_validate -- the host-only argument check of attn_bwd_strided. */
int attn_bwd_strided_validate(const void *q, const int64_t *q_strides, const void *k,
                              const int64_t *k_strides, const void *v, const int64_t *v_strides,
                              const void *out, const int64_t *out_strides, const void *dout,
                              const int64_t *dout_strides, const float *lse, const void *dq,
                              const int64_t *dq_strides, const void *dk,
                              const int64_t *dk_strides, const void *dv,
                              const int64_t *dv_strides, const float *ws, int B, int Hq, int Hkv,
                              int N, int D, float scale, int causal, const int32_t *valid_len,
                              int dtype);

/*
 * attn_bwd_masked -- attn_bwd_strided plus the explicit mask of attn_fwd_masked (the same mask,
 * type and strides the forward was given; the article's §2.1-2.2 masks): the gradients of that
 * masked forward. The mask is a constant (no gradient). Any dtype (with ATTN_F32 an additive
 * mask is fp32, as in the forward). Returns as attn_bwd_strided; mask
 * errors as attn_fwd_masked (ATTN_ERR_MASK, ATTN_ERR_NULL, ATTN_ERR_LAYOUT, ATTN_ERR_SHAPE, and
 * ATTN_ERR_ALIAS when an output overlaps the mask).
 */
int attn_bwd_masked(const void *q, const int64_t *q_strides, const void *k,
                    const int64_t *k_strides, const void *v, const int64_t *v_strides,
                    const void *out, const int64_t *out_strides, const void *dout,
                    const int64_t *dout_strides, const float *lse, void *dq,
                    const int64_t *dq_strides, void *dk, const int64_t *dk_strides, void *dv,
                    const int64_t *dv_strides, float *ws, int B, int Hq, int Hkv, int N, int D,
                    float scale, int causal, const int32_t *valid_len, const void *mask,
                    int mask_type, const int64_t *mask_strides, int dtype, void *stream);

/* attn_bwd_masked_validate -- the host-only argument check of attn_bwd_masked. */
int attn_bwd_masked_validate(const void *q, const int64_t *q_strides, const void *k,
                             const int64_t *k_strides, const void *v, const int64_t *v_strides,
                             const void *out, const int64_t *out_strides, const void *dout,
                             const int64_t *dout_strides, const float *lse, const void *dq,
                             const int64_t *dq_strides, const void *dk,
                             const int64_t *dk_strides, const void *dv,
                             const int64_t *dv_strides, const float *ws, int B, int Hq, int Hkv,
                             int N, int D, float scale, int causal, const int32_t *valid_len,
                             const void *mask, int mask_type, const int64_t *mask_strides,
                             int dtype);

/*
 * attn_bwd_ws -- attn_bwd_masked with the workspace's size, so that the library may use more of
 * it: with room for fp32 partial sums the dK/dV kernel splits each 128-key tile's (query head,
 * query tile) iterations over up to 16 workgroups (enough for at least four workgroups per
 * compute unit, 1024 on a whole MI355X), and a third kernel adds the parts in a fixed order
 * (deterministic) and rounds once. This fills the device where few key tiles exist (MQA, short
 * sequences, small batches). mask_type
 * ATTN_MASK_NONE (mask and mask_strides ignored) gives attn_bwd_strided; NULL strides mean
 * contiguous tensors, as there.
 *
 *   ws, ws_floats  device float32 workspace of ws_floats values (>= 2 * B * Hq * N, else
 *                  ATTN_ERR_WORKSPACE); attn_bwd_workspace_floats gives the size that allows
 *                  the split, smaller sizes use a smaller split or none. On return ws holds
 *                  Delta and the base-2 LSE as in attn_bwd; the partial sums follow from the
 *                  next 16-byte boundary and are scratch.
 *   others         as in attn_bwd_masked.
 */
int attn_bwd_ws(const void *q, const int64_t *q_strides, const void *k,
                const int64_t *k_strides, const void *v, const int64_t *v_strides,
                const void *out, const int64_t *out_strides, const void *dout,
                const int64_t *dout_strides, const float *lse, void *dq,
                const int64_t *dq_strides, void *dk, const int64_t *dk_strides, void *dv,
                const int64_t *dv_strides, float *ws, int64_t ws_floats, int B, int Hq,
                int Hkv, int N, int D, float scale, int causal, const int32_t *valid_len,
                const void *mask, int mask_type, const int64_t *mask_strides, int dtype,
                void *stream);

/* attn_bwd_ws_validate -- the host-only argument check of attn_bwd_ws. */
int attn_bwd_ws_validate(const void *q, const int64_t *q_strides, const void *k,
                         const int64_t *k_strides, const void *v, const int64_t *v_strides,
                         const void *out, const int64_t *out_strides, const void *dout,
                         const int64_t *dout_strides, const float *lse, const void *dq,
                         const int64_t *dq_strides, const void *dk, const int64_t *dk_strides,
                         const void *dv, const int64_t *dv_strides, const float *ws,
                         int64_t ws_floats, int B, int Hq, int Hkv, int N, int D, float scale,
                         int causal, const int32_t *valid_len, const void *mask, int mask_type,
                         const int64_t *mask_strides, int dtype);

/*
 * attn_bwd_workspace_floats -- the workspace size (float32 values) with which attn_bwd_ws uses
 * its full split for these sizes: 2 * B * Hq * N when no split is needed, else that plus
 * 4 + 2 * split * B * Hkv * N * D. -1 when a size is below 1. Host only.
 */
int64_t attn_bwd_workspace_floats(int B, int Hq, int Hkv, int N, int D);

/*
 * attn_bwd_scratch -- attn_bwd_ws without a workspace argument and without any allocation, for
 * callers that cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). The workspace is a static device array of
 * ATTN_SCRATCH_FLOATS float32 values inside the library: each device the library runs on holds
 * its own copy (32 MiB) until the process ends; its address is looked up once per device, on
 * the first call for a stream of that device. The call allocates nothing (no hipMalloc, no
 * hipFree, no allocating library routine) and, like attn_bwd_ws, only queues kernels.
 *
 * Every call on one device shares that device's array and leaves its contents behind (Delta and
 * the base-2 LSE of its last call, then scratch); nothing in it needs to start at zero. Calls
 * that overlap in time on one device (several streams or host threads) race on the array: the
 * caller orders them, e.g. by one stream.
 *
 *   all arguments  as in attn_bwd_ws (same layouts, masks, dtypes; ws is the static array and
 *                  ws_floats is ATTN_SCRATCH_FLOATS, so small shapes still get the dK/dV split).
 *   returns        ATTN_ERR_SCRATCH when 2 * B * Hq * N > ATTN_SCRATCH_FLOATS (the sizes need
 *                  more workspace than the array holds: use attn_bwd_ws), ATTN_ERR_LAUNCH when
 *                  the runtime cannot give the array's device address, else as attn_bwd_ws.
 */
#define ATTN_SCRATCH_FLOATS (1 << 23)
int attn_bwd_scratch(const void *q, const int64_t *q_strides, const void *k,
                     const int64_t *k_strides, const void *v, const int64_t *v_strides,
                     const void *out, const int64_t *out_strides, const void *dout,
                     const int64_t *dout_strides, const float *lse, void *dq,
                     const int64_t *dq_strides, void *dk, const int64_t *dk_strides, void *dv,
                     const int64_t *dv_strides, int B, int Hq, int Hkv, int N, int D,
                     float scale, int causal, const int32_t *valid_len, const void *mask,
                     int mask_type, const int64_t *mask_strides, int dtype, void *stream);

/* attn_status_string -- a static, NUL-terminated description of a return code (never NULL);
 * the error codes and the failure modes they stand for are listed at attn_status_t (the
 * article's sections 5.2 and 6.2 on launch configuration and failure symptoms). */
const char *attn_status_string(int status);

/* attn_version -- the library's interface version, currently 14 (2 added attn_fwd_strided, 3
 * attn_fwd_masked, 4 attn_bwd, 5 attn_bwd_strided, 6 attn_bwd_masked, 7 ATTN_F32 in attn_bwd
 * and attn_bwd_strided, 8 attn_bwd_ws and attn_bwd_workspace_floats, 9 lowered ATTN_MAX_TILES
 * to what one launch can hold, 10 ATTN_F32 in attn_fwd_masked, 11 ATTN_F32 with a mask in
 * attn_bwd_masked and attn_bwd_ws, 12 ATTN_F32 at D = 256 in the backward, 13
 * attn_bwd_scratch, 14 attn_fwd_ws, attn_fwd_ws_validate and attn_fwd_workspace_floats). */
int attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
