/*
 * attn.h -- C ABI of libattn.so, the MI355X (gfx950) online-softmax attention
 * forward and row-wise online softmax.
 *
 * Plain C: pointers, sizes and a stream handle; no C++ or framework types.
 * Every tensor pointer is a DEVICE pointer owned by the caller; the library
 * never frees, retains or reallocates it.  All calls are asynchronous on the
 * given HIP stream (a hipStream_t passed as void*, NULL = the null stream) and
 * never synchronise the host.  A return of ATTN_OK means "validated and
 * enqueued": a fault while the kernels run surfaces at the caller's next
 * synchronisation, as for any HIP launch.  Argument validation happens before
 * any HIP call, so invalid arguments are reported without touching a device.
 * No exception crosses this boundary.  The library keeps no global state
 * besides a per-thread error detail string, so it is safe to call from
 * several host threads.
 */
#ifndef ONLINE_SOFTMAX_ATTN_H
#define ONLINE_SOFTMAX_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v and o. */
typedef enum {
    ATTN_F32 = 0,          /* IEEE binary32 */
    ATTN_BF16 = 1,         /* bfloat16 (8-bit significand), stored as 16-bit words */
    ATTN_BF16_OUT_F32 = 2  /* q, k, v bfloat16 as ATTN_BF16; o float32 (not rounded to bf16) */
} attn_dtype;

/* Return codes. */
enum {
    ATTN_OK = 0,
    ATTN_ERR_NULL = -1,      /* a required pointer is NULL */
    ATTN_ERR_SHAPE = -2,     /* a size is negative, or M < 1 / n < 1 with work to do */
    ATTN_ERR_HEADDIM = -3,   /* d is not one of the compiled head dims (64, 128) */
    ATTN_ERR_DTYPE = -4,     /* dtype is not an attn_dtype */
    ATTN_ERR_ALIGN = -5,     /* a pointer is not 16-byte aligned */
    ATTN_ERR_OVERFLOW = -6,  /* sizes exceed the kernels' index range */
    ATTN_ERR_HIP = -7,       /* a HIP launch or allocation failed (see attn_last_error_detail) */
    ATTN_ERR_SCALE = -8,     /* scale is NaN or infinite */
    ATTN_ERR_SPLITS = -9,    /* num_splits outside [0, ATTN_MAX_SPLITS] */
    ATTN_ERR_MASK = -10,     /* attn_mask.causal is not one of attn_causal */
    ATTN_ERR_WORKSPACE = -11 /* attn_fwd_masked_noalloc: the split workspace exceeds its static scratch */
};

/* Largest split count attn_fwd_splits accepts. */
#define ATTN_MAX_SPLITS 256

/*
 * attn_fwd -- exact attention forward with the online-softmax recurrence.
 *
 * For every batch b < B, head h < H and query row i < N:
 *   s_j   = scale * <q[b,h,i,:], k[b,h,j,:]>        for visible keys j,
 *   o[b,h,i,:] = sum_j softmax(s)_j * v[b,h,j,:],
 *   lse[b,h,i] = log sum_j e^{s_j}                  (natural log),
 * computed block by block with a running max m and running exponential sum l
 * that rescale the unnormalised accumulator by e^{m_old - m_new} whenever a
 * new key block raises the max; the N x M score matrix never reaches memory.
 * Source: "Online Softmax and Flash Attention" page, eq. (8) (definition and
 * shapes Q [N,K], K and V [M,K]); "从原始Softmax到在线Softmax" page, the
 * online softmax derivation (m, l, o~ recurrences, o = o~/l) and the LSE
 * definition.
 *
 * Visible keys: all j < M when causal == 0; j <= i (and j < M) when causal != 0,
 * i.e. key index greater than query index is masked, counted from 0 in both
 * (top-left aligned when N != M).
 *
 * Arguments
 *   q      [B,H,N,d] dtype, contiguous row-major        (device, read)
 *   k, v   [B,H,M,d] dtype, contiguous row-major        (device, read)
 *   o      [B,H,N,d] dtype, contiguous row-major        (device, written)
 *   lse    [B,H,N] float32                              (device, written)
 *   B, H, N >= 0 (B*H*N == 0 is a no-op returning ATTN_OK); M >= 1
 *   d      head dim, 64 or 128 (compile-time instantiations)
 *   scale  finite float32 used exactly as passed (1/sqrt(d) for the usual form)
 *   causal 0 or non-zero
 *   dtype  ATTN_F32 (fp32 products and accumulation throughout), ATTN_BF16
 *          (bf16 products, fp32 accumulation, probabilities rounded to bf16
 *          before the P.V product, o rounded to nearest-even bf16) or
 *          ATTN_BF16_OUT_F32 (the same arithmetic with o written as float32:
 *          the output keeps the fp32 accumulation's precision)
 *   stream hipStream_t as void*
 * o must not overlap q, k, v or lse.  q, k, v, o and lse must be 16-byte
 * aligned.  Per-head sizes N*d and M*d must each be below 2^31 elements and
 * B*H below 2^31.
 *
 * Errors: ATTN_ERR_NULL, _SHAPE, _HEADDIM, _DTYPE, _ALIGN, _OVERFLOW, _SCALE
 * before any HIP call; ATTN_ERR_HIP if a launch or the split workspace
 * allocation fails.  Outputs are unspecified after an error.
 */
int attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
             int64_t B, int64_t H, int64_t N, int64_t M, int d,
             float scale, int causal, int dtype, void *stream);

/*
 * attn_fwd_splits -- attn_fwd with an explicit split count over the keys.
 *
 * num_splits == 0 lets the library choose (what attn_fwd does).  num_splits
 * == 1 forces the single-pass kernel.  num_splits >= 2 divides the keys into
 * that many contiguous ranges, computes each range's normalised partial
 * output O_s and log-sum-exp lse_s, and merges them:
 *   lse = log sum_s e^{lse_s},   o = sum_s e^{lse_s - lse} O_s,
 * which is the block merge of the online recurrence (the "从原始Softmax到在线
 * Softmax" page, merge form of the m / l / o~ update).  An empty range has
 * lse_s = -inf and weight 0.  The partials live in a workspace allocated
 * with hipMallocAsync and freed with hipFreeAsync on the same stream.
 * Every split count gives the same result up to rounding.
 *
 * Arguments and errors as attn_fwd, plus ATTN_ERR_SPLITS when num_splits < 0
 * or num_splits > ATTN_MAX_SPLITS.
 */
int attn_fwd_splits(const void *q, const void *k, const void *v, void *o, float *lse,
                    int64_t B, int64_t H, int64_t N, int64_t M, int d,
                    float scale, int causal, int dtype, int num_splits, void *stream);

/*
 * Masks for attn_fwd_masked.  The pages leave mask() open ("Online Softmax and
 * Flash Attention" page, eq. (8)).  Two kinds: masks whose visible keys form
 * a prefix of each row (causal alignments, key lengths), and an additive
 * score bias, the elementwise reading of mask(): the score of query i and
 * key j becomes scale * <q_i, k_j> + bias_ij, and a bias of -inf masks.
 */
typedef enum {
    ATTN_CAUSAL_NONE = 0,         /* no causal mask */
    ATTN_CAUSAL_TOP_LEFT = 1,     /* key j masked for query i when j > i (as attn_fwd's causal) */
    ATTN_CAUSAL_BOTTOM_RIGHT = 2  /* key j masked when j > i + M - N: the last query sees every key */
} attn_causal;

typedef struct attn_mask {
    int causal;             /* one of attn_causal */
    const int32_t *kv_len;  /* [B] valid key count per batch (device, int32, 4-byte aligned): keys
                               j >= kv_len[b] are masked (values clamped to [0, M]); NULL = M for all */
    const float *bias;      /* additive score bias, fp32 (device, 16-byte aligned), or NULL: the
                               bias of (b, h, i, j) is bias[b*bias_stride_b + h*bias_stride_h +
                               i*bias_stride_n + j], j < M contiguous.  Values finite or -inf. */
    int64_t bias_stride_b;  /* strides in elements: >= 0 (0 broadcasts) and multiples of 4 */
    int64_t bias_stride_h;
    int64_t bias_stride_n;
} attn_mask;

/*
 * attn_fwd_masked -- attn_fwd_splits with a mask.
 *
 * The masks combine: key j of batch b is visible to query i when j < kv_len[b]
 * and the causal rule (if any) allows it; the visible scores get the bias
 * added.  A query row with no visible key, or whose visible scores are all
 * -inf, gets o = 0 and lse = -inf (an empty softmax sum).  lse is taken over
 * the biased scores.  mask == NULL means no mask.
 *
 * Arguments and errors as attn_fwd_splits, plus ATTN_ERR_MASK for an unknown
 * causal mode, ATTN_ERR_ALIGN for a misaligned kv_len or bias (pointer or a
 * stride not a multiple of 4), ATTN_ERR_SHAPE for a negative bias stride and
 * ATTN_ERR_OVERFLOW when the bias spans 4 GiB or more from its base (the
 * kernels address it with 32-bit offsets).  kv_len and bias are read by the
 * kernels (asynchronously, on `stream`); they are not validated on the host.
 * Calls with a bias run on the bias instantiations of the bf16 kernels (or
 * the fp32 kernel), never the decode kernel, and attn_fwd_plan does not
 * describe them.
 */
int attn_fwd_masked(const void *q, const void *k, const void *v, void *o, float *lse,
                    int64_t B, int64_t H, int64_t N, int64_t M, int d,
                    float scale, const attn_mask *mask, int dtype, int num_splits, void *stream);

/*
 * attn_fwd_masked_noalloc -- attn_fwd_masked for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.
 *
 * Same arguments, plan, kernels and results as attn_fwd_masked (bit for
 * bit), but a split plan's partials (num_splits * B*H*N * (d + 1) * 4 bytes)
 * go to a static device array of ATTN_NOALLOC_SCRATCH_BYTES bytes that the
 * library holds on each GPU it runs on until the process ends; nothing is
 * allocated or freed.  The array of the current device is used (the stream
 * must belong to it).  Every call on one GPU shares that GPU's array: calls
 * that overlap on one GPU (other streams, other host threads) race, so the
 * caller orders them.  Nothing in the array needs clearing between calls.
 *
 * Errors as attn_fwd_masked, plus ATTN_ERR_WORKSPACE, before any HIP call,
 * when the split workspace would exceed ATTN_NOALLOC_SCRATCH_BYTES (choose
 * fewer splits, or num_splits = 1 for the single pass, which needs none).
 */
#define ATTN_NOALLOC_SCRATCH_BYTES 33554432
int attn_fwd_masked_noalloc(const void *q, const void *k, const void *v, void *o, float *lse,
                            int64_t B, int64_t H, int64_t N, int64_t M, int d,
                            float scale, const attn_mask *mask, int dtype, int num_splits, void *stream);

/*
 * attn_fwd_kv_outer -- the same attention as attn_fwd, computed in the
 * key/value-outer loop order of the first FlashAttention formulation
 * ("从原始Softmax到在线Softmax" page, the blocked online-softmax code under
 * "softmax实际代码实现": key/value blocks outer, query blocks inner, each
 * query block's normalised output, max and sum written back after every
 * key/value block).  Provided to measure what the query-outer order of
 * attn_fwd saves: per query tile and key block, the row state makes a round
 * trip through HBM.  One kernel launch per 64-key block.
 *
 * Arguments as attn_fwd (causal = top-left); bf16 only (ATTN_ERR_DTYPE
 * otherwise).  Allocates its fp32 row-state workspace (B*H*N*(d+2)*4 bytes)
 * stream-ordered on `stream`.
 */
int attn_fwd_kv_outer(const void *q, const void *k, const void *v, void *o, float *lse,
                      int64_t B, int64_t H, int64_t N, int64_t M, int d,
                      float scale, int causal, int dtype, void *stream);

/*
 * online_softmax -- row-wise softmax with the one-pass normaliser.
 *
 * For each row r < rows of x [rows, n] (float32, row-major):
 *   pass 1: running max m and running sum s over the row,
 *           m_i = max(m_{i-1}, x_i), s_i = s_{i-1} e^{m_{i-1}-m_i} + e^{x_i-m_i},
 *           kept per lane over strided elements and merged across lanes with
 *           the same rule;
 *   pass 2: y[r,i] = e^{x[r,i] - m} / s.
 * Source: "Online Softmax and Flash Attention" page, section "Online softmax",
 * eq. (3)-(7); "Softmax与Flash-Attention" page, online-softmax derivation.
 *
 * Arguments
 *   x     [rows, n] float32 (device, read);  y [rows, n] float32 (device, written)
 *   rows >= 0 (0 is a no-op), n >= 1 when rows > 0
 *   stream hipStream_t as void*
 * x and y must be 16-byte aligned and may be the same buffer (in place).
 * rows * n must be below 2^62 and n below 2^31.
 * Errors: ATTN_ERR_NULL, _SHAPE, _ALIGN, _OVERFLOW before any HIP call;
 * ATTN_ERR_HIP if the launch fails.  A row whose entries are all -inf gives NaN.
 */
int online_softmax(const float *x, float *y, int64_t rows, int64_t n, void *stream);

/*
 * online_softmax_lse -- online_softmax that also returns each row's
 * log-sum-exp, LSE_r = m + log s = log sum_i e^{x[r,i]} (natural log), the
 * normaliser's two numbers folded into one ("从原始Softmax到在线Softmax" page,
 * "softmax形式推导": log-softmax = x - LSE).
 *
 * Arguments as online_softmax, plus
 *   lse   [rows] float32 (device, written, 4-byte aligned), or NULL;
 *   y     may be NULL: then only the LSE is computed, in one read of x
 *         (pass 2 is skipped); y and lse must not both be NULL.
 * Errors as online_softmax (ATTN_ERR_NULL when x is NULL or both outputs
 * are).  A row whose entries are all -inf has LSE = -inf (and y NaN).
 */
int online_softmax_lse(const float *x, float *y, float *lse, int64_t rows, int64_t n, void *stream);

/* Static, human-readable text for a return code (never NULL). */
const char *attn_strerror(int code);

/*
 * softmax_xent -- softmax cross-entropy of each row against a class label,
 * with the log-sum-exp taken in one pass by the online normaliser.
 *
 *   loss[i] = LSE_i - x[i, labels[i]],   LSE_i = log sum_j e^{x[i,j]}  (natural log)
 *   mean    = (1/rows) sum_i loss[i]
 *
 * The loss of a row is the negated log probability of its label under the
 * row's softmax, and the batch loss is their mean ("从原始Softmax到在线Softmax"
 * page, "softmax实际代码实现" and "softmax形式推导"); the LSE is formed with
 * the one-pass normaliser of the "Online Softmax and Flash Attention" page,
 * section "Online softmax", eq. (3)-(7), so the logits are read once.
 *
 * x      [rows, n] fp32 logits, row-major, device, 16-byte aligned (read only)
 * labels [rows] int64 class indices, device, 8-byte aligned (read only); a
 *        label outside [0, n) makes that row's loss NaN (and so the mean)
 * loss   [rows] fp32, device, written
 * lse    [rows] fp32, device, written; may be NULL
 * mean   one fp32, device, written; may be NULL.  Added in fp64 in a fixed
 *        order (deterministic).
 * All buffers are caller-owned; the call is asynchronous on `stream` (a
 * hipStream_t; NULL = the null stream) and allocates nothing.
 *
 * Errors (before any HIP call): ATTN_ERR_SHAPE for rows < 0, n < 0, or
 * n < 1 with rows > 0; ATTN_ERR_NULL for a NULL x, labels or loss;
 * ATTN_ERR_ALIGN for misaligned pointers; ATTN_ERR_OVERFLOW when rows * n
 * or n exceeds the index range.  rows == 0 is a no-op returning ATTN_OK
 * (mean is not written).  A row of only -inf logits has LSE -inf and a NaN
 * loss.
 */
int softmax_xent(const float *x, const int64_t *labels, float *loss, float *lse, float *mean, int64_t rows,
                 int64_t n, void *stream);

/*
 * attn_fwd_plan -- the work decomposition attn_fwd_splits would use, without
 * launching anything (host only; needs no GPU).
 *
 * Returns the name of the kernel that computes the attention itself (one of
 * "attn_fwd_bf16_w8_kernel", "attn_fwd_bf16_kh_kernel", "attn_fwd_bf16_kernel",
 * "attn_fwd_f32_kernel", "attn_fwd_f32_small_kernel", "attn_decode_kernel"; a
 * static string, not to be freed) and stores in
 * *splits (if splits is not NULL) the number of key splits: 1 for a single
 * pass, >= 2 when the kernel writes partials that the merge kernel combines.
 * Returns NULL (and *splits = 0) for arguments attn_fwd_splits would reject
 * or for which it has nothing to compute (B, H or N zero).
 */
const char *attn_fwd_plan(int64_t B, int64_t H, int64_t N, int64_t M, int d, int dtype, int num_splits,
                          int *splits);

/* Detail of the last ATTN_ERR_HIP on the calling thread ("" if none). */
const char *attn_last_error_detail(void);

#ifdef __cplusplus
}
#endif

#endif /* ONLINE_SOFTMAX_ATTN_H */
