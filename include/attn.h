/*
 * attn.h -- C ABI of libattn: the fused attention forward with a pluggable
 * normalizer, for AMD Instinct MI355X (gfx950).
 *
 *     out = N( mask( softcap( scaling * Q K^T ) ) ) V        (grouped-query)
 *
 * N is one of softmax, softmax1, sparsemax, 1.5-entmax ("HF Attention
 * Normalizers", section "Supported Normalizers").  The arguments follow the
 * backend contract of the transformers "Attention" wiki page (factory.ai,
 * "What every backend must support": query/key/value after rotary, the mask,
 * scaling and is_causal; the output) and the paged signature of "HF Attention
 * Normalizers", "Differentiable Paged Attention" (query, key_cache,
 * value_cache, block_table, sequence_lengths, block_size, normalizer).
 *
 * Conventions shared by every entry point
 *   - Ownership: the caller owns every buffer.  The library never allocates,
 *     frees or synchronizes inside attn_fwd; it validates, enqueues kernels on
 *     the caller's stream and returns.  It keeps no mutable global state apart
 *     from a thread-local error message, so calls on different streams and
 *     threads are independent.
 *   - Pointers: every data pointer is a DEVICE pointer unless stated
 *     otherwise; the descriptor structs themselves are HOST memory and are only
 *     read during the call.
 *   - Errors: strict.  Every entry point returns an attn_status; nothing falls
 *     back to another path ("HF Attention Normalizers", "Strict vs Fallback
 *     Mode": unsupported requests raise a clear error).  On an error no kernel
 *     has been enqueued, except ATTN_E_LAUNCH, which reports the HIP error of
 *     a launch.  attn_last_error_detail() names the failing check.
 *   - Dropout and returned attention weights are not part of this forward.
 */
#ifndef ATTN_H_
#define ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_ABI_VERSION 8

/* Status codes. */
typedef enum attn_status {
  ATTN_OK = 0,
  ATTN_E_INVALID = 1,      /* null pointer, shape/stride/param inconsistency          */
  ATTN_E_UNSUPPORTED = 2,  /* valid request outside what this library implements      */
  ATTN_E_WORKSPACE = 3,    /* workspace missing or smaller than attn_fwd_workspace_bytes */
  ATTN_E_LAUNCH = 4        /* a HIP kernel launch failed                               */
} attn_status;

/* The normalizer N ("Supported Normalizers"):
 *   SOFTMAX   exp(s_i) / sum_j exp(s_j)
 *   SOFTMAX1  exp(s_i) / (1 + sum_j exp(s_j))         (Softmax-N with n = 1)
 *   SPARSEMAX max(s_i - tau, 0),        tau such that the weights sum to 1
 *   ENTMAX15  max(s_i / 2 - tau, 0)^2,  tau such that the weights sum to 1   */
typedef enum attn_normalizer {
  ATTN_SOFTMAX = 0,
  ATTN_SOFTMAX1 = 1,
  ATTN_SPARSEMAX = 2,
  ATTN_ENTMAX15 = 3
} attn_normalizer;

typedef enum attn_dtype {
  ATTN_F32 = 0,   /* IEEE binary32                              */
  ATTN_BF16 = 1   /* bfloat16 (upper half of a binary32)        */
} attn_dtype;

/* A strided 4-D device tensor.  Strides are in ELEMENTS; the last dimension
 * must be contiguous (stride[3] == 1) and the other strides >= 0.
 *   q, out : [B, Hq, Lq, D]
 *   k, v   : contiguous KV  -> [B, Hkv, Lk, D]
 *            paged KV       -> caches [num_blocks, block_size, Hkv, D]      */
typedef struct attn_tensor {
  void* data;
  int32_t dtype;         /* attn_dtype; q, k, v and out must agree */
  int32_t reserved;      /* must be 0 */
  int64_t shape[4];
  int64_t stride[4];
} attn_tensor;

/* Paged KV cache ("Differentiable Paged Attention": the kernel reads the
 * physical pages through the block table; no gathered K/V is built).
 * Logical token t of sequence b lives in physical page
 * block_table[b * max_blocks + t / block_size], slot t % block_size.
 * Entries past ceil(seq_lens[b] / block_size) are never read (use -1);
 * slots past seq_lens[b] in the last page are never read.  The host cannot
 * see seq_lens, so max_blocks * block_size bounds every sequence: a larger
 * seq_lens[b] is a caller error the kernels clamp to that bound.          */
typedef struct attn_paged_kv {
  const int32_t* block_table;  /* device, int32 [B, max_blocks], row-major */
  const int32_t* seq_lens;     /* device, int32 [B], 0 <= seq_lens[b]      */
  int32_t block_size;          /* tokens per page, > 0; equals k->shape[1]  */
  int32_t max_blocks;          /* > 0; row length of block_table           */
} attn_paged_kv;

/* Block-sparse key mask in compressed-row form: FlexAttention's
 * BlockMask.from_kv_blocks with a no-op mask_mod, i.e. explicit full-block
 * CSR masks ("HF Attention Normalizers", "Important Limitations": such
 * masks run without dense-mask expansion).  Query rows are grouped in
 * blocks of block_q (row i in block i / block_q), keys in blocks of block_k;
 * query block r of (b, h) may attend to the key blocks
 * kv_indices[b, h', r, 0 .. kv_num_blocks[b, h', r] - 1] (h' = h, or 0 when
 * num_heads == 1), every key of a listed block included.  Causal, window and
 * live-length masking still apply on top.  Entries must be ascending; an
 * entry outside [0, ceil(Lk / block_k)) or not above its predecessor is
 * ignored, and counts are clamped to [0, max_kv_blocks].  Block indices
 * count from key 0 and query 0 (top-left), independently of the
 * bottom-right causal alignment.  Contiguous K/V only (no paged cache, no
 * packed batch).  block_q == 128 with block_k a multiple of 64 runs on the
 * matrix-core kernels (bf16, head dim 64/128/256); any other block shape on
 * the per-row kernel (at most 16384 key blocks).                           */
typedef struct attn_block_mask {
  const int32_t* kv_num_blocks;  /* device int32 [B, num_heads, ceil(Lq / block_q)] */
  const int32_t* kv_indices;     /* device int32 [B, num_heads, ceil(Lq / block_q), max_kv_blocks] */
  int32_t block_q;               /* > 0 */
  int32_t block_k;               /* > 0 */
  int32_t num_heads;             /* 1 (shared by all query heads) or Hq */
  int32_t max_kv_blocks;         /* >= 0 */
} attn_block_mask;

/* Forward parameters.
 *   causal  : keep key j for query i iff j <= i + (L - Lq), L the live key
 *             count (bottom-right alignment: "Packed Variable-Length
 *             Attention"; mask_mod "q_idx >= k_idx" of the "attention
 *             interface" page, "flexattention patterns").
 *   window  : 0 = none; else also keep only (i + L - Lq) - j < window (the
 *             sliding-window pattern of the same page).  Requires causal.
 *   softcap : 0 = none; else score <- softcap * tanh(score / softcap),
 *             applied after scaling and before the mask ("Attention
 *             variants", parameter table: logit_softcap).  Must be >= 0.
 *   scaling : multiplies Q K^T; must be finite.
 *   sinks   : NULL, or (softmax1 only) device float32 [Hq]: per query head
 *             h the logit of softmax1's virtual key (value 0) in place of 0,
 *             i.e. learned attention sinks, one more per-head term in the
 *             softmax's denominator ("Attention variants: what to open up,
 *             and how far", "What cannot be drawn today"):
 *             w_j = exp(s_j) / (exp(sinks[h]) + sum_k exp(s_k)).  The logit
 *             is used as given (no scaling, no softcap); values must be
 *             finite.  Any other normalizer with sinks != NULL is
 *             ATTN_E_INVALID.
 *   block_mask : NULL, or a host descriptor of a block-sparse key mask
 *             (attn_block_mask; its arrays are on the device).            */
typedef struct attn_params {
  int32_t normalizer;  /* attn_normalizer */
  int32_t causal;      /* 0 or 1 */
  int32_t window;      /* >= 0 */
  float softcap;
  float scaling;
  const float* sinks;  /* NULL or device float32 [Hq] (softmax1) */
  const attn_block_mask* block_mask;  /* NULL or host descriptor */
} attn_params;

/* attn_fwd -- enqueue the forward on `stream` (a hipStream_t; NULL = the
 * default stream).
 *
 *   q, k, v   : input descriptors (see attn_tensor).  Hq % Hkv == 0; query
 *               head h reads key/value head h / (Hq / Hkv).
 *   paged     : NULL for contiguous K/V, else the paged cache descriptor
 *               (then k, v are the caches; queries align bottom-right
 *               against each sequence's own length).
 *   p         : parameters (host struct).
 *   out       : [B, Hq, Lq, D], same dtype as q, written in full (rows with
 *               no visible key get zeros).
 *   row_stats : NULL, or device float32 [B, Hq, Lq, 2], contiguous:
 *               softmax / softmax1 -> (m, l): the weights are exp(s - m) / l
 *               (softmax1: m = max(b, max s), l includes exp(b - m), with
 *               b = 0 or the head's sink logit);
 *               sparsemax / entmax15 -> (tau, k): threshold (in the s/2
 *               domain for entmax15) and support size, as a float.
 *               Rows with no visible key: (-inf, 0), (b, 1), (+inf, 0).
 *   workspace : device scratch of at least attn_fwd_workspace_bytes(...)
 *               bytes (may be NULL when that size is 0); its contents on entry
 *               are ignored and on return are unspecified.  It must not be
 *               used by another call that runs concurrently.
 *
 * Supported: dtype F32 or BF16, D in 1..256, contiguous or paged, any Lq.
 * BF16 prefill with D in {64, 128, 256} runs on the matrix-core (MFMA)
 * kernels and BF16 paged decode (Lq == 1) on the split-KV kernels; every
 * other supported case runs on a plain per-row kernel.
 * Returns ATTN_OK, or an error code (see attn_status); inputs are not read
 * and outputs not written on an error other than ATTN_E_LAUNCH.           */
int attn_fwd(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
             const attn_paged_kv* paged, const attn_params* p,
             const attn_tensor* out, float* row_stats,
             void* workspace, size_t workspace_bytes, void* stream);

/* attn_fwd_noalloc -- attn_fwd for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same arguments minus the workspace, the same
 * kernels and results.  Where attn_fwd needs a workspace (paged decode), it
 * uses a fixed 128 MiB array of this library in device memory instead (one
 * per GPU the library runs on, held until the process ends); a request
 * whose attn_fwd_workspace_bytes exceeds 128 MiB returns ATTN_E_WORKSPACE.
 * Nothing is allocated or freed: no hipMalloc, hipFree or allocating
 * library routine.  Its contents on entry are ignored (every byte a call
 * reads is written by that call first).  All calls on one GPU share that
 * array: calls that overlap in time on one GPU (on different streams, or
 * from different threads) race and produce undefined results -- serialize
 * them.  Errors as attn_fwd.                                               */
int attn_fwd_noalloc(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                     const attn_paged_kv* paged, const attn_params* p,
                     const attn_tensor* out, float* row_stats, void* stream);

/* Packed variable-length batch ("HF Attention Normalizers", "Packed
 * Variable-Length Attention": FlashAttention-style packed Q/K/V with
 * cumulative sequence lengths, GQA, different Q/K lengths and per-request
 * bottom-right causal alignment).  Request r owns query tokens
 * [cu_seqlens_q[r], cu_seqlens_q[r+1]) and key tokens
 * [cu_seqlens_k[r], cu_seqlens_k[r+1]); it attends like a batch entry of
 * its own (causal / window aligned bottom-right against its key count).
 * The arrays must start at 0 and be non-decreasing, with the last entries
 * at most the packed token counts; values outside that range are clamped
 * into it on the device.  max_seqlen_q must be >= every request's query
 * count (rows of a longer request beyond it are not computed); query tokens
 * outside every request are not written.                                   */
typedef struct attn_varlen {
  const int32_t* cu_seqlens_q;  /* device, int32 [num_seqs + 1] */
  const int32_t* cu_seqlens_k;  /* device, int32 [num_seqs + 1] */
  int32_t num_seqs;             /* >= 0 */
  int32_t max_seqlen_q;         /* >= 0 */
} attn_varlen;

/* attn_fwd_varlen -- attn_fwd over a packed variable-length batch.
 *   q, out : [1, Hq, total_q, D] (a packed [total_q, Hq, D] array is the
 *            view with strides {., D, Hq*D, 1});
 *   k, v   : [1, Hkv, total_k, D] likewise;
 *   row_stats : NULL or device float32 [1, Hq, total_q, 2], contiguous.
 * Parameters, dtypes, kernels and errors as attn_fwd (no paged cache; no
 * workspace is needed: workspace may be NULL).                             */
int attn_fwd_varlen(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                    const attn_varlen* varlen, const attn_params* p,
                    const attn_tensor* out, float* row_stats,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Kernel family a call runs on (attn_fwd_path, attn_fwd_varlen_path,
 * attn_bwd_path).  The selection is a fixed function of dtype, head dim,
 * layout, alignment and size; it never changes at run time ("HF Attention
 * Normalizers", "Strict vs Fallback Mode").  The per-row kernels (one wave
 * per query row, fp32 arithmetic, scores recomputed per pass) are the
 * correctness path for everything the tiled kernels do not take, one to two
 * orders of magnitude slower on large bf16 problems.                       */
typedef enum attn_path {
  ATTN_PATH_NONE = 0,          /* nothing to compute (an empty extent)          */
  ATTN_PATH_PREFILL_MFMA = 1,  /* tiled matrix-core prefill kernels             */
  ATTN_PATH_DECODE_SPLIT = 2,  /* split-KV paged decode kernels                 */
  ATTN_PATH_PER_ROW = 3,       /* per-row forward kernel                        */
  ATTN_PATH_BWD_MFMA = 4,      /* matrix-core backward kernels                  */
  ATTN_PATH_BWD_PER_ROW = 5    /* per-row backward kernels                      */
} attn_path;

/* attn_fwd_path -- the attn_path that attn_fwd would take for exactly these
 * arguments (host computation only: nothing is read from or written to
 * device memory, nothing is enqueued).  Validates like attn_fwd (the data
 * pointers enter only through their alignment) and writes the path to
 * *path (host pointer).  Returns ATTN_OK or the error attn_fwd would give
 * before launching.                                                        */
int attn_fwd_path(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                  const attn_paged_kv* paged, const attn_params* p,
                  const attn_tensor* out, int* path);

/* attn_fwd_varlen_path -- the same for attn_fwd_varlen. */
int attn_fwd_varlen_path(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                         const attn_varlen* varlen, const attn_params* p,
                         const attn_tensor* out, int* path);

/* attn_fwd_workspace_bytes -- workspace size attn_fwd needs for these
 * arguments (host computation only; no device access).  Validates the same
 * way attn_fwd does and writes the size to *bytes (host pointer).          */
int attn_fwd_workspace_bytes(const attn_tensor* q, const attn_tensor* k,
                             const attn_tensor* v, const attn_paged_kv* paged,
                             const attn_params* p, size_t* bytes);

/* attn_bwd -- gradients of attn_fwd ("HF Attention Normalizers",
 * "Important Limitations": the fused backward recomputes the weights from
 * the saved row statistics -- row max and denominator for softmax1, one
 * threshold per row for the sparse normalizers).  For the same q, k, v and
 * parameters as a forward that wrote `row_stats` (and optionally its output
 * `out`), and the upstream gradient dout of that output:
 *   dq   [B, Hq, Lq, D]  <- dL/dq
 *   dk, dv [B, Hkv, Lk, D] <- dL/dk, dL/dv (summed over each key/value
 *                            head's query heads)
 *   dsinks : NULL, or (softmax1) device float32 [Hq] <- dL/d(sink logit)
 *            (the logits are p->sinks, or 0 when that is NULL).
 * dout, dq match q in shape and dtype; dk, dv match k, v; last dimension
 * contiguous.  The sparse normalizers' gradients are the usual ones of the
 * piecewise-smooth maps (sparsemax: dP minus its mean over the support, on
 * the support; 1.5-entmax: sqrt(p) (dP - sum sqrt(p) dP / sum sqrt(p))).
 * out : NULL, or the forward's output [B, Hq, Lq, D] (dtype of q, last
 *       dimension contiguous, 16-byte aligned).  softmax / softmax1 then take
 *       the row constant of the Jacobian, sum_j p dP = dout . out, from it
 *       and skip one pass over the keys; the sparse normalizers ignore it.
 * Contiguous K/V.  p->block_mask as in the forward: keys outside the listed
 * blocks carry no weight and receive no gradient (at most 16384 query
 * blocks and 16384 key blocks; the per-row kernels).  bf16 inputs with
 * D = 64, 128 or 256 (16-byte aligned, strides multiples of 8 elements) and
 * no block mask run on the matrix cores (bf16 operands, fp32
 * accumulation); everything else on per-row fp32 kernels.
 * Every output is written in full.  workspace: attn_bwd_workspace_bytes
 * (the larger of 8 bytes per query row, and 384 bytes per 32 query rows of
 * each (batch, head) plus 4 bytes per query row, rounded up to 256 bytes,
 * plus, with grouped-query heads and fewer than 1024 blocks of 128 keys
 * over (batch, kv head), 8 bytes per (batch, query head, key, dim)).
 * Errors as attn_fwd.                                                     */
int attn_bwd(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
             const attn_tensor* out, const attn_tensor* dout, const float* row_stats,
             const attn_params* p,
             const attn_tensor* dq, const attn_tensor* dk, const attn_tensor* dv,
             float* dsinks, void* workspace, size_t workspace_bytes, void* stream);

/* attn_bwd_varlen -- attn_bwd over a packed variable-length batch ("HF
 * Attention Normalizers", "Packed Variable-Length Attention": the packed
 * path carries a full backward).  Layouts as attn_fwd_varlen: q, out,
 * dout, dq [1, Hq, total_q, D]; k, v, dk, dv [1, Hkv, total_k, D];
 * row_stats [1, Hq, total_q, 2] from the attn_fwd_varlen call with the same
 * q, k, v, varlen and parameters.  Each request is differentiated as a
 * batch entry of its own; dk / dv sum over the request's query heads of
 * each key/value head only.  Tokens outside every request get zero
 * gradients (every output is written in full); dsinks sums over all
 * requests.  max_seqlen_q is not used.  No block mask.  Runs on the per-row
 * fp32 kernels.  workspace: 8 bytes per (query head, packed query token)
 * (attn_bwd_workspace_bytes of the packed descriptors is enough).  Errors
 * as attn_bwd.                                                            */
int attn_bwd_varlen(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                    const attn_tensor* out, const attn_tensor* dout, const float* row_stats,
                    const attn_varlen* varlen, const attn_params* p,
                    const attn_tensor* dq, const attn_tensor* dk, const attn_tensor* dv,
                    float* dsinks, void* workspace, size_t workspace_bytes, void* stream);

/* attn_bwd_path -- the attn_path (ATTN_PATH_BWD_MFMA or ATTN_PATH_BWD_PER_ROW,
 * ATTN_PATH_NONE when there is nothing to compute) that attn_bwd would take
 * for these arguments; host computation only, as attn_fwd_path.            */
int attn_bwd_path(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                  const attn_tensor* out, const attn_tensor* dout, const attn_params* p,
                  const attn_tensor* dq, const attn_tensor* dk, const attn_tensor* dv,
                  int* path);

/* attn_bwd_workspace_bytes -- workspace size attn_bwd needs (host only). */
int attn_bwd_workspace_bytes(const attn_tensor* q, const attn_tensor* k,
                             const attn_tensor* v, const attn_params* p, size_t* bytes);

/* Static, human-readable name of a status code (never NULL). */
const char* attn_strerror(int status);

/* Detail of the last error returned on the calling thread ("" if none).
 * The pointer stays valid until the next call on that thread. */
const char* attn_last_error_detail(void);

/* ATTN_ABI_VERSION of the built library. */
int attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H_ */
