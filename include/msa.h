/*
 * msa.h -- C ABI of libmsa: the MiniMax Sparse Attention (MSA) forward hot
 * path on AMD MI355X (gfx950).
 *
 * The method (MiniMax Sparse Attention abstract; paper summary page, "Method";
 * zhichai.net write-up, section 2):
 *   Index Branch, per GQA group g and query i at position p = q_offset + i:
 *     token score  s_t = <idx_q[b,i,g,:], idx_k[b,t,g,:]>          (no scale)
 *     block score  S_j = max over the tokens t of key block j of s_t
 *                  (Block Max Pooling) for the candidate blocks j < L,
 *                  L = floor(p / Bk) being the block holding the query;
 *     selection    {L} plus the k-1 best candidates by (S desc, id asc);
 *                  every candidate when there are at most k-1.  The
 *                  selection is exp-free: it uses the raw scores (zhichai.net
 *                  write-up, section 4.1).
 *   Main Branch: each query head h of group g = h / (Hq/Hkv) attends with
 *     exact softmax (scale 1/sqrt(d) unless given) over the tokens t <= p of
 *     the group's selected blocks.
 *
 * Tensor layouts (contiguous, token-major "BNHD"; element type = dtype):
 *   q      [B, Nq, Hq,  d]          k, v   [B, Nk, Hkv, d]
 *   idx_q  [B, Nq, Hkv, d_idx]      idx_k  [B, Nk, Hkv, d_idx]
 *   out    [B, Nq, Hq,  d]          lse    [B, Nq, Hq]        (fp32, natural log)
 *   block_ids [B, Nq, Hkv, topk]    int32, ascending, -1 padded
 *   scores [B, Hkv, Nq, nblk]       fp32, nblk = ceil(Nk / Bk)
 *
 * Conventions for every call:
 *   - All tensor pointers are device pointers, 16-byte aligned, owned by the
 *     caller.  Inputs are read only; outputs are fully overwritten and must not
 *     alias inputs.  `ws` is caller-owned device scratch of `ws_bytes` bytes
 *     (its contents on entry do not matter and are clobbered).
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is queued
 *     asynchronously on it; the library never allocates device memory and
 *     never synchronises the device.
 *   - Arguments are validated before any HIP call.  Errors: MSA_ERR_INVALID_ARG
 *     (inconsistent or out-of-range shape, NULL pointer, misalignment),
 *     MSA_ERR_UNSUPPORTED (valid but not built: see below), MSA_ERR_WORKSPACE
 *     (ws_bytes below what msa_workspace_size reports as the minimum),
 *     MSA_ERR_HIP (a HIP call failed; msa_last_hip_error gives its code).
 *     No C++ exception crosses this boundary.
 *   - Results are bitwise reproducible for identical inputs and do not depend
 *     on how the library splits the work (query chunks, workspace size).
 *
 * Block id tables.  The ids msa_index_topk / msa_forward / msa_topk_from_scores
 * write hold, per (b, i, g) row, min(topk, L+1) distinct blocks in ascending
 * order -- the local block L and the best candidates -- then -1.  The calls
 * that take a table (msa_invert, msa_sparse_attention,
 * msa_sparse_attention_backward, msa_indexer_kl) accept any int32 values and
 * define the result for every one of them:
 *   - an id outside [0, nblk) (-1 or any other) selects nothing;
 *   - a block named twice in a row counts twice: its visible tokens enter the
 *     softmax once per listing (the output is unchanged and lse grows by
 *     ln 2; each listing gets its own gradient share), and msa_invert lists
 *     the row once per listing, in slot order;
 *   - tokens past the query position are never visible, so a block after the
 *     query's own contributes nothing;
 *   - a row with no visible selected token gets out = 0 and lse = -inf, zero
 *     dq, no dk / dv share, kl = 0 and zero index gradients.
 * Every schedule gives the same result for such a table, and no id makes a
 * kernel read or write outside the caller's buffers.
 *
 * Block scores given to msa_topk_from_scores may be non-finite: -inf and NaN
 * rank below every finite score (NaN as -inf), ties to the lower id.
 *
 * Supported: dtype MSA_BF16 or MSA_F32; block_size in {32, 64, 128} (the
 * pages use 128 and ablate the smaller sizes); d in {64, 128};
 * d_idx in {32, 64, 128}; 1 <= topk <= 32; Hq / Hkv a power of two <= 32;
 * 0 <= q_offset and q_offset + Nq <= Nk; nblk = ceil(Nk / Bk) <= 16384 (2M
 * tokens at Bk = 128); B * Hkv <= 65535; Nq * topk and Nq * Hkv below 2^31.
 * Outside these (but otherwise valid) a call returns MSA_ERR_UNSUPPORTED.
 *
 * Index keys may instead be an MXFP8 cache (idx_format = MSA_IDX_MXFP8; the
 * MiniMax write-up pairs MSA with MXFP8 caches for long-context decode,
 * zhichai.net section 9).  Format: OCP Microscaling Formats v1.0 -- blocks of
 * 32 consecutive elements of a row share one E8M0 scale byte s (value
 * 2^(s-127)); elements are OCP FP8 E4M3 codes.  Layout: the idx_k pointer
 * holds the codes [B, Nk, Hkv, d_idx] (uint8) immediately followed by the
 * scales [B, Nk, Hkv, d_idx/32] (uint8), i.e. the scales start
 * B*Nk*Hkv*d_idx bytes after idx_k.  idx_q stays in `dtype`; scores are
 * computed from the exactly decoded keys in fp32.  msa_mxfp8_quantize writes
 * such a cache.
 *
 * K and V may likewise be MXFP8 caches (kv_format = MSA_IDX_MXFP8, the same
 * write-up's MXFP8 KV cache): the k (v) pointer holds the codes [B, Nk, Hkv, d]
 * followed by the scales [B, Nk, Hkv, d/32].  The attention entry points
 * (msa_sparse_attention, msa_forward) decode them exactly into `dtype` while
 * staging a key block, so the products are those of the decoded cache; q, the
 * output and lse stay in `dtype` / fp32.  The training entry points
 * (msa_sparse_attention_backward, msa_indexer_kl) need plain K and V
 * (MSA_ERR_UNSUPPORTED otherwise).
 */
#ifndef MSA_H
#define MSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MSA_OK = 0,
  MSA_ERR_INVALID_ARG = -1,
  MSA_ERR_UNSUPPORTED = -2,
  MSA_ERR_WORKSPACE = -3,
  MSA_ERR_HIP = -4
} msa_status_t;

typedef enum { MSA_F32 = 0, MSA_BF16 = 1 } msa_dtype_t;

/* Attention schedule.  KV_OUTER keeps one selected KV block resident and
 * streams the queries that chose it (KV-stationary; the paper's co-designed
 * path, abstract and "Key Contributions").  Q_OUTER keeps the query resident
 * and gathers its blocks (the query-stationary baseline of the Fireworks note
 * on KV-stationary attention, "The design space").  AUTO picks KV_OUTER when
 * the average number of times a selected KV token is re-read,
 * Nq*topk*Bk/Nk, exceeds 0.75 -- where the two schedules cross on MI355X
 * (the note quotes 2.85 for its Blackwell kernels) -- and Q_OUTER otherwise. */
typedef enum { MSA_SCHED_AUTO = 0, MSA_SCHED_KV_OUTER = 1, MSA_SCHED_Q_OUTER = 2 } msa_sched_t;

/* How idx_k (idx_format) or K and V (kv_format) are stored: in `dtype` like the
 * other tensors, or as an MXFP8 cache. */
typedef enum { MSA_IDX_PLAIN = 0, MSA_IDX_MXFP8 = 1 } msa_idx_format_t;

typedef struct {
  int32_t batch, n_q, n_k, h_q, h_kv, d, d_idx, block_size, topk;
  int32_t dtype;         /* msa_dtype_t */
  int64_t q_offset;      /* query i sits at position q_offset + i */
  float softmax_scale;   /* <= 0 means 1/sqrt(d) */
  int32_t sched;         /* msa_sched_t */
  int32_t idx_format;    /* msa_idx_format_t */
  int32_t kv_format;     /* msa_idx_format_t, for K and V */
} msa_problem_t;

typedef enum {
  MSA_OP_INDEX_TOPK = 0,
  MSA_OP_ATTENTION = 1,
  MSA_OP_FORWARD = 2,
  MSA_OP_INVERT = 3,
  MSA_OP_BACKWARD = 4,
  MSA_OP_INDEXER_KL = 5
} msa_op_t;

/* Human-readable name of a status code (static storage). */
const char* msa_status_string(msa_status_t status);

/* The hipError_t of the last failing HIP call on this thread (0 if none). */
int msa_last_hip_error(void);

/* Validate a problem without touching the GPU. */
msa_status_t msa_validate(const msa_problem_t* prob);

/* Workspace for one call of `op`: *bytes = size that lets the whole problem
 * run in one pass; *min_bytes (may be NULL) = the least the call accepts (it
 * then processes the queries in chunks). */
msa_status_t msa_workspace_size(const msa_problem_t* prob, int op, size_t* bytes, size_t* min_bytes);

/* Index Branch step 1+2 alone: block scores (Block Max Pooling of the
 * index-q . index-k token scores; paper summary "Method").  Writes `scores`
 * [B, Hkv, Nq, nblk] fp32: S_j for candidate blocks j < L(i), -inf elsewhere. */
msa_status_t msa_block_scores(const msa_problem_t* prob, const void* idx_q, const void* idx_k,
                              float* scores, void* stream);

/* Index Branch step 3 alone: exp-free Top-k over given block scores (laid out
 * as msa_block_scores writes them; only j < L(i) is read), forcing the local
 * block, ties to the lower id (zhichai.net write-up, sections 2 and 4.1).
 * Writes block_ids [B, Nq, Hkv, topk]. */
msa_status_t msa_topk_from_scores(const msa_problem_t* prob, const float* scores, int32_t* block_ids,
                                  void* stream);

/* Index Branch, steps 1 to 3 in one call (paper summary page, "Method": the
 * index-q . index-k token scores, Block Max Pooling over each candidate
 * block, Top-k with the local block always kept; zhichai.net write-up,
 * sections 2 and 4.1: one index head pair per GQA group, exp-free selection).
 * Writes block_ids [B, Nq, Hkv, topk] as described under "Block id tables".
 * Needs the MSA_OP_INDEX_TOPK workspace (zero bytes for most prefill shapes,
 * where scoring and selection run fused; the block scores otherwise).
 * Errors: as listed under "Conventions". */
msa_status_t msa_index_topk(const msa_problem_t* prob, const void* idx_q, const void* idx_k,
                            int32_t* block_ids, void* ws, size_t ws_bytes, void* stream);

/* Block -> query inversion used by the KV-outer schedule (the paper's
 * skew-tolerant, atomic-free bookkeeping, "Key Contributions"): for each
 * (b, g), offsets [B, Hkv, nblk+1] (int32, exclusive prefix of the number of
 * (query, slot) pairs that chose each block) and entries [B, Hkv, Nq*topk]
 * (int32 i*topk + slot, grouped by block, ascending within a block; entries
 * past offsets[nblk] are unspecified).  Ids outside [0, nblk) are not listed;
 * a block named twice in a row is listed once per slot.  Deterministic.  Needs the
 * MSA_OP_INVERT workspace (the whole problem in one pass). */
msa_status_t msa_invert(const msa_problem_t* prob, const int32_t* block_ids, int32_t* offsets,
                        int32_t* entries, void* ws, size_t ws_bytes, void* stream);

/* Main Branch: exact softmax attention of every query head over the visible
 * tokens of its group's blocks in block_ids (paper summary "Method"), in the
 * schedule prob->sched.  Writes out (dtype of the inputs) and, if lse is not
 * NULL, the log-sum-exp of the scaled logits.  block_ids may be any int32
 * table (see "Block id tables"). */
msa_status_t msa_sparse_attention(const msa_problem_t* prob, const void* q, const void* k, const void* v,
                                  const int32_t* block_ids, void* out, float* lse, void* ws, size_t ws_bytes,
                                  void* stream);

/* The whole MSA forward (paper summary page, "Method"; zhichai.net write-up,
 * section 2): the Index Branch of msa_index_topk, then the Main Branch of
 * msa_sparse_attention over the blocks it selected, in one call on one
 * stream.  Writes block_ids, out and, if lse is not NULL, lse.  Needs the
 * MSA_OP_FORWARD workspace; given less than the full size (but at least the
 * minimum msa_workspace_size reports) it processes the queries in chunks
 * with bitwise the same results.  Errors: as listed under "Conventions". */
msa_status_t msa_forward(const msa_problem_t* prob, const void* q, const void* k, const void* v,
                         const void* idx_q, const void* idx_k, int32_t* block_ids, void* out, float* lse,
                         void* ws, size_t ws_bytes, void* stream);

/* msa_forward for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * same arguments as msa_forward without the workspace: the library uses its
 * own scratch, one array of MSA_NOALLOC_SCRATCH_BYTES in each GPU's memory
 * (held from the first call on that GPU until the process ends), processing
 * the queries in chunks when the whole problem does not fit.  Results are
 * bitwise those of msa_forward.  The call allocates nothing and calls no
 * allocating routine.  Every call on one GPU shares that GPU's array: calls
 * that overlap on one GPU (other host threads, or other streams not ordered
 * with this one) race and must not be issued.  Errors: as msa_forward, and
 * MSA_ERR_WORKSPACE when the problem's minimum workspace (msa_workspace_size,
 * MSA_OP_FORWARD) exceeds MSA_NOALLOC_SCRATCH_BYTES. */
#define MSA_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
msa_status_t msa_forward_noalloc(const msa_problem_t* prob, const void* q, const void* k, const void* v,
                                 const void* idx_q, const void* idx_k, int32_t* block_ids, void* out, float* lse,
                                 void* stream);

/* Gradients of the Main Branch for the fixed selection block_ids (the
 * selection is not differentiable; the pages train the Index Branch by a
 * separate loss -- paper summary page, "Method").  Given the forward's out and
 * lse (as msa_sparse_attention / msa_forward wrote them for these inputs and
 * ids) and the upstream gradient dout = dL/dout (layout and dtype of q), writes
 *   dq [B, Nq, Hq, d], dk, dv [B, Nk, Hkv, d]    (dtype of the inputs)
 * with, per (b, i, h) over its visible selected tokens: P = softmax of
 * scale <q, k_t>, D = <dout, out>, dS_t = P_t (<dout, v_t> - D), dq = scale
 * sum dS_t k_t, dk_t += scale dS_t q, dv_t += P_t dout.  Tokens no query
 * attends get zero gradients.  Sums are formed in fixed orders (no atomics), so
 * results are bitwise reproducible.  Needs the MSA_OP_BACKWARD workspace (the
 * whole problem in one pass).  Errors as for msa_sparse_attention. */
msa_status_t msa_sparse_attention_backward(const msa_problem_t* prob, const void* q, const void* k, const void* v,
                                           const void* out, const float* lse, const void* dout,
                                           const int32_t* block_ids, void* dq, void* dk, void* dv, void* ws,
                                           size_t ws_bytes, void* stream);

/* The Index-Branch alignment loss (paper summary page, "Method"; zhichai.net
 * write-up, section 5.1): the KL divergence from the Main Branch's
 * group-averaged attention distribution to the Index Branch's distribution,
 * both over the visible selected tokens T of (b, i, g).  With P_h the Main
 * Branch softmax of head h (recomputed from q, k and the forward's lse) and
 * s_t = <idx_q, idx_k_t> the raw token scores:
 *   pm(t) = mean over the group's heads of P_h(t),  pi = softmax over T of s,
 *   kl[b, i, g] = sum_t pm(t) log(pm(t) / pi(t))          (fp32 [B, Nq, Hkv])
 * and the gradients of loss_scale * sum(kl) with respect to the index inputs,
 *   d_iq [B, Nq, Hkv, d_idx], d_ik [B, Nk, Hkv, d_idx]    (dtype of the inputs)
 * (d kl / d s_t = pi(t) - pm(t)).  The Main Branch and the selection are fixed
 * targets: nothing flows to q or k (the pages' gradient detach).  Keys no query
 * selects get zero d_ik.  Sums in fixed orders (no atomics).  Needs plain
 * (not MXFP8) index keys and the MSA_OP_INDEXER_KL workspace (whole problem).
 * Errors as for msa_sparse_attention. */
msa_status_t msa_indexer_kl(const msa_problem_t* prob, const void* q, const void* k, const void* idx_q,
                            const void* idx_k, const float* lse, const int32_t* block_ids, float loss_scale,
                            float* kl, void* d_iq, void* d_ik, void* ws, size_t ws_bytes, void* stream);

/* Quantise n_rows rows of row_len elements (row_len a multiple of 32) of src
 * (device, `src_dtype` MSA_F32 or MSA_BF16, row-major) to MXFP8 following the
 * OCP MX v1.0 conversion: per 32-element block, shared exponent
 * e = floor(log2(max |v|)) - 8 clamped to [-127, 127] (-127 for an all-zero
 * block), scale byte e + 127, codes = E4M3(v / 2^e) rounded to nearest even
 * with magnitudes above 448 saturating to 448 (-0 keeps its sign).  codes:
 * n_rows*row_len bytes; scales: n_rows*row_len/32 bytes (device, caller-owned;
 * codes 16-byte aligned).  For an idx_k cache pass rows = B*Nk*Hkv,
 * row_len = d_idx and scales = codes + B*Nk*Hkv*d_idx.  Errors:
 * MSA_ERR_INVALID_ARG (NULL or misaligned pointer, bad sizes or dtype). */
msa_status_t msa_mxfp8_quantize(const void* src, int32_t src_dtype, int64_t n_rows, int32_t row_len, uint8_t* codes,
                                uint8_t* scales, void* stream);

/* Kernel timing for measurement.  While enabled, every kernel launch is
 * bracketed by two hipEvents on its stream (a small overhead per launch).
 * msa_profile_read synchronises on those events and returns, for kernel
 * number `index` (0 <= index < msa_profile_count()), its name (static
 * storage), the summed duration in milliseconds and the launch count since the
 * last reset.  These are the only calls that wait on the GPU. */
msa_status_t msa_profile_enable(int on);
msa_status_t msa_profile_reset(void);
int msa_profile_count(void);
msa_status_t msa_profile_read(int index, const char** name, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif
#endif /* MSA_H */
