/*
 * msa_oracle.h -- plain fp64 CPU oracle for the MiniMax Sparse Attention (MSA)
 * forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  This library is what the GPU kernels are checked
 * against.  Only the test-suite, the smoke check and the CPU-baseline leg of
 * the benchmark may load it; the product path never does.  It shares no code,
 * header or table with the HIP library.
 *
 * What it computes (MiniMax Sparse Attention, arXiv 2606.13392 summary page,
 * "Method"; the same paper's abstract; the zhichai.net write-up, section 2):
 *   1. token score  s_t = <idx_q[b,i,g,:], idx_k[b,t,g,:]>  (no scale)
 *   2. block score  S_j = max over the tokens t of key block j of s_t
 *      (Block Max Pooling), for every candidate block j < L(i), where
 *      L(i) = floor(p(i)/Bk) is the block holding the query position
 *      p(i) = q_offset + i.  Candidates are the blocks wholly before L(i).
 *   3. selection    {L(i)} plus the (k-1) best candidates ordered by
 *      (S descending, block id ascending); all candidates when there are at
 *      most k-1 of them.  Emitted ascending, padded with -1 to length k.
 *   4. attention    exact softmax attention of every query head h of group
 *      g = h / (Hq/Hkv) over the visible tokens (t <= p(i), t < Nk) of the
 *      selected blocks, softmax scale 1/sqrt(d) unless given.
 * Every sum and product is carried out in IEEE fp64; bf16 and fp32 inputs are
 * widened exactly.
 *
 * Tensor layouts (all contiguous, token-major):
 *   q  [B, Nq, Hq,  d]      k, v [B, Nk, Hkv, d]
 *   iq [B, Nq, Hkv, d_idx]  ik   [B, Nk, Hkv, d_idx]
 *
 * Query subsets: every routine takes `rows`, a list of n_rows (b, i) pairs
 * stored as rows[2r] = b, rows[2r+1] = i.  rows == NULL means every (b, i)
 * in batch-major order (n_rows must then equal B*Nq).  Outputs are indexed by
 * r, the position in that list.
 *
 * Return value: 0 on success, a negative number for an invalid argument.
 */
#ifndef MSA_ORACLE_H
#define MSA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { MO_F32 = 0, MO_BF16 = 1, MO_F64 = 2 };

typedef struct {
  int32_t batch, n_q, n_k, h_q, h_kv, d, d_idx, block_size, topk;
  int64_t q_offset;
  double softmax_scale; /* <= 0 means 1/sqrt(d) */
} mo_problem;

/* Block scores.  scores: double [n_rows][h_kv][nblk], nblk = ceil(Nk/Bk).
 * Entries for non-candidate blocks (j >= L(i)) are set to -INFINITY. */
int mo_block_scores(const mo_problem* p, const void* iq, const void* ik, int dtype,
                    const int64_t* rows, int64_t n_rows, double* scores);

/* Selection from block scores laid out as mo_block_scores writes them.
 * ids: int32 [n_rows][h_kv][topk], ascending, -1 padded.  A NaN score ranks
 * with -inf: below every finite score, ties to the lower id. */
int mo_select(const mo_problem* p, const double* scores, const int64_t* rows, int64_t n_rows,
              int32_t* ids);

/* Exact softmax attention over the tokens of the blocks listed in ids
 * (int32 [n_rows][h_kv][topk]).  Any int32 is accepted: ids outside
 * [0, nblk) are ignored, a block listed twice enters T twice (the output is
 * unchanged, lse grows by ln 2), tokens past the query position are not
 * visible.  A row with no visible listed token gets out = 0, lse = -inf.
 * out: double [n_rows][h_q][d]; lse: double [n_rows][h_q] (may be NULL). */
int mo_attend(const mo_problem* p, const void* q, const void* k, const void* v, int dtype,
              const int32_t* ids, const int64_t* rows, int64_t n_rows, double* out, double* lse);

/* Gradients of the attention step for a fixed selection: given the upstream
 * gradient dout = dL/dO (same layout and dtype as q), returns dq = dL/dq,
 * dk = dL/dk, dv = dL/dv of L through O of mo_attend (the selection itself is
 * not differentiable; the pages train the index branch separately).  For each
 * (b, i, h) over its visible selected tokens T:
 *   P = softmax(x), x_t = scale <q, k_t>;  O = sum_t P_t v_t;
 *   dP_t = <dout, v_t>;  dS_t = P_t (dP_t - <dout, O>);
 *   dq += scale sum_t dS_t k_t;  dk_t += scale dS_t q;  dv_t += P_t dout.
 * Over the listed rows: ids [n_rows][h_kv][topk], dq [n_rows][h_q][d];
 * dk, dv [B, Nk, h_kv, d] hold the contributions of those rows only (all
 * rows: the full gradients; tokens no listed query attends get zeros).  All
 * fp64. */
int mo_attend_backward(const mo_problem* p, const void* q, const void* k, const void* v, const void* dout,
                       int dtype, const int32_t* ids, const int64_t* rows, int64_t n_rows, double* dq, double* dk,
                       double* dv);

/* Index-Branch alignment loss (KL divergence from the Main Branch's
 * group-averaged distribution to the Index Branch's, on the selected tokens;
 * the selection and the Main Branch are fixed targets).  Per listed row and
 * group g, over the visible selected tokens T:
 *   pm(t) = (1/G) sum_{h in g} P_h(t)   (P_h as in mo_attend)
 *   pi(t) = exp(s_t) / sum_{u in T} exp(s_u),  s_t = <iq[b,i,g], ik[b,t,g]>
 *   kl    = sum_t pm(t) log(pm(t) / pi(t))
 * kl: [n_rows][h_kv]; d_iq: [n_rows][h_kv][d_idx]; d_ik: [B, Nk, h_kv, d_idx]
 * (the listed rows' contributions) -- the gradients of
 * loss_scale * sum(kl).  ids: [n_rows][h_kv][topk].  All fp64. */
int mo_indexer_kl(const mo_problem* p, const void* q, const void* k, const void* iq, const void* ik, int dtype,
                  const int32_t* ids, const int64_t* rows, int64_t n_rows, double loss_scale, double* kl,
                  double* d_iq, double* d_ik);

/* Block -> query lists (the bookkeeping a KV-outer schedule needs; the paper
 * summary's "Key Contributions" name KV-outer attention): for each (b, g),
 * offsets[(b*h_kv+g)*(nblk+1) + j] = number of (i, slot) pairs with
 * ids[b,i,g,slot] < j and >= 0 (so offsets[.., nblk] = all valid picks), and
 * entries[(b*h_kv+g)*(n_q*topk) + ...] = i*topk + slot for every pick, grouped
 * by block j, ascending in (i, slot) within a block.  ids: [B, Nq, h_kv, topk]
 * covering every query (no row subset). */
int mo_invert(const mo_problem* p, const int32_t* ids, int32_t* offsets, int32_t* entries);

/* MXFP8 index-key caches (OCP Microscaling Formats v1.0, section 6: blocks of
 * 32 elements share one E8M0 power-of-two scale X = 2^(s - 127); elements are
 * OCP FP8 E4M3, i.e. bias 7, no infinities, S.1111.111 = NaN, largest finite
 * 448).  The MiniMax pages name MXFP8 for the long-context cache (zhichai.net
 * write-up, section 9, decode KV-cache); the spec fixes the rest.
 *
 * Value of one E4M3 code (NaN for the two NaN codes). */
double mo_e4m3_value(uint8_t code);
/* The E4M3 code nearest to y, ties to the even code, magnitudes above 448
 * saturating to +-448 (the spec's conversion of a scaled element); -0 keeps
 * its sign bit. */
uint8_t mo_e4m3_encode(double y);
/* Quantise rows of row_len elements (a multiple of 32) block by block:
 * shared exponent e = floor(log2(max |v|)) - 8 (8 = the largest exponent of
 * E4M3), clamped to [-127, 127] (e = -127 for an all-zero block); codes =
 * encode(v / 2^e), scales = e + 127.  src holds n_rows*row_len elements of
 * `dtype`; codes: n_rows*row_len bytes; scales: n_rows*row_len/32 bytes. */
int mo_mxfp8_quantize(const void* src, int dtype, int64_t n_rows, int32_t row_len, uint8_t* codes, uint8_t* scales);
/* out[r*row_len + c] = value(codes[...]) * 2^(scales[r*row_len/32 + c/32] - 127). */
int mo_mxfp8_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t n_rows, int32_t row_len, double* out);

/* Number of OpenMP threads the routines above use. */
int mo_num_threads(void);

/* Threads the following calls may use (n >= 1; results do not depend on it). */
void mo_set_num_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
