// msa_internal.h -- host-side launchers of the MSA kernels (not part of the
// public ABI; the C entry points in msa.cpp validate and plan, then call these).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace msa {

enum DType { kF32 = 0, kBF16 = 1 };

// Shape of one call after validation (all sizes in elements).
struct Shape {
  int B, Nq, Nk, Hq, Hkv, D, DI, topk, dtype;
  bool idx_mx;  // idx_k is an MXFP8 cache: codes, then one scale byte per 32 elements
  bool kv_mx;   // K and V are MXFP8 caches (same layout)
  int64_t q_offset;
  int Bk;       // key block size: 32, 64 or 128
  int nblk;     // ceil(Nk / Bk)
  float scale;  // softmax scale (natural-log domain)
};

// Keeps e as this thread's last HIP error (msa_last_hip_error) and returns MSA_ERR_HIP.
int record_hip_error(hipError_t e);

// Kernel launch bookkeeping for the optional event-based timing.
void prof_begin(hipStream_t s, int kernel_id);
void prof_end(hipStream_t s, int kernel_id);
int prof_register(const char* name);

// Index Branch ---------------------------------------------------------------
// Query tile (MFMA) path: block scores for a tile of queries against every
// candidate key block, fused with per-query Top-k.  Writes ids and/or scores.
hipError_t launch_index_tile(const Shape& s, const void* iq, const void* ik, int32_t* ids, float* scores,
                             hipStream_t st);
// Streaming scan for few queries (decode): writes block scores only.
hipError_t launch_index_scan(const Shape& s, const void* iq, const void* ik, float* scores, hipStream_t st);
// MXFP8 quantisation of n_rows rows of row_len elements (src in `dtype`).
hipError_t launch_mxfp8_quantize(const void* src, int dtype, int64_t n_rows, int row_len, uint8_t* codes,
                                 uint8_t* scales, hipStream_t st);
// Fill scores with -inf.
hipError_t launch_fill_neg_inf(float* p, size_t n, hipStream_t st);
// Top-k over score rows (one wave per (b, g, i) row).
hipError_t launch_topk_rows(const Shape& s, const float* scores, int32_t* ids, hipStream_t st);
// True when the MFMA tile path is used for this shape.
bool index_use_tile(const Shape& s);

// Inversion (KV-outer bookkeeping) --------------------------------------------
struct InvertPlan {
  int nq_chunk;      // queries per chunk
  int n_tiles;       // ceil(nq_chunk / kInvTile)
  int items_cap;     // work-item capacity per (b, g), a multiple of 8
  int qi;            // queries per work item
};
constexpr int kInvTile = 256;
// Words per query row of block ids in the scatter's LDS copy (whole 16-byte chunks).
__host__ __device__ constexpr int inv_row_pitch(int topk) { return (topk + 3) & ~3; }
// A KV-outer work item holds at most kItemRows (query, head) rows and at most
// kItemEntries (query, slot) entries (the entries are staged in LDS).
constexpr int kItemRows = 2048;
constexpr int kItemEntries = 1024;
InvertPlan invert_plan(const Shape& s, int nq_chunk);
size_t invert_ws_bytes(const Shape& s, const InvertPlan& p);
// Builds offsets/entries (and work items) for queries [q0, q0 + nq) of every
// batch.  Offsets [B, Hkv, nblk+1]; entries [B, Hkv, nq*topk] hold
// (i - q0)*topk + slot.  ws must hold invert_ws_bytes.
struct InvertOut {
  int32_t* offsets;
  int32_t* entries;
  int32_t* item_count;  // [B*Hkv]
  int4* items;          // [B*Hkv][items_cap]: (block, e_begin, e_end, 0)
};
hipError_t launch_invert(const Shape& s, const InvertPlan& p, const int32_t* ids, int q0, int nq, InvertOut out,
                         void* ws, hipStream_t st);

// Main Branch -----------------------------------------------------------------
// Partial results per (b, i, h, slot): normalised output o (D values in the
// input dtype) and the log-sum-exp (fp32) of the slot's scaled logits.  The
// lse of one (query, slot) is contiguous over heads, so the G heads of a group
// write one run.
struct Partials {
  void* o;     // [B, nq, Hq, S, D]
  float* lse;  // [B, nq, S, Hq]
  int S;       // slots per (query, head)
  void* trash; // kTrashBytes written (never read) by KV-outer for padding rows
};
constexpr int kTrashBytes = 1024;
hipError_t launch_attn_kvouter(const Shape& s, const InvertPlan& p, int q0, int nq, const void* q, const void* k,
                               const void* v, const InvertOut& inv, Partials part, hipStream_t st);
// Query-outer: each workgroup handles (b, i, g, split); nsplit == 1 writes out/lse
// directly, otherwise partials with S = nsplit.
hipError_t launch_attn_qouter(const Shape& s, int q0, int nq, int nsplit, const void* q, const void* k,
                              const void* v, const int32_t* ids, void* out, float* lse, Partials part,
                              hipStream_t st);
// Merge S partials per (b, i, h) into out/lse.  Slots whose block id is -1
// are skipped when ids_slots is true (KV-outer); with ids_slots false all
// S partials are valid unless their lse is -inf (Q-outer splits).
hipError_t launch_combine(const Shape& s, int q0, int nq, const Partials& part, const int32_t* ids,
                          bool ids_slots, void* out, float* lse, hipStream_t st);

// Backward of the Main Branch ------------------------------------------------
// D = <dO, O> per (b, i, h) row (fp32).
hipError_t launch_bwd_rowdot(const Shape& s, const void* out, const void* dout, float* drow, hipStream_t st);
// Bytes of the per-work-item fp32 dk/dv partials.
size_t bwd_dkv_bytes(const Shape& s, const InvertPlan& p);
// dq (via per-(row, slot) partials in the input type, [B, Nq, Hq, topk, D])
// and dk, dv (via per-item fp32 partials) for the work items of `inv` (whole problem, q0 = 0).
hipError_t launch_bwd_attention(const Shape& s, const InvertPlan& p, const void* q, const void* k, const void* v,
                                const void* dout, const float* lse, const float* drow, const int32_t* ids,
                                const InvertOut& inv, void* dq_part, void* dkv_part, void* trash, void* dq, void* dk,
                                void* dv, hipStream_t st);

// Index-Branch alignment loss -----------------------------------------------
struct KlWorkspace {
  size_t plse, lse_s, kl_part, diq_part, dik_part;
};
// Bytes of the loss's scratch after the inversion (layout in *w when given).
size_t kl_bytes(const Shape& s, const InvertPlan& p, KlWorkspace* w);
// kl per (b, i, g) and the gradients of loss_scale * sum(kl) for idx_q / idx_k,
// for the work items of `inv` (whole problem); ws holds kl_bytes() bytes.
hipError_t launch_indexer_kl(const Shape& s, const InvertPlan& p, const void* q, const void* k, const void* iq,
                             const void* ik, const float* lse, const int32_t* ids, const InvertOut& inv, char* ws,
                             float loss_scale, float* kl, void* d_iq, void* d_ik, hipStream_t st);

}  // namespace msa
