// msa.cpp -- the C ABI of libmsa (declared in include/msa.h): validation,
// workspace planning, schedule choice and kernel dispatch.  Everything here
// runs on the host and only enqueues work on the caller's stream.
#include "msa.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <new>
#include <vector>

#include "msa_internal.h"

namespace {

thread_local int t_last_hip_error = 0;

msa_status_t hip_fail(hipError_t e) {
  t_last_hip_error = (int)e;
  return MSA_ERR_HIP;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

msa_status_t validate(const msa_problem_t* p) {
  if (!p) return MSA_ERR_INVALID_ARG;
  if (p->batch < 1 || p->n_q < 1 || p->n_k < 1 || p->h_q < 1 || p->h_kv < 1 || p->d < 1 || p->d_idx < 1 ||
      p->block_size < 1 || p->topk < 1)
    return MSA_ERR_INVALID_ARG;
  if (p->h_q % p->h_kv) return MSA_ERR_INVALID_ARG;
  if (p->q_offset < 0 || p->q_offset + p->n_q > p->n_k) return MSA_ERR_INVALID_ARG;
  if (p->dtype != MSA_F32 && p->dtype != MSA_BF16) return MSA_ERR_INVALID_ARG;
  if (p->sched != MSA_SCHED_AUTO && p->sched != MSA_SCHED_KV_OUTER && p->sched != MSA_SCHED_Q_OUTER)
    return MSA_ERR_INVALID_ARG;
  if (!std::isfinite(p->softmax_scale)) return MSA_ERR_INVALID_ARG;
  if (p->idx_format != MSA_IDX_PLAIN && p->idx_format != MSA_IDX_MXFP8) return MSA_ERR_INVALID_ARG;
  if (p->kv_format != MSA_IDX_PLAIN && p->kv_format != MSA_IDX_MXFP8) return MSA_ERR_INVALID_ARG;
  // Valid but outside what the kernels are built for.
  if (p->block_size != 32 && p->block_size != 64 && p->block_size != 128) return MSA_ERR_UNSUPPORTED;
  if (p->d != 64 && p->d != 128) return MSA_ERR_UNSUPPORTED;
  if (p->d_idx != 32 && p->d_idx != 64 && p->d_idx != 128) return MSA_ERR_UNSUPPORTED;
  if (p->topk > 32) return MSA_ERR_UNSUPPORTED;
  const int G = p->h_q / p->h_kv;
  if (!is_pow2(G) || G > 32) return MSA_ERR_UNSUPPORTED;
  const int64_t nblk = ((int64_t)p->n_k + p->block_size - 1) / p->block_size;
  if (nblk > 16384) return MSA_ERR_UNSUPPORTED;
  if ((int64_t)p->n_q * p->topk >= (int64_t)1 << 31) return MSA_ERR_UNSUPPORTED;
  if ((int64_t)p->batch * p->h_kv > 65535 || (int64_t)p->n_q * p->h_kv >= (int64_t)1 << 31)
    return MSA_ERR_UNSUPPORTED;
  return MSA_OK;
}

msa::Shape shape_of(const msa_problem_t* p) {
  msa::Shape s;
  s.B = p->batch;
  s.Nq = p->n_q;
  s.Nk = p->n_k;
  s.Hq = p->h_q;
  s.Hkv = p->h_kv;
  s.D = p->d;
  s.DI = p->d_idx;
  s.topk = p->topk;
  s.dtype = p->dtype == MSA_BF16 ? msa::kBF16 : msa::kF32;
  s.idx_mx = p->idx_format == MSA_IDX_MXFP8;
  s.kv_mx = p->kv_format == MSA_IDX_MXFP8;
  s.q_offset = p->q_offset;
  s.Bk = p->block_size;
  s.nblk = (p->n_k + s.Bk - 1) / s.Bk;
  s.scale = p->softmax_scale > 0 ? p->softmax_scale : 1.0f / std::sqrt((float)p->d);
  return s;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Average number of reads of a selected KV token above which keeping the KV
// block resident (KV-outer) beats keeping the query resident.  The Fireworks
// note on KV-stationary attention puts this crossover near 2.85 for its
// Blackwell kernels; on MI355X the two schedules here cross between 0.5 and
// 1.0 (1M-token cache, 256..16384-query chunks).
constexpr double kReuseCrossover = 0.75;

bool use_kv_outer(const msa_problem_t* p) {
  if (p->sched == MSA_SCHED_KV_OUTER) return true;
  if (p->sched == MSA_SCHED_Q_OUTER) return false;
  const double reuse = (double)p->n_q * p->topk * p->block_size / (double)p->n_k;
  return reuse > kReuseCrossover;
}

// Split factor of the query-outer schedule: enough workgroups to fill the chip.
int qouter_splits(const msa::Shape& s) {
  const int64_t items = (int64_t)s.B * s.Nq * s.Hkv;
  int ns = 1;
  while (ns < s.topk && items * ns < 2048) ns *= 2;
  return std::min(ns, s.topk);
}

// ---- workspace layout ------------------------------------------------------

// Partial outputs are kept in the input dtype (bf16 partials add one bf16
// rounding of a normalised output, well inside the bf16 output tolerance).
size_t elem_bytes(const msa::Shape& s) { return s.dtype == msa::kBF16 ? 2 : 4; }

struct KvLayout {
  size_t offsets, entries, item_count, items, inv_scratch, part_o, part_lse, trash, total;
};

KvLayout kv_layout(const msa::Shape& s, int nc) {
  const msa::InvertPlan p = msa::invert_plan(s, nc);
  const size_t BG = (size_t)s.B * s.Hkv;
  KvLayout L;
  size_t off = 0;
  L.offsets = off;
  off += align_up(BG * (s.nblk + 1) * 4);
  L.entries = off;
  off += align_up(BG * (size_t)nc * s.topk * 4);
  L.item_count = off;
  off += align_up(BG * 4);
  L.items = off;
  off += align_up(BG * (size_t)p.items_cap * 16);
  L.inv_scratch = off;
  off += align_up(msa::invert_ws_bytes(s, p));
  L.part_o = off;
  off += align_up((size_t)s.B * nc * s.Hq * s.topk * s.D * elem_bytes(s));
  L.part_lse = off;
  off += align_up((size_t)s.B * nc * s.Hq * s.topk * 4);
  L.trash = off;
  off += align_up(msa::kTrashBytes);
  L.total = off;
  return L;
}

// Backward workspace: D rows, the inversion of the whole problem, dq partials,
// per-item dk/dv partials and a scratch line.
struct BwdLayout {
  size_t drow, offsets, entries, item_count, items, inv_scratch, dq_part, dkv_part, trash, total;
};

BwdLayout bwd_layout(const msa::Shape& s) {
  const msa::InvertPlan p = msa::invert_plan(s, s.Nq);
  const size_t BG = (size_t)s.B * s.Hkv, rows = (size_t)s.B * s.Nq * s.Hq;
  BwdLayout L;
  size_t off = 0;
  L.drow = off;
  off += align_up(rows * 4);
  L.offsets = off;
  off += align_up(BG * (s.nblk + 1) * 4);
  L.entries = off;
  off += align_up(BG * (size_t)s.Nq * s.topk * 4);
  L.item_count = off;
  off += align_up(BG * 4);
  L.items = off;
  off += align_up(BG * (size_t)p.items_cap * 16);
  L.inv_scratch = off;
  off += align_up(msa::invert_ws_bytes(s, p));
  L.dq_part = off;
  off += align_up(rows * s.topk * s.D * elem_bytes(s));
  L.dkv_part = off;
  off += align_up(msa::bwd_dkv_bytes(s, p));
  L.trash = off;
  off += align_up(msa::kTrashBytes);
  L.total = off;
  return L;
}

// Indexer KL workspace: the inversion of the whole problem, then the loss's
// partials.
struct KlLayout {
  size_t offsets, entries, item_count, items, inv_scratch, kl, total;
};

KlLayout kl_layout(const msa::Shape& s) {
  const msa::InvertPlan p = msa::invert_plan(s, s.Nq);
  const size_t BG = (size_t)s.B * s.Hkv;
  KlLayout L;
  size_t off = 0;
  L.offsets = off;
  off += align_up(BG * (s.nblk + 1) * 4);
  L.entries = off;
  off += align_up(BG * (size_t)s.Nq * s.topk * 4);
  L.item_count = off;
  off += align_up(BG * 4);
  L.items = off;
  off += align_up(BG * (size_t)p.items_cap * 16);
  L.inv_scratch = off;
  off += align_up(msa::invert_ws_bytes(s, p));
  L.kl = off;
  off += align_up(msa::kl_bytes(s, p, nullptr));
  L.total = off;
  return L;
}

size_t qo_bytes(const msa::Shape& s, int nc, int nsplit) {
  if (nsplit <= 1) return 0;
  return align_up((size_t)s.B * nc * s.Hq * nsplit * s.D * elem_bytes(s)) + align_up((size_t)s.B * nc * s.Hq * nsplit * 4);
}

size_t attn_bytes(const msa_problem_t* p, const msa::Shape& s, int nc) {
  if (use_kv_outer(p)) return kv_layout(s, nc).total;
  return qo_bytes(s, nc, qouter_splits(s));
}

size_t index_bytes(const msa::Shape& s) {
  if (msa::index_use_tile(s)) return 0;
  return align_up((size_t)s.B * s.Hkv * s.Nq * s.nblk * 4);
}

// Largest query chunk whose attention workspace fits in ws_bytes (0 if none).
int attn_chunk(const msa_problem_t* p, const msa::Shape& s, size_t ws_bytes) {
  if (attn_bytes(p, s, s.Nq) <= ws_bytes) return s.Nq;
  int lo = 0, hi = (s.Nq - 1) / msa::kInvTile;  // chunks are multiples of the inversion tile
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (attn_bytes(p, s, mid * msa::kInvTile) <= ws_bytes) lo = mid;
    else hi = mid - 1;
  }
  return lo * msa::kInvTile;
}

int min_chunk(const msa::Shape& s) { return std::min(s.Nq, msa::kInvTile); }

// ---- the work itself -------------------------------------------------------

msa_status_t run_index(const msa::Shape& s, const void* iq, const void* ik, int32_t* ids, void* ws, size_t ws_bytes,
                       hipStream_t st) {
  hipError_t e;
  if (msa::index_use_tile(s)) {
    e = msa::launch_index_tile(s, iq, ik, ids, nullptr, st);
  } else {
    if (ws_bytes < index_bytes(s) || (index_bytes(s) && !ws)) return MSA_ERR_WORKSPACE;
    float* S = static_cast<float*>(ws);
    e = msa::launch_index_scan(s, iq, ik, S, st);
    if (e == hipSuccess) e = msa::launch_topk_rows(s, S, ids, st);
  }
  return e == hipSuccess ? MSA_OK : hip_fail(e);
}

msa_status_t run_attention(const msa_problem_t* p, const msa::Shape& s, const void* q, const void* k, const void* v,
                           const int32_t* ids, void* out, float* lse, void* ws, size_t ws_bytes, hipStream_t st) {
  const int nc = attn_chunk(p, s, ws_bytes);
  if (nc <= 0) return MSA_ERR_WORKSPACE;
  char* w = static_cast<char*>(ws);
  hipError_t e = hipSuccess;
  if (use_kv_outer(p)) {
    const KvLayout L = kv_layout(s, nc);
    const msa::InvertPlan plan = msa::invert_plan(s, nc);
    msa::InvertOut inv;
    inv.offsets = reinterpret_cast<int32_t*>(w + L.offsets);
    inv.entries = reinterpret_cast<int32_t*>(w + L.entries);
    inv.item_count = reinterpret_cast<int32_t*>(w + L.item_count);
    inv.items = reinterpret_cast<int4*>(w + L.items);
    msa::Partials part;
    part.o = w + L.part_o;
    part.lse = reinterpret_cast<float*>(w + L.part_lse);
    part.S = s.topk;
    part.trash = w + L.trash;
    for (int q0 = 0; q0 < s.Nq && e == hipSuccess; q0 += nc) {
      const int nq = std::min(nc, s.Nq - q0);
      e = msa::launch_invert(s, plan, ids, q0, nq, inv, w + L.inv_scratch, st);
      if (e == hipSuccess) e = msa::launch_attn_kvouter(s, plan, q0, nq, q, k, v, inv, part, st);
      if (e == hipSuccess) e = msa::launch_combine(s, q0, nq, part, ids, true, out, lse, st);
    }
  } else {
    const int ns = qouter_splits(s);
    msa::Partials part;
    part.o = w;
    part.lse = reinterpret_cast<float*>(w + (ns > 1 ? align_up((size_t)s.B * nc * s.Hq * ns * s.D * elem_bytes(s)) : 0));
    part.S = ns;
    part.trash = nullptr;
    for (int q0 = 0; q0 < s.Nq && e == hipSuccess; q0 += nc) {
      const int nq = std::min(nc, s.Nq - q0);
      e = msa::launch_attn_qouter(s, q0, nq, ns, q, k, v, ids, out, lse, part, st);
      if (e == hipSuccess && ns > 1) e = msa::launch_combine(s, q0, nq, part, ids, false, out, lse, st);
    }
  }
  return e == hipSuccess ? MSA_OK : hip_fail(e);
}

// ---- kernel timing -----------------------------------------------------------

struct ProfKernel {
  const char* name;
  double ms;
  int64_t launches;
};
struct ProfPending {
  int id;
  hipEvent_t a, b;
};

std::mutex g_prof_mu;
std::vector<ProfKernel>& prof_kernels() {
  static std::vector<ProfKernel> v;
  return v;
}
std::vector<ProfPending> g_pending;
std::vector<hipEvent_t> g_pool;
bool g_prof_on = false;
thread_local int t_open_id = -1;
thread_local hipEvent_t t_open_ev = nullptr;

hipEvent_t pool_get() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

msa_status_t prof_flush() {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  msa_status_t rc = MSA_OK;
  for (const ProfPending& pp : g_pending) {
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(pp.b);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, pp.a, pp.b);
    if (e != hipSuccess) rc = hip_fail(e);
    else {
      prof_kernels()[pp.id].ms += ms;
      prof_kernels()[pp.id].launches += 1;
    }
    g_pool.push_back(pp.a);
    g_pool.push_back(pp.b);
  }
  g_pending.clear();
  return rc;
}

}  // namespace

namespace msa {

int record_hip_error(hipError_t e) { return hip_fail(e); }

int prof_register(const char* name) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  prof_kernels().push_back(ProfKernel{name, 0.0, 0});
  return (int)prof_kernels().size() - 1;
}

void prof_begin(hipStream_t s, int kernel_id) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (!g_prof_on) return;
  hipEvent_t e = pool_get();
  if (!e || hipEventRecord(e, s) != hipSuccess) return;
  t_open_id = kernel_id;
  t_open_ev = e;
}

void prof_end(hipStream_t s, int kernel_id) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (!g_prof_on || t_open_id != kernel_id) return;
  hipEvent_t e = pool_get();
  if (e && hipEventRecord(e, s) == hipSuccess) g_pending.push_back(ProfPending{kernel_id, t_open_ev, e});
  t_open_id = -1;
  t_open_ev = nullptr;
}

}  // namespace msa

extern "C" {

const char* msa_status_string(msa_status_t status) {
  switch (status) {
    case MSA_OK: return "ok";
    case MSA_ERR_INVALID_ARG: return "invalid argument";
    case MSA_ERR_UNSUPPORTED: return "unsupported problem";
    case MSA_ERR_WORKSPACE: return "workspace too small";
    case MSA_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

int msa_last_hip_error(void) { return t_last_hip_error; }

msa_status_t msa_validate(const msa_problem_t* prob) { return validate(prob); }

msa_status_t msa_workspace_size(const msa_problem_t* prob, int op, size_t* bytes, size_t* min_bytes) {
  msa_status_t rc = validate(prob);
  if (rc != MSA_OK) return rc;
  if (!bytes || op < MSA_OP_INDEX_TOPK || op > MSA_OP_INDEXER_KL) return MSA_ERR_INVALID_ARG;
  const msa::Shape s = shape_of(prob);
  size_t full = 0, least = 0;
  if (op == MSA_OP_INVERT) {
    full = least = msa::invert_ws_bytes(s, msa::invert_plan(s, s.Nq));
  }
  if (op == MSA_OP_BACKWARD) {
    full = least = bwd_layout(s).total;
  }
  if (op == MSA_OP_INDEXER_KL) {
    full = least = kl_layout(s).total;
  }
  if (op == MSA_OP_INDEX_TOPK || op == MSA_OP_FORWARD) {
    full = std::max(full, index_bytes(s));
    least = std::max(least, index_bytes(s));
  }
  if (op == MSA_OP_ATTENTION || op == MSA_OP_FORWARD) {
    full = std::max(full, attn_bytes(prob, s, s.Nq));
    least = std::max(least, attn_bytes(prob, s, min_chunk(s)));
  }
  *bytes = full;
  if (min_bytes) *min_bytes = least;
  return MSA_OK;
}

msa_status_t msa_block_scores(const msa_problem_t* prob, const void* idx_q, const void* idx_k, float* scores,
                              void* stream) {
  msa_status_t rc = validate(prob);
  if (rc != MSA_OK) return rc;
  if (!idx_q || !idx_k || !scores || !aligned16(idx_q) || !aligned16(idx_k) || !aligned16(scores))
    return MSA_ERR_INVALID_ARG;
  const msa::Shape s = shape_of(prob);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = msa::launch_fill_neg_inf(scores, (size_t)s.B * s.Hkv * s.Nq * s.nblk, st);
  if (e == hipSuccess) {
    if (msa::index_use_tile(s)) e = msa::launch_index_tile(s, idx_q, idx_k, nullptr, scores, st);
    else e = msa::launch_index_scan(s, idx_q, idx_k, scores, st);
  }
  return e == hipSuccess ? MSA_OK : hip_fail(e);
}

msa_status_t msa_sparse_attention_backward(const msa_problem_t* prob, const void* q, const void* k, const void* v,
                                           const void* out, const float* lse, const void* dout,
                                           const int32_t* block_ids, void* dq, void* dk, void* dv, void* ws,
                                           size_t ws_bytes, void* stream) {
  msa_status_t rc = validate(prob);
  if (rc != MSA_OK) return rc;
  if (prob->kv_format != MSA_IDX_PLAIN) return MSA_ERR_UNSUPPORTED;
  const void* ptrs[] = {q, k, v, out, lse, dout, block_ids, dq, dk, dv, ws};
  for (const void* x : ptrs)
    if (!x || !aligned16(x)) return MSA_ERR_INVALID_ARG;
  const msa::Shape s = shape_of(prob);
  const BwdLayout L = bwd_layout(s);
  if (ws_bytes < L.total) return MSA_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  float* drow = reinterpret_cast<float*>(w + L.drow);
  const msa::InvertPlan plan = msa::invert_plan(s, s.Nq);
  msa::InvertOut inv;
  inv.offsets = reinterpret_cast<int32_t*>(w + L.offsets);
  inv.entries = reinterpret_cast<int32_t*>(w + L.entries);
  inv.item_count = reinterpret_cast<int32_t*>(w + L.item_count);
  inv.items = reinterpret_cast<int4*>(w + L.items);
  hipError_t e = msa::launch_bwd_rowdot(s, out, dout, drow, st);
  if (e == hipSuccess) e = msa::launch_invert(s, plan, block_ids, 0, s.Nq, inv, w + L.inv_scratch, st);
  if (e == hipSuccess)
    e = msa::launch_bwd_attention(s, plan, q, k, v, dout, lse, drow, block_ids, inv,
                                  w + L.dq_part, w + L.dkv_part,
                                  w + L.trash, dq, dk, dv, st);
  return e == hipSuccess ? MSA_OK : hip_fail(e);
}

msa_status_t msa_indexer_kl(const msa_problem_t* prob, const void* q, const void* k, const void* idx_q,
                            const void* idx_k, const float* lse, const int32_t* block_ids, float loss_scale,
                            float* kl, void* d_iq, void* d_ik, void* ws, size_t ws_bytes, void* stream) {
  msa_status_t rc = validate(prob);
  if (rc != MSA_OK) return rc;
  if (prob->idx_format != MSA_IDX_PLAIN || prob->kv_format != MSA_IDX_PLAIN) return MSA_ERR_UNSUPPORTED;
  if (!std::isfinite(loss_scale)) return MSA_ERR_INVALID_ARG;
  const void* ptrs[] = {q, k, idx_q, idx_k, lse, block_ids, kl, d_iq, d_ik, ws};
  for (const void* x : ptrs)
    if (!x || !aligned16(x)) return MSA_ERR_INVALID_ARG;
  const msa::Shape s = shape_of(prob);
  const KlLayout L = kl_layout(s);
  if (ws_bytes < L.total) return MSA_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  const msa::InvertPlan plan = msa::invert_plan(s, s.Nq);
  msa::InvertOut inv;
  inv.offsets = reinterpret_cast<int32_t*>(w + L.offsets);
  inv.entries = reinterpret_cast<int32_t*>(w + L.entries);
  inv.item_count = reinterpret_cast<int32_t*>(w + L.item_count);
  inv.items = reinterpret_cast<int4*>(w + L.items);
  hipError_t e = msa::launch_invert(s, plan, block_ids, 0, s.Nq, inv, w + L.inv_scratch, st);
  if (e == hipSuccess)
    e = msa::launch_indexer_kl(s, plan, q, k, idx_q, idx_k, lse, block_ids, inv, w + L.kl, loss_scale, kl, d_iq,
                               d_ik, st);
  return e == hipSuccess ? MSA_OK : hip_fail(e);
}

msa_status_t msa_mxfp8_quantize(const void* src, int32_t src_dtype, int64_t n_rows, int32_t row_len, uint8_t* codes,
                                uint8_t* scales, void* stream) {
  if (!src || !codes || !scales || !aligned16(src) || !aligned16(codes)) return MSA_ERR_INVALID_ARG;
  if (src_dtype != MSA_F32 && src_dtype != MSA_BF16) return MSA_ERR_INVALID_ARG;
  if (n_rows < 0 || row_len <= 0 || row_len % 32 || n_rows > ((int64_t)1 << 40) / row_len) return MSA_ERR_INVALID_ARG;
  if (n_rows == 0) return MSA_OK;
  const hipError_t e = msa::launch_mxfp8_quantize(src, src_dtype == MSA_BF16 ? msa::kBF16 : msa::kF32, n_rows,
                                                  row_len, codes, scales, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MSA_OK : hip_fail(e);
}

msa_status_t msa_topk_from_scores(const msa_problem_t* prob, const float* scores, int32_t* block_ids, void* stream) {
  msa_status_t rc = validate(prob);
  if (rc != MSA_OK) return rc;
  if (!scores || !block_ids || !aligned16(scores) || !aligned16(block_ids)) return MSA_ERR_INVALID_ARG;
  const msa::Shape s = shape_of(prob);
  const hipError_t e = msa::launch_topk_rows(s, scores, block_ids, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MSA_OK : hip_fail(e);
}

msa_status_t msa_index_topk(const msa_problem_t* prob, const void* idx_q, const void* idx_k, int32_t* block_ids,
                            void* ws, size_t ws_bytes, void* stream) {
  msa_status_t rc = validate(prob);
  if (rc != MSA_OK) return rc;
  if (!idx_q || !idx_k || !block_ids || !aligned16(idx_q) || !aligned16(idx_k) || !aligned16(block_ids))
    return MSA_ERR_INVALID_ARG;
  if (ws && !aligned16(ws)) return MSA_ERR_INVALID_ARG;
  const msa::Shape s = shape_of(prob);
  return run_index(s, idx_q, idx_k, block_ids, ws, ws_bytes, static_cast<hipStream_t>(stream));
}

msa_status_t msa_invert(const msa_problem_t* prob, const int32_t* block_ids, int32_t* offsets, int32_t* entries,
                        void* ws, size_t ws_bytes, void* stream) {
  msa_status_t rc = validate(prob);
  if (rc != MSA_OK) return rc;
  if (!block_ids || !offsets || !entries || !ws || !aligned16(block_ids) || !aligned16(ws)) return MSA_ERR_INVALID_ARG;
  const msa::Shape s = shape_of(prob);
  const msa::InvertPlan plan = msa::invert_plan(s, s.Nq);
  if (ws_bytes < msa::invert_ws_bytes(s, plan)) return MSA_ERR_WORKSPACE;
  msa::InvertOut inv;
  inv.offsets = offsets;
  inv.entries = entries;
  inv.item_count = nullptr;
  inv.items = nullptr;
  const hipError_t e = msa::launch_invert(s, plan, block_ids, 0, s.Nq, inv, ws, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MSA_OK : hip_fail(e);
}

msa_status_t msa_sparse_attention(const msa_problem_t* prob, const void* q, const void* k, const void* v,
                                  const int32_t* block_ids, void* out, float* lse, void* ws, size_t ws_bytes,
                                  void* stream) {
  msa_status_t rc = validate(prob);
  if (rc != MSA_OK) return rc;
  if (!q || !k || !v || !block_ids || !out) return MSA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(block_ids) || !aligned16(out) ||
      (lse && !aligned16(lse)) || (ws && !aligned16(ws)))
    return MSA_ERR_INVALID_ARG;
  const msa::Shape s = shape_of(prob);
  size_t full = 0, least = 0;
  msa_workspace_size(prob, MSA_OP_ATTENTION, &full, &least);
  if (ws_bytes < least || (least && !ws)) return MSA_ERR_WORKSPACE;
  return run_attention(prob, s, q, k, v, block_ids, out, lse, ws, ws_bytes, static_cast<hipStream_t>(stream));
}

msa_status_t msa_forward(const msa_problem_t* prob, const void* q, const void* k, const void* v, const void* idx_q,
                         const void* idx_k, int32_t* block_ids, void* out, float* lse, void* ws, size_t ws_bytes,
                         void* stream) {
  msa_status_t rc = validate(prob);
  if (rc != MSA_OK) return rc;
  if (!q || !k || !v || !idx_q || !idx_k || !block_ids || !out) return MSA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(idx_q) || !aligned16(idx_k) ||
      !aligned16(block_ids) || !aligned16(out) || (lse && !aligned16(lse)) || (ws && !aligned16(ws)))
    return MSA_ERR_INVALID_ARG;
  const msa::Shape s = shape_of(prob);
  size_t full = 0, least = 0;
  msa_workspace_size(prob, MSA_OP_FORWARD, &full, &least);
  if (ws_bytes < least || (least && !ws)) return MSA_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  rc = run_index(s, idx_q, idx_k, block_ids, ws, ws_bytes, st);
  if (rc != MSA_OK) return rc;
  return run_attention(prob, s, q, k, v, block_ids, out, lse, ws, ws_bytes, st);
}

msa_status_t msa_profile_enable(int on) {
  {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof_on = on != 0;
  }
  return MSA_OK;
}

msa_status_t msa_profile_reset(void) {
  msa_status_t rc = prof_flush();
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (ProfKernel& k : prof_kernels()) {
    k.ms = 0.0;
    k.launches = 0;
  }
  return rc;
}

int msa_profile_count(void) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  return (int)prof_kernels().size();
}

msa_status_t msa_profile_read(int index, const char** name, double* total_ms, int64_t* launches) {
  msa_status_t rc = prof_flush();
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (index < 0 || index >= (int)prof_kernels().size()) return MSA_ERR_INVALID_ARG;
  const ProfKernel& k = prof_kernels()[index];
  if (name) *name = k.name;
  if (total_ms) *total_ms = k.ms;
  if (launches) *launches = k.launches;
  return rc;
}

}  // extern "C"
