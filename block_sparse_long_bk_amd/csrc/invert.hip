// invert.hip -- block -> query inversion for the KV-outer schedule (gfx950).
//
// The KV-outer path keeps one selected key block resident and streams the
// queries that chose it (paper summary page, "Key Contributions": KV-outer
// sparse attention, skewed block popularity handled without atomic updates).
// It needs, for every (b, g), the list of (query, slot) pairs that selected
// each block: a CSR transpose of the block-id table, built here as a
// deterministic counting sort keyed by block id:
//   1. k_inv_hist     per 256-query tile: count picks of every block
//                     (LDS counters; counts do not depend on order);
//   2. k_inv_colscan  per block: exclusive prefix of the tile counts;
//   3. k_inv_blkscan  per (b, g): exclusive prefix over blocks -> offsets, and
//                     of ceil(count/QI) -> work-item offsets;
//   4. k_inv_scatter  per tile, one wave walks its queries in order and
//                     places each pick at offsets[j] + (earlier picks of j):
//                     entries of a block come out in ascending (query, slot)
//                     order.  A row may name a block more than once (the
//                     attention then counts it once per listing): the lanes
//                     of one step rank themselves among the lower lanes with
//                     the same id, and the last of them advances the cursor,
//                     so every entry slot and every cursor has one writer and
//                     no atomics are needed;
//   5. k_inv_items    splits each block's entries into work items of at most
//                     QI queries; a hot block yields many items, which is
//                     what absorbs the skew.
// Every output word has exactly one writer.
#include "msa_device.h"
#include "msa_internal.h"

namespace msa {
namespace {

struct InvArgs {
  const int32_t* ids;  // [B, Nq, Hkv, topk]
  int32_t* hist;       // [B*Hkv][n_tiles][nblk]
  int32_t* totals;     // [B*Hkv][nblk]
  int32_t* item_off;   // [B*Hkv][nblk+1]
  int32_t* offsets;    // [B*Hkv][nblk+1]
  int32_t* entries;    // [B*Hkv][nq*topk]
  int32_t* item_count; // [B*Hkv]
  int4* items;         // [B*Hkv][items_cap]
  int Nq, Hkv, topk, nblk, q0, nq, n_tiles, items_cap, qi;
};

__global__ void __launch_bounds__(kInvTile) k_inv_hist(InvArgs a) {
  extern __shared__ int32_t cnt[];
  const int tile = blockIdx.x, bg = blockIdx.y;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  for (int j = threadIdx.x; j < a.nblk; j += blockDim.x) cnt[j] = 0;
  __syncthreads();
  const int qq = tile * kInvTile + threadIdx.x;  // chunk-relative query
  if (qq < a.nq) {
    const int32_t* row = a.ids + (((int64_t)b * a.Nq + a.q0 + qq) * a.Hkv + g) * a.topk;
    for (int s = 0; s < a.topk; ++s) {
      const int j = row[s];
      if (j >= 0 && j < a.nblk) atomicAdd(&cnt[j], 1);
    }
  }
  __syncthreads();
  int32_t* out = a.hist + ((int64_t)bg * a.n_tiles + tile) * a.nblk;
  for (int j = threadIdx.x; j < a.nblk; j += blockDim.x) out[j] = cnt[j];
}

__global__ void __launch_bounds__(256) k_inv_colscan(InvArgs a) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x, bg = blockIdx.y;
  if (j >= a.nblk) return;
  int32_t run = 0;
  int32_t* h = a.hist + (int64_t)bg * a.n_tiles * a.nblk + j;
  for (int t = 0; t < a.n_tiles; ++t) {
    const int32_t c = h[(int64_t)t * a.nblk];
    h[(int64_t)t * a.nblk] = run;
    run += c;
  }
  a.totals[(int64_t)bg * a.nblk + j] = run;
}

// Exclusive scan of v over the workgroup (1024 threads); returns the prefix
// and leaves the workgroup total in *total.
__device__ int32_t block_exclusive_scan(int32_t v, int32_t* tmp, int32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int32_t inc = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int32_t o = __shfl_up(inc, d, 64);
    if (lane >= d) inc += o;
  }
  if (lane == 63) tmp[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    int32_t w = lane < nw ? tmp[lane] : 0;
    int32_t wi = w;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int32_t o = __shfl_up(wi, d, 64);
      if (lane >= d) wi += o;
    }
    if (lane < nw) tmp[lane] = wi - w;
    if (lane == nw - 1) tmp[64] = wi;
  }
  __syncthreads();
  const int32_t res = tmp[wave] + inc - v;
  *total = tmp[64];
  __syncthreads();
  return res;
}

__global__ void __launch_bounds__(1024) k_inv_blkscan(InvArgs a) {
  __shared__ int32_t tmp[65];
  const int bg = blockIdx.x;
  const int per = (a.nblk + blockDim.x - 1) / blockDim.x;
  const int j0 = threadIdx.x * per;
  const int32_t* tot = a.totals + (int64_t)bg * a.nblk;
  int32_t s = 0, si = 0;
  for (int j = j0; j < min(j0 + per, a.nblk); ++j) {
    s += tot[j];
    si += (tot[j] + a.qi - 1) / a.qi;
  }
  int32_t all, all_i;
  int32_t base = block_exclusive_scan(s, tmp, &all);
  int32_t base_i = block_exclusive_scan(si, tmp, &all_i);
  int32_t* off = a.offsets + (int64_t)bg * (a.nblk + 1);
  int32_t* ioff = a.item_off + (int64_t)bg * (a.nblk + 1);
  for (int j = j0; j < min(j0 + per, a.nblk); ++j) {
    off[j] = base;
    ioff[j] = base_i;
    base += tot[j];
    base_i += (tot[j] + a.qi - 1) / a.qi;
  }
  if (threadIdx.x == 0) {
    off[a.nblk] = all;
    ioff[a.nblk] = all_i;
    if (a.item_count) a.item_count[bg] = all_i;
  }
}

// One wave per (b, g, tile).  LDS: cursors [nblk], then the tile's ids, one
// row of inv_row_pitch(topk) words per query (rows padded to whole 16-byte
// chunks with -1, so that a step reads its row with 16-byte broadcasts), then
// one flag per row: set where the row's valid ids are not strictly ascending,
// the only rows that can name a block twice (the Index Branch writes its rows
// ascending, so for them every flag is clear and each step is a single pass).
__global__ void __launch_bounds__(64) k_inv_scatter(InvArgs a) {
  extern __shared__ __attribute__((aligned(16))) int32_t sm[];
  int32_t* cur = sm;
  const int tp = inv_row_pitch(a.topk);
  int32_t* tids = sm + ((a.nblk + 3) & ~3);
  int32_t* unsorted = tids + kInvTile * tp;
  const int tile = blockIdx.x, bg = blockIdx.y;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int lane = threadIdx.x;
  const int32_t* off = a.offsets + (int64_t)bg * (a.nblk + 1);
  const int32_t* pre = a.hist + ((int64_t)bg * a.n_tiles + tile) * a.nblk;
  for (int j = lane; j < a.nblk; j += 64) cur[j] = off[j] + pre[j];
  const int qbeg = tile * kInvTile;
  const int nt = min(kInvTile, a.nq - qbeg);
  for (int e = lane; e < nt * tp; e += 64) {
    const int qq = qbeg + e / tp, s = e % tp;
    tids[e] = s < a.topk ? a.ids[(((int64_t)b * a.Nq + a.q0 + qq) * a.Hkv + g) * a.topk + s] : -1;
  }
  __syncthreads();
  for (int t = lane; t < nt; t += 64) {
    const int32_t* row = tids + t * tp;
    int last = -1, bad = 0;
    for (int s = 0; s < a.topk; ++s) {
      const int v = row[s];
      if (v >= 0 && v < a.nblk) {
        bad |= v <= last ? 1 : 0;
        last = v;
      }
    }
    unsorted[t] = bad;
  }
  __syncthreads();
  int32_t* ent = a.entries + (int64_t)bg * a.nq * a.topk;
  for (int t = 0; t < nt; ++t) {
    const int32_t* row = tids + t * tp;
    const int j = lane < a.topk ? row[lane] : -1;
    const bool ok = j >= 0 && j < a.nblk;
    if (!__builtin_amdgcn_readfirstlane(unsorted[t])) {  // distinct blocks: one cursor per lane
      if (ok) {
        const int32_t pos = cur[j];
        cur[j] = pos + 1;
        ent[pos] = (qbeg + t) * a.topk + lane;
      }
      wave_lds_sync();  // the next step may read a cursor another lane just advanced
      continue;
    }
    // rank among the lower slots of this row that name the same block, and
    // how many slots name it
    int rank = 0, cnt = 0;
    for (int c = 0; c < tp; c += 4) {
      const int4 v = *reinterpret_cast<const int4*>(row + c);
      const int vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int eq = vv[u] == j ? 1 : 0;
        cnt += eq;
        rank += c + u < lane ? eq : 0;
      }
    }
    const int32_t base = ok ? cur[j] : 0;
    wave_lds_sync();  // every lane has read its cursor before any is advanced
    if (ok) {
      ent[base + rank] = (qbeg + t) * a.topk + lane;
      if (rank == cnt - 1) cur[j] = base + cnt;
    }
    wave_lds_sync();  // the next step may read a cursor another lane just advanced
  }
}

__global__ void __launch_bounds__(256) k_inv_items(InvArgs a) {
  const int it = blockIdx.x * blockDim.x + threadIdx.x, bg = blockIdx.y;
  const int n = a.item_count[bg];
  if (it >= n) return;
  const int32_t* ioff = a.item_off + (int64_t)bg * (a.nblk + 1);
  const int32_t* off = a.offsets + (int64_t)bg * (a.nblk + 1);
  // largest j with ioff[j] <= it (blocks with no items share their offset)
  int lo = 0, hi = a.nblk - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (ioff[mid] <= it) lo = mid;
    else hi = mid - 1;
  }
  const int j = lo;
  const int m = it - ioff[j];
  const int e0 = off[j] + m * a.qi;
  const int e1 = min(e0 + a.qi, off[j + 1]);
  a.items[(int64_t)bg * a.items_cap + it] = make_int4(j, e0, e1, 0);
}

}  // namespace

InvertPlan invert_plan(const Shape& s, int nq_chunk) {
  InvertPlan p;
  p.nq_chunk = nq_chunk;
  p.n_tiles = (nq_chunk + kInvTile - 1) / kInvTile;
  const int G = s.Hq / s.Hkv;
  p.qi = kItemRows / G < kItemEntries ? kItemRows / G : kItemEntries;
  const int64_t cap = ((int64_t)nq_chunk * s.topk + p.qi - 1) / p.qi + s.nblk;
  p.items_cap = (int)((cap + 7) / 8 * 8);
  return p;
}

// Internal scratch: hist, totals, item offsets.
size_t invert_ws_bytes(const Shape& s, const InvertPlan& p) {
  const size_t bg = (size_t)s.B * s.Hkv;
  return bg * (size_t)p.n_tiles * s.nblk * 4 + bg * s.nblk * 4 + bg * (s.nblk + 1) * 4;
}

hipError_t launch_invert(const Shape& s, const InvertPlan& p, const int32_t* ids, int q0, int nq, InvertOut out,
                         void* ws, hipStream_t st) {
  static const int k1 = prof_register("inv_hist");
  static const int k2 = prof_register("inv_colscan");
  static const int k3 = prof_register("inv_blkscan");
  static const int k4 = prof_register("inv_scatter");
  static const int k5 = prof_register("inv_items");
  const int BG = s.B * s.Hkv;
  InvArgs a;
  a.ids = ids;
  char* w = static_cast<char*>(ws);
  a.hist = reinterpret_cast<int32_t*>(w);
  w += (size_t)BG * p.n_tiles * s.nblk * 4;
  a.totals = reinterpret_cast<int32_t*>(w);
  w += (size_t)BG * s.nblk * 4;
  a.item_off = reinterpret_cast<int32_t*>(w);
  a.offsets = out.offsets;
  a.entries = out.entries;
  a.item_count = out.item_count;
  a.items = out.items;
  a.Nq = s.Nq;
  a.Hkv = s.Hkv;
  a.topk = s.topk;
  a.nblk = s.nblk;
  a.q0 = q0;
  a.nq = nq;
  a.n_tiles = (nq + kInvTile - 1) / kInvTile;
  a.items_cap = p.items_cap;
  a.qi = p.qi;
  hipError_t e;
#define MSA_INV_LAUNCH(kid, ...)        \
  prof_begin(st, kid);                  \
  hipLaunchKernelGGL(__VA_ARGS__);      \
  e = hipGetLastError();                \
  prof_end(st, kid);                    \
  if (e != hipSuccess) return e;
  MSA_INV_LAUNCH(k1, k_inv_hist, dim3(a.n_tiles, BG), dim3(kInvTile), (size_t)s.nblk * 4, st, a)
  MSA_INV_LAUNCH(k2, k_inv_colscan, dim3((s.nblk + 255) / 256, BG), dim3(256), 0, st, a)
  MSA_INV_LAUNCH(k3, k_inv_blkscan, dim3(BG), dim3(1024), 0, st, a)
  MSA_INV_LAUNCH(k4, k_inv_scatter, dim3(a.n_tiles, BG), dim3(64),
                 (size_t)(((s.nblk + 3) & ~3) + kInvTile * (inv_row_pitch(s.topk) + 1)) * 4, st, a)
  if (out.items) {
    MSA_INV_LAUNCH(k5, k_inv_items, dim3(p.items_cap / 256 + 1, BG), dim3(256), 0, st, a)
  }
#undef MSA_INV_LAUNCH
  return hipSuccess;
}

}  // namespace msa
