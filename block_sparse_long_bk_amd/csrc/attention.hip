// attention.hip -- Main Branch of MiniMax Sparse Attention on gfx950.
//
// Exact scaled-dot-product softmax attention of every query head over the
// visible tokens (t <= position) of its GQA group's selected 128-token key
// blocks (paper summary page, "Method"; zhichai.net write-up, section 2: the
// heads of a group share the group's blocks but keep their own queries).
//
// Both schedules compute, per (query head, selected block), the block's
// online-softmax partial (max m, sum l, normalised output o = acc/l) and merge
// the partials of a row with a log-sum-exp combine -- the standard
// FlashAttention recurrence (cited by the Fireworks note on KV-stationary
// attention), which is exact up to rounding order.
//
//  * k_attn_kvouter -- KV-stationary (the paper's KV-outer path, abstract and
//    "Key Contributions").  One workgroup per work item (block j, up to 1024
//    (query, head) rows that chose j).  K_j (row-major) and V_j (transposed) are
//    staged once in LDS; 32-row tiles of the gathered queries stream through
//        S^T = K_j Q^T      (MFMA: A = K rows from LDS, B = Q rows from HBM)
//        O^T = V_j^T P^T    (MFMA: A = V^T rows from LDS, B = P from registers)
//    Computing the transposed products keeps each query row inside one lane
//    pair, so the softmax is in-register (plus one swap between wave halves)
//    and P never touches LDS.  Each (query, head, slot) partial has exactly one
//    writer: no atomics.
//  * k_attn_qouter -- query-stationary (the baseline schedule of the Fireworks
//    note, "The design space").  One workgroup per (query, group, split) keeps
//    the group's query heads resident and walks its selected blocks; the four
//    waves split each block's 128 keys and merge their states at the end.
//  * k_combine -- log-sum-exp merge of the partials into the output.
#include <type_traits>

#include "attn_common.h"

namespace msa {
namespace {

// One 32-row tile of one key block: S^T = K Q^T, mask, softmax statistics,
// O^T = V^T P^T.  Lane (c = lane%32, h = lane/32) ends with the tile row c's
// block max (log2 domain, already scaled) m, sum l, and its 64 of the D output
// values in o[dt][e] for d = 32dt + 8(e/4) + 4h + e%4.
// Keys at offsets >= vis (0..BK) inside the block are masked when need_mask.
template <typename T, int D, int BK>
__device__ __forceinline__ void block_tile(const char* lds, const frag_t<T> (&qf)[D / 16], float c_log2, int vis,
                                           bool need_mask, float& m, float& l, f32x16 (&o)[D / 32]) {
  using L = KvLds<T, D, BK>;
  constexpr int MT = BK / 32;  // 32-key M-tiles per block
  const int lane = threadIdx.x & 63, half = lane >> 5;
  f32x16 s[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const T* arow = reinterpret_cast<const T*>(lds + (mt * 32 + (lane & 31)) * L::KPITCH) + 8 * half;
    s[mt] = mma0(load8(arow), qf[0]);
#pragma unroll
    for (int ks = 1; ks < D / 16; ++ks) mma(load8(arow + 16 * ks), qf[ks], s[mt]);
  }
  if (need_mask) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int t = 32 * mt + 8 * (e / 4) + 4 * half + (e % 4);
        if (t >= vis) s[mt][e] = -__builtin_huge_valf();
      }
  }
  float mx = -__builtin_huge_valf();
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) mx = max16(s[mt], mx);
  mx = pair32_max(mx);
  const float mref = mx == -__builtin_huge_valf() ? 0.f : mx * c_log2;
  float sum = 0.f;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float p = exp2_fast(fmaf(s[mt][e], c_log2, -mref));
      s[mt][e] = p;
      sum += p;
    }
  sum = pair32_sum(sum);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      frag_t<T> pb;
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[e] = from_f32<T>(s[mt][8 * a + e]);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const frag_t<T> va = vt_frag<T, D, BK>(lds, 32 * dt + (lane & 31), mt, a, half);
        if (mt == 0 && a == 0) o[dt] = mma0(va, pb);
        else mma(va, pb, o[dt]);
      }
    }
  m = mx == -__builtin_huge_valf() ? -__builtin_huge_valf() : mref;
  l = sum;
}

struct KvArgs {
  const void* q;
  const void* k;    // K rows, or MXFP8 codes
  const void* v;
  const uint8_t* ksc;  // MXFP8 scale rows of K and V (KVMX kernels only)
  const uint8_t* vsc;
  const int32_t* entries;
  const int32_t* item_count;
  const int4* items;
  void* part_o;  // [B, nq, Hq, S, D] in the input dtype
  float* part_lse;
  void* trash;      // kTrashBytes of scratch for the stores of rows past an item's end
  float* trash_lse;
  int Nq, Nk, Hq, Hkv, G, topk, S, q0, nq, items_cap, gshift;
  int64_t q_offset;
  uint64_t topk_magic;  // ceil(2^40 / topk)
  float c_log2;  // softmax scale * log2(e)
};

// One 32-row tile of a KV-outer work item: prefetches the query rows of tile
// `tile + 4` into (nxt, qn), computes the tile's partials from (cur, qf) and
// writes them out.  Partial rows leave through LDS (`ob`, this wave's 8-row
// buffer), 8 rows per pass, so that each store instruction writes four whole
// rows instead of an 8-byte piece of 32.
template <typename T, int D, bool NT, int BK>
__device__ __forceinline__ void kv_tile(const KvArgs& a, const char* lds, const int32_t* ent_lds, char* ob, int tile,
                                        int nrows, int b, int g, int64_t key0, const TileRows& cur,
                                        const frag_t<T> (&qf)[D / 16], TileRows& nxt, frag_t<T> (&qn)[D / 16]) {
  constexpr int ROWB = D * (int)sizeof(T);   // bytes of one partial row
  constexpr int OPITCH = ROWB + 16;          // padded LDS row
  constexpr int LPR = ROWB / 16;             // lanes per row on the way out
  constexpr int RPS = 64 / LPR;              // rows per store instruction
  const int lane = threadIdx.x & 63, half = lane >> 5;
  const int rn = (tile + 4) * 32 + (lane & 31);
  const int en = ent_lds[min(rn >> a.gshift, kMaxItemEntries - 1)];
  nxt = rows_of(rn < nrows ? en : 0, rn < nrows, rn, a.gshift, a.topk, a.topk_magic, g);
  load_q_rows<T, D>(qn, static_cast<const T*>(a.q), nxt, b, a.Nq, a.Hq, a.q0, half);
  const int64_t pos = a.q_offset + a.q0 + cur.qq;
  const int64_t vis_end = min(pos + 1, (int64_t)a.Nk);  // keys t < vis_end are visible
  const int vis = (int)max((int64_t)0, min((int64_t)BK, vis_end - key0));
  // Masking is only needed where the block reaches past a row's position.
  const int need = __any(cur.valid && vis < BK);
  float m, l;
  f32x16 o[D / 32];
  block_tile<T, D, BK>(lds, qf, a.c_log2, vis, need != 0, m, l, o);
  const int64_t prow = (((int64_t)b * a.nq + cur.qq) * a.Hq + cur.h) * a.S + cur.slot;
  const int64_t lrow = (((int64_t)b * a.nq + cur.qq) * a.S + cur.slot) * a.Hq + cur.h;
  // Every store below is issued by every lane (rows past the item's end write
  // to a scratch line instead): with no store under a branch the compiler
  // counts the outstanding memory operations exactly, and the wait for the
  // next tile's query rows does not also wait for these stores.  Both halves
  // of the wave hold the row's m and l, so both write the same lse.
  store_partial<NT>(cur.valid ? a.part_lse + lrow : a.trash_lse, (m + log2_fast(l)) * kLn2);
  const float inv = 1.f / l;
  // The normalised row in the output type, converted once (the passes below
  // only pick which lanes write it).
  typename Pack4<T>::type ow[D / 32][4];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) ow[dt][i][rr] = from_f32<T>(o[dt][4 * i + rr] * inv);
#pragma unroll
  for (int ps = 0; ps < 4; ++ps) {
    if (((lane & 31) >> 3) == ps) {
      char* orow = ob + ((lane & 7) * OPITCH);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *reinterpret_cast<typename Pack4<T>::type*>(orow + (32 * dt + 8 * i + 4 * half) * (int)sizeof(T)) = ow[dt][i];
    }
    wave_lds_sync();  // the rows written above are read by other lanes below
    // lane -> (row ps*8 + lane/LPR + k*RPS, 16-byte chunk lane%LPR)
#pragma unroll
    for (int k = 0; k < 8 / RPS; ++k) {
      const int rl = lane / LPR + k * RPS;
      const int src = ps * 8 + rl;
      const int64_t dst_row = __shfl(prow, src, 64);
      const int ok = __shfl((int)cur.valid, src, 64);
      const u32x4 v = *reinterpret_cast<const u32x4*>(ob + rl * OPITCH + (lane % LPR) * 16);
      char* dst = ok ? static_cast<char*>(a.part_o) + dst_row * ROWB : static_cast<char*>(a.trash);
      store_partial<NT>(reinterpret_cast<u32x4*>(dst + (lane % LPR) * 16), v);
    }
    wave_lds_sync();  // the next pass overwrites the rows just read
  }
}

// KVMX: K and V are MXFP8 caches, decoded while staged.
template <typename T, int D, bool NT, int BK, bool KVMX>
__global__ void __launch_bounds__(256, 2) k_attn_kvouter(KvArgs a) {
  using L = KvLds<T, D, BK>;
  __shared__ __attribute__((aligned(16))) char lds[L::BYTES];
  __shared__ int32_t ent_lds[kMaxItemEntries];
  __shared__ __attribute__((aligned(16))) char obuf[4][8 * (D * (int)sizeof(T) + 16)];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5;
  const int bg = blockIdx.y, b = bg / a.Hkv, g = bg % a.Hkv;
  // Items of one (b, g) are spread so that each XCD (workgroup id mod 8) runs a
  // contiguous run of them: neighbouring items share their key block in L2.
  const int n = a.item_count[bg];
  const int per = (n + 7) / 8;
  const int x = blockIdx.x;
  const int item = (x % 8) * per + x / 8;
  if (x / 8 >= per || item >= n) return;
  const int4 it = a.items[(int64_t)bg * a.items_cap + item];
  const int j = it.x, e0 = it.y, e1 = it.z;
  const int nrows = (e1 - e0) * a.G;

  const int64_t tok_stride = (int64_t)a.Hkv * D;
  const T* kb = static_cast<const T*>(a.k) + (int64_t)b * a.Nk * tok_stride + g * D;
  const T* vb = static_cast<const T*>(a.v) + (int64_t)b * a.Nk * tok_stride + g * D;
  const int32_t* ent = a.entries + (int64_t)bg * a.nq * a.topk + e0;
  const int nent = e1 - e0;
  const T* qbase = static_cast<const T*>(a.q);
  const int64_t key0 = (int64_t)j * BK;

  // Prologue, ordered so that the loads overlap: (1) the entries (this lane's
  // first row, and the item's list for LDS), (2) K_j / V_j into registers,
  // (3) the first tile's query rows, then the LDS stores.  Vector-memory
  // counters retire in order, so each wait only covers the older loads.
  const int r0 = wave * 32 + (lane & 31);
  const int e_first = r0 < nrows ? ent[r0 >> a.gshift] : 0;
  constexpr int EPT = kMaxItemEntries / 256;  // entries per thread
  static_assert(kMaxItemEntries % 256 == 0, "whole entries per thread");
  int e_mine[EPT];
#pragma unroll
  for (int u = 0; u < EPT; ++u) e_mine[u] = tid + 256 * u < nent ? ent[tid + 256 * u] : 0;
  __builtin_amdgcn_sched_barrier(0);
  std::conditional_t<KVMX, KvStageMx<T, D, BK>, KvStage<T, D, BK>> stg;
  if constexpr (KVMX) {
    const int64_t r0 = (int64_t)b * a.Nk * a.Hkv + g;  // first (token, group) row of this (b, g)
    stg.load(static_cast<const uint8_t*>(a.k) + r0 * D, static_cast<const uint8_t*>(a.v) + r0 * D,
             a.ksc + r0 * (D / 32), a.vsc + r0 * (D / 32), (int64_t)a.Hkv * D, j, a.Nk, tid);
  } else {
    stg.load(kb, vb, tok_stride, j, a.Nk, tid);
  }
  __builtin_amdgcn_sched_barrier(0);
  // Gathered query rows of tile t: row r = t*32 + lane%32 <-> (entry r/G, head r%G).
  TileRows cur = rows_of(e_first, r0 < nrows, r0, a.gshift, a.topk, a.topk_magic, g);
  frag_t<T> qf[D / 16];
  load_q_rows<T, D>(qf, qbase, cur, b, a.Nq, a.Hq, a.q0, half);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int u = 0; u < EPT; ++u)
    if (tid + 256 * u < nent) ent_lds[tid + 256 * u] = e_mine[u];
  stg.store(lds, tid);
  __syncthreads();

  // Tiles alternate between two query-fragment buffers: tile t computes from
  // one while the rows of tile t+4 load into the other.  (A single buffer
  // refilled by register copies made the wave wait at every copy for all of
  // its outstanding memory operations, the partial stores included.)
  // The first tile is peeled so that the loop is entered with the same
  // outstanding operations (one tile's query loads, then its stores) on both
  // paths; otherwise the merged count makes the first wait cover the stores.
  frag_t<T> qg[D / 16];
  TileRows nx;
  if (wave * 32 >= nrows) return;
  kv_tile<T, D, NT, BK>(a, lds, ent_lds, obuf[wave], wave, nrows, b, g, key0, cur, qf, nx, qg);
  for (int tile = wave + 4; tile * 32 < nrows; tile += 8) {
    kv_tile<T, D, NT, BK>(a, lds, ent_lds, obuf[wave], tile, nrows, b, g, key0, nx, qg, cur, qf);
    if ((tile + 4) * 32 >= nrows) break;
    kv_tile<T, D, NT, BK>(a, lds, ent_lds, obuf[wave], tile + 4, nrows, b, g, key0, cur, qf, nx, qg);
  }
}

struct QoArgs {
  const void* q;
  const void* k;    // K rows, or MXFP8 codes
  const void* v;
  const uint8_t* ksc;  // MXFP8 scale rows of K and V (KVMX kernels only)
  const uint8_t* vsc;
  const int32_t* ids;
  void* out;
  float* lse;
  void* part_o;
  float* part_lse;
  int Nq, Nk, Hq, Hkv, G, topk, nsplit, q0, nq;
  int64_t q_offset;
  float c_log2;
};

// grid: x = nq * Hkv, y = nsplit, z = B.  256 threads; wave w owns keys
// [32w, 32w + 32) of every block (waves past the block's BK / 32 tiles idle).
template <typename T, int D, int BK, bool KVMX>
__global__ void __launch_bounds__(256, 2) k_attn_qouter(QoArgs a) {
  using L = KvLds<T, D, BK>;
  constexpr int MERGE_BYTES = 4 * D * 32 * (int)sizeof(float);  // the final merge reuses the staging area
  __shared__ __attribute__((aligned(16))) char lds[L::BYTES > MERGE_BYTES ? L::BYTES : MERGE_BYTES];
  __shared__ float stat[4][2][32];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5;
  const int qq = blockIdx.x / a.Hkv, g = blockIdx.x % a.Hkv;
  const int split = blockIdx.y, b = blockIdx.z;
  const int64_t qglob = (int64_t)a.q0 + qq;
  const int64_t pos = a.q_offset + qglob;
  const int64_t vis_end = min(pos + 1, (int64_t)a.Nk);
  const int per = (a.topk + a.nsplit - 1) / a.nsplit;
  const int s0 = split * per, s1 = min(a.topk, s0 + per);

  const int c = lane & 31;
  const bool valid = c < a.G;
  const int h = g * a.G + (valid ? c : 0);
  const T* qrow = static_cast<const T*>(a.q) + ((((int64_t)b * a.Nq + qglob) * a.Hq + h) * D) + 8 * half;
  frag_t<T> qf[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) qf[ks] = valid ? load8(qrow + 16 * ks) : zero_frag<T>();

  const int64_t tok_stride = (int64_t)a.Hkv * D;
  const T* kb = static_cast<const T*>(a.k) + (int64_t)b * a.Nk * tok_stride + g * D;
  const T* vb = static_cast<const T*>(a.v) + (int64_t)b * a.Nk * tok_stride + g * D;
  const int32_t* sel = a.ids + ((((int64_t)b * a.Nq + qglob) * a.Hkv) + g) * a.topk;

  float m = -__builtin_huge_valf(), l = 0.f;
  f32x16 o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) o[dt] = f32x16{};

  for (int s = s0; s < s1; ++s) {
    const int j = sel[s];
    if (j < 0) continue;  // uniform across the workgroup
    __syncthreads();
    if constexpr (KVMX) {
      const int64_t r0 = (int64_t)b * a.Nk * a.Hkv + g;
      KvStageMx<T, D, BK> stg;
      stg.load(static_cast<const uint8_t*>(a.k) + r0 * D, static_cast<const uint8_t*>(a.v) + r0 * D,
               a.ksc + r0 * (D / 32), a.vsc + r0 * (D / 32), (int64_t)a.Hkv * D, j, a.Nk, tid);
      stg.store(lds, tid);
    } else {
      stage_kv<T, D, BK>(lds, kb, vb, tok_stride, j, a.Nk, tid);
    }
    __syncthreads();
    if (wave * 32 >= BK) continue;  // no keys for this wave (uniform per wave)
    // wave's 32 keys: S^T tile for M-tile `wave`
    f32x16 sc = f32x16{};
    const T* arow = reinterpret_cast<const T*>(lds + (wave * 32 + c) * L::KPITCH) + 8 * half;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) mma(load8(arow + 16 * ks), qf[ks], sc);
    const int64_t kbase = (int64_t)j * BK + wave * 32;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int64_t t = kbase + 8 * (e / 4) + 4 * half + (e % 4);
      if (t >= vis_end) sc[e] = -__builtin_huge_valf();
    }
    float mx = max16(sc);
    mx = pair32_max(mx);
    const float mnew = fmaxf(m, mx == -__builtin_huge_valf() ? -__builtin_huge_valf() : mx * a.c_log2);
    const float mref = mnew == -__builtin_huge_valf() ? 0.f : mnew;
    const float alpha = exp2_fast(m - mref);
    float sum = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float p = exp2_fast(fmaf(sc[e], a.c_log2, -mref));
      sc[e] = p;
      sum += p;
    }
    sum = pair32_sum(sum);
    l = l * alpha + sum;
    m = mnew;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[dt][e] *= alpha;
#pragma unroll
    for (int aa = 0; aa < 2; ++aa) {
      frag_t<T> pb;
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[e] = from_f32<T>(sc[8 * aa + e]);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) mma(vt_frag<T, D, BK>(lds, 32 * dt + c, wave, aa, half), pb, o[dt]);
    }
  }
  // Merge the four waves' states through LDS (reusing the staging area).
  __syncthreads();
  float* ob = reinterpret_cast<float*>(lds);  // [4 waves][D][32]
  if (half == 0) {
    stat[wave][0][c] = m;
    stat[wave][1][c] = l;
  }
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int d = 32 * dt + 8 * (e / 4) + 4 * half + (e % 4);
      ob[(wave * D + d) * 32 + c] = o[dt][e];
    }
  __syncthreads();
  // threads: row c2 = tid % 32, d-range split over tid / 32 (8 groups)
  const int c2 = tid & 31, dg = tid >> 5;
  if (c2 < a.G) {
    float M = -__builtin_huge_valf();
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, stat[w][0][c2]);
    const float Mref = M == -__builtin_huge_valf() ? 0.f : M;
    float wgt[4], Ls = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      wgt[w] = exp2_fast(stat[w][0][c2] - Mref);
      Ls += wgt[w] * stat[w][1][c2];
    }
    const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
    const int h2 = g * a.G + c2;
    const float lse_v = Ls > 0.f ? (M + log2_fast(Ls)) * kLn2 : -__builtin_huge_valf();
    constexpr int DPG = D / 8;
    if (a.nsplit == 1) {
      T* orow = static_cast<T*>(a.out) + (((int64_t)b * a.Nq + qglob) * a.Hq + h2) * D;
      for (int d = dg * DPG; d < (dg + 1) * DPG; ++d) {
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) acc += wgt[w] * ob[(w * D + d) * 32 + c2];
        orow[d] = from_f32<T>(acc * inv);
      }
      if (dg == 0 && a.lse) a.lse[((int64_t)b * a.Nq + qglob) * a.Hq + h2] = lse_v;
    } else {
      const int64_t prow = (((int64_t)b * a.nq + qq) * a.Hq + h2) * a.nsplit + split;
      const int64_t lrow = (((int64_t)b * a.nq + qq) * a.nsplit + split) * a.Hq + h2;
      T* po = static_cast<T*>(a.part_o) + prow * D;
      for (int d = dg * DPG; d < (dg + 1) * DPG; ++d) {
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) acc += wgt[w] * ob[(w * D + d) * 32 + c2];
        po[d] = from_f32<T>(acc * inv);
      }
      if (dg == 0) a.part_lse[lrow] = lse_v;
    }
  }
}

struct CombArgs {
  const void* part_o;
  const float* part_lse;
  const int32_t* ids;
  void* out;
  float* lse;
  int Nq, Hq, Hkv, G, topk, S, q0, nq, ids_slots, nblk;
};

template <typename T> struct Pack8;
template <> struct Pack8<bf16_t> { using type = bf16x8; };
template <> struct Pack8<float> { using type = f32x8; };

// D/8 lanes per (b, query, head) row, 8 output values per lane: merge the S
// partials of the row by log-sum-exp weights.  Slots whose block id lies
// outside [0, nblk) (KV-outer: the inversion gave them no partial) or whose
// lse is -inf (no visible key, or an empty query-outer split) carry no weight.
template <typename T, int D, int SMAX>
__global__ void __launch_bounds__(256) k_combine(CombArgs a) {
  constexpr int LPH = D / 8;     // lanes per row
  constexpr int RPW = 64 / LPH;  // rows per wave
  const int lane = threadIdx.x & 63;
  const int sub = lane % LPH;
  const int64_t row = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW + lane / LPH;  // (qq, h)
  const int b = blockIdx.y;
  if (row >= (int64_t)a.nq * a.Hq) return;  // no cross-lane work below
  const int qq = (int)(row / a.Hq), h = (int)(row % a.Hq), g = h / a.G;
  const int64_t prow = ((int64_t)b * a.nq + qq) * a.Hq + h;
  const int32_t* sel = a.ids + (((int64_t)b * a.Nq + a.q0 + qq) * a.Hkv + g) * a.topk;
  const float* pl = a.part_lse + ((int64_t)b * a.nq + qq) * a.S * a.Hq + h;
  // All slot statistics are loaded at once (S <= SMAX); the slot ids four at
  // a time where a row of them is 16-byte aligned (topk a multiple of 4).
  int idv[SMAX];
  if (a.ids_slots && (a.topk & 3) == 0) {
#pragma unroll
    for (int s4 = 0; s4 < SMAX / 4; ++s4) {
      const int4 t = 4 * s4 < a.S ? *reinterpret_cast<const int4*>(sel + 4 * s4) : int4{0, 0, 0, 0};
      idv[4 * s4] = t.x;
      idv[4 * s4 + 1] = t.y;
      idv[4 * s4 + 2] = t.z;
      idv[4 * s4 + 3] = t.w;
    }
  } else {
#pragma unroll
    for (int s = 0; s < SMAX; ++s) idv[s] = a.ids_slots && s < a.S ? sel[s] : 0;
  }
  float ls[SMAX];
#pragma unroll
  for (int s = 0; s < SMAX; ++s) {
    ls[s] = -__builtin_huge_valf();
    if (s < a.S) {
      const float x = pl[(int64_t)s * a.Hq];
      if ((unsigned)idv[s] < (unsigned)a.nblk) ls[s] = x;
    }
  }
  float M = -__builtin_huge_valf();
#pragma unroll
  for (int s = 0; s < SMAX; ++s) M = fmaxf(M, ls[s]);
  const float Mref = M == -__builtin_huge_valf() ? 0.f : M;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  float W = 0.f;
  const T* po = static_cast<const T*>(a.part_o) + prow * a.S * D + sub * 8;
  // Eight slots per round: all their loads are issued before any is used.
  // Partials are read exactly once, so the loads are non-temporal.
#pragma unroll
  for (int s0 = 0; s0 < SMAX; s0 += 8) {
    if (s0 < a.S) {
      frag_t<T> v[8];
      float w[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int s = s0 + u;
        w[u] = ls[s] == -__builtin_huge_valf() ? 0.f : exp2_fast((ls[s] - Mref) * kLog2e);
        v[u] = s < a.S ? __builtin_nontemporal_load(reinterpret_cast<const frag_t<T>*>(po + (int64_t)s * D))
                       : zero_frag<T>();
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        W += w[u];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = w[u] != 0.f ? fmaf(w[u], to_f32(v[u][e]), acc[e]) : acc[e];
      }
    }
  }
  const float inv = W > 0.f ? 1.f / W : 0.f;
  T* orow = static_cast<T*>(a.out) + (((int64_t)b * a.Nq + a.q0 + qq) * a.Hq + h) * D + sub * 8;
  typename Pack8<T>::type ov;
#pragma unroll
  for (int e = 0; e < 8; ++e) ov[e] = from_f32<T>(acc[e] * inv);
  if constexpr (sizeof(T) == 2) {
    *reinterpret_cast<bf16x8*>(orow) = ov;
  } else {
    *reinterpret_cast<f32x4*>(orow) = f32x4{ov[0], ov[1], ov[2], ov[3]};
    *reinterpret_cast<f32x4*>(orow + 4) = f32x4{ov[4], ov[5], ov[6], ov[7]};
  }
  if (sub == 0 && a.lse)
    a.lse[((int64_t)b * a.Nq + a.q0 + qq) * a.Hq + h] = W > 0.f ? M + log2_fast(W) * kLn2 : -__builtin_huge_valf();
}

template <typename T, int D, int BK, bool KVMX>
void kvouter_launch_bk(bool nt, dim3 grid, hipStream_t st, const KvArgs& a) {
  if (nt) hipLaunchKernelGGL((k_attn_kvouter<T, D, true, BK, KVMX>), grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((k_attn_kvouter<T, D, false, BK, KVMX>), grid, dim3(256), 0, st, a);
}

template <typename T, int D, bool KVMX>
void kvouter_launch_mx(int bk, bool nt, dim3 grid, hipStream_t st, const KvArgs& a) {
  if (bk == 32) kvouter_launch_bk<T, D, 32, KVMX>(nt, grid, st, a);
  else if (bk == 64) kvouter_launch_bk<T, D, 64, KVMX>(nt, grid, st, a);
  else kvouter_launch_bk<T, D, 128, KVMX>(nt, grid, st, a);
}

template <typename T, int D>
void kvouter_launch(int bk, bool kv_mx, bool nt, dim3 grid, hipStream_t st, const KvArgs& a) {
  if (kv_mx) kvouter_launch_mx<T, D, true>(bk, nt, grid, st, a);
  else kvouter_launch_mx<T, D, false>(bk, nt, grid, st, a);
}

template <typename T, int D, bool KVMX>
void qouter_launch_mx(int bk, dim3 grid, hipStream_t st, const QoArgs& a) {
  if (bk == 32) hipLaunchKernelGGL((k_attn_qouter<T, D, 32, KVMX>), grid, dim3(256), 0, st, a);
  else if (bk == 64) hipLaunchKernelGGL((k_attn_qouter<T, D, 64, KVMX>), grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((k_attn_qouter<T, D, 128, KVMX>), grid, dim3(256), 0, st, a);
}

template <typename T, int D>
void qouter_launch(int bk, bool kv_mx, dim3 grid, hipStream_t st, const QoArgs& a) {
  if (kv_mx) qouter_launch_mx<T, D, true>(bk, grid, st, a);
  else qouter_launch_mx<T, D, false>(bk, grid, st, a);
}

// MXFP8 K / V caches: the codes [B, Nk, Hkv, D] are followed by the scales.
const uint8_t* mx_scales_of(const Shape& s, const void* codes) {
  return s.kv_mx ? static_cast<const uint8_t*>(codes) + (size_t)s.B * s.Nk * s.Hkv * s.D : nullptr;
}

}  // namespace

hipError_t launch_attn_kvouter(const Shape& s, const InvertPlan& p, int q0, int nq, const void* q, const void* k,
                               const void* v, const InvertOut& inv, Partials part, hipStream_t st) {
  static const int kid = prof_register("attn_kvouter");
  KvArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.ksc = mx_scales_of(s, k);
  a.vsc = mx_scales_of(s, v);
  a.entries = inv.entries;
  a.item_count = inv.item_count;
  a.items = inv.items;
  a.part_o = part.o;
  a.part_lse = part.lse;
  a.trash = part.trash;
  a.trash_lse = reinterpret_cast<float*>(static_cast<char*>(part.trash) + kTrashBytes - 16);
  a.Nq = s.Nq;
  a.Nk = s.Nk;
  a.Hq = s.Hq;
  a.Hkv = s.Hkv;
  a.G = s.Hq / s.Hkv;
  a.topk = s.topk;
  a.S = part.S;
  a.q0 = q0;
  a.nq = nq;
  a.items_cap = p.items_cap;
  a.q_offset = s.q_offset;
  a.c_log2 = s.scale * kLog2e;
  a.gshift = __builtin_ctz((unsigned)a.G);
  a.topk_magic = ((uint64_t)1 << 40) / (uint64_t)s.topk + 1;
  const dim3 grid(p.items_cap, s.B * s.Hkv);
  // Non-temporal partial stores pay off when the average selected block
  // carries at least a full work item of rows.
  const bool nt = (double)nq * s.topk * a.G >= (double)kItemRows * s.nblk;
  prof_begin(st, kid);
  if (s.dtype == kBF16) {
    if (s.D == 64) kvouter_launch<bf16_t, 64>(s.Bk, s.kv_mx, nt, grid, st, a);
    else kvouter_launch<bf16_t, 128>(s.Bk, s.kv_mx, nt, grid, st, a);
  } else {
    if (s.D == 64) kvouter_launch<float, 64>(s.Bk, s.kv_mx, nt, grid, st, a);
    else kvouter_launch<float, 128>(s.Bk, s.kv_mx, nt, grid, st, a);
  }
  const hipError_t e = hipGetLastError();
  prof_end(st, kid);
  return e;
}

hipError_t launch_attn_qouter(const Shape& s, int q0, int nq, int nsplit, const void* q, const void* k,
                              const void* v, const int32_t* ids, void* out, float* lse, Partials part,
                              hipStream_t st) {
  static const int kid = prof_register("attn_qouter");
  QoArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.ksc = mx_scales_of(s, k);
  a.vsc = mx_scales_of(s, v);
  a.ids = ids;
  a.out = out;
  a.lse = lse;
  a.part_o = part.o;
  a.part_lse = part.lse;
  a.Nq = s.Nq;
  a.Nk = s.Nk;
  a.Hq = s.Hq;
  a.Hkv = s.Hkv;
  a.G = s.Hq / s.Hkv;
  a.topk = s.topk;
  a.nsplit = nsplit;
  a.q0 = q0;
  a.nq = nq;
  a.q_offset = s.q_offset;
  a.c_log2 = s.scale * kLog2e;
  const dim3 grid(nq * s.Hkv, nsplit, s.B);
  prof_begin(st, kid);
  if (s.dtype == kBF16) {
    if (s.D == 64) qouter_launch<bf16_t, 64>(s.Bk, s.kv_mx, grid, st, a);
    else qouter_launch<bf16_t, 128>(s.Bk, s.kv_mx, grid, st, a);
  } else {
    if (s.D == 64) qouter_launch<float, 64>(s.Bk, s.kv_mx, grid, st, a);
    else qouter_launch<float, 128>(s.Bk, s.kv_mx, grid, st, a);
  }
  const hipError_t e = hipGetLastError();
  prof_end(st, kid);
  return e;
}

template <int SMAX>
static void combine_dispatch(const Shape& s, dim3 grid, const CombArgs& a, hipStream_t st) {
  if (s.dtype == kBF16) {
    if (s.D == 64) hipLaunchKernelGGL((k_combine<bf16_t, 64, SMAX>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((k_combine<bf16_t, 128, SMAX>), grid, dim3(256), 0, st, a);
  } else {
    if (s.D == 64) hipLaunchKernelGGL((k_combine<float, 64, SMAX>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((k_combine<float, 128, SMAX>), grid, dim3(256), 0, st, a);
  }
}

hipError_t launch_combine(const Shape& s, int q0, int nq, const Partials& part, const int32_t* ids,
                          bool ids_slots, void* out, float* lse, hipStream_t st) {
  static const int kid = prof_register("combine");
  CombArgs a;
  a.part_o = part.o;
  a.part_lse = part.lse;
  a.ids = ids;
  a.out = out;
  a.lse = lse;
  a.Nq = s.Nq;
  a.Hq = s.Hq;
  a.Hkv = s.Hkv;
  a.G = s.Hq / s.Hkv;
  a.topk = s.topk;
  a.S = part.S;
  a.q0 = q0;
  a.nq = nq;
  a.ids_slots = ids_slots ? 1 : 0;
  a.nblk = s.nblk;
  const int64_t rows = (int64_t)nq * s.Hq;
  const int rows_per_wg = 4 * (64 / (s.D / 8));
  const dim3 grid((unsigned)((rows + rows_per_wg - 1) / rows_per_wg), s.B);
  prof_begin(st, kid);
  if (part.S <= 8) combine_dispatch<8>(s, grid, a, st);
  else if (part.S <= 16) combine_dispatch<16>(s, grid, a, st);
  else combine_dispatch<32>(s, grid, a, st);
  const hipError_t e = hipGetLastError();
  prof_end(st, kid);
  return e;
}

}  // namespace msa
