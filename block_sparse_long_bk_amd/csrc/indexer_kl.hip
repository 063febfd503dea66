// indexer_kl.hip -- the Index-Branch alignment loss and its gradients (gfx950).
//
// The pages train the Index Branch with a KL divergence that pulls its
// distribution towards the Main Branch's group-averaged one on the selected
// tokens; the Main Branch and the selection are fixed targets (gradient
// detach), so only the index queries and keys receive gradients (paper
// summary page, "Method"; zhichai.net write-up, section 5.1).  Per (b, i, g)
// over the visible selected tokens T:
//     pm(t) = (1/G) sum_{h in g} P_h(t)            P_h from the forward's LSE
//     pi(t) = exp(s_t - lse_s),  s_t = <iq, ik_t>,  lse_s = log sum_T exp(s)
//     kl    = sum_t pm(t) (log pm(t) - s_t + lse_s)
//     d kl / d s_t = pi(t) - pm(t)
// Work is organised on the KV-outer work items of the forward (block j and the
// (query, slot) entries that chose it), each entry once for all its heads:
//   k_kl_lse      entry = lane: the block's index scores -> a partial lse_s
//                 per (query, group, slot)
//   k_kl_lse_sum  lse_s per (query, group) over its slots
//   k_kl_main     (fp32; k_kl_main8 with eight waves for 16-bit inputs)
//                 a lane owns a key (wave w: keys 32w..): index scores and the
//                 G heads' probabilities for a 32-entry tile, the per-element
//                 KL term and gradient g = loss_scale (pi - pm); d ik += g^T iq
//                 in registers over the item's tiles; g goes through LDS to
//                 form d iq^T = ik^T g^T per entry (fp32 partial per slot)
//   k_kl_finish   kl and d iq per (query, group): slot partials summed in slot
//                 order;  k_kl_dik_reduce: d ik summed over a block's items in
//                 item order.  No atomics: results are bitwise reproducible.
#include "attn_common.h"

namespace msa {
namespace {

struct KlArgs {
  const void* q;
  const void* k;
  const void* iq;
  const void* ik;
  const float* lse;      // [B, Nq, Hq] Main Branch log-sum-exp (natural log)
  const int32_t* ids;    // [B, Nq, Hkv, topk]
  const int32_t* entries;
  const int32_t* item_count;
  const int4* items;
  float* plse;           // [B, Nq, Hkv, topk] partial index lse per slot
  float* lse_s;          // [B, Nq, Hkv]
  float* kl_part;        // [B, Nq, Hkv, topk]
  void* diq_part;        // [B, Nq, Hkv, topk, DI] in the input type
  void* dik_part;        // [B*Hkv][items_cap][BK][DI] in the input type
  int Nq, Nk, Hq, Hkv, G, topk, items_cap;
  int64_t q_offset;
  uint64_t topk_magic;
  float c_log2;      // Main Branch softmax scale * log2(e)
  float loss_scale;
};

__device__ __forceinline__ void split_entry(int e, int topk, uint64_t magic, int& qq, int& slot) {
  qq = (int)(((uint64_t)(uint32_t)e * magic) >> 40);
  slot = e - qq * topk;
}

// ---- partial index lse per (query, group, slot): entry = lane ---------------
template <typename T, int DI, int BK>
__global__ void __launch_bounds__(256) k_kl_lse(KlArgs a) {
  using L = KvLds<T, DI, BK>;
  constexpr int MT = BK / 32;
  __shared__ __attribute__((aligned(16))) char lds[BK * L::KPITCH];
  __shared__ int32_t ent_lds[kMaxItemEntries];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5;
  const int bg = blockIdx.y, b = bg / a.Hkv, g = bg % a.Hkv;
  const int n = a.item_count[bg];
  const int per = (n + 7) / 8;
  const int x = blockIdx.x;
  const int item = (x % 8) * per + x / 8;
  if (x / 8 >= per || item >= n) return;
  const int4 it = a.items[(int64_t)bg * a.items_cap + item];
  const int j = it.x, e0 = it.y, nent = it.z - it.y;
  const int32_t* ent = a.entries + (int64_t)bg * a.Nq * a.topk + e0;
  for (int u = tid; u < nent; u += 256) ent_lds[u] = ent[u];
  const int64_t tok_stride = (int64_t)a.Hkv * DI;
  const T* ikb = static_cast<const T*>(a.ik) + (int64_t)b * a.Nk * tok_stride + g * DI;
  {
    KvStage<T, DI, BK> st;  // all loads issued before the stores
    st.load_k(ikb, tok_stride, j, a.Nk, tid);
    st.store_k(lds, tid);
  }
  __syncthreads();
  const int64_t key0 = (int64_t)j * BK;
  // The index query rows of a wave's next tile are fetched while the current
  // one is scored (rows past the item's end read entry 0's row).
  auto fetch = [&](int tile, frag_t<T> (&qf)[DI / 16]) {
    const int r = tile * 32 + (lane & 31);
    int qq, slot;
    split_entry(r < nent ? ent_lds[r] : ent_lds[0], a.topk, a.topk_magic, qq, slot);
    const T* iqr = static_cast<const T*>(a.iq) + (((int64_t)b * a.Nq + qq) * a.Hkv + g) * DI + 8 * half;
#pragma unroll
    for (int ks = 0; ks < DI / 16; ++ks) qf[ks] = load8(iqr + 16 * ks);
  };
  frag_t<T> qnext[DI / 16];
  if (wave * 32 < nent) fetch(wave, qnext);
  for (int tile = wave; tile * 32 < nent; tile += 4) {
    const int r = tile * 32 + (lane & 31);
    const bool valid = r < nent;
    int qq, slot;
    split_entry(valid ? ent_lds[r] : ent_lds[0], a.topk, a.topk_magic, qq, slot);
    frag_t<T> qf[DI / 16];
#pragma unroll
    for (int ks = 0; ks < DI / 16; ++ks) qf[ks] = qnext[ks];
    if ((tile + 4) * 32 < nent) fetch(tile + 4, qnext);
    const int64_t pos = a.q_offset + qq;
    const int vis = (int)max((int64_t)0, min((int64_t)BK, min(pos + 1, (int64_t)a.Nk) - key0));
    // online over the M-tiles (one 32-key tile of scores live at a time); the
    // key fragments are read anew per tile (kept over the loop they would
    // hold 128 registers and leave one wave per SIMD)
    asm volatile("" ::: "memory");
    float m = -__builtin_huge_valf(), l = 0.f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const T* kr = reinterpret_cast<const T*>(lds + (mt * 32 + (lane & 31)) * L::KPITCH) + 8 * half;
      f32x16 s = mma0(load8(kr), qf[0]);
#pragma unroll
      for (int ks = 1; ks < DI / 16; ++ks) mma(load8(kr + 16 * ks), qf[ks], s);
      float mt_max = -__builtin_huge_valf();
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int t = 32 * mt + 8 * (e / 4) + 4 * half + (e % 4);
        if (t < vis) mt_max = fmaxf(mt_max, s[e]);
      }
      const float mn = fmaxf(m, mt_max);
      if (mn != -__builtin_huge_valf()) {
        float add = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int t = 32 * mt + 8 * (e / 4) + 4 * half + (e % 4);
          if (t < vis) add += exp2_fast((s[e] - mn) * kLog2e);
        }
        l = (m == -__builtin_huge_valf() ? 0.f : l * exp2_fast((m - mn) * kLog2e)) + add;
        m = mn;
      }
    }
    // merge the two halves' keys (a block that lies wholly past the query --
    // only a caller's table can name one -- has no visible key: -inf)
    const float2 mp = lane_pair32(m), lp = lane_pair32(l);  // (half 0's, half 1's)
    const float mm = fmaxf(mp.x, mp.y);
    const float lt = lp.x * exp2_fast((mp.x - mm) * kLog2e) + lp.y * exp2_fast((mp.y - mm) * kLog2e);
    const float pl = mm == -__builtin_huge_valf() ? -__builtin_huge_valf() : mm + __logf(lt);
    if (half == 0 && valid) a.plse[(((int64_t)b * a.Nq + qq) * a.Hkv + g) * a.topk + slot] = pl;
  }
}

// ---- lse_s per (query, group) over its selected slots -----------------------
// Slots whose id lies outside [0, nblk) have no partial; a row with no
// visible selected key (every partial -inf) gets -inf.
__global__ void __launch_bounds__(256) k_kl_lse_sum(const float* __restrict__ plse, const int32_t* __restrict__ ids,
                                                    float* __restrict__ lse_s, int topk, int nblk, int64_t nrows) {
  const int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (row >= nrows) return;
  const int32_t* sel = ids + row * topk;
  const float* p = plse + row * topk;
  float m = -__builtin_huge_valf();
  for (int s = 0; s < topk; ++s)
    if ((unsigned)sel[s] < (unsigned)nblk) m = fmaxf(m, p[s]);
  float l = 0.f;
  if (m != -__builtin_huge_valf())
    for (int s = 0; s < topk; ++s)
      if ((unsigned)sel[s] < (unsigned)nblk) l += exp2_fast((p[s] - m) * kLog2e);
  lse_s[row] = l > 0.f ? m + __logf(l) : -__builtin_huge_valf();
}

// ---- the main pass: a lane owns a key ---------------------------------------
template <typename T, int D, int DI, int BK>
struct KlLds {
  using LI = KvLds<T, DI, BK>;
  static constexpr int QPITCH = D * (int)sizeof(T) + 16;    // a Main Branch query row
  static constexpr int IPITCH = DI * (int)sizeof(T) + 16;   // an index query row
  static constexpr int TPITCH = 32 * (int)sizeof(T) + (sizeof(T) == 2 ? 8 : 16);  // 32 entries, transposed
  // g row [entry][key]: for 16-bit types an odd multiple of 8 bytes past BK keys, so that the 32 rows read by a
  // half-wave fall on distinct banks, and 3 mod 8 of them so that the two half-waves' writes (4 rows apart) do too
  static constexpr int GPITCH = BK * (int)sizeof(T) + (sizeof(T) == 2 ? 24 : 16);
  static constexpr bool SWZ = sizeof(T) == 2;  // the transposed tile uses the chunk swizzle
  static constexpr int IKT_OFF = 0;                          // ik^T [DI][BK]
  static constexpr int IQ_OFF = IKT_OFF + DI * LI::VPITCH;   // iq tile [32][DI]
  static constexpr int IQT_OFF = IQ_OFF + 32 * IPITCH;       // iq^T tile [DI][32]
  static constexpr int G_OFF = IQT_OFF + DI * TPITCH;        // g [32][BK]
  static constexpr int Q_OFF = G_OFF + 32 * GPITCH;          // HC heads x 32 query rows
  static constexpr int FIXED = Q_OFF + 4 * kMaxItemEntries + 32 * 4 * 4 + 32 * 4 * 4 + 512;
  static constexpr int BUDGET = 160 * 1024;
  static constexpr int HC_FIT = (BUDGET - FIXED) / (32 * QPITCH);
  static constexpr int HC = HC_FIT >= 8 ? 8 : HC_FIT >= 4 ? 4 : HC_FIT >= 2 ? 2 : 1;  // heads per staged chunk
  static constexpr int BYTES = Q_OFF + HC * 32 * QPITCH;
  static constexpr int TPM = BK * 4 + 16;  // a row of fp32 KL terms, kept in the query-row area
  static_assert(HC * 32 * QPITCH >= 32 * TPM, "KL terms fit in the query-row area");
  static_assert(HC_FIT >= 1, "LDS budget");
};

template <typename T, int D, int DI, int BK>
__global__ void __launch_bounds__(256, 1) k_kl_main(KlArgs a) {
  using X = KlLds<T, D, DI, BK>;
  constexpr int HC = X::HC;
  __shared__ __attribute__((aligned(16))) char lds[X::BYTES];
  __shared__ int32_t ent_lds[kMaxItemEntries];
  __shared__ float row_lse_s[32];
  __shared__ __attribute__((aligned(16))) int row_pos[32];  // -1 past the item's end
  __shared__ int row_q[32], row_slot[32];
  __shared__ __attribute__((aligned(16))) float row_lsm[HC][32];  // Main Branch lse * log2(e) per (head, entry)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5;
  const int bg = blockIdx.y, b = bg / a.Hkv, g = bg % a.Hkv;
  const int n = a.item_count[bg];
  const int per = (n + 7) / 8;
  const int x = blockIdx.x;
  const int item = (x % 8) * per + x / 8;
  if (x / 8 >= per || item >= n) return;
  const int4 it = a.items[(int64_t)bg * a.items_cap + item];
  const int j = it.x, e0 = it.y, nent = it.z - it.y;
  const int32_t* ent = a.entries + (int64_t)bg * a.Nq * a.topk + e0;
  for (int u = tid; u < nent; u += 256) ent_lds[u] = ent[u];

  const int64_t ik_stride = (int64_t)a.Hkv * DI, k_stride = (int64_t)a.Hkv * D;
  const T* ikb = static_cast<const T*>(a.ik) + (int64_t)b * a.Nk * ik_stride + g * DI;
  const T* kb = static_cast<const T*>(a.k) + (int64_t)b * a.Nk * k_stride + g * D;
  const T* iqb = static_cast<const T*>(a.iq);
  const T* qb = static_cast<const T*>(a.q);
  {
    KvStage<T, DI, BK> st;
    st.load_v(ikb, ik_stride, j, a.Nk, tid);
    st.store_vt(lds + X::IKT_OFF, tid);
  }
  const int64_t key0 = (int64_t)j * BK;
  const bool has_keys = wave * 32 < BK;
  const int kk = wave * 32 + (lane & 31);                 // this lane's key in the block
  const int64_t my_key = key0 + kk;
  const int64_t kt = min(my_key, (int64_t)a.Nk - 1);      // keys past n_k are masked below
  // this lane's key rows (B operands of the score products)
  frag_t<T> kf[D / 16], ikf[DI / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) kf[ks] = load8(kb + kt * k_stride + 8 * half + 16 * ks);
#pragma unroll
  for (int ks = 0; ks < DI / 16; ++ks) ikf[ks] = load8(ikb + kt * ik_stride + 8 * half + 16 * ks);

  f32x16 dik[DI / 32];
#pragma unroll
  for (int dt = 0; dt < DI / 32; ++dt) dik[dt] = f32x16{};
  constexpr int ICPR = DI * (int)sizeof(T) / 16;
  constexpr int QCPR = D * (int)sizeof(T) / 16;
  const float inv_g = 1.f / (float)a.G;

  for (int tile = 0; tile * 32 < nent; ++tile) {
    __syncthreads();  // the previous tile's LDS is no longer read
    // All of a thread's loads are issued before any of them is used, so the
    // tile costs one memory latency rather than one per chunk.  A task is one
    // 16-byte column chunk of two consecutive rows, so that the transposed
    // copy gets both rows per store.  Rows past the item's end read entry 0
    // and store zeros.
    {
      constexpr int NI = (16 * ICPR + 255) / 256;
      constexpr int EPC = 16 / (int)sizeof(T);  // elements per chunk
      u32x4 v[NI][2];
      float ls[NI][2];
#pragma unroll
      for (int u = 0; u < NI; ++u) {
        const int c = min(tid + 256 * u, 16 * ICPR - 1);
        const int rp = c / ICPR, col = c % ICPR;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int r = tile * 32 + 2 * rp + h;
          int qq, slot;
          split_entry(r < nent ? ent_lds[r] : ent_lds[0], a.topk, a.topk_magic, qq, slot);
          const int64_t row = ((int64_t)b * a.Nq + qq) * a.Hkv + g;
          v[u][h] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(iqb + row * DI) + col * 16);
          ls[u][h] = a.lse_s[row];
        }
      }
#pragma unroll
      for (int u = 0; u < NI; ++u) {
        const int c = tid + 256 * u;
        if (c >= 16 * ICPR) continue;
        const int rp = c / ICPR, col = c % ICPR;
        u32x4 w[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int rr = 2 * rp + h, r = tile * 32 + rr;
          const bool valid = r < nent;
          w[h] = valid ? v[u][h] : u32x4{};
          *reinterpret_cast<u32x4*>(lds + X::IQ_OFF + rr * X::IPITCH + col * 16) = w[h];
          if (col == 0) {
            int qq, slot;
            split_entry(valid ? ent_lds[r] : ent_lds[0], a.topk, a.topk_magic, qq, slot);
            row_lse_s[rr] = valid ? ls[u][h] : 0.f;
            row_pos[rr] = valid ? (int)min(a.q_offset + qq, (int64_t)a.Nk - 1) : -1;
            row_q[rr] = qq;
            row_slot[rr] = slot;
          }
        }
        if constexpr (sizeof(T) == 2) {
          // element pairs 2i, 2i+1 of the two rows: 2x2 transposes
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int c0 = col * EPC + 2 * i;  // columns c0 and c0 + 1 share the swizzle
            const int pos = tile_t_chunk<X::SWZ>(c0, rp >> 1) * 8 + (rp & 1) * 4;
            *reinterpret_cast<uint32_t*>(lds + X::IQT_OFF + c0 * X::TPITCH + pos) =
                __builtin_amdgcn_perm(w[1][i], w[0][i], 0x05040100u);
            *reinterpret_cast<uint32_t*>(lds + X::IQT_OFF + (c0 + 1) * X::TPITCH + pos) =
                __builtin_amdgcn_perm(w[1][i], w[0][i], 0x07060302u);
          }
        } else {
#pragma unroll
          for (int e = 0; e < EPC; ++e)
            *reinterpret_cast<uint2*>(lds + X::IQT_OFF + (col * EPC + e) * X::TPITCH + rp * 8) =
                make_uint2(w[0][e], w[1][e]);
        }
      }
    }
    __syncthreads();
    // index scores s[entry][key] (accumulator rows = entries)
    f32x16 si = f32x16{}, pm = f32x16{};
    if (has_keys) {
      const T* ir = reinterpret_cast<const T*>(lds + X::IQ_OFF + (lane & 31) * X::IPITCH) + 8 * half;
#pragma unroll
      for (int ks = 0; ks < DI / 16; ++ks) mma(load8(ir + 16 * ks), ikf[ks], si);
    }
    // the group's heads, HC at a time: pm += P_h
    for (int h0 = 0; h0 < a.G; h0 += HC) {
      const int hn = min(HC, a.G - h0);
      __syncthreads();  // the previous chunk's query rows are no longer read
      {
        constexpr int NQ = (HC * 32 * QCPR + 255) / 256;
        u32x4 v[NQ];
        float ls[NQ];
#pragma unroll
        for (int u = 0; u < NQ; ++u) {
          const int c = min(tid + 256 * u, hn * 32 * QCPR - 1);
          const int hr = c / QCPR, col = c % QCPR;  // hr = hl * 32 + rr
          const int hl = hr >> 5, rr = hr & 31;
          const int64_t qrow = ((int64_t)b * a.Nq + row_q[rr]) * a.Hq + g * a.G + h0 + hl;
          v[u] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(qb + qrow * D) + col * 16);
          ls[u] = a.lse[qrow];
        }
#pragma unroll
        for (int u = 0; u < NQ; ++u) {
          const int c = tid + 256 * u;
          if (c >= hn * 32 * QCPR) continue;
          const int hr = c / QCPR, col = c % QCPR;
          const int hl = hr >> 5, rr = hr & 31;
          const bool valid = tile * 32 + rr < nent;
          *reinterpret_cast<u32x4*>(lds + X::Q_OFF + hr * X::QPITCH + col * 16) = valid ? v[u] : u32x4{};
          if (col == 0) row_lsm[hl][rr] = valid ? ls[u] * kLog2e : 0.f;
        }
      }
      __syncthreads();
      if (has_keys) {
        for (int hl = 0; hl < hn; ++hl) {
          const T* qr = reinterpret_cast<const T*>(lds + X::Q_OFF + (hl * 32 + (lane & 31)) * X::QPITCH) + 8 * half;
          f32x16 s = mma0(load8(qr), kf[0]);
#pragma unroll
          for (int ks = 1; ks < D / 16; ++ks) mma(load8(qr + 16 * ks), kf[ks], s);
          // masked positions: the exponent is clamped at 0 (visible ones never
          // exceed it) so that the product with the 0/1 mask stays finite
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int r0 = 8 * q4 + 4 * half;
            const f32x4 l4 = *reinterpret_cast<const f32x4*>(&row_lsm[hl][r0]);
            const int4 p4 = *reinterpret_cast<const int4*>(row_pos + r0);
            const int pp[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              const int e = 4 * q4 + c;
              const float m = my_key <= pp[c] ? 1.f : 0.f;
              pm[e] = fmaf(m, exp2_fast(fminf(fmaf(s[e], a.c_log2, -l4[c]), 0.f)), pm[e]);
            }
          }
        }
      }
    }
    __syncthreads();  // every wave is past the heads: the query-row area is free
    if (has_keys) {
      // per element: KL term and gradient; g to LDS as [entry][key]
      f32x16 gs;
      float term[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int rr = 8 * (e / 4) + 4 * half + (e % 4);
        const bool vis = row_pos[rr] >= 0 && my_key <= row_pos[rr];
        const float p = pm[e] * inv_g;
        const float logpi = si[e] - row_lse_s[rr];
        const float pi = exp2_fast(logpi * kLog2e);
        term[e] = (vis && p > 0.f) ? p * (__logf(p) - logpi) : 0.f;
        gs[e] = vis ? a.loss_scale * (pi - p) : 0.f;
        *reinterpret_cast<T*>(lds + X::G_OFF + rr * X::GPITCH + kk * (int)sizeof(T)) = from_f32<T>(gs[e]);
      }
      // the per-element KL terms go to LDS as [entry][key] (fp32, in the
      // query-row area, free once every wave is past the heads: the barrier
      // above the element loop) and are summed per entry after the barrier
#pragma unroll
      for (int e = 0; e < 16; ++e)
        *reinterpret_cast<float*>(lds + X::Q_OFF + (8 * (e / 4) + 4 * half + (e % 4)) * X::TPM + kk * 4) = term[e];
      // d ik[key][c] += sum over entries g^T[key][e] iq[e][c]
#pragma unroll
      for (int aa = 0; aa < 2; ++aa) {
        frag_t<T> ga;
#pragma unroll
        for (int e = 0; e < 8; ++e) ga[e] = from_f32<T>(gs[8 * aa + e]);
#pragma unroll
        for (int dt = 0; dt < DI / 32; ++dt)
          mma(ga, tile_t_frag<T, X::TPITCH, X::SWZ>(lds + X::IQT_OFF, 32 * dt + (lane & 31), aa, half), dik[dt]);
      }
    }
    __syncthreads();  // g and the KL partials of every wave are in LDS
    // d iq^T[c][entry] = sum over the block's keys ik^T[c][key] g^T[key][entry];
    // wave w takes c in [32w, 32w + 32)
    if (wave < DI / 32) {
      f32x16 o = f32x16{};
      const int c = 32 * wave + (lane & 31);
      const T* grow = reinterpret_cast<const T*>(lds + X::G_OFF + (lane & 31) * X::GPITCH);
#pragma unroll
      for (int mt = 0; mt < BK / 32; ++mt)
#pragma unroll
        for (int aa = 0; aa < 2; ++aa) {
          const frag_t<T> ka = vt_frag_at<T, DI, BK>(lds + X::IKT_OFF, c, mt, aa, half);
          const int k0 = 32 * mt + 16 * aa + 4 * half;
          const typename Pack4<T>::type lo = *reinterpret_cast<const typename Pack4<T>::type*>(grow + k0);
          const typename Pack4<T>::type hi = *reinterpret_cast<const typename Pack4<T>::type*>(grow + k0 + 8);
          frag_t<T> gb;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            gb[e] = lo[e];
            gb[4 + e] = hi[e];
          }
          mma(ka, gb, o);
        }
      const int rr = lane & 31;
      if (row_pos[rr] >= 0) {
        T* dst = static_cast<T*>(a.diq_part) +
                 ((((int64_t)b * a.Nq + row_q[rr]) * a.Hkv + g) * a.topk + row_slot[rr]) * DI;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          typename Pack4<T>::type w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = from_f32<T>(o[4 * i + e]);
          *reinterpret_cast<typename Pack4<T>::type*>(dst + 32 * wave + 8 * i + 4 * half) = w;
        }
      }
    }
    {
      // KL partial per entry: 8 threads per entry, BK / 8 keys each, then a
      // fixed-order combination of the 8 sums
      const int rr = tid >> 3, part = tid & 7;
      const float* trow = reinterpret_cast<const float*>(lds + X::Q_OFF + rr * X::TPM) + part * (BK / 8);
      float acc = 0.f;
#pragma unroll
      for (int u = 0; u < BK / 8; u += 4) {
        const f32x4 t4 = *reinterpret_cast<const f32x4*>(trow + u);
        acc += (t4[0] + t4[1]) + (t4[2] + t4[3]);
      }
      acc = group_sum<8>(acc);
      if (part == 0 && row_pos[rr] >= 0)
        a.kl_part[(((int64_t)b * a.Nq + row_q[rr]) * a.Hkv + g) * a.topk + row_slot[rr]] = acc;
    }
  }
  if (!has_keys) return;
  // this item's d ik: lane holds key 32w + 8(e/4) + 4h + e%4, c = 32 dt + lane%32
  T* dst = static_cast<T*>(a.dik_part) + ((int64_t)bg * a.items_cap + item) * BK * DI;
#pragma unroll
  for (int dt = 0; dt < DI / 32; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int key = wave * 32 + 8 * (e / 4) + 4 * half + (e % 4);
      dst[key * DI + 32 * dt + (lane & 31)] = from_f32<T>(dik[dt][e]);
    }
}

// ---- the main pass for 16-bit inputs: eight waves ---------------------------
// Waves w and w + 4 share the keys [32 (w % 4), +32) of the block.  Of each
// head chunk, wave w takes the even heads and wave w + 4 the odd ones; their
// partial sums of P meet in LDS (even + odd, a fixed order).  Wave w holds
// the index keys and forms the index scores, the KL terms, g and the first
// half of d idx_k; wave w + 4 takes g from LDS for the second half and forms
// d idx_q.  Two waves per SIMD where the four-wave pass holds one.
template <typename T, int D, int DI, int BK>
struct KlLds8 {
  using LI = KvLds<T, DI, BK>;
  static constexpr int QPITCH = D * 2 + 16;   // a Main Branch query row
  static constexpr int IPITCH = DI * 2 + 16;  // an index query row
  static constexpr int TPITCH = 32 * 2 + 8;   // 32 entries, transposed
  static constexpr int GPITCH = BK * 2 + 24;  // g row [entry][key] (padded as the backward's dS rows)
  static constexpr bool SWZ = true;           // the transposed tile uses the chunk swizzle
  static constexpr int TPM = BK * 4 + 16;     // a row of fp32 KL terms
  static constexpr int PMX = 4 * 16 * 64 * 4;  // partial sums of P of the odd-head waves, [key group][e][lane]
  static constexpr int GX = 4 * 16 * 64 * 2;   // g of the even-head waves, same layout, in the input type
  static constexpr int AUX = 32 * TPM + PMX + GX;  // kept in the query-row area once the heads are done
  static constexpr int KPITCH = KvLds<T, D, BK>::KPITCH;     // a Main Branch key row
  static constexpr int IKT_OFF = 0;                          // ik^T [DI][BK]
  static constexpr int K_OFF = IKT_OFF + DI * LI::VPITCH;    // k [BK][D]
  static constexpr int IQ_OFF = K_OFF + BK * KPITCH;         // iq tile [32][DI]
  static constexpr int IQT_OFF = IQ_OFF + 32 * IPITCH;       // iq^T tile [DI][32]
  static constexpr int G_OFF = IQT_OFF + DI * TPITCH;        // g [32][BK]
  static constexpr int Q_OFF = G_OFF + 32 * GPITCH;          // HC heads x 32 query rows, later AUX
  static constexpr int OTHER = 4 * kMaxItemEntries + 4 * 32 * 4 + 8 * 32 * 4;  // the other shared arrays
  static constexpr int BUDGET = 160 * 1024;
  static constexpr int HC_FIT = (BUDGET - OTHER - Q_OFF) / (32 * QPITCH);
  // heads per staged chunk: at most four 16-byte loads per thread in flight (registers), and what LDS holds
  static constexpr int HC_REG = 4 * 512 / (32 * D * 2 / 16);
  static constexpr int HC_MAX = HC_FIT < HC_REG ? HC_FIT : HC_REG;
  static constexpr int HC = HC_MAX >= 8 ? 8 : HC_MAX >= 4 ? 4 : HC_MAX >= 2 ? 2 : 1;
  static constexpr int QAREA = HC * 32 * QPITCH > AUX ? HC * 32 * QPITCH : AUX;
  static constexpr int TPM_OFF = Q_OFF;
  static constexpr int PMX_OFF = TPM_OFF + 32 * TPM;
  static constexpr int GX_OFF = PMX_OFF + PMX;
  static constexpr int BYTES = Q_OFF + QAREA;
  static_assert(HC_FIT >= 1 && BYTES + OTHER <= BUDGET, "LDS budget");
};

// B fragment (column = key, k = 8 consecutive rows of d) of a 16-bit tile
// stored transposed in the V^T layout of KvLds ([d][key], 4-key chunks
// swizzled), read with two ds_read_b64_tr_b16.  Within each 16-lane group that
// instruction gives lane 4a + w word w of the 8-byte chunks addressed by lanes
// a, a + 4, a + 8 and a + 12 of the group (one element from each, in that
// order), so lane a + 4e of a group points at row k0 + e, keys 4a..4a+3 of the
// group's 16 keys.  Lane l gets key kcol0 + l%32, rows 16 ks + 8(l/32) + [0, 8).
template <int DI, int BK>
__device__ __forceinline__ bf16x8 vt_frag_tr(const char* vt, int kcol0, int ks, int lane) {
  using L = KvLds<bf16_t, DI, BK>;
  typedef short v4s __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4s* lds_v4s;
  const int grp = lane >> 4, a = lane & 3, e = (lane >> 2) & 3;
  const int c = (kcol0 >> 2) + 4 * (grp & 1) + a;  // 4-key chunk
  const int k = 16 * ks + 8 * (grp >> 1) + e;
  const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(const_cast<char*>(vt) + L::vt_off(k, c)));
  const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(const_cast<char*>(vt) + L::vt_off(k + 4, c)));
  struct Pair {
    v4s x, y;
  } pr{lo, hi};
  return __builtin_bit_cast(bf16x8, pr);
}

template <typename T, int D, int DI, int BK>
__global__ void __launch_bounds__(512, 1) k_kl_main8(KlArgs a) {
  static_assert(sizeof(T) == 2, "the eight-wave pass is laid out for 16-bit inputs");
  using X = KlLds8<T, D, DI, BK>;
  constexpr int HC = X::HC;
  constexpr int DT = DI / 32;        // d idx_k accumulator tiles in all
  constexpr int DT0 = (DT + 1) / 2;  // of which the even-head wave keeps the first DT0
  __shared__ __attribute__((aligned(16))) char lds[X::BYTES];
  __shared__ int32_t ent_lds[kMaxItemEntries];
  __shared__ float row_lse_s[32];
  __shared__ __attribute__((aligned(16))) int row_pos[32];  // -1 past the item's end
  __shared__ int row_q[32], row_slot[32];
  __shared__ __attribute__((aligned(16))) float row_lsm[8][32];  // Main Branch lse * log2(e) per (head, entry)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5;
  const int kg = wave & 3, hs = wave >> 2;  // key group; 0 = even heads, 1 = odd heads
  const int bg = blockIdx.y, b = bg / a.Hkv, g = bg % a.Hkv;
  const int n = a.item_count[bg];
  const int per = (n + 7) / 8;
  const int x = blockIdx.x;
  const int item = (x % 8) * per + x / 8;
  if (x / 8 >= per || item >= n) return;
  const int4 it = a.items[(int64_t)bg * a.items_cap + item];
  const int j = it.x, e0 = it.y, nent = it.z - it.y;
  const int32_t* ent = a.entries + (int64_t)bg * a.Nq * a.topk + e0;
  for (int u = tid; u < nent; u += 512) ent_lds[u] = ent[u];

  const int64_t ik_stride = (int64_t)a.Hkv * DI, k_stride = (int64_t)a.Hkv * D;
  const T* ikb = static_cast<const T*>(a.ik) + (int64_t)b * a.Nk * ik_stride + g * DI;
  const T* kb = static_cast<const T*>(a.k) + (int64_t)b * a.Nk * k_stride + g * D;
  const T* iqb = static_cast<const T*>(a.iq);
  const T* qb = static_cast<const T*>(a.q);
  if (tid < 256) {
    KvStage<T, DI, BK> st;
    st.load_v(ikb, ik_stride, j, a.Nk, tid);
    st.store_vt(lds + X::IKT_OFF, tid);
  } else {
    KvStage<T, D, BK> st;  // the Main Branch key rows, row-major
    st.load_k(kb, k_stride, j, a.Nk, tid - 256);
    st.store_k(lds + X::K_OFF, tid - 256);
  }
  const int64_t key0 = (int64_t)j * BK;
  const bool has_keys = kg * 32 < BK;
  const int kk = kg * 32 + (lane & 31);                 // this lane's key in the block
  const int64_t my_key = key0 + kk;
  // this lane's Main Branch key row in LDS (B operands of the score products;
  // the index keys are read from the transposed copy when needed)
  const T* krow = reinterpret_cast<const T*>(lds + X::K_OFF + kk * X::KPITCH) + 8 * half;
  f32x16 dik[DT0];
#pragma unroll
  for (int i = 0; i < DT0; ++i) dik[i] = f32x16{};
  constexpr int ICPR = DI * 2 / 16;
  constexpr int QCPR = D * 2 / 16;
  const float inv_g = 1.f / (float)a.G;
  float* pmx = reinterpret_cast<float*>(lds + X::PMX_OFF) + kg * 16 * 64 + lane;
  T* gx = reinterpret_cast<T*>(lds + X::GX_OFF) + kg * 16 * 64 + lane;

  // The index query rows and the first head chunk of a tile are fetched into
  // registers during the previous tile (all threads, branch-free: rows past
  // the item's end read entry 0, tasks past the end repeat the last one) and
  // written to LDS at the start of the tile.
  constexpr int IQ_TASKS = 16 * ICPR;  // 16-byte chunks of two consecutive rows
  constexpr int NQ = (HC * 32 * QCPR + 511) / 512;
  const int hn0 = min(HC, a.G);
  struct Prefetch {
    u32x4 iq[2];
    float ils[2];
    u32x4 q[NQ];
    float qls[NQ];
  } pf;
  auto fetch = [&](int tile) {
    {
      const int c = min(tid, IQ_TASKS - 1);
      const int rp = c / ICPR, col = c % ICPR;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = tile * 32 + 2 * rp + h;
        int qq, slot;
        split_entry(r < nent ? ent_lds[r] : ent_lds[0], a.topk, a.topk_magic, qq, slot);
        const int64_t row = ((int64_t)b * a.Nq + qq) * a.Hkv + g;
        pf.iq[h] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(iqb + row * DI) + col * 16);
        pf.ils[h] = a.lse_s[row];
      }
    }
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
      const int c = min(tid + 512 * u, hn0 * 32 * QCPR - 1);
      const int hr = c / QCPR, col = c % QCPR;  // hr = hl * 32 + rr
      const int hl = hr >> 5, r = tile * 32 + (hr & 31);
      int qq, slot;
      split_entry(r < nent ? ent_lds[r] : ent_lds[0], a.topk, a.topk_magic, qq, slot);
      const int64_t qrow = ((int64_t)b * a.Nq + qq) * a.Hq + g * a.G + hl;
      pf.q[u] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(qb + qrow * D) + col * 16);
      pf.qls[u] = a.lse[qrow];
    }
  };
  // masked: some row of the tile sits before one of this wave's keys (its
  // local block, or a row past the item's end); otherwise every product is
  // visible and both the mask and the clamp are skipped (a visible exponent
  // exceeds 0 only by the rounding of the recomputed score).
  auto heads = [&](int hn, f32x16& pm, bool masked) {
    for (int hl = hs; hl < hn; hl += 2) {
      // the key fragments are read anew for each head: kept from one head to
      // the next they would hold 32 registers through the whole tile
      asm volatile("" ::: "memory");
      const T* qr = reinterpret_cast<const T*>(lds + X::Q_OFF + (hl * 32 + (lane & 31)) * X::QPITCH) + 8 * half;
      f32x16 s = mma0(load8(qr), load8(krow));
#pragma unroll
      for (int ks = 1; ks < D / 16; ++ks) mma(load8(qr + 16 * ks), load8(krow + 16 * ks), s);
      // masked positions: the exponent is clamped at 0 (visible ones never
      // exceed it) so that the product with the 0/1 mask stays finite
      if (masked) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int r0 = 8 * q4 + 4 * half;
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(&row_lsm[hl][r0]);
          const int4 p4 = *reinterpret_cast<const int4*>(row_pos + r0);
          const int pp[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int e = 4 * q4 + c;
            const float m = my_key <= pp[c] ? 1.f : 0.f;
            pm[e] = fmaf(m, exp2_fast(fminf(fmaf(s[e], a.c_log2, -l4[c]), 0.f)), pm[e]);
          }
        }
      } else {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(&row_lsm[hl][8 * q4 + 4 * half]);
#pragma unroll
          for (int c = 0; c < 4; ++c) pm[4 * q4 + c] += exp2_fast(fmaf(s[4 * q4 + c], a.c_log2, -l4[c]));
        }
      }
    }
  };
  __builtin_amdgcn_s_waitcnt(0);  // the staging loads have landed: the wait below then covers the fetch alone
  fetch(0);

  for (int tile = 0; tile * 32 < nent; ++tile) {
    __syncthreads();  // the previous tile's LDS is no longer read
    {
      // the prefetched rows to LDS: index query rows (row-major and
      // transposed, two rows per task) and the first head chunk
      const int rp = tid / ICPR, col = tid % ICPR;
      if (tid < IQ_TASKS) {
        u32x4 w[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int rr = 2 * rp + h, r = tile * 32 + rr;
          const bool valid = r < nent;
          w[h] = valid ? pf.iq[h] : u32x4{};
          *reinterpret_cast<u32x4*>(lds + X::IQ_OFF + rr * X::IPITCH + col * 16) = w[h];
          if (col == 0) {
            int qq, slot;
            split_entry(valid ? ent_lds[r] : ent_lds[0], a.topk, a.topk_magic, qq, slot);
            row_lse_s[rr] = valid ? pf.ils[h] : 0.f;
            row_pos[rr] = valid ? (int)min(a.q_offset + qq, (int64_t)a.Nk - 1) : -1;
            row_q[rr] = qq;
            row_slot[rr] = slot;
          }
        }
        // element pairs 2i, 2i+1 of the two rows: 2x2 transposes
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c0 = col * 8 + 2 * i;  // columns c0 and c0 + 1 share the swizzle
          const int pos = tile_t_chunk<X::SWZ>(c0, rp >> 1) * 8 + (rp & 1) * 4;
          *reinterpret_cast<uint32_t*>(lds + X::IQT_OFF + c0 * X::TPITCH + pos) =
              __builtin_amdgcn_perm(w[1][i], w[0][i], 0x05040100u);
          *reinterpret_cast<uint32_t*>(lds + X::IQT_OFF + (c0 + 1) * X::TPITCH + pos) =
              __builtin_amdgcn_perm(w[1][i], w[0][i], 0x07060302u);
        }
      }
#pragma unroll
      for (int u = 0; u < NQ; ++u) {
        const int c = tid + 512 * u;
        if (c >= hn0 * 32 * QCPR) continue;
        const int hr = c / QCPR, col = c % QCPR;
        const int hl = hr >> 5, rr = hr & 31;
        const bool valid = tile * 32 + rr < nent;
        *reinterpret_cast<u32x4*>(lds + X::Q_OFF + hr * X::QPITCH + col * 16) = valid ? pf.q[u] : u32x4{};
        if (col == 0) row_lsm[hl][rr] = valid ? pf.qls[u] * kLog2e : 0.f;
      }
    }
    __syncthreads();
    fetch(tile + 1);  // past the last tile: entry 0's rows, never stored
    const bool masked = __any((int64_t)row_pos[lane & 31] < key0 + kg * 32 + 31);
    f32x16 pm = f32x16{};
    if (has_keys) heads(hn0, pm, masked);
    // further head chunks (groups of more than HC heads), fetched here
    for (int h0 = HC; h0 < a.G; h0 += HC) {
      const int hn = min(HC, a.G - h0);
      __syncthreads();  // the previous chunk's query rows are no longer read
      {
        u32x4 v[NQ];
        float ls[NQ];
#pragma unroll
        for (int u = 0; u < NQ; ++u) {
          const int c = min(tid + 512 * u, hn * 32 * QCPR - 1);
          const int hr = c / QCPR, col = c % QCPR;
          const int hl = hr >> 5, rr = hr & 31;
          const int64_t qrow = ((int64_t)b * a.Nq + row_q[rr]) * a.Hq + g * a.G + h0 + hl;
          v[u] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(qb + qrow * D) + col * 16);
          ls[u] = a.lse[qrow];
        }
#pragma unroll
        for (int u = 0; u < NQ; ++u) {
          const int c = tid + 512 * u;
          if (c >= hn * 32 * QCPR) continue;
          const int hr = c / QCPR, col = c % QCPR;
          const int hl = hr >> 5, rr = hr & 31;
          const bool valid = tile * 32 + rr < nent;
          *reinterpret_cast<u32x4*>(lds + X::Q_OFF + hr * X::QPITCH + col * 16) = valid ? v[u] : u32x4{};
          if (col == 0) row_lsm[hl][rr] = valid ? ls[u] * kLog2e : 0.f;
        }
      }
      __syncthreads();
      if (has_keys) heads(hn, pm, masked);
    }
    __syncthreads();  // every wave is past the heads: the query-row area is free
    if (has_keys && hs == 1) {
#pragma unroll
      for (int e = 0; e < 16; ++e) pmx[e * 64] = pm[e];
    }
    __syncthreads();  // the odd heads' sums are in LDS
    f32x16 gs;
    if (has_keys && hs == 0) {
      // index scores s[entry][key] (accumulator rows = entries)
      f32x16 si = f32x16{};
      const T* ir = reinterpret_cast<const T*>(lds + X::IQ_OFF + (lane & 31) * X::IPITCH) + 8 * half;
#pragma unroll
      for (int ks = 0; ks < DI / 16; ++ks) mma(load8(ir + 16 * ks), vt_frag_tr<DI, BK>(lds + X::IKT_OFF, kg * 32, ks, lane), si);
      // per element: the KL term and the gradient; g to LDS as [entry][key]
      // (for d iq) and in this layout (for the odd-head wave's half of d ik)
      float term[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int rr = 8 * (e / 4) + 4 * half + (e % 4);
        const bool vis = row_pos[rr] >= 0 && my_key <= row_pos[rr];
        const float p = (pm[e] + pmx[e * 64]) * inv_g;
        const float logpi = si[e] - row_lse_s[rr];
        const float pi = exp2_fast(logpi * kLog2e);
        term[e] = (vis && p > 0.f) ? p * (__logf(p) - logpi) : 0.f;
        gs[e] = vis ? a.loss_scale * (pi - p) : 0.f;
        const T gt = from_f32<T>(gs[e]);
        *reinterpret_cast<T*>(lds + X::G_OFF + rr * X::GPITCH + kk * 2) = gt;
        gx[e * 64] = gt;
      }
#pragma unroll
      for (int e = 0; e < 16; ++e)
        *reinterpret_cast<float*>(lds + X::TPM_OFF + (8 * (e / 4) + 4 * half + (e % 4)) * X::TPM + kk * 4) = term[e];
    }
    __syncthreads();  // g and the KL terms are in LDS
    if (has_keys) {
      if (hs == 1) {
#pragma unroll
        for (int e = 0; e < 16; ++e) gs[e] = to_f32(gx[e * 64]);
      }
      // d ik[key][c] += sum over entries g^T[key][e] iq[e][c], this wave's tiles of c
#pragma unroll
      for (int aa = 0; aa < 2; ++aa) {
        frag_t<T> ga;
#pragma unroll
        for (int e = 0; e < 8; ++e) ga[e] = from_f32<T>(gs[8 * aa + e]);
#pragma unroll
        for (int i = 0; i < DT0; ++i) {
          const int dt = hs * DT0 + i;
          if (dt < DT)
            mma(ga, tile_t_frag<T, X::TPITCH, X::SWZ>(lds + X::IQT_OFF, 32 * dt + (lane & 31), aa, half), dik[i]);
        }
      }
    }
    // d iq^T[c][entry] = sum over the block's keys ik^T[c][key] g^T[key][entry];
    // odd-head wave w + 4 takes c in [32w, 32w + 32)
    if (hs == 1 && kg < DI / 32) {
      f32x16 o = f32x16{};
      const int c = 32 * kg + (lane & 31);
      const T* grow = reinterpret_cast<const T*>(lds + X::G_OFF + (lane & 31) * X::GPITCH);
#pragma unroll
      for (int mt = 0; mt < BK / 32; ++mt)
#pragma unroll
        for (int aa = 0; aa < 2; ++aa) {
          const frag_t<T> ka = vt_frag_at<T, DI, BK>(lds + X::IKT_OFF, c, mt, aa, half);
          const int k0 = 32 * mt + 16 * aa + 4 * half;
          const typename Pack4<T>::type lo = *reinterpret_cast<const typename Pack4<T>::type*>(grow + k0);
          const typename Pack4<T>::type hi = *reinterpret_cast<const typename Pack4<T>::type*>(grow + k0 + 8);
          frag_t<T> gb;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            gb[e] = lo[e];
            gb[4 + e] = hi[e];
          }
          mma(ka, gb, o);
        }
      const int rr = lane & 31;
      if (row_pos[rr] >= 0) {
        T* dst = static_cast<T*>(a.diq_part) +
                 ((((int64_t)b * a.Nq + row_q[rr]) * a.Hkv + g) * a.topk + row_slot[rr]) * DI;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          typename Pack4<T>::type w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = from_f32<T>(o[4 * i + e]);
          *reinterpret_cast<typename Pack4<T>::type*>(dst + 32 * kg + 8 * i + 4 * half) = w;
        }
      }
    }
    if (tid < 256) {
      // KL partial per entry: 8 threads per entry, BK / 8 keys each, then a
      // fixed-order combination of the 8 sums
      const int rr = tid >> 3, part = tid & 7;
      const float* trow = reinterpret_cast<const float*>(lds + X::TPM_OFF + rr * X::TPM) + part * (BK / 8);
      float acc = 0.f;
#pragma unroll
      for (int u = 0; u < BK / 8; u += 4) {
        const f32x4 t4 = *reinterpret_cast<const f32x4*>(trow + u);
        acc += (t4[0] + t4[1]) + (t4[2] + t4[3]);
      }
      acc = group_sum<8>(acc);
      if (part == 0 && row_pos[rr] >= 0)
        a.kl_part[(((int64_t)b * a.Nq + row_q[rr]) * a.Hkv + g) * a.topk + row_slot[rr]] = acc;
    }
  }
  if (!has_keys) return;
  // this item's d ik: lane holds key 32 kg + 8(e/4) + 4h + e%4, c = 32 dt + lane%32
  T* dst = static_cast<T*>(a.dik_part) + ((int64_t)bg * a.items_cap + item) * BK * DI;
#pragma unroll
  for (int i = 0; i < DT0; ++i) {
    const int dt = hs * DT0 + i;
    if (dt >= DT) continue;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int key = kg * 32 + 8 * (e / 4) + 4 * half + (e % 4);
      dst[key * DI + 32 * dt + (lane & 31)] = from_f32<T>(dik[i][e]);
    }
  }
}

// ---- kl and d iq per (query, group): slot partials in slot order ------------
template <typename T, int DI>
__global__ void __launch_bounds__(256) k_kl_finish(const float* __restrict__ kl_part,
                                                   const T* __restrict__ diq_part,
                                                   const int32_t* __restrict__ ids, float* __restrict__ kl,
                                                   T* __restrict__ d_iq, int topk, int nblk, int64_t nrows) {
  constexpr int LPR = DI / 8;
  const int lane = threadIdx.x & 63;
  const int64_t row = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * (64 / LPR) + lane / LPR;  // (b, i, g)
  if (row >= nrows) return;
  const int32_t* sel = ids + row * topk;
  const T* p = diq_part + row * topk * DI + (lane % LPR) * 8;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  float kacc = 0.f;
  for (int s = 0; s < topk; ++s) {
    if ((unsigned)sel[s] >= (unsigned)nblk) continue;  // no partial for ids outside [0, nblk)
    const frag_t<T> x = load8(p + (int64_t)s * DI);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += to_f32(x[e]);
    kacc += kl_part[row * topk + s];
  }
  if (lane % LPR == 0) kl[row] = kacc;
  frag_t<T> o;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = from_f32<T>(acc[e]);
  T* dst = d_iq + row * DI + (lane % LPR) * 8;
  if constexpr (sizeof(T) == 2) {
    *reinterpret_cast<frag_t<T>*>(dst) = o;
  } else {
    *reinterpret_cast<f32x4*>(dst) = f32x4{o[0], o[1], o[2], o[3]};
    *reinterpret_cast<f32x4*>(dst + 4) = f32x4{o[4], o[5], o[6], o[7]};
  }
}

// ---- d ik: item partials of each block in item order ------------------------
template <typename T, int DI, int BK>
__global__ void __launch_bounds__(256) k_kl_dik_reduce(const T* __restrict__ part, const int4* __restrict__ items,
                                                       const int32_t* __restrict__ item_count, T* __restrict__ d_ik,
                                                       int Nk, int Hkv, int nblk, int items_cap) {
  constexpr int CH = DI / 8;
  const int bg = blockIdx.y, b = bg / Hkv, g = bg % Hkv;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // over nblk * BK * CH
  if (idx >= (int64_t)nblk * BK * CH) return;
  const int j = (int)(idx / (BK * CH));
  const int tk = (int)(idx / CH % BK), c = (int)(idx % CH);
  const int64_t t = (int64_t)j * BK + tk;
  if (t >= Nk) return;
  const int4* its = items + (int64_t)bg * items_cap;
  const int n = item_count[bg];
  int lo = 0, hi = n;  // first item of block j (items are in block order)
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (its[mid].x < j) lo = mid + 1;
    else hi = mid;
  }
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  for (int u = lo; u < n && its[u].x == j; ++u) {
    const frag_t<T> x = load8(part + ((int64_t)bg * items_cap + u) * BK * DI + tk * DI + c * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += to_f32(x[e]);
  }
  frag_t<T> o;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = from_f32<T>(acc[e]);
  T* dst = d_ik + (((int64_t)b * Nk + t) * Hkv + g) * DI + c * 8;
  if constexpr (sizeof(T) == 2) {
    *reinterpret_cast<frag_t<T>*>(dst) = o;
  } else {
    *reinterpret_cast<f32x4*>(dst) = f32x4{o[0], o[1], o[2], o[3]};
    *reinterpret_cast<f32x4*>(dst + 4) = f32x4{o[4], o[5], o[6], o[7]};
  }
}

struct KlKernels {
  int lse, lse_sum, main, finish, reduce;
};

template <typename T, int D, int DI, int BK>
void kl_launch_bk(const Shape& s, const KlArgs& a, const InvertPlan& p, float* kl, void* d_iq, void* d_ik,
                  hipStream_t st, const KlKernels& kid) {
  const dim3 grid(p.items_cap, s.B * s.Hkv);
  const int64_t nrows = (int64_t)s.B * s.Nq * s.Hkv;
  prof_begin(st, kid.lse);
  hipLaunchKernelGGL((k_kl_lse<T, DI, BK>), grid, dim3(256), 0, st, a);
  prof_end(st, kid.lse);
  prof_begin(st, kid.lse_sum);
  hipLaunchKernelGGL(k_kl_lse_sum, dim3((unsigned)((nrows + 255) / 256)), dim3(256), 0, st, a.plse, a.ids, a.lse_s,
                     s.topk, s.nblk, nrows);
  prof_end(st, kid.lse_sum);
  prof_begin(st, kid.main);
  if constexpr (sizeof(T) == 2) hipLaunchKernelGGL((k_kl_main8<T, D, DI, BK>), grid, dim3(512), 0, st, a);
  else hipLaunchKernelGGL((k_kl_main<T, D, DI, BK>), grid, dim3(256), 0, st, a);
  prof_end(st, kid.main);
  const int rpb = 4 * (64 / (DI / 8));
  prof_begin(st, kid.finish);
  hipLaunchKernelGGL((k_kl_finish<T, DI>), dim3((unsigned)((nrows + rpb - 1) / rpb)), dim3(256), 0, st, a.kl_part,
                     static_cast<const T*>(a.diq_part), a.ids, kl, static_cast<T*>(d_iq), s.topk, s.nblk, nrows);
  prof_end(st, kid.finish);
  const int64_t nthr = (int64_t)s.nblk * BK * (DI / 8);
  prof_begin(st, kid.reduce);
  hipLaunchKernelGGL((k_kl_dik_reduce<T, DI, BK>), dim3((unsigned)((nthr + 255) / 256), s.B * s.Hkv), dim3(256), 0,
                     st, static_cast<const T*>(a.dik_part), a.items, a.item_count, static_cast<T*>(d_ik), s.Nk, s.Hkv, s.nblk, p.items_cap);
  prof_end(st, kid.reduce);
}

template <typename T, int D, int DI>
void kl_launch_di(const Shape& s, const KlArgs& a, const InvertPlan& p, float* kl, void* d_iq, void* d_ik,
                  hipStream_t st, const KlKernels& kid) {
  if (s.Bk == 32) kl_launch_bk<T, D, DI, 32>(s, a, p, kl, d_iq, d_ik, st, kid);
  else if (s.Bk == 64) kl_launch_bk<T, D, DI, 64>(s, a, p, kl, d_iq, d_ik, st, kid);
  else kl_launch_bk<T, D, DI, 128>(s, a, p, kl, d_iq, d_ik, st, kid);
}

template <typename T, int D>
void kl_launch_d(const Shape& s, const KlArgs& a, const InvertPlan& p, float* kl, void* d_iq, void* d_ik,
                 hipStream_t st, const KlKernels& kid) {
  if (s.DI == 32) kl_launch_di<T, D, 32>(s, a, p, kl, d_iq, d_ik, st, kid);
  else if (s.DI == 64) kl_launch_di<T, D, 64>(s, a, p, kl, d_iq, d_ik, st, kid);
  else kl_launch_di<T, D, 128>(s, a, p, kl, d_iq, d_ik, st, kid);
}

}  // namespace

size_t kl_bytes(const Shape& s, const InvertPlan& p, KlWorkspace* w) {
  const size_t rows = (size_t)s.B * s.Nq * s.Hkv;
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  size_t off = 0;
  KlWorkspace L;
  L.plse = off;
  off += up(rows * s.topk * 4);
  L.lse_s = off;
  off += up(rows * 4);
  L.kl_part = off;
  off += up(rows * s.topk * 4);
  L.diq_part = off;
  off += up(rows * s.topk * s.DI * (s.dtype == kBF16 ? 2 : 4));  // in the input type
  L.dik_part = off;
  off += up((size_t)s.B * s.Hkv * p.items_cap * s.Bk * s.DI * (s.dtype == kBF16 ? 2 : 4));  // in the input type
  if (w) *w = L;
  return off;
}

hipError_t launch_indexer_kl(const Shape& s, const InvertPlan& p, const void* q, const void* k, const void* iq,
                             const void* ik, const float* lse, const int32_t* ids, const InvertOut& inv, char* ws,
                             float loss_scale, float* kl, void* d_iq, void* d_ik, hipStream_t st) {
  static const KlKernels kid{prof_register("kl_lse"), prof_register("kl_lse_sum"), prof_register("kl_main"),
                             prof_register("kl_finish"), prof_register("kl_dik_reduce")};
  KlWorkspace L;
  kl_bytes(s, p, &L);
  KlArgs a;
  a.q = q;
  a.k = k;
  a.iq = iq;
  a.ik = ik;
  a.lse = lse;
  a.ids = ids;
  a.entries = inv.entries;
  a.item_count = inv.item_count;
  a.items = inv.items;
  a.plse = reinterpret_cast<float*>(ws + L.plse);
  a.lse_s = reinterpret_cast<float*>(ws + L.lse_s);
  a.kl_part = reinterpret_cast<float*>(ws + L.kl_part);
  a.diq_part = ws + L.diq_part;
  a.dik_part = ws + L.dik_part;
  a.Nq = s.Nq;
  a.Nk = s.Nk;
  a.Hq = s.Hq;
  a.Hkv = s.Hkv;
  a.G = s.Hq / s.Hkv;
  a.topk = s.topk;
  a.items_cap = p.items_cap;
  a.q_offset = s.q_offset;
  a.topk_magic = ((uint64_t)1 << 40) / (uint64_t)s.topk + 1;
  a.c_log2 = s.scale * kLog2e;
  a.loss_scale = loss_scale;
  if (s.dtype == kBF16) {
    if (s.D == 64) kl_launch_d<bf16_t, 64>(s, a, p, kl, d_iq, d_ik, st, kid);
    else kl_launch_d<bf16_t, 128>(s, a, p, kl, d_iq, d_ik, st, kid);
  } else {
    if (s.D == 64) kl_launch_d<float, 64>(s, a, p, kl, d_iq, d_ik, st, kid);
    else kl_launch_d<float, 128>(s, a, p, kl, d_iq, d_ik, st, kid);
  }
  return hipGetLastError();
}

}  // namespace msa
