// backward.hip -- gradients of the Main Branch on gfx950.
//
// The selection is not differentiable (the pages train the Index Branch with a
// separate loss, paper summary page "Method"), so the backward pass is that of
// exact softmax attention restricted to the selected blocks, for the fixed
// block ids of the forward pass.  Per (b, i, h) over its visible selected
// tokens T, with P the softmax of x_t = scale <q, k_t> and O = sum P_t v_t
// (the chain rule through the softmax; the same recurrence as FlashAttention's
// backward, which the Fireworks note on KV-stationary attention cites):
//     D    = <dO, O>                         (k_bwd_rowdot)
//     dP_t = <dO, v_t>,  dS_t = P_t (dP_t - D)
//     dq   = scale sum_t dS_t k_t            (k_bwd_dq, then k_bwd_dq_sum)
//     dk_t = scale sum dS_t q,  dv_t = sum P_t dO   (k_bwd_dkdv, then reduce)
// P is recomputed from the forward's log-sum-exp, so nothing of the forward
// but O and LSE is kept.
//
// Both heavy kernels walk the KV-outer work items of the forward (block j and
// the (query, head) rows that chose it; msa_invert's lists):
//  * k_bwd_dq keeps the forward's orientation -- each query row in a lane pair,
//    S^T = K Q^T, dP^T = V dO^T, dQ^T = K^T dS^T (dS taken straight from the
//    accumulators) -- and writes one fp32 dq partial per (row, slot), summed
//    in slot order afterwards: no atomics.
//  * k_bwd_dkdv turns the products around so that a lane owns a key: wave w
//    takes keys [32w, 32w+32) of the block, S = Q K^T and dP = dO V^T per
//    32-row tile, and accumulates dV += P^T dO and dK += dS^T Q in registers
//    over the item's tiles (the tile's Q and dO are staged in LDS, row-major
//    and transposed).  Each item writes fp32 dk/dv partials of its block;
//    k_bwd_dkdv_reduce sums the items of every block in item order.
#include "attn_common.h"

namespace msa {
namespace {

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  const float* lse;      // [B, Nq, Hq] forward log-sum-exp (natural log)
  const float* drow;     // [B, Nq, Hq] <dO, O>
  const int32_t* entries;
  const int32_t* item_count;
  const int4* items;
  float* dq_part;        // [B, Nq, Hq, topk, D] fp32
  float* dkv_part;       // [B*Hkv][items_cap][2][BK][D] fp32 (dk, then dv)
  void* trash;           // scratch line for the stores of rows past an item's end
  int Nq, Nk, Hq, Hkv, G, topk, items_cap, gshift;
  int64_t q_offset;
  uint64_t topk_magic;
  float scale;   // softmax scale
  float c_log2;  // softmax scale * log2(e)
};

// ---- D = <dO, O> per (b, i, h): D/8 lanes per row ---------------------------
template <typename T, int D>
__global__ void __launch_bounds__(256) k_bwd_rowdot(const T* __restrict__ out, const T* __restrict__ dout,
                                                    float* __restrict__ drow, int64_t nrows) {
  constexpr int LPR = D / 8;
  const int lane = threadIdx.x & 63;
  const int64_t row = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * (64 / LPR) + lane / LPR;
  if (row >= nrows) return;  // rows are whole lane groups: no cross-lane work below is cut short
  const frag_t<T> o = load8(out + row * D + (lane % LPR) * 8);
  const frag_t<T> g = load8(dout + row * D + (lane % LPR) * 8);
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) acc = fmaf(to_f32(o[e]), to_f32(g[e]), acc);
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) acc += xor_shfl(acc, m);
  if (lane % LPR == 0) drow[row] = acc;
}

// Rows of one key block (BK rows of D elements at a token stride) staged into
// LDS with the row pitch of KvLds.  Rows past n_k are zero-filled.
template <typename T, int D, int BK>
__device__ __forceinline__ void stage_rows(char* dst, const T* base, int64_t tok_stride, int j, int n_k, int tid) {
  using L = KvLds<T, D, BK>;
  constexpr int CPR = D * (int)sizeof(T) / 16;
  constexpr int CH = BK * CPR;
#pragma unroll
  for (int u = 0; u < (CH + 255) / 256; ++u) {
    const int c = tid + u * 256;
    if (c < CH) {
      const int row = c / CPR, col = c % CPR;
      const int64_t t = (int64_t)j * BK + row;
      u32x4 x = u32x4{};
      if (t < n_k) x = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(base + t * tok_stride) + col * 16);
      *reinterpret_cast<u32x4*>(dst + row * L::KPITCH + col * 16) = x;
    }
  }
}

// ---- dq partials: forward orientation ---------------------------------------
// LDS: K rows | K^T (the KvLds "V^T" region, filled with K) | V rows | obuf.
template <typename T, int D, int BK>
__global__ void __launch_bounds__(256, 1) k_bwd_dq(BwdArgs a) {
  using L = KvLds<T, D, BK>;
  constexpr int MT = BK / 32;
  constexpr int ROWB = D * 4;           // one fp32 dq partial row
  constexpr int OPITCH = ROWB + 16;
  constexpr int LPR = ROWB / 16;        // lanes per row on the way out
  constexpr int RPS = 64 / LPR;         // rows per store instruction
  // fp32 with d = 128 and 128-token blocks: V rows would not fit beside K and
  // K^T, so its fragments are read from global memory instead.
  constexpr bool V_LDS = !(sizeof(T) == 4 && D == 128 && BK == 128);
  __shared__ __attribute__((aligned(16))) char lds[L::BYTES + (V_LDS ? BK * L::KPITCH : 16)];
  __shared__ int32_t ent_lds[kMaxItemEntries];
  __shared__ __attribute__((aligned(16))) char obuf[4][8 * OPITCH];
  char* vrows = lds + L::BYTES;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5;
  const int bg = blockIdx.y, b = bg / a.Hkv, g = bg % a.Hkv;
  const int n = a.item_count[bg];
  const int per = (n + 7) / 8;
  const int x = blockIdx.x;
  const int item = (x % 8) * per + x / 8;  // each XCD runs a contiguous run of items
  if (x / 8 >= per || item >= n) return;
  const int4 it = a.items[(int64_t)bg * a.items_cap + item];
  const int j = it.x, e0 = it.y, e1 = it.z;
  const int nrows = (e1 - e0) * a.G;
  const int nent = e1 - e0;
  const int32_t* ent = a.entries + (int64_t)bg * a.Nq * a.topk + e0;
  for (int u = tid; u < nent; u += 256) ent_lds[u] = ent[u];

  const int64_t tok_stride = (int64_t)a.Hkv * D;
  const T* kb = static_cast<const T*>(a.k) + (int64_t)b * a.Nk * tok_stride + g * D;
  const T* vb = static_cast<const T*>(a.v) + (int64_t)b * a.Nk * tok_stride + g * D;
  stage_kv<T, D, BK>(lds, kb, kb, tok_stride, j, a.Nk, tid);  // K rows and K^T
  if constexpr (V_LDS) stage_rows<T, D, BK>(vrows, vb, tok_stride, j, a.Nk, tid);
  __syncthreads();
  const int64_t key0 = (int64_t)j * BK;
  const T* qbase = static_cast<const T*>(a.q);
  const T* dobase = static_cast<const T*>(a.dout);
  char* ob = obuf[wave];

  for (int tile = wave; tile * 32 < nrows; tile += 4) {
    const int r = tile * 32 + (lane & 31);
    const bool valid = r < nrows;
    const TileRows cur = rows_of(valid ? ent_lds[r >> a.gshift] : 0, valid, r, a.gshift, a.topk, a.topk_magic, g);
    frag_t<T> qf[D / 16], dof[D / 16];
    load_q_rows<T, D>(qf, qbase, cur, b, a.Nq, a.Hq, 0, half);
    load_q_rows<T, D>(dof, dobase, cur, b, a.Nq, a.Hq, 0, half);
    const int64_t rowi = ((int64_t)b * a.Nq + cur.qq) * a.Hq + cur.h;
    const float lse2 = a.lse[rowi] * kLog2e;
    const float dr = a.drow[rowi];
    const int64_t pos = a.q_offset + cur.qq;
    const int vis = (int)max((int64_t)0, min((int64_t)BK, min(pos + 1, (int64_t)a.Nk) - key0));
    // S^T = K Q^T and dP^T = V dO^T (each lane pair holds row c's keys)
    f32x16 s[MT], dp[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int kk = mt * 32 + (lane & 31);  // key of this lane's A rows
      const T* krow = reinterpret_cast<const T*>(lds + kk * L::KPITCH) + 8 * half;
      // V rows past n_k read token n_k - 1: their keys are masked below
      const T* vrow = V_LDS ? reinterpret_cast<const T*>(vrows + kk * L::KPITCH) + 8 * half
                            : vb + min(key0 + kk, (int64_t)a.Nk - 1) * tok_stride + 8 * half;
      s[mt] = mma0(load8(krow), qf[0]);
      dp[mt] = mma0(load8(vrow), dof[0]);
#pragma unroll
      for (int ks = 1; ks < D / 16; ++ks) {
        mma(load8(krow + 16 * ks), qf[ks], s[mt]);
        mma(load8(vrow + 16 * ks), dof[ks], dp[mt]);
      }
    }
    // dS = P (dP - D), P = exp2(x log2e - lse log2e); masked keys give P = 0
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int t = 32 * mt + 8 * (e / 4) + 4 * half + (e % 4);
        const float p = t < vis ? exp2_fast(fmaf(s[mt][e], a.c_log2, -lse2)) : 0.f;
        s[mt][e] = p * (dp[mt][e] - dr);
      }
    // dQ^T = K^T dS^T, dS taken from the accumulators (k permuted as in the forward)
    f32x16 o[D / 32];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int aa = 0; aa < 2; ++aa) {
        frag_t<T> pb;
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[e] = from_f32<T>(s[mt][8 * aa + e]);
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          const frag_t<T> ka = vt_frag<T, D, BK>(lds, 32 * dt + (lane & 31), mt, aa, half);
          if (mt == 0 && aa == 0) o[dt] = mma0(ka, pb);
          else mma(ka, pb, o[dt]);
        }
      }
    // fp32 partial rows out through LDS, 8 rows per pass (whole rows per store)
    const int64_t prow = rowi * a.topk + cur.slot;
#pragma unroll
    for (int ps = 0; ps < 4; ++ps) {
      if (((lane & 31) >> 3) == ps) {
        char* orow = ob + ((lane & 7) * OPITCH);
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const f32x4 w = f32x4{o[dt][4 * i] * a.scale, o[dt][4 * i + 1] * a.scale, o[dt][4 * i + 2] * a.scale,
                                  o[dt][4 * i + 3] * a.scale};
            *reinterpret_cast<f32x4*>(orow + (32 * dt + 8 * i + 4 * half) * 4) = w;
          }
      }
      wave_lds_sync();
#pragma unroll
      for (int kk = 0; kk < 8 / RPS; ++kk) {
        const int rl = lane / LPR + kk * RPS;
        const int src = ps * 8 + rl;
        const int64_t dst_row = __shfl(prow, src, 64);
        const int ok = __shfl((int)cur.valid, src, 64);
        const u32x4 v = *reinterpret_cast<const u32x4*>(ob + rl * OPITCH + (lane % LPR) * 16);
        char* dst = ok ? reinterpret_cast<char*>(a.dq_part) + dst_row * ROWB : static_cast<char*>(a.trash);
        *reinterpret_cast<u32x4*>(dst + (lane % LPR) * 16) = v;
      }
      wave_lds_sync();
    }
  }
}

// ---- dq = sum of the slot partials, in slot order ---------------------------
template <typename T, int D>
__global__ void __launch_bounds__(256) k_bwd_dq_sum(const float* __restrict__ part, const int32_t* __restrict__ ids,
                                                    T* __restrict__ dq, int Nq, int Hq, int Hkv, int G, int topk,
                                                    int64_t nrows) {
  constexpr int LPR = D / 8;
  const int lane = threadIdx.x & 63;
  const int64_t row = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * (64 / LPR) + lane / LPR;  // (b, i, h)
  if (row >= nrows) return;
  const int h = (int)(row % Hq);
  const int64_t bi = row / Hq;
  const int32_t* sel = ids + (bi * Hkv + h / G) * topk;
  const float* p = part + row * topk * D + (lane % LPR) * 8;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  for (int s = 0; s < topk; ++s) {
    if (sel[s] < 0) continue;
    const f32x4 lo = *reinterpret_cast<const f32x4*>(p + (int64_t)s * D);
    const f32x4 hi = *reinterpret_cast<const f32x4*>(p + (int64_t)s * D + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[e] += lo[e];
      acc[4 + e] += hi[e];
    }
  }
  frag_t<T> o;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = from_f32<T>(acc[e]);
  T* dst = dq + row * D + (lane % LPR) * 8;
  if constexpr (sizeof(T) == 2) {
    *reinterpret_cast<frag_t<T>*>(dst) = o;
  } else {
    *reinterpret_cast<f32x4*>(dst) = f32x4{o[0], o[1], o[2], o[3]};
    *reinterpret_cast<f32x4*>(dst + 4) = f32x4{o[4], o[5], o[6], o[7]};
  }
}

// ---- dk / dv partials: a lane owns a key ------------------------------------
// LDS: K rows | V rows | the tile's Q and dO rows (row-major) | their
// transposes | per-row log-sum-exp, D and position.
template <typename T, int D, int BK>
struct DkdvLds {
  using L = KvLds<T, D, BK>;
  // fp32 with d = 128 and 128-token blocks: K and V fragments come from global
  // memory (the block would not fit beside the tile buffers).
  static constexpr bool KV_LDS = !(sizeof(T) == 4 && D == 128 && BK == 128);
  static constexpr int RPITCH = D * (int)sizeof(T) + 16;            // a tile row
  static constexpr int TPITCH = 32 * (int)sizeof(T) + (sizeof(T) == 2 ? 8 : 16);  // a transposed row (32 rows)
  static constexpr int K_OFF = 0;
  static constexpr int V_OFF = KV_LDS ? BK * L::KPITCH : 0;
  static constexpr int Q_OFF = KV_LDS ? V_OFF + BK * L::KPITCH : 0;
  static constexpr int DO_OFF = Q_OFF + 32 * RPITCH;
  static constexpr int QT_OFF = DO_OFF + 32 * RPITCH;
  static constexpr int DOT_OFF = QT_OFF + D * TPITCH;
  static constexpr int BYTES = DOT_OFF + D * TPITCH;
};

// A fragment of a transposed tile for k-step a: row d, tile rows
// 16a + 4h + [0..3] and 16a + 8 + 4h + [0..3] (the accumulator order).
template <typename T, int D, int BK>
__device__ __forceinline__ frag_t<T> tile_t_frag(const char* base, int d, int a, int half) {
  using X = DkdvLds<T, D, BK>;
  const T* row = reinterpret_cast<const T*>(base + d * X::TPITCH);
  const int r0 = 16 * a + 4 * half;
  const typename Pack4<T>::type lo = *reinterpret_cast<const typename Pack4<T>::type*>(row + r0);
  const typename Pack4<T>::type hi = *reinterpret_cast<const typename Pack4<T>::type*>(row + r0 + 8);
  frag_t<T> f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[e] = lo[e];
    f[4 + e] = hi[e];
  }
  return f;
}

template <typename T, int D, int BK>
__global__ void __launch_bounds__(256, 1) k_bwd_dkdv(BwdArgs a) {
  using L = KvLds<T, D, BK>;
  using X = DkdvLds<T, D, BK>;
  __shared__ __attribute__((aligned(16))) char lds[X::BYTES];
  __shared__ int32_t ent_lds[kMaxItemEntries];
  __shared__ float row_lse2[32], row_d[32];
  __shared__ int row_pos[32];  // -1 for rows past the item's end
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5;
  const int bg = blockIdx.y, b = bg / a.Hkv, g = bg % a.Hkv;
  const int n = a.item_count[bg];
  const int per = (n + 7) / 8;
  const int x = blockIdx.x;
  const int item = (x % 8) * per + x / 8;
  if (x / 8 >= per || item >= n) return;
  const int4 it = a.items[(int64_t)bg * a.items_cap + item];
  const int j = it.x, e0 = it.y, e1 = it.z;
  const int nrows = (e1 - e0) * a.G;
  const int nent = e1 - e0;
  const int32_t* ent = a.entries + (int64_t)bg * a.Nq * a.topk + e0;
  for (int u = tid; u < nent; u += 256) ent_lds[u] = ent[u];

  const int64_t tok_stride = (int64_t)a.Hkv * D;
  const T* kb = static_cast<const T*>(a.k) + (int64_t)b * a.Nk * tok_stride + g * D;
  const T* vb = static_cast<const T*>(a.v) + (int64_t)b * a.Nk * tok_stride + g * D;
  if constexpr (X::KV_LDS) {
    stage_rows<T, D, BK>(lds + X::K_OFF, kb, tok_stride, j, a.Nk, tid);
    stage_rows<T, D, BK>(lds + X::V_OFF, vb, tok_stride, j, a.Nk, tid);
  }
  const T* qbase = static_cast<const T*>(a.q);
  const T* dobase = static_cast<const T*>(a.dout);
  const int64_t key0 = (int64_t)j * BK;
  const bool has_keys = wave * 32 < BK;  // waves past the block's keys only help staging
  const int64_t my_key = key0 + wave * 32 + (lane & 31);

  f32x16 dkacc[D / 32], dvacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    dkacc[dt] = f32x16{};
    dvacc[dt] = f32x16{};
  }
  constexpr int CPR = D * (int)sizeof(T) / 16;  // 16-byte chunks per tile row
  for (int tile = 0; tile * 32 < nrows; ++tile) {
    __syncthreads();  // the previous tile's staging is no longer read
    // Stage the tile's 32 (query, head) rows of Q and dO, row-major and transposed.
    for (int c = tid; c < 32 * CPR * 2; c += 256) {
      const int which = c / (32 * CPR);  // 0: Q, 1: dO
      const int cc = c % (32 * CPR);
      const int rr = cc / CPR, col = cc % CPR;
      const int r = tile * 32 + rr;
      const bool valid = r < nrows;
      const TileRows t = rows_of(valid ? ent_lds[r >> a.gshift] : 0, valid, r, a.gshift, a.topk, a.topk_magic, g);
      const T* src = (which ? dobase : qbase) + (((int64_t)b * a.Nq + t.qq) * a.Hq + t.h) * D;
      u32x4 v = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(src) + col * 16);
      if (!valid) v = u32x4{};
      *reinterpret_cast<u32x4*>(lds + (which ? X::DO_OFF : X::Q_OFF) + rr * X::RPITCH + col * 16) = v;
      T el[16 / sizeof(T)];
      __builtin_memcpy(el, &v, 16);
      char* tb = lds + (which ? X::DOT_OFF : X::QT_OFF);
#pragma unroll
      for (int e = 0; e < (int)(16 / sizeof(T)); ++e)
        *reinterpret_cast<T*>(tb + (col * (16 / (int)sizeof(T)) + e) * X::TPITCH + rr * (int)sizeof(T)) = el[e];
      if (which == 0 && col == 0) {
        const int64_t rowi = ((int64_t)b * a.Nq + t.qq) * a.Hq + t.h;
        row_lse2[rr] = valid ? a.lse[rowi] * kLog2e : 0.f;
        row_d[rr] = valid ? a.drow[rowi] : 0.f;
        row_pos[rr] = valid ? (int)min(a.q_offset + t.qq, (int64_t)a.Nk - 1) : -1;
      }
    }
    __syncthreads();
    if (!has_keys) continue;
    // S = Q K^T and dP = dO V^T for this wave's 32 keys: lane = key, rows in the accumulator
    f32x16 s = f32x16{}, dp = f32x16{};
    const T* qr = reinterpret_cast<const T*>(lds + X::Q_OFF + (lane & 31) * X::RPITCH) + 8 * half;
    const T* dr = reinterpret_cast<const T*>(lds + X::DO_OFF + (lane & 31) * X::RPITCH) + 8 * half;
    const int kk = wave * 32 + (lane & 31);  // this lane's key in the block
    const int64_t kt = min(key0 + kk, (int64_t)a.Nk - 1);  // keys past n_k are masked below
    const T* kr = X::KV_LDS ? reinterpret_cast<const T*>(lds + X::K_OFF + kk * L::KPITCH) + 8 * half
                            : kb + kt * tok_stride + 8 * half;
    const T* vr = X::KV_LDS ? reinterpret_cast<const T*>(lds + X::V_OFF + kk * L::KPITCH) + 8 * half
                            : vb + kt * tok_stride + 8 * half;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      mma(load8(qr + 16 * ks), load8(kr + 16 * ks), s);
      mma(load8(dr + 16 * ks), load8(vr + 16 * ks), dp);
    }
    // P and dS; position e of the accumulator is tile row 8(e/4) + 4h + e%4
    f32x16 pm, dsm;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int rr = 8 * (e / 4) + 4 * half + (e % 4);
      const int pos = row_pos[rr];
      const float p = (pos >= 0 && my_key <= pos) ? exp2_fast(fmaf(s[e], a.c_log2, -row_lse2[rr])) : 0.f;
      pm[e] = p;
      dsm[e] = p * (dp[e] - row_d[rr]);
    }
    // dV += P^T dO, dK += dS^T Q: A from the accumulators, B from the transposed tile
#pragma unroll
    for (int aa = 0; aa < 2; ++aa) {
      frag_t<T> pa, sa;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pa[e] = from_f32<T>(pm[8 * aa + e]);
        sa[e] = from_f32<T>(dsm[8 * aa + e]);
      }
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        mma(pa, tile_t_frag<T, D, BK>(lds + X::DOT_OFF, 32 * dt + (lane & 31), aa, half), dvacc[dt]);
        mma(sa, tile_t_frag<T, D, BK>(lds + X::QT_OFF, 32 * dt + (lane & 31), aa, half), dkacc[dt]);
      }
    }
  }
  if (!has_keys) return;
  // Partials of this item: lane holds key 32w + 8(e/4) + 4h + e%4, d = 32 dt + lane%32.
  float* dst = a.dkv_part + ((int64_t)bg * a.items_cap + item) * 2 * BK * D;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int key = wave * 32 + 8 * (e / 4) + 4 * half + (e % 4);
      const int d = 32 * dt + (lane & 31);
      dst[key * D + d] = dkacc[dt][e] * a.scale;
      dst[BK * D + key * D + d] = dvacc[dt][e];
    }
}

// ---- dk, dv = sum of the item partials of each block, in item order ---------
// One thread per (token of the block, 8 channels); blocks no query selected
// (and tokens no query can see) get zeros.
template <typename T, int D, int BK>
__global__ void __launch_bounds__(256) k_bwd_dkdv_reduce(const float* __restrict__ part, const int4* __restrict__ items,
                                                         const int32_t* __restrict__ item_count, T* __restrict__ dk,
                                                         T* __restrict__ dv, int Nk, int Hkv, int nblk, int items_cap) {
  constexpr int CH = D / 8;
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
  float ak[8], av[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) ak[e] = av[e] = 0.f;
  for (int u = lo; u < n && its[u].x == j; ++u) {
    const float* p = part + ((int64_t)bg * items_cap + u) * 2 * BK * D + tk * D + c * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ak[e] += p[e];
      av[e] += p[BK * D + e];
    }
  }
  frag_t<T> ok, ov;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    ok[e] = from_f32<T>(ak[e]);
    ov[e] = from_f32<T>(av[e]);
  }
  const int64_t off = (((int64_t)b * Nk + t) * Hkv + g) * D + c * 8;
  if constexpr (sizeof(T) == 2) {
    *reinterpret_cast<frag_t<T>*>(dk + off) = ok;
    *reinterpret_cast<frag_t<T>*>(dv + off) = ov;
  } else {
    *reinterpret_cast<f32x4*>(dk + off) = f32x4{ok[0], ok[1], ok[2], ok[3]};
    *reinterpret_cast<f32x4*>(dk + off + 4) = f32x4{ok[4], ok[5], ok[6], ok[7]};
    *reinterpret_cast<f32x4*>(dv + off) = f32x4{ov[0], ov[1], ov[2], ov[3]};
    *reinterpret_cast<f32x4*>(dv + off + 4) = f32x4{ov[4], ov[5], ov[6], ov[7]};
  }
}

template <typename T, int D, int BK>
void bwd_launch_bk(const Shape& s, const BwdArgs& a, const InvertPlan& p, const void* ids, void* dq, void* dk, void* dv,
                   hipStream_t st, int kid_dq, int kid_sum, int kid_dkdv, int kid_red) {
  const dim3 grid(p.items_cap, s.B * s.Hkv);
  prof_begin(st, kid_dq);
  hipLaunchKernelGGL((k_bwd_dq<T, D, BK>), grid, dim3(256), 0, st, a);
  prof_end(st, kid_dq);
  const int64_t nrows = (int64_t)s.B * s.Nq * s.Hq;
  const int rpb = 4 * (64 / (D / 8));
  prof_begin(st, kid_sum);
  hipLaunchKernelGGL((k_bwd_dq_sum<T, D>), dim3((unsigned)((nrows + rpb - 1) / rpb)), dim3(256), 0, st, a.dq_part,
                     static_cast<const int32_t*>(ids), static_cast<T*>(dq), s.Nq, s.Hq, s.Hkv, s.Hq / s.Hkv, s.topk,
                     nrows);
  prof_end(st, kid_sum);
  prof_begin(st, kid_dkdv);
  hipLaunchKernelGGL((k_bwd_dkdv<T, D, BK>), grid, dim3(256), 0, st, a);
  prof_end(st, kid_dkdv);
  const int64_t nthr = (int64_t)s.nblk * BK * (D / 8);
  prof_begin(st, kid_red);
  hipLaunchKernelGGL((k_bwd_dkdv_reduce<T, D, BK>), dim3((unsigned)((nthr + 255) / 256), s.B * s.Hkv), dim3(256), 0,
                     st, a.dkv_part, a.items, a.item_count, static_cast<T*>(dk), static_cast<T*>(dv), s.Nk, s.Hkv,
                     s.nblk, p.items_cap);
  prof_end(st, kid_red);
}

template <typename T, int D>
void bwd_launch(const Shape& s, const BwdArgs& a, const InvertPlan& p, const void* ids, void* dq, void* dk, void* dv,
                hipStream_t st, int k1, int k2, int k3, int k4) {
  if (s.Bk == 32) bwd_launch_bk<T, D, 32>(s, a, p, ids, dq, dk, dv, st, k1, k2, k3, k4);
  else if (s.Bk == 64) bwd_launch_bk<T, D, 64>(s, a, p, ids, dq, dk, dv, st, k1, k2, k3, k4);
  else bwd_launch_bk<T, D, 128>(s, a, p, ids, dq, dk, dv, st, k1, k2, k3, k4);
}

}  // namespace

size_t bwd_dkv_bytes(const Shape& s, const InvertPlan& p) {
  return (size_t)s.B * s.Hkv * p.items_cap * 2 * s.Bk * s.D * sizeof(float);
}

hipError_t launch_bwd_rowdot(const Shape& s, const void* out, const void* dout, float* drow, hipStream_t st) {
  static const int kid = prof_register("bwd_rowdot");
  const int64_t nrows = (int64_t)s.B * s.Nq * s.Hq;
  const int rpb = 4 * (64 / (s.D / 8));
  const dim3 grid((unsigned)((nrows + rpb - 1) / rpb));
  prof_begin(st, kid);
  if (s.dtype == kBF16) {
    if (s.D == 64) hipLaunchKernelGGL((k_bwd_rowdot<bf16_t, 64>), grid, dim3(256), 0, st, static_cast<const bf16_t*>(out), static_cast<const bf16_t*>(dout), drow, nrows);
    else hipLaunchKernelGGL((k_bwd_rowdot<bf16_t, 128>), grid, dim3(256), 0, st, static_cast<const bf16_t*>(out), static_cast<const bf16_t*>(dout), drow, nrows);
  } else {
    if (s.D == 64) hipLaunchKernelGGL((k_bwd_rowdot<float, 64>), grid, dim3(256), 0, st, static_cast<const float*>(out), static_cast<const float*>(dout), drow, nrows);
    else hipLaunchKernelGGL((k_bwd_rowdot<float, 128>), grid, dim3(256), 0, st, static_cast<const float*>(out), static_cast<const float*>(dout), drow, nrows);
  }
  const hipError_t e = hipGetLastError();
  prof_end(st, kid);
  return e;
}

hipError_t launch_bwd_attention(const Shape& s, const InvertPlan& p, const void* q, const void* k, const void* v,
                                const void* dout, const float* lse, const float* drow, const int32_t* ids,
                                const InvertOut& inv, float* dq_part, float* dkv_part, void* trash, void* dq, void* dk,
                                void* dv, hipStream_t st) {
  static const int k1 = prof_register("bwd_dq");
  static const int k2 = prof_register("bwd_dq_sum");
  static const int k3 = prof_register("bwd_dkdv");
  static const int k4 = prof_register("bwd_dkdv_reduce");
  BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.dout = dout;
  a.lse = lse;
  a.drow = drow;
  a.entries = inv.entries;
  a.item_count = inv.item_count;
  a.items = inv.items;
  a.dq_part = dq_part;
  a.dkv_part = dkv_part;
  a.trash = trash;
  a.Nq = s.Nq;
  a.Nk = s.Nk;
  a.Hq = s.Hq;
  a.Hkv = s.Hkv;
  a.G = s.Hq / s.Hkv;
  a.topk = s.topk;
  a.items_cap = p.items_cap;
  a.gshift = __builtin_ctz((unsigned)a.G);
  a.q_offset = s.q_offset;
  a.topk_magic = ((uint64_t)1 << 40) / (uint64_t)s.topk + 1;
  a.scale = s.scale;
  a.c_log2 = s.scale * kLog2e;
  if (s.dtype == kBF16) {
    if (s.D == 64) bwd_launch<bf16_t, 64>(s, a, p, ids, dq, dk, dv, st, k1, k2, k3, k4);
    else bwd_launch<bf16_t, 128>(s, a, p, ids, dq, dk, dv, st, k1, k2, k3, k4);
  } else {
    if (s.D == 64) bwd_launch<float, 64>(s, a, p, ids, dq, dk, dv, st, k1, k2, k3, k4);
    else bwd_launch<float, 128>(s, a, p, ids, dq, dk, dv, st, k1, k2, k3, k4);
  }
  return hipGetLastError();
}

}  // namespace msa
