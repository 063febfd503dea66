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
// The heavy kernel walks the KV-outer work items of the forward (block j and
// the (query, head) rows that chose it; msa_invert's lists) with a lane owning
// a key of the block: S = Q K^T and dP = dO V^T per 32-row tile, dV += P^T dO
// and dK += dS^T Q accumulated in registers over the item's tiles, and
// dQ = dS K formed per tile from dS passed through LDS (k_bwd_split for
// 16-bit inputs, k_bwd_fused for fp32).  dq goes
// out as one partial per (row, slot), summed in slot order (k_bwd_dq_sum); dk
// and dv as fp32 partials per item, summed per block in item order
// (k_bwd_dkdv_reduce).  No atomics.
#include <type_traits>

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
  void* dq_part;         // [B, Nq, Hq, topk, D] in the input type
  void* dkv_part;        // [B*Hkv][items_cap][2][BK][D] in the input type (dk, then dv)
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
  acc = group_sum<LPR>(acc);
  if (lane % LPR == 0) drow[row] = acc;
}

// ---- the fused pass over one work item -------------------------------------
// A lane owns a key (wave w: keys [32w, 32w+32) of the block, held in
// registers as MFMA B operands); the item's (query, head) rows go by in tiles
// of 32.  Per tile: S = Q K^T and dP = dO V^T (rows in the accumulator), P and
// dS = P (dP - D) in place, dV += P^T dO and dK += dS^T Q with the
// accumulators as A operands and the tile's transposed rows as B operands.
// dS is written to LDS as [row][key]; after a barrier wave w forms
// dQ^T[32w..32w+32) = K^T dS^T over the whole block (K^T staged once per item)
// and stores it as the (row, slot) partial.  The next tile's rows are fetched
// into registers before the current tile's products and written to LDS while
// the dQ products run.
template <typename T, int D, int BK>
struct FusedLds {
  using L = KvLds<T, D, BK>;
  static constexpr int RPITCH = D * (int)sizeof(T) + 16;                          // a tile row
  static constexpr int TPITCH = 32 * (int)sizeof(T) + (sizeof(T) == 2 ? 8 : 16);  // a transposed tile row
  // a dS row [row][key]: for 16-bit types an odd multiple of 8 bytes past BK keys, so that the 32 rows read by a
  // half-wave fall on distinct banks, and 3 mod 8 of them so that the two half-waves' writes (4 rows apart) do too
  static constexpr int SPITCH = BK * (int)sizeof(T) + (sizeof(T) == 2 ? 24 : 16);
  static constexpr bool SWZ = sizeof(T) == 2;  // transposed tiles use the chunk swizzle
  static constexpr int KT_OFF = 0;                                                 // K^T [D][BK]
  static constexpr int Q_OFF = KT_OFF + D * L::VPITCH;
  static constexpr int DO_OFF = Q_OFF + 32 * RPITCH;
  static constexpr int QT_OFF = DO_OFF + 32 * RPITCH;
  static constexpr int DOT_OFF = QT_OFF + D * TPITCH;
  static constexpr int DS_OFF = DOT_OFF + D * TPITCH;
  static constexpr int BYTES = DS_OFF + 32 * SPITCH;
};

// The Q and dO rows of one tile: each task moves a 16-byte column chunk of
// four consecutive rows of one tensor, so that the transposed copy is written
// four rows at a time.
template <typename T, int D>
struct TileStage {
  static constexpr int CPR = D * (int)sizeof(T) / 16;  // chunks per row
  static constexpr int EPC = 16 / (int)sizeof(T);      // elements per chunk
  static constexpr int TASKS = 2 * 8 * CPR;
  static constexpr int NT = (TASKS + 255) / 256;
  // Loaded values are left untouched until store(): any use right after the
  // loads would make the compiler wait for them there, and the fetch would no
  // longer overlap the current tile's products.
  u32x4 v[NT][4];
  float lse[4], dr[4];
  uint32_t valid_mask;

  __device__ __forceinline__ void load(const BwdArgs& a, const int32_t* ent_lds, int tile, int nrows, int b, int g,
                                       int tid) {
    valid_mask = 0;
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      const int task = tid + 256 * u;
      if (task >= TASKS) continue;
      const int tensor = task / (8 * CPR), rg = task / CPR % 8, col = task % CPR;
      const T* base = static_cast<const T*>(tensor ? a.dout : a.q);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int rr = tile * 32 + 4 * rg + r;
        const bool valid = rr < nrows;
        const TileRows t = rows_of(valid ? ent_lds[rr >> a.gshift] : ent_lds[0], valid, rr, a.gshift, a.topk,
                                   a.topk_magic, g);
        const int64_t rowi = ((int64_t)b * a.Nq + t.qq) * a.Hq + t.h;
        // rows past the item's end read a valid row (entry 0) and store zeros
        v[u][r] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(base + rowi * D) + col * 16);
        valid_mask |= (uint32_t)valid << (4 * u + r);
        if (u == 0 && tensor == 0 && col == 0) {
          lse[r] = a.lse[rowi];
          dr[r] = a.drow[rowi];
        }
      }
    }
  }

  // Row positions and partial rows are recomputed here from the entries
  // rather than held in registers across the products.
  template <int BK>
  __device__ __forceinline__ void store(const BwdArgs& a, const int32_t* ent_lds, int tile, int b, int g, char* lds,
                                        float* row_lse2, float* row_d, int* row_pos, int64_t* row_prow,
                                        int tid) const {
    using X = FusedLds<T, D, BK>;
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      const int task = tid + 256 * u;
      if (task >= TASKS) continue;
      const int tensor = task / (8 * CPR), rg = task / CPR % 8, col = task % CPR;
      char* rows = lds + (tensor ? X::DO_OFF : X::Q_OFF);
      char* tr = lds + (tensor ? X::DOT_OFF : X::QT_OFF);
      u32x4 vv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        vv[r] = (valid_mask >> (4 * u + r)) & 1 ? v[u][r] : u32x4{};
        *reinterpret_cast<u32x4*>(rows + (4 * rg + r) * X::RPITCH + col * 16) = vv[r];
      }
      if constexpr (sizeof(T) == 2) {
        // elements 2w and 2w+1 of the chunk for the four rows: 2x2 transposes
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t x0 = vv[0][w], x1 = vv[1][w], x2 = vv[2][w], x3 = vv[3][w];
          const uint2 lo = make_uint2(__builtin_amdgcn_perm(x1, x0, 0x05040100u), __builtin_amdgcn_perm(x3, x2, 0x05040100u));
          const uint2 hi = make_uint2(__builtin_amdgcn_perm(x1, x0, 0x07060302u), __builtin_amdgcn_perm(x3, x2, 0x07060302u));
          const int c0 = col * EPC + 2 * w;  // columns c0 and c0 + 1 share the swizzle
          const int pos = tile_t_chunk<X::SWZ>(c0, rg) * 8;
          *reinterpret_cast<uint2*>(tr + c0 * X::TPITCH + pos) = lo;
          *reinterpret_cast<uint2*>(tr + (c0 + 1) * X::TPITCH + pos) = hi;
        }
      } else {
#pragma unroll
        for (int w = 0; w < 4; ++w)
          *reinterpret_cast<u32x4*>(tr + (col * EPC + w) * X::TPITCH + 4 * rg * 4) =
              u32x4{vv[0][w], vv[1][w], vv[2][w], vv[3][w]};
      }
      if (u == 0 && tensor == 0 && col == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool ok = (valid_mask >> r) & 1;
          const int rr = tile * 32 + 4 * rg + r;
          const TileRows t = rows_of(ok ? ent_lds[rr >> a.gshift] : ent_lds[0], ok, rr, a.gshift, a.topk,
                                     a.topk_magic, g);
          row_lse2[4 * rg + r] = ok ? lse[r] * kLog2e : 0.f;
          row_d[4 * rg + r] = ok ? dr[r] : 0.f;
          row_pos[4 * rg + r] = ok ? (int)min(a.q_offset + t.qq, (int64_t)a.Nk - 1) : -1;
          row_prow[4 * rg + r] = (((int64_t)b * a.Nq + t.qq) * a.Hq + t.h) * a.topk + t.slot;
        }
      }
    }
  }
};

// fp32 inputs: four waves, wave w owns keys [32w, 32w+32) and all of d.
template <typename T, int D, int BK>
__global__ void __launch_bounds__(256, 1) k_bwd_fused(BwdArgs a) {
  using X = FusedLds<T, D, BK>;
  constexpr int NTHR = 256;
  constexpr int DT = D / 32;  // dK / dV accumulator tiles per wave
  __shared__ __attribute__((aligned(16))) char lds[X::BYTES];
  __shared__ int32_t ent_lds[kMaxItemEntries];
  __shared__ __attribute__((aligned(16))) float row_lse2[32];
  __shared__ __attribute__((aligned(16))) float row_d[32];
  __shared__ __attribute__((aligned(16))) int row_pos[32];  // -1 for rows past the item's end
  __shared__ int64_t row_prow[32];                           // dq partial row: (b, i, h) * topk + slot
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
  for (int u = tid; u < nent; u += NTHR) ent_lds[u] = ent[u];

  const int64_t tok_stride = (int64_t)a.Hkv * D;
  const T* kb = static_cast<const T*>(a.k) + (int64_t)b * a.Nk * tok_stride + g * D;
  const T* vb = static_cast<const T*>(a.v) + (int64_t)b * a.Nk * tok_stride + g * D;
  if (tid < 256) {
    KvStage<T, D, BK> st;
    st.load_v(kb, tok_stride, j, a.Nk, tid);
    st.store_vt(lds + X::KT_OFF, tid);
  }
  const int kg = wave;  // key group
  const int64_t key0 = (int64_t)j * BK;
  const bool has_keys = kg * 32 < BK;  // waves past the block's keys stage and form dQ only
  const int kk = kg * 32 + (lane & 31);
  const int64_t my_key = key0 + kk;
  const int64_t kt = min(my_key, (int64_t)a.Nk - 1);  // keys past n_k are masked below
  frag_t<T> kf[D / 16], vf[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    kf[ks] = load8(kb + kt * tok_stride + 8 * half + 16 * ks);
    vf[ks] = load8(vb + kt * tok_stride + 8 * half + 16 * ks);
  }
  f32x16 dkacc[DT], dvacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    dkacc[dt] = f32x16{};
    dvacc[dt] = f32x16{};
  }
  __syncthreads();  // ent_lds
  TileStage<T, D> stg;
  stg.load(a, ent_lds, 0, nrows, b, g, tid);
  stg.template store<BK>(a, ent_lds, 0, b, g, lds, row_lse2, row_d, row_pos, row_prow, tid);
  // Every load so far (the key rows included) has landed: without this the
  // compiler's wait before the first use of kf / vf inside the loop also
  // covers the next tile's fetch, which would then no longer overlap.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  const int ntiles = (nrows + 31) / 32;
  for (int tile = 0; tile < ntiles; ++tile) {
    const bool more = tile + 1 < ntiles;
    if (more) stg.load(a, ent_lds, tile + 1, nrows, b, g, tid);
    const int my_pos = row_pos[lane & 31];
    const int64_t my_prow = row_prow[lane & 31];
    if (has_keys) {
      // S = Q K^T, dP = dO V^T: lane = key, accumulator rows = tile rows
      f32x16 s = f32x16{}, dp = f32x16{};
      const T* qr = reinterpret_cast<const T*>(lds + X::Q_OFF + (lane & 31) * X::RPITCH) + 8 * half;
      const T* dr = reinterpret_cast<const T*>(lds + X::DO_OFF + (lane & 31) * X::RPITCH) + 8 * half;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        mma(load8(qr + 16 * ks), kf[ks], s);
        mma(load8(dr + 16 * ks), vf[ks], dp);
      }
      // P and dS in place; accumulator position e is tile row 8(e/4) + 4h + e%4.
      // The mask is applied only when some row of the tile sits before one of
      // this wave's keys (its local block, or a row past the item's end).
      auto p_ds = [&](auto masked) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int r0 = 8 * q4 + 4 * half;
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(row_lse2 + r0);
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(row_d + r0);
          int4 p4{};
          if constexpr (decltype(masked)::value) p4 = *reinterpret_cast<const int4*>(row_pos + r0);
          const int pp[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int e = 4 * q4 + c;
            const float x = exp2_fast(fmaf(s[e], a.c_log2, -l4[c]));
            float p = x;
            if constexpr (decltype(masked)::value) p = my_key <= pp[c] ? x : 0.f;
            s[e] = p;
            dp[e] = p * (dp[e] - d4[c]);
            *reinterpret_cast<T*>(lds + X::DS_OFF + (r0 + c) * X::SPITCH + kk * (int)sizeof(T)) = from_f32<T>(dp[e]);
          }
        }
      };
      if (__any((int64_t)my_pos < key0 + kg * 32 + 31)) p_ds(std::true_type{});
      else p_ds(std::false_type{});
      // dV += P^T dO, dK += dS^T Q
#pragma unroll
      for (int aa = 0; aa < 2; ++aa) {
        frag_t<T> pa, sa;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pa[e] = from_f32<T>(s[8 * aa + e]);
          sa[e] = from_f32<T>(dp[8 * aa + e]);
        }
#pragma unroll
        for (int i = 0; i < DT; ++i) {
          const int c = 32 * i + (lane & 31);
          mma(pa, tile_t_frag<T, X::TPITCH, X::SWZ>(lds + X::DOT_OFF, c, aa, half), dvacc[i]);
          mma(sa, tile_t_frag<T, X::TPITCH, X::SWZ>(lds + X::QT_OFF, c, aa, half), dkacc[i]);
        }
      }
    }
    __syncthreads();  // dS complete; the tile's rows are no longer read
    if (more) stg.template store<BK>(a, ent_lds, tile + 1, b, g, lds, row_lse2, row_d, row_pos, row_prow, tid);
    if (wave < D / 32) {
      // dQ^T[c][row] = sum over the block's keys of K^T[c][key] dS^T[key][row]
      f32x16 o = f32x16{};
      const int c = 32 * wave + (lane & 31);
      const T* srow = reinterpret_cast<const T*>(lds + X::DS_OFF + (lane & 31) * X::SPITCH);
#pragma unroll
      for (int mt = 0; mt < BK / 32; ++mt)
#pragma unroll
        for (int aa = 0; aa < 2; ++aa) {
          const frag_t<T> ka = vt_frag_at<T, D, BK>(lds + X::KT_OFF, c, mt, aa, half);
          const int k0 = 32 * mt + 16 * aa + 4 * half;
          const typename Pack4<T>::type lo = *reinterpret_cast<const typename Pack4<T>::type*>(srow + k0);
          const typename Pack4<T>::type hi = *reinterpret_cast<const typename Pack4<T>::type*>(srow + k0 + 8);
          frag_t<T> sb;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            sb[e] = lo[e];
            sb[4 + e] = hi[e];
          }
          mma(ka, sb, o);
        }
      if (my_pos >= 0) {
        // o[e]: d = 32 w + 8(e/4) + 4h + e%4 of row lane%32
        T* dst = static_cast<T*>(a.dq_part) + my_prow * D + 32 * wave + 4 * half;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          typename Pack4<T>::type w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = from_f32<T>(o[4 * i + e] * a.scale);
          *reinterpret_cast<typename Pack4<T>::type*>(dst + 8 * i) = w;
        }
      }
    }
    __syncthreads();  // the next tile's rows are in LDS; dS is no longer read
  }
  if (!has_keys) return;
  // Partials of this item: lane holds key 32 kg + 8(e/4) + 4h + e%4,
  // d = 32 i + lane%32.
  T* dst = static_cast<T*>(a.dkv_part) + ((int64_t)bg * a.items_cap + item) * 2 * BK * D;
#pragma unroll
  for (int i = 0; i < DT; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int key = kg * 32 + 8 * (e / 4) + 4 * half + (e % 4);
      const int d = 32 * i + (lane & 31);
      dst[key * D + d] = from_f32<T>(dkacc[i][e] * a.scale);
      dst[BK * D + key * D + d] = from_f32<T>(dvacc[i][e]);
    }
}

// 16-bit inputs: eight waves, where waves w and w + 4 share keys
// [32 (w % 4), +32) and split the work by product rather than by d.  Wave w
// (the P wave) holds the block's K rows, forms S = Q K^T and P, and keeps dV
// for all of d; wave w + 4 (the dS wave) holds the V rows, forms dP = dO V^T,
// takes P from LDS (accumulator layout, fp32), forms dS = P (dP - D) and keeps
// dK for all of d.  Each product is formed once, and each wave holds one set of
// key rows and one set of accumulators.  Waves 0..3 form dQ after each tile
// while waves 4..7 write the next tile's rows, fetched before the products.
template <typename T, int D, int BK>
__global__ void __launch_bounds__(512, 1) k_bwd_split(BwdArgs a) {
  static_assert(sizeof(T) == 2, "the split schedule is laid out for 16-bit inputs");
  using X = FusedLds<T, D, BK>;
  constexpr int DT = D / 32;  // dK or dV accumulator tiles per wave
  __shared__ __attribute__((aligned(16))) char lds[X::BYTES];
  __shared__ int32_t ent_lds[kMaxItemEntries];
  __shared__ __attribute__((aligned(16))) float row_lse2[32];
  __shared__ __attribute__((aligned(16))) float row_d[32];
  __shared__ __attribute__((aligned(16))) int row_pos[32];  // -1 for rows past the item's end
  __shared__ int64_t row_prow[32];                           // dq partial row: (b, i, h) * topk + slot
  __shared__ float pex[4][16][64];                           // P of each key group, [e][lane] of the P wave
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
  for (int u = tid; u < nent; u += 512) ent_lds[u] = ent[u];

  const int64_t tok_stride = (int64_t)a.Hkv * D;
  const T* kb = static_cast<const T*>(a.k) + (int64_t)b * a.Nk * tok_stride + g * D;
  const T* vb = static_cast<const T*>(a.v) + (int64_t)b * a.Nk * tok_stride + g * D;
  if (tid < 256) {
    KvStage<T, D, BK> st;
    st.load_v(kb, tok_stride, j, a.Nk, tid);
    st.store_vt(lds + X::KT_OFF, tid);
  }
  const int kg = wave % 4, role = wave / 4;  // key group; 0 = P wave, 1 = dS wave
  const bool stager = role == 1;
  const int stid = tid - 256;
  const int64_t key0 = (int64_t)j * BK;
  const bool has_keys = kg * 32 < BK;  // waves past the block's keys stage and form dQ only
  const int kk = kg * 32 + (lane & 31);
  const int64_t my_key = key0 + kk;
  const int64_t kt = min(my_key, (int64_t)a.Nk - 1);  // keys past n_k are masked below
  const T* rb = role ? vb : kb;
  frag_t<T> kv[D / 16];  // K rows (P wave) or V rows (dS wave) as B operands
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) kv[ks] = load8(rb + kt * tok_stride + 8 * half + 16 * ks);
  f32x16 acc[DT];  // dV (P wave) or dK (dS wave)
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};
  __syncthreads();  // ent_lds, K^T
  // The P waves (0..3) also form dQ^T = K^T dS^T; their K^T fragments (A
  // operands, columns 32 w.. of d) are the same for every tile of the item.
  frag_t<T> ktf[BK / 32][2];
  if (wave < D / 32) {
#pragma unroll
    for (int mt = 0; mt < BK / 32; ++mt)
#pragma unroll
      for (int aa = 0; aa < 2; ++aa) ktf[mt][aa] = vt_frag_at<T, D, BK>(lds + X::KT_OFF, 32 * wave + (lane & 31), mt, aa, half);
  }
  TileStage<T, D> stg;
  if (stager) {
    stg.load(a, ent_lds, 0, nrows, b, g, stid);
    stg.template store<BK>(a, ent_lds, 0, b, g, lds, row_lse2, row_d, row_pos, row_prow, stid);
  }
  // Every load so far (the key rows included) has landed: without this the
  // compiler's wait before the first use of kv inside the loop also covers
  // the next tile's fetch, which would then no longer overlap.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  const int ntiles = (nrows + 31) / 32;
  for (int tile = 0; tile < ntiles; ++tile) {
    const bool more = tile + 1 < ntiles;
    if (more && stager) stg.load(a, ent_lds, tile + 1, nrows, b, g, stid);
    const int my_pos = row_pos[lane & 31];
    const int64_t my_prow = row_prow[lane & 31];
    // S = Q K^T (P wave) or dP = dO V^T (dS wave): lane = key, accumulator rows = tile rows
    f32x16 xs = f32x16{};
    if (has_keys) {
      const T* xr = reinterpret_cast<const T*>(lds + (role ? X::DO_OFF : X::Q_OFF) + (lane & 31) * X::RPITCH) + 8 * half;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) mma(load8(xr + 16 * ks), kv[ks], xs);
      if (role == 0) {
        // P in place; accumulator position e is tile row 8(e/4) + 4h + e%4.
        // The mask is applied only when some row of the tile sits before one
        // of this wave's keys (its local block, or a row past the item's end).
        auto p_of = [&](auto masked) {
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int r0 = 8 * q4 + 4 * half;
            const f32x4 l4 = *reinterpret_cast<const f32x4*>(row_lse2 + r0);
            int4 p4{};
            if constexpr (decltype(masked)::value) p4 = *reinterpret_cast<const int4*>(row_pos + r0);
            const int pp[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              const int e = 4 * q4 + c;
              const float x = exp2_fast(fmaf(xs[e], a.c_log2, -l4[c]));
              float p = x;
              if constexpr (decltype(masked)::value) p = my_key <= pp[c] ? x : 0.f;
              xs[e] = p;
              pex[kg][e][lane] = p;
            }
          }
        };
        if (__any((int64_t)my_pos < key0 + kg * 32 + 31)) p_of(std::true_type{});
        else p_of(std::false_type{});
      }
    }
    __syncthreads();  // P of every key group is in LDS
    if (has_keys) {
      if (role == 1) {
        // dS = P (dP - D) in place, and to LDS as [row][key] for dQ
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int r0 = 8 * q4 + 4 * half;
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(row_d + r0);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int e = 4 * q4 + c;
            xs[e] = pex[kg][e][lane] * (xs[e] - d4[c]);
            *reinterpret_cast<T*>(lds + X::DS_OFF + (r0 + c) * X::SPITCH + kk * (int)sizeof(T)) = from_f32<T>(xs[e]);
          }
        }
      }
      // dV += P^T dO (P wave), dK += dS^T Q (dS wave)
      const char* tt = lds + (role ? X::QT_OFF : X::DOT_OFF);
#pragma unroll
      for (int aa = 0; aa < 2; ++aa) {
        frag_t<T> xa;
#pragma unroll
        for (int e = 0; e < 8; ++e) xa[e] = from_f32<T>(xs[8 * aa + e]);
#pragma unroll
        for (int i = 0; i < DT; ++i)
          mma(xa, tile_t_frag<T, X::TPITCH, X::SWZ>(tt, 32 * i + (lane & 31), aa, half), acc[i]);
      }
    }
    __syncthreads();  // dS complete; the tile's rows and P are no longer read
    if (more && stager) stg.template store<BK>(a, ent_lds, tile + 1, b, g, lds, row_lse2, row_d, row_pos, row_prow, stid);
    if (wave < D / 32) {
      // dQ^T[c][row] = sum over the block's keys of K^T[c][key] dS^T[key][row]
      f32x16 o = f32x16{};
      const int c = 32 * wave + (lane & 31);
      const T* srow = reinterpret_cast<const T*>(lds + X::DS_OFF + (lane & 31) * X::SPITCH);
#pragma unroll
      for (int mt = 0; mt < BK / 32; ++mt)
#pragma unroll
        for (int aa = 0; aa < 2; ++aa) {
          const frag_t<T> ka = ktf[mt][aa];
          const int k0 = 32 * mt + 16 * aa + 4 * half;
          const typename Pack4<T>::type lo = *reinterpret_cast<const typename Pack4<T>::type*>(srow + k0);
          const typename Pack4<T>::type hi = *reinterpret_cast<const typename Pack4<T>::type*>(srow + k0 + 8);
          frag_t<T> sb;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            sb[e] = lo[e];
            sb[4 + e] = hi[e];
          }
          mma(ka, sb, o);
        }
      if (my_pos >= 0) {
        // o[e]: d = 32 w + 8(e/4) + 4h + e%4 of row lane%32
        T* dst = static_cast<T*>(a.dq_part) + my_prow * D + 32 * wave + 4 * half;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          typename Pack4<T>::type w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = from_f32<T>(o[4 * i + e] * a.scale);
          *reinterpret_cast<typename Pack4<T>::type*>(dst + 8 * i) = w;
        }
      }
    }
    __syncthreads();  // the next tile's rows are in LDS; dS is no longer read
  }
  if (!has_keys) return;
  // Partials of this item: lane holds key 32 kg + 8(e/4) + 4h + e%4, d = 32 i + lane%32.
  T* dst = static_cast<T*>(a.dkv_part) + ((int64_t)bg * a.items_cap + item) * 2 * BK * D + (role ? 0 : BK * D);
  const float f = role ? a.scale : 1.f;
#pragma unroll
  for (int i = 0; i < DT; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int key = kg * 32 + 8 * (e / 4) + 4 * half + (e % 4);
      dst[key * D + 32 * i + (lane & 31)] = from_f32<T>(acc[i][e] * f);
    }
}

// ---- dq = sum of the slot partials, in slot order ---------------------------
template <typename T, int D>
__global__ void __launch_bounds__(256) k_bwd_dq_sum(const T* __restrict__ part, const int32_t* __restrict__ ids,
                                                    T* __restrict__ dq, int Hq, int Hkv, int G, int topk,
                                                    int nblk, int64_t nrows) {
  constexpr int LPR = D / 8;
  const int lane = threadIdx.x & 63;
  const int64_t row = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * (64 / LPR) + lane / LPR;  // (b, i, h)
  if (row >= nrows) return;
  const int h = (int)(row % Hq);
  const int64_t bi = row / Hq;
  const int32_t* sel = ids + (bi * Hkv + h / G) * topk;
  const T* p = part + row * topk * D + (lane % LPR) * 8;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  // Sixteen slots per round, all their loads issued before any is used (a
  // slot past topk re-reads the last one, an unselected slot is read and not
  // added); the sum runs in slot order.  Partials are read exactly once, so
  // the loads are non-temporal.
  // The slot ids are read four per load where a row of them is 16-byte
  // aligned (topk a multiple of 4).
  constexpr int RND = 16;
  for (int s0 = 0; s0 < topk; s0 += RND) {
    int idv[RND];
    if ((topk & 3) == 0) {
#pragma unroll
      for (int q = 0; q < RND / 4; ++q) {
        const int4 t = s0 + 4 * q < topk ? *reinterpret_cast<const int4*>(sel + s0 + 4 * q) : int4{-1, -1, -1, -1};
        idv[4 * q] = t.x;
        idv[4 * q + 1] = t.y;
        idv[4 * q + 2] = t.z;
        idv[4 * q + 3] = t.w;
      }
    } else {
#pragma unroll
      for (int u = 0; u < RND; ++u) idv[u] = s0 + u < topk ? sel[s0 + u] : -1;
    }
    frag_t<T> x[RND];
    bool ok[RND];
#pragma unroll
    for (int u = 0; u < RND; ++u) {
      const int sl = min(s0 + u, topk - 1);
      ok[u] = (unsigned)idv[u] < (unsigned)nblk;  // slots past topk and ids outside [0, nblk) have no partial
      x[u] = __builtin_nontemporal_load(reinterpret_cast<const frag_t<T>*>(p + (int64_t)sl * D));
    }
#pragma unroll
    for (int u = 0; u < RND; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = ok[u] ? acc[e] + to_f32(x[u][e]) : acc[e];
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

// ---- dk, dv = sum of the item partials of each block, in item order ---------
// One thread per (token of the block, 8 channels); blocks no query selected
// (and tokens no query can see) get zeros.
template <typename T, int D, int BK>
__global__ void __launch_bounds__(256) k_bwd_dkdv_reduce(const T* __restrict__ part, const int4* __restrict__ items,
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
    const T* p = part + ((int64_t)bg * items_cap + u) * 2 * BK * D + tk * D + c * 8;
    const frag_t<T> xk = load8(p), xv = load8(p + BK * D);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ak[e] += to_f32(xk[e]);
      av[e] += to_f32(xv[e]);
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
                   hipStream_t st, int kid_main, int kid_sum, int kid_red) {
  const dim3 grid(p.items_cap, s.B * s.Hkv);
  prof_begin(st, kid_main);
  if constexpr (sizeof(T) == 2) hipLaunchKernelGGL((k_bwd_split<T, D, BK>), grid, dim3(512), 0, st, a);
  else hipLaunchKernelGGL((k_bwd_fused<T, D, BK>), grid, dim3(256), 0, st, a);
  prof_end(st, kid_main);
  const int64_t nrows = (int64_t)s.B * s.Nq * s.Hq;
  const int rpb = 4 * (64 / (D / 8));
  prof_begin(st, kid_sum);
  hipLaunchKernelGGL((k_bwd_dq_sum<T, D>), dim3((unsigned)((nrows + rpb - 1) / rpb)), dim3(256), 0, st,
                     static_cast<const T*>(a.dq_part), static_cast<const int32_t*>(ids), static_cast<T*>(dq), s.Hq,
                     s.Hkv, s.Hq / s.Hkv, s.topk, s.nblk, nrows);
  prof_end(st, kid_sum);
  const int64_t nthr = (int64_t)s.nblk * BK * (D / 8);
  prof_begin(st, kid_red);
  hipLaunchKernelGGL((k_bwd_dkdv_reduce<T, D, BK>), dim3((unsigned)((nthr + 255) / 256), s.B * s.Hkv), dim3(256), 0,
                     st, static_cast<const T*>(a.dkv_part), a.items, a.item_count, static_cast<T*>(dk), static_cast<T*>(dv), s.Nk, s.Hkv,
                     s.nblk, p.items_cap);
  prof_end(st, kid_red);
}

template <typename T, int D>
void bwd_launch(const Shape& s, const BwdArgs& a, const InvertPlan& p, const void* ids, void* dq, void* dk, void* dv,
                hipStream_t st, int k1, int k2, int k3) {
  if (s.Bk == 32) bwd_launch_bk<T, D, 32>(s, a, p, ids, dq, dk, dv, st, k1, k2, k3);
  else if (s.Bk == 64) bwd_launch_bk<T, D, 64>(s, a, p, ids, dq, dk, dv, st, k1, k2, k3);
  else bwd_launch_bk<T, D, 128>(s, a, p, ids, dq, dk, dv, st, k1, k2, k3);
}

}  // namespace

size_t bwd_dkv_bytes(const Shape& s, const InvertPlan& p) {
  return (size_t)s.B * s.Hkv * p.items_cap * 2 * s.Bk * s.D * (s.dtype == kBF16 ? 2 : 4);  // in the input type
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
                                const InvertOut& inv, void* dq_part, void* dkv_part, void* trash, void* dq, void* dk,
                                void* dv, hipStream_t st) {
  static const int k1 = prof_register("bwd_fused");
  static const int k2 = prof_register("bwd_dq_sum");
  static const int k3 = prof_register("bwd_dkdv_reduce");
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
    if (s.D == 64) bwd_launch<bf16_t, 64>(s, a, p, ids, dq, dk, dv, st, k1, k2, k3);
    else bwd_launch<bf16_t, 128>(s, a, p, ids, dq, dk, dv, st, k1, k2, k3);
  } else {
    if (s.D == 64) bwd_launch<float, 64>(s, a, p, ids, dq, dk, dv, st, k1, k2, k3);
    else bwd_launch<float, 128>(s, a, p, ids, dq, dk, dv, st, k1, k2, k3);
  }
  return hipGetLastError();
}

}  // namespace msa
