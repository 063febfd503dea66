// attn_common.h -- device helpers shared by the Main Branch kernels (forward
// attention in attention.hip, gradients in backward.hip): LDS staging of one
// key block (rows and transposed rows), MFMA fragment reads of the transposed
// block, the gathered query rows of a KV-outer work item, partial stores.
#pragma once

#include "msa_device.h"
#include "msa_internal.h"

namespace msa {
namespace {

template <typename T> struct Pack4;
template <> struct Pack4<bf16_t> { using type = bf16x4; };
template <> struct Pack4<float> { using type = f32x4; };

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) { return static_cast<bf16_t>(x); }
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }

// Eight elements to (16-byte aligned) memory.
__device__ __forceinline__ void store8(bf16_t* p, const bf16x8& v) { *reinterpret_cast<bf16x8*>(p) = v; }
__device__ __forceinline__ void store8(float* p, const f32x8& v) {
  *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
  *reinterpret_cast<f32x4*>(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
}

// LDS geometry of one staged key block of BK tokens: K row-major [BK][D], V
// transposed [D][BK].  Pitches are padded so the 32 rows read by a half-wave
// fall on distinct banks.
template <typename T, int D, int BK>
struct KvLds {
  static constexpr int KPITCH = D * (int)sizeof(T) + 16;
  static constexpr int VPITCH = BK * (int)sizeof(T) + (sizeof(T) == 2 ? 8 : 16);
  static constexpr int KBYTES = BK * KPITCH;
  static constexpr int BYTES = KBYTES + D * VPITCH;
  // Byte offset of keys [4c, 4c+4) in V^T row d.  For 16-bit types the
  // 4-key chunks are XOR-swizzled by (d / 32) % 4: the staging stores write
  // rows 8 apart from neighbouring lanes, which would otherwise share banks;
  // the MFMA fragment reads take 32 consecutive rows, which share the swizzle.
  __device__ static __forceinline__ int vt_off(int d, int c) {
    if constexpr (sizeof(T) == 2) return d * VPITCH + ((c ^ ((d >> 5) & 3)) * 4 * (int)sizeof(T));
    else return d * VPITCH + c * 4 * (int)sizeof(T);
  }
};

// Staging of K_j and V_j^T of one (b, g) into LDS by 256 threads, split into
// a global-load phase (into registers) and an LDS-store phase so that callers
// can overlap other loads with it.  Rows past n_k are zero-filled (they are
// masked anyway).
template <typename T, int D, int BK>
struct KvStage {
  using L = KvLds<T, D, BK>;
  static constexpr int CPR = D * (int)sizeof(T) / 16;  // 16-byte chunks per K row
  static constexpr int KCH = BK * CPR;
  static constexpr int KLD = (KCH + 255) / 256;
  static constexpr int DCH = D / 8;         // 8-element chunks per V row
  static constexpr int KG = 256 / DCH;      // groups of 4 keys per pass
  static constexpr int PASSES = (BK + 4 * KG - 1) / (4 * KG);  // the last pass may be partial
  u32x4 kr[KLD];
  frag_t<T> vr[PASSES][4];

  __device__ __forceinline__ void load(const T* kbase, const T* vbase, int64_t tok_stride, int j, int n_k, int tid) {
    load_k(kbase, tok_stride, j, n_k, tid);
    load_v(vbase, tok_stride, j, n_k, tid);
  }
  __device__ __forceinline__ void load_k(const T* kbase, int64_t tok_stride, int j, int n_k, int tid) {
#pragma unroll
    for (int u = 0; u < KLD; ++u) {
      const int c = tid + u * 256;
      const int row = c / CPR, col = c % CPR;
      const int64_t t = (int64_t)j * BK + row;
      kr[u] = u32x4{};
      if (c < KCH && t < n_k)
        kr[u] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(kbase + t * tok_stride) + col * 16);
    }
  }
  __device__ __forceinline__ void load_v(const T* vbase, int64_t tok_stride, int j, int n_k, int tid) {
    const int dch = tid % DCH, kg = tid / DCH;
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = (ps * KG + kg) * 4 + r;
        const int64_t t = (int64_t)j * BK + key;
        vr[ps][r] = key < BK && t < n_k ? load8(vbase + t * tok_stride + dch * 8) : zero_frag<T>();
      }
  }

  // V^T rows get four consecutive keys per store.
  __device__ __forceinline__ void store(char* lds, int tid) const {
    store_k(lds, tid);
    store_vt(lds + L::KBYTES, tid);
  }
  // The key rows alone, at lds (BK rows of KPITCH bytes).
  __device__ __forceinline__ void store_k(char* lds, int tid) const {
#pragma unroll
    for (int u = 0; u < KLD; ++u) {
      const int c = tid + u * 256;
      if (c < KCH) *reinterpret_cast<u32x4*>(lds + (c / CPR) * L::KPITCH + (c % CPR) * 16) = kr[u];
    }
  }
  // The transposed rows alone, at vt (D rows of VPITCH bytes).
  __device__ __forceinline__ void store_vt(char* vt, int tid) const {
    const int dch = tid % DCH, kg = tid / DCH;
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
      const int key0 = (ps * KG + kg) * 4;
      if (key0 >= BK) continue;  // a partial last pass (blocks smaller than 4 * KG keys)
      if constexpr (sizeof(T) == 2) {
        // 2x2 transposes of 16-bit halves with byte permutes (v_perm_b32).
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          uint32_t x0 = __builtin_bit_cast(u32x4, vr[ps][0])[w], x1 = __builtin_bit_cast(u32x4, vr[ps][1])[w];
          uint32_t x2 = __builtin_bit_cast(u32x4, vr[ps][2])[w], x3 = __builtin_bit_cast(u32x4, vr[ps][3])[w];
          const uint2 lo = make_uint2(__builtin_amdgcn_perm(x1, x0, 0x05040100u), __builtin_amdgcn_perm(x3, x2, 0x05040100u));
          const uint2 hi = make_uint2(__builtin_amdgcn_perm(x1, x0, 0x07060302u), __builtin_amdgcn_perm(x3, x2, 0x07060302u));
          *reinterpret_cast<uint2*>(vt + L::vt_off(dch * 8 + 2 * w, key0 / 4)) = lo;
          *reinterpret_cast<uint2*>(vt + L::vt_off(dch * 8 + 2 * w + 1, key0 / 4)) = hi;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          typename Pack4<T>::type w;
          w[0] = vr[ps][0][e];
          w[1] = vr[ps][1][e];
          w[2] = vr[ps][2][e];
          w[3] = vr[ps][3][e];
          *reinterpret_cast<typename Pack4<T>::type*>(vt + L::vt_off(dch * 8 + e, key0 / 4)) = w;
        }
      }
    }
  }
};

// The same staging from MXFP8 K and V caches (OCP MX v1.0: E4M3 codes, one
// E8M0 scale byte per 32 elements of a row).  The loads keep the codes and
// scale bytes; the stores decode them exactly (fp8 conversion, then a power
// of two) into the dtype layout of KvLds, so the products are unchanged.
// kc / vc: code rows (D bytes) and ks / vs: scale rows (D/32 bytes) of this
// (b, g) at token strides of cstride / cstride/32 bytes.
template <typename T, int D, int BK>
struct KvStageMx {
  using L = KvLds<T, D, BK>;
  static constexpr int KT = BK * (D / 16);  // K tasks: 16 codes of one row
  static constexpr int KLD = (KT + 255) / 256;
  static constexpr int DCH = D / 8;
  static constexpr int KG = 256 / DCH;
  static constexpr int PASSES = (BK + 4 * KG - 1) / (4 * KG);
  u32x4 kc[KLD];
  uint32_t ksc[KLD];
  uint2 vc[PASSES][4];
  uint32_t vsc[PASSES][4];

  __device__ __forceinline__ void load(const uint8_t* kcb, const uint8_t* vcb, const uint8_t* ksb,
                                       const uint8_t* vsb, int64_t cstride, int j, int n_k, int tid) {
    const int64_t sstride = cstride / 32;
#pragma unroll
    for (int u = 0; u < KLD; ++u) {
      const int c = tid + u * 256;
      const int row = c / (D / 16), col = c % (D / 16);
      const int64_t t = (int64_t)j * BK + row;
      kc[u] = u32x4{};
      ksc[u] = 127;
      if (c < KT && t < n_k) {
        kc[u] = *reinterpret_cast<const u32x4*>(kcb + t * cstride + col * 16);
        ksc[u] = ksb[t * sstride + col / 2];
      }
    }
    const int dch = tid % DCH, kg = tid / DCH;
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = (ps * KG + kg) * 4 + r;
        const int64_t t = (int64_t)j * BK + key;
        vc[ps][r] = make_uint2(0, 0);
        vsc[ps][r] = 127;
        if (key < BK && t < n_k) {
          vc[ps][r] = *reinterpret_cast<const uint2*>(vcb + t * cstride + dch * 8);
          vsc[ps][r] = vsb[t * sstride + dch / 4];
        }
      }
  }

  __device__ __forceinline__ void store(char* lds, int tid) const {
#pragma unroll
    for (int u = 0; u < KLD; ++u) {
      const int c = tid + u * 256;
      if (c >= KT) continue;
      const int row = c / (D / 16), col = c % (D / 16);
      float f[16];
      e4m3_decode16(kc[u], f);
      const int sh = (int)ksc[u] - 127;
      T* dst = reinterpret_cast<T*>(lds + row * L::KPITCH) + col * 16;
      frag_t<T> lo, hi;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        lo[e] = from_f32<T>(__builtin_ldexpf(f[e], sh));
        hi[e] = from_f32<T>(__builtin_ldexpf(f[8 + e], sh));
      }
      store8(dst, lo);
      store8(dst + 8, hi);
    }
    KvStage<T, D, BK> tmp;  // V^T through the plain stager's transposing store
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float f[8];
        e4m3_decode8(vc[ps][r], f);
        const int sh = (int)vsc[ps][r] - 127;
#pragma unroll
        for (int e = 0; e < 8; ++e) tmp.vr[ps][r][e] = from_f32<T>(__builtin_ldexpf(f[e], sh));
      }
    tmp.store_vt(lds + L::KBYTES, tid);
  }
};

template <typename T, int D, int BK>
__device__ __forceinline__ void stage_kv(char* lds, const T* kbase, const T* vbase, int64_t tok_stride, int j,
                                         int n_k, int tid) {
  KvStage<T, D, BK> st;
  st.load(kbase, vbase, tok_stride, j, n_k, tid);
  st.store(lds, tid);
}

// A fragment of V^T for k-step (mt, a): row d, keys 32mt+16a+4h+[0..3] and +8.
template <typename T, int D, int BK>
__device__ __forceinline__ frag_t<T> vt_frag_at(const char* vt, int d, int mt, int a, int half) {
  using L = KvLds<T, D, BK>;
  const int c0 = 8 * mt + 4 * a + half;  // chunk of keys 32mt+16a+4h .. +3
  const typename Pack4<T>::type lo = *reinterpret_cast<const typename Pack4<T>::type*>(vt + L::vt_off(d, c0));
  const typename Pack4<T>::type hi = *reinterpret_cast<const typename Pack4<T>::type*>(vt + L::vt_off(d, c0 + 2));
  frag_t<T> f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[e] = lo[e];
    f[4 + e] = hi[e];
  }
  return f;
}
template <typename T, int D, int BK>
__device__ __forceinline__ frag_t<T> vt_frag(const char* lds, int d, int mt, int a, int half) {
  return vt_frag_at<T, D, BK>(lds + KvLds<T, D, BK>::KBYTES, d, mt, a, half);
}


// Position of the 4-row chunk q (rows 4q..4q+3) in column c of a transposed
// 32-row tile.  With SWZ (16-bit types) the chunks of columns 32 apart are
// XOR-permuted by ((c / 32) % 4) * 2: the staging stores write columns 8
// apart from neighbouring lanes, which would otherwise fall on 4 banks per
// 64; the fragment reads take 32 consecutive columns, which share the swizzle.
template <bool SWZ>
__device__ __forceinline__ int tile_t_chunk(int c, int q) {
  return SWZ ? q ^ (((c >> 5) & 3) << 1) : q;
}

// A fragment of a transposed 32-row tile (rows of TPITCH bytes, one per
// column) for k-step a: column c, tile rows 16a + 4h + [0..3] and
// 16a + 8 + 4h + [0..3] -- the order of an accumulator's rows, so that a
// product whose other operand comes straight from an accumulator lines up.
template <typename T, int TPITCH, bool SWZ = false>
__device__ __forceinline__ frag_t<T> tile_t_frag(const char* base, int c, int a, int half) {
  static_assert(!SWZ || sizeof(T) == 2, "the chunk swizzle is laid out for 16-bit tiles");
  const T* row = reinterpret_cast<const T*>(base + c * TPITCH);
  const int q0 = 4 * a + half;
  const typename Pack4<T>::type lo = *reinterpret_cast<const typename Pack4<T>::type*>(row + 4 * tile_t_chunk<SWZ>(c, q0));
  const typename Pack4<T>::type hi =
      *reinterpret_cast<const typename Pack4<T>::type*>(row + 4 * tile_t_chunk<SWZ>(c, q0 + 2));
  frag_t<T> f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[e] = lo[e];
    f[4 + e] = hi[e];
  }
  return f;
}

// Query rows of one 32-row tile of a KV-outer work item.
struct TileRows {
  bool valid;
  int qq, slot, h;
};
// e = qq*topk + slot is split with a multiply by ceil(2^40/topk): exact for
// 0 <= e < 2^31 and topk <= 32 (the rounding error stays below 2^-9 < 1/topk).
__device__ __forceinline__ TileRows rows_of(int e, bool valid, int r, int gshift, int topk, uint64_t topk_magic,
                                           int g) {
  TileRows t;
  t.valid = valid;
  t.qq = (int)(((uint64_t)(uint32_t)e * topk_magic) >> 40);
  t.slot = e - t.qq * topk;
  t.h = (g << gshift) + (r & ((1 << gshift) - 1));
  return t;
}
// A work item holds at most min(kItemRows / G, kItemEntries) entries.
constexpr int kMaxItemEntries = kItemEntries;
// Rows past the item's end read a valid row (entry 0 of the chunk): their
// results are never stored, so no branch is needed around the loads.
template <typename T, int D>
__device__ __forceinline__ void load_q_rows(frag_t<T> (&qf)[D / 16], const T* qbase, const TileRows& t, int b, int Nq,
                                            int Hq, int q0, int half) {
  const T* qrow = qbase + (((int64_t)b * Nq + q0 + t.qq) * Hq + t.h) * D + 8 * half;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) qf[ks] = load8(qrow + 16 * ks);
}
// Partial store.  A partial is written once and read back only by the
// combine.  With NT the store is marked non-temporal, which keeps partials
// from displacing the query rows that other blocks of the same queries re-read
// from the caches: measured faster where work items are full (many rows per
// staged block), slower where most items are small and the staging of K/V
// dominates, so the launcher chooses.  Every partial store writes whole rows
// or whole runs of lse values (partial-line non-temporal writes measured
// several times slower than plain ones).
template <bool NT, typename V>
__device__ __forceinline__ void store_partial(V* p, const V& v) {
  if constexpr (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

}  // namespace
}  // namespace msa
