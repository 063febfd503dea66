// msa_device.h -- device-side building blocks shared by the MSA kernels
// (gfx950 / CDNA4, wave64).
//
// MFMA operand layout used throughout (v_mfma_f32_32x32x16_bf16, and eight
// v_mfma_f32_32x32x2_f32 issued back to back for fp32 inputs):
//   A (32 x 16): lane l holds row l%32, k = 8*(l/32) + e, e = 0..7
//   B (16 x 32): lane l holds col l%32, k = 8*(l/32) + e
//   C (32 x 32): lane l holds col l%32, rows 8*(e/4) + 4*(l/32) + e%4, e = 0..15
// For fp32 the eight 32x32x2 steps take element e of A and B in step e; any
// fixed assignment of the 16 k-values works as long as A and B agree.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

typedef __bf16 bf16_t;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(8 * sizeof(float)))) float f32x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

constexpr int kChunk = 128;     // tokens per key chunk the index kernels stage at a time
constexpr int kMaxBk = 128;     // largest key block size (block sizes 32, 64, 128 divide a chunk)
constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <typename T> struct FragOf;
template <> struct FragOf<bf16_t> { using type = bf16x8; };
template <> struct FragOf<float> { using type = f32x8; };
// Eight consecutive k-values of one MFMA operand row/column.
template <typename T> using frag_t = typename FragOf<T>::type;

__device__ __forceinline__ void mma(const bf16x8& a, const bf16x8& b, f32x16& c) {
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ void mma(const f32x8& a, const f32x8& b, f32x16& c) {
#pragma unroll
  for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], b[e], c, 0, 0, 0);
}

// Product with a zero accumulator (no register zeroing needed).
__device__ __forceinline__ f32x16 mma0(const bf16x8& a, const bf16x8& b) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, f32x16{}, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mma0(const f32x8& a, const f32x8& b) {
  f32x16 c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[0], b[0], f32x16{}, 0, 0, 0);
#pragma unroll
  for (int e = 1; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], b[e], c, 0, 0, 0);
  return c;
}

// 8 elements from a 16-byte aligned address (global or LDS).
__device__ __forceinline__ bf16x8 load8(const bf16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ f32x8 load8(const float* p) {
  const f32x4 lo = *reinterpret_cast<const f32x4*>(p);
  const f32x4 hi = *reinterpret_cast<const f32x4*>(p + 4);
  return f32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
template <typename T> __device__ __forceinline__ frag_t<T> zero_frag() { return frag_t<T>{}; }

__device__ __forceinline__ float to_f32(bf16_t x) { return static_cast<float>(x); }
__device__ __forceinline__ float to_f32(float x) { return x; }

// Hardware base-2 exponential / logarithm (v_exp_f32, v_log_f32).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// s_waitcnt immediate: wait until at most N vector-memory operations of this
// wave are outstanding (expcnt and lgkmcnt left at their maximum).  Loads
// complete in issue order, so after it every load but the N most recent has
// landed, whatever stores are still in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// Running max over 16 values as a chain of three-input maxima (v_max3_f32).
__device__ __forceinline__ float max16(const f32x16& v, float m = -__builtin_huge_valf()) {
#pragma unroll
  for (int e = 0; e < 16; e += 2) m = fmaxf(fmaxf(m, v[e]), v[e + 1]);
  return m;
}

// Sixteen OCP E4M3 codes (one 16-byte chunk, little-endian bytes) decoded
// exactly to fp32 by the hardware conversion (which follows the OCP encoding
// on gfx950: checked against a reference table of all 256 codes).
__device__ __forceinline__ void e4m3_decode16(const u32x4& c, float (&out)[16]) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[w], false);
    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[w], true);
    out[4 * w + 0] = lo[0];
    out[4 * w + 1] = lo[1];
    out[4 * w + 2] = hi[0];
    out[4 * w + 3] = hi[1];
  }
}

// Eight E4M3 codes (8 bytes, little-endian) decoded exactly to fp32.
__device__ __forceinline__ void e4m3_decode8(const uint2& c, float (&out)[8]) {
  const uint32_t w[2] = {c.x, c.y};
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], false);
    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], true);
    out[4 * i + 0] = lo[0];
    out[4 * i + 1] = lo[1];
    out[4 * i + 2] = hi[0];
    out[4 * i + 3] = hi[1];
  }
}

// Lanes of one wave that exchange data through LDS without a workgroup
// barrier must separate the writes from the reads with this: the wave runs in
// lockstep and LDS accesses of one wave complete in order, but without a fence
// the compiler may treat another lane's write as invisible and move or forward
// the read (a wavefront-scope fence costs nothing in hardware).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float xor_shfl(float v, int mask) { return __shfl_xor(v, mask, kWave); }
__device__ __forceinline__ int xor_shfl(int v, int mask) { return __shfl_xor(v, mask, kWave); }

// v of lanes l and l ^ 32 as (lower-half lane's, upper-half lane's), from one
// v_permlane32_swap: lane l < 32 gets (v[l], v[l + 32]), lane l >= 32 gets
// (v[l - 32], v[l]), with no LDS round trip (a shuffle through ds_bpermute
// would also make the next LDS wait cover every LDS read in flight).  Both
// lanes of a pair see the same pair in the same order, so a sum of the two
// is bitwise equal on both.
__device__ __forceinline__ float2 lane_pair32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair32_max(float v) {
  const float2 p = lane_pair32(v);
  return fmaxf(p.x, p.y);
}
__device__ __forceinline__ float pair32_sum(float v) {
  const float2 p = lane_pair32(v);
  return p.x + p.y;
}

// Sum over aligned groups of C lanes (C in {1, 2, 4, 8, 16}); every lane of a
// group gets the group's total.  DPP lane moves within rows of 16 lanes (no
// LDS): swap neighbours, swap lane pairs, then add the mirror image within 8
// and within 16 lanes -- the mirror of a lane lies in the other half of its
// group, whose total it already holds, and both lanes add the same two values.
template <int C>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(C == 1 || C == 2 || C == 4 || C == 8 || C == 16, "groups of 1..16 lanes");
  if constexpr (C >= 2) v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
  if constexpr (C >= 4) v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));
  if constexpr (C >= 8) v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, true));
  if constexpr (C >= 16) v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, true));
  return v;
}

// Per-lane list of the KMAX best (score, block id) pairs seen so far, best
// first; order = score descending, id ascending.  Ids must be offered in
// increasing order, so a newcomer only passes an entry with a strictly lower
// score (equal scores keep the earlier, lower id in front).  Empty slots hold
// (-inf, INT32_MAX); only finite scores are ever admitted.
template <int KMAX>
struct TopList {
  float s[KMAX];
  int j[KMAX];

  __device__ __forceinline__ void init() {
#pragma unroll
    for (int p = 0; p < KMAX; ++p) {
      s[p] = -__builtin_huge_valf();
      j[p] = INT32_MAX;
    }
  }

  __device__ __forceinline__ void offer(float x, int id) {
    if (x > s[KMAX - 1]) {
      s[KMAX - 1] = x;
      j[KMAX - 1] = id;
#pragma unroll
      for (int p = KMAX - 1; p > 0; --p) {
        const bool up = s[p] > s[p - 1];
        const float ts = s[p], tp = s[p - 1];
        const int js = j[p], jp = j[p - 1];
        s[p - 1] = up ? ts : tp;
        s[p] = up ? tp : ts;
        j[p - 1] = up ? js : jp;
        j[p] = up ? jp : js;
      }
    }
  }

  // Drop the front entry (used by the wave-level merge).
  __device__ __forceinline__ void pop() {
#pragma unroll
    for (int p = 0; p < KMAX - 1; ++p) {
      s[p] = s[p + 1];
      j[p] = j[p + 1];
    }
    s[KMAX - 1] = -__builtin_huge_valf();
    j[KMAX - 1] = INT32_MAX;
  }
};

// Sort N ints ascending in registers (bitonic network; N a power of two).
template <int N>
__device__ __forceinline__ void sort_asc(int (&a)[N]) {
#pragma unroll
  for (int size = 2; size <= N; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const int p = i ^ stride;
        if (p > i) {
          const bool asc = (i & size) == 0;
          const int x = a[i], y = a[p];
          const bool sw = asc ? (x > y) : (x < y);
          a[i] = sw ? y : x;
          a[p] = sw ? x : y;
        }
      }
    }
  }
}

// Write one selection row: the first `nsel` (<= k-1) ids of `cand` (KMAX
// entries; unused ones are INT32_MAX), then the local block L, then -1 up to
// topk.  `cand` is sorted here.  All candidate ids are < L.
// The lists admit finite scores only (-inf and NaN never pass the -inf of an
// empty slot), so a row with fewer than nsel finite scores comes with missing
// picks; they go to the lowest candidate ids not yet picked -- the order that
// puts -inf (and NaN, ranked with it) below every finite score, ties to the
// lower id.
template <int KMAX>
__device__ __forceinline__ void write_selection(int (&cand)[KMAX], int nsel, int L, int topk, int32_t* out) {
#pragma unroll
  for (int p = 0; p < KMAX; ++p)
    if (p >= nsel) cand[p] = INT32_MAX;
  sort_asc<KMAX>(cand);
  int nv = 0;
#pragma unroll
  for (int p = 0; p < KMAX; ++p) nv += cand[p] != INT32_MAX ? 1 : 0;
  if (nv < nsel) {
    // The f-th smallest id outside the sorted picks: start at f and step past
    // every pick at or below the running value (missing picks are INT32_MAX
    // and never step).
    int fill[KMAX];
#pragma unroll
    for (int p = 0; p < KMAX; ++p) {
      int c = p - nv;
#pragma unroll
      for (int q = 0; q < KMAX; ++q) c += cand[q] <= c ? 1 : 0;
      fill[p] = p >= nv && p < nsel ? c : cand[p];
    }
#pragma unroll
    for (int p = 0; p < KMAX; ++p) cand[p] = fill[p];
    sort_asc<KMAX>(cand);
  }
#pragma unroll
  for (int p = 0; p <= KMAX; ++p) {
    if (p < topk) {
      int v = -1;
      if (p < nsel) v = cand[p < KMAX ? p : KMAX - 1];
      else if (p == nsel) v = L;
      out[p] = v;
    }
  }
}

}  // namespace msa
