// index.hip -- Index Branch of MiniMax Sparse Attention on gfx950.
//
// Block score of key block j for query i of GQA group g (paper summary page,
// "Method"; zhichai.net write-up, section 2: one index-q and one index-k head
// per group):
//     S[b,g,i,j] = max_{t in block j} <idx_q[b,i,g,:], idx_k[b,t,g,:]>
// for the candidate blocks j < L(i) = floor((q_offset + i) / 128), followed by
// an exp-free Top-(k-1) that always adds the local block L(i) (write-up,
// section 4.1: only the order of the scores matters, so no exponential).
//
// Two kernels:
//  * k_index_tile -- prefill.  A workgroup owns 512 consecutive queries of one
//    group (their index queries stay in VGPRs as the MFMA B operand) and sweeps
//    the candidate key blocks in order.  Each 128 x d_idx key block is staged
//    once in LDS (global -> LDS transfers three blocks ahead where rows are
//    256 bytes, else through registers, double buffered) and multiplied on the
//    matrix cores as S^T = K_blk * Q^T, so each lane's accumulators hold one
//    query's scores for 16 keys and the max pool is an in-register max plus
//    one lane swap.  The token scores never leave registers; the block score
//    goes straight into the lane's running Top-k list, so the score matrix
//    never reaches HBM.  The 32-key M-tiles of all blocks run as one pipeline
//    (the products of the next M-tile are issued before the max-pool and
//    Top-k insertion of the current one, across block boundaries too).
//  * k_index_scan -- decode / few queries.  Streams idx_k block by block (each
//    128-token block of all groups is one contiguous span), VALU dot products
//    against the few index queries kept in LDS; writes block scores, which
//    k_topk_rows then selects from.
#include <type_traits>

#include "msa_device.h"
#include "msa_internal.h"

namespace msa {
namespace {

struct TileArgs {
  const void* iq;
  const void* ik;          // keys in the dtype, or MXFP8 codes
  const uint8_t* iks;      // MXFP8 scales (one per 32 key elements), else null
  int32_t* ids;
  float* scores;
  int Nq, Nk, Hkv, topk, nblk, n_tiles, bk;
  int64_t q_offset;
};

constexpr int kTileWaves = 8;  // waves per workgroup of the MFMA tile kernel

// Global -> registers -> LDS staging of one 128-token key block (16-byte
// chunks; CPR chunks per token row, row stride `rowb` bytes in HBM).
// Chunk j covers tokens [128 j, 128 j + 128); tokens past n_k (only in the last
// chunk, and only when blocks are smaller than a chunk) re-read token n_k - 1:
// they belong to the last, partial block, which is never a candidate.
template <int LOADS, int CPR, int CHUNKS, int NTHR>
__device__ __forceinline__ void tile_gload(u32x4 (&stage)[LOADS], const char* base, int j, int64_t rowb, int nk,
                                           int tid) {
#pragma unroll
  for (int u = 0; u < LOADS; ++u) {
    const int c = tid + u * NTHR;
    if (c < CHUNKS) {
      const int row = c / CPR, col = c % CPR;
      const int64_t t = min((int64_t)j * kChunk + row, (int64_t)nk - 1);
      stage[u] = *reinterpret_cast<const u32x4*>(base + t * rowb + col * 16);
    }
  }
}
template <int LOADS, int CPR, int CHUNKS, int NTHR, int PITCH>
__device__ __forceinline__ void tile_lstore(const u32x4 (&stage)[LOADS], char* buf, int tid) {
#pragma unroll
  for (int u = 0; u < LOADS; ++u) {
    const int c = tid + u * NTHR;
    if (c < CHUNKS) {
      const int row = c / CPR, col = c % CPR;
      *reinterpret_cast<u32x4*>(buf + row * PITCH + col * 16) = stage[u];
    }
  }
}

// MXFP8 keys: 16-byte chunks of codes (16 elements, inside one 32-element
// scale block) and their scale byte are loaded, decoded exactly and stored to
// LDS in the dtype layout the MFMA path reads (each element times 2^(s-127) is
// representable in the dtype: E4M3 carries 3 mantissa bits).
template <int LOADS, int MCPR, int CHUNKS, int NTHR, int DI>
__device__ __forceinline__ void mx_gload(u32x4 (&stage)[LOADS], uint32_t (&scl)[LOADS], const uint8_t* codes,
                                         const uint8_t* scales, int j, int hkv, int nk, int tid) {
#pragma unroll
  for (int u = 0; u < LOADS; ++u) {
    const int c = tid + u * NTHR;
    if (c < CHUNKS) {
      const int row = c / MCPR, col = c % MCPR;
      const int64_t r = min((int64_t)j * kChunk + row, (int64_t)nk - 1) * hkv;
      stage[u] = *reinterpret_cast<const u32x4*>(codes + r * DI + col * 16);
      scl[u] = scales[r * (DI / 32) + col / 2];
    }
  }
}
template <typename T, int LOADS, int MCPR, int CHUNKS, int NTHR, int PITCH>
__device__ __forceinline__ void mx_lstore(const u32x4 (&stage)[LOADS], const uint32_t (&scl)[LOADS], char* buf,
                                          int tid) {
#pragma unroll
  for (int u = 0; u < LOADS; ++u) {
    const int c = tid + u * NTHR;
    if (c < CHUNKS) {
      const int row = c / MCPR, col = c % MCPR;
      float f[16];
      e4m3_decode16(stage[u], f);
      const int ex = (int)scl[u] - 127;
      T* dst = reinterpret_cast<T*>(buf + row * PITCH) + col * 16;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        frag_t<T> o;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = static_cast<T>(__builtin_ldexpf(f[8 * h + e], ex));
        if constexpr (sizeof(T) == 2) {
          *reinterpret_cast<frag_t<T>*>(dst + 8 * h) = o;
        } else {
          *reinterpret_cast<f32x4*>(dst + 8 * h) = f32x4{o[0], o[1], o[2], o[3]};
          *reinterpret_cast<f32x4*>(dst + 8 * h + 4) = f32x4{o[4], o[5], o[6], o[7]};
        }
      }
    }
  }
}

// Key blocks whose rows are 256 bytes (bf16 d_idx = 128, fp32 d_idx = 64) are
// staged with direct global -> LDS loads (global_load_lds_dwordx4: lane L of
// a wave writes 16 bytes at the wave's LDS base + 16 L), four blocks deep, no
// staging registers.  Rows are unpadded; chunk c of row r sits at position
// c ^ (r % 16), so the 16 rows read by a quarter-wave hit distinct banks.
constexpr int kDmaRowBytes = 256;
// Blocks in flight: four with eight waves (one workgroup per CU), two with four
// waves (two workgroups per CU, 64 KB of LDS each).
template <int WAVES> constexpr int dma_bufs() { return WAVES == 8 ? 4 : 2; }

// One wave's share of a key block's transfer: PER 1 KB slots of 4 rows each
// (32 / WAVES slots per wave).  Tokens past n_k (a partial last block, only
// when blocks are smaller than a chunk) re-read token n_k - 1.
template <int WAVES>
struct DmaLane {
  static constexpr int PER = 32 / WAVES;
  __device__ __forceinline__ void issue(char* buf, const char* ikb, int j, int64_t rowb, int nk, int wave,
                                        int lane) const {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int slot = wave * PER + u;
      const int r = slot * 4 + lane / 16;
      const int c = (lane & 15) ^ (r & 15);
      const char* src = ikb + min((int64_t)j * kChunk + r, (int64_t)nk - 1) * rowb + c * 16;
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src), buf + slot * 1024, 16, 0, 0);
    }
  }
};

// Fragment of 8 elements starting at element e (multiple of 8) of row r of a
// swizzled 256-byte-row buffer.
template <typename T>
__device__ __forceinline__ frag_t<T> dma_frag(const char* buf, int r, int e) {
  const int c = e * (int)sizeof(T) / 16;
  if constexpr (sizeof(T) == 2) {
    return *reinterpret_cast<const bf16x8*>(buf + r * kDmaRowBytes + ((c ^ (r & 15)) << 4));
  } else {
    const f32x4 lo = *reinterpret_cast<const f32x4*>(buf + r * kDmaRowBytes + ((c ^ (r & 15)) << 4));
    const f32x4 hi = *reinterpret_cast<const f32x4*>(buf + r * kDmaRowBytes + (((c + 1) ^ (r & 15)) << 4));
    return f32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
}

template <typename T, int DI, int NT, int KMAX, bool WRITE_S, bool TOPK, bool MX, int WAVES>
__global__ void __launch_bounds__(WAVES * 64, 2) k_index_tile(TileArgs a) {
  constexpr int TQ = WAVES * NT * 32;  // queries per workgroup
  constexpr int ROW_BYTES = DI * (int)sizeof(T);
  constexpr int PITCH = ROW_BYTES + 16;  // padded LDS row: conflict-free 16-byte reads
  constexpr int KSTEPS = DI / 16;
  constexpr int CPR = ROW_BYTES / 16;  // 16-byte chunks per key row
  constexpr int CHUNKS = kChunk * CPR;
  constexpr int NTHR = WAVES * 64;
  constexpr int LOADS = (CHUNKS + NTHR - 1) / NTHR;
  constexpr bool DMA = !MX && ROW_BYTES == kDmaRowBytes && (WAVES == 8 || WAVES == 4);  // 32 loads = one block
  constexpr int DPW = 32 / WAVES;  // DMA loads per wave per block
  constexpr int MCPR = DI / 16;  // MXFP8: 16-byte code chunks per key row
  constexpr int MCHUNKS = kChunk * MCPR;
  constexpr int MLOADS = (MCHUNKS + NTHR - 1) / NTHR;
  constexpr int NBUF = DMA ? dma_bufs<WAVES>() : 2;
  constexpr int BUFB = DMA ? kChunk * kDmaRowBytes : kChunk * PITCH;
  __shared__ __attribute__((aligned(16))) char lds[NBUF][BUFB];

  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: slot arithmetic on the scalar unit
  const int g = blockIdx.x % a.Hkv;
  const int tile = a.n_tiles - 1 - (int)(blockIdx.x / a.Hkv);  // heaviest tiles first
  const int b = blockIdx.y;
  const int q0 = tile * TQ;
  const int q_last = min(q0 + TQ, a.Nq) - 1;
  // Key chunks holding a candidate block of some query of the tile.
  const int j_end = (int)(((a.q_offset + q_last) / a.bk * a.bk + kChunk - 1) / kChunk);
  const int bpm = a.bk / 32;              // 32-key M-tiles per block
  const int bpc = kChunk / a.bk;          // blocks per chunk

  const T* iq = static_cast<const T*>(a.iq);
  const int64_t krow = (int64_t)a.Hkv * DI;  // elements between consecutive tokens
  const char* ikb = reinterpret_cast<const char*>(static_cast<const T*>(a.ik) + (int64_t)b * a.Nk * krow + g * DI);
  const uint8_t* ikc = static_cast<const uint8_t*>(a.ik) + ((int64_t)b * a.Nk * a.Hkv + g) * DI;  // MXFP8 codes
  const uint8_t* iks = a.iks + ((int64_t)b * a.Nk * a.Hkv + g) * (DI / 32);                       // MXFP8 scales

  // Index queries of this wave as B operands: column = query, k = d_idx.
  frag_t<T> bq[NT][KSTEPS];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int q = q0 + wave * NT * 32 + nt * 32 + (lane & 31);
    const T* p = iq + (((int64_t)b * a.Nq + q) * a.Hkv + g) * DI + 8 * half;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) bq[nt][ks] = q < a.Nq ? load8(p + 16 * ks) : zero_frag<T>();
  }

  // Query owned by this lane after the max-pool exchange.
  const int q_own = q0 + wave * NT * 32 + (NT == 2 ? lane : (lane & 31));
  const bool own_valid = q_own < a.Nq && (NT == 2 || half == 0);
  const int L_own = own_valid ? (int)((a.q_offset + q_own) / a.bk) : 0;

  TopList<KMAX> list;
  list.init();

  if constexpr (DMA && KMAX <= 16) {
    // The M-tiles of all key blocks as one pipeline (two accumulator sets,
    // two fragment sets): the products of M-tile m + 1 are issued before the
    // max-pool of m, and the fragments of m + 2 are read meanwhile -- across
    // block boundaries too.  The barrier that makes block j + 1 visible sits
    // in block j, after the products of its last M-tile are issued (every LDS
    // read of block j has then been consumed, so block j + 4's transfer can
    // reuse its buffer), and the block's last max-pool and Top-k insertion run
    // while the first products of block j + 1 are on the matrix core.
    if (j_end > 0) {
      DmaLane<WAVES> dl;
      const int64_t rowb = krow * (int64_t)sizeof(T);
#pragma unroll
      for (int sb = 0; sb < NBUF - 1; ++sb)
        if (sb < j_end) dl.issue(lds[sb], ikb, sb, rowb, a.Nk, wave, lane);
      // block j has landed and is visible; then block j + NBUF - 1 is issued
      // into the buffer of block j - 1
      auto gate = [&](int j) {
        if (!WRITE_S && j + NBUF - 2 < j_end) wait_vmcnt<DPW * (NBUF - 2)>();
        else wait_vmcnt<0>();
        __syncthreads();
        if (j + NBUF - 1 < j_end) dl.issue(lds[(j + NBUF - 1) % NBUF], ikb, j + NBUF - 1, rowb, a.Nk, wave, lane);
      };
      const int arow = lane & 31;
      auto frag = [&](const char* buf, int mt, int ks) -> frag_t<T> {
        return dma_frag<T>(buf, mt * 32 + arow, 16 * ks + 8 * half);
      };
      frag_t<T> A[2][KSTEPS];
      f32x16 acc[2][NT];
      auto products = [&](int set) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[set][nt] = mma0(A[set][0], bq[nt][0]);
#pragma unroll
        for (int ks = 1; ks < KSTEPS; ++ks)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) mma(A[set][ks], bq[nt][ks], acc[set][nt]);
      };
      gate(0);
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) A[0][ks] = frag(lds[0], 0, ks);
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) A[1][ks] = frag(lds[0], 1, ks);
      products(0);
      for (int j = 0; j < j_end; ++j) {
        const char* bufc = lds[j % NBUF];
        const char* bufn = lds[(j + 1) % NBUF];
        const bool more = j + 1 < j_end;
        float run[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) run[nt] = -__builtin_huge_valf();
        const int bpm = a.bk / 32, bpc = kChunk / a.bk;
        auto pool = [&](int set, int mt) {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) run[nt] = max16(acc[set][nt], run[nt]);
          if (((mt + 1) & (bpm - 1)) == 0) {
            float own;
            if (NT == 2) {
              const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(run[0]), __float_as_uint(run[1]), false,
                                                              false);
              own = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
            } else {
              own = pair32_max(run[0]);
            }
            const int jb = j * bpc + mt / bpm;
            if (jb < L_own) {
              if (TOPK) list.offer(own, jb);
              if (WRITE_S) a.scores[(((int64_t)b * a.Hkv + g) * a.Nq + q_own) * a.nblk + jb] = own;
            }
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) run[nt] = -__builtin_huge_valf();
          }
        };
        // M-tile 0 of block j was issued in the previous round (or above).
        products(1);
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) A[0][ks] = frag(bufc, 2, ks);
        pool(0, 0);
        products(0);
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) A[1][ks] = frag(bufc, 3, ks);
        pool(1, 1);
        products(1);
        if (more) {
          gate(j + 1);
#pragma unroll
          for (int ks = 0; ks < KSTEPS; ++ks) A[0][ks] = frag(bufn, 0, ks);
        }
        pool(0, 2);
        if (more) {
          products(0);
#pragma unroll
          for (int ks = 0; ks < KSTEPS; ++ks) A[1][ks] = frag(bufn, 1, ks);
        }
        pool(1, 3);
      }
    }
  } else if (j_end > 0) {
    DmaLane<WAVES> dl;
    u32x4 stage[LOADS];
    u32x4 mstage[MLOADS];
    uint32_t mscl[MLOADS];
    if constexpr (MX) {
      mx_gload<MLOADS, MCPR, MCHUNKS, NTHR, DI>(mstage, mscl, ikc, iks, 0, a.Hkv, a.Nk, tid);
      mx_lstore<T, MLOADS, MCPR, MCHUNKS, NTHR, PITCH>(mstage, mscl, lds[0], tid);
      __syncthreads();
    } else if constexpr (DMA) {
#pragma unroll
      for (int sb = 0; sb < NBUF - 1; ++sb)
        if (sb < j_end) dl.issue(lds[sb], ikb, sb, krow * (int64_t)sizeof(T), a.Nk, wave, lane);
    } else {
      tile_gload<LOADS, CPR, CHUNKS, NTHR>(stage, ikb, 0, krow * (int64_t)sizeof(T), a.Nk, tid);
      tile_lstore<LOADS, CPR, CHUNKS, NTHR, PITCH>(stage, lds[0], tid);
      __syncthreads();
    }
    for (int j = 0; j < j_end; ++j) {
      const int cur = j % NBUF;
      if constexpr (DMA) {
        // Block j has landed once at most the loads of the later blocks in
        // flight remain; then every wave's share is visible after the barrier.
        if (!WRITE_S && j + NBUF - 2 < j_end) wait_vmcnt<DPW * (NBUF - 2)>();
        else wait_vmcnt<0>();
        __syncthreads();
        if (j + NBUF - 1 < j_end)
          dl.issue(lds[(j + NBUF - 1) % NBUF], ikb, j + NBUF - 1, krow * (int64_t)sizeof(T), a.Nk, wave, lane);
      } else if constexpr (MX) {
        if (j + 1 < j_end) mx_gload<MLOADS, MCPR, MCHUNKS, NTHR, DI>(mstage, mscl, ikc, iks, j + 1, a.Hkv, a.Nk, tid);
      } else {
        if (j + 1 < j_end) tile_gload<LOADS, CPR, CHUNKS, NTHR>(stage, ikb, j + 1, krow * (int64_t)sizeof(T), a.Nk, tid);
      }
      float run[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) run[nt] = -__builtin_huge_valf();
      // The key fragments of M-tile mt+1 are read from LDS while mt multiplies.
      const char* bufc = lds[cur];
      const int arow = lane & 31;
      auto frag = [&](int mt, int ks) -> frag_t<T> {
        if constexpr (DMA) return dma_frag<T>(bufc, mt * 32 + arow, 16 * ks + 8 * half);
        else return load8(reinterpret_cast<const T*>(bufc + (mt * 32 + arow) * PITCH) + 8 * half + 16 * ks);
      };
      // Max-pool of M-tile mt (accumulator set mt & 1) and, after the last
      // M-tile of a key block, the block score into the Top-k list.
      auto pool = [&](const f32x16 (&accm)[NT], int mt) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) run[nt] = max16(accm[nt], run[nt]);
        if (((mt + 1) & (bpm - 1)) == 0) {
          // Last M-tile of a key block.  Each half of the wave saw half of the
          // block's keys; swap halves so that lane l ends with the full block
          // max of query q0 + wave*NT*32 + l.
          float own;
          if (NT == 2) {
            // one v_permlane32_swap: lane l < 32 pairs run[0] of lanes l and
            // l + 32, lane l >= 32 pairs run[1] of lanes l - 32 and l
            const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(run[0]), __float_as_uint(run[1]), false,
                                                            false);
            own = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
          } else {
            own = pair32_max(run[0]);
          }
          const int jb = j * bpc + mt / bpm;  // blocks arrive in increasing order
          if (jb < L_own) {
            if (TOPK) list.offer(own, jb);
            if (WRITE_S) a.scores[(((int64_t)b * a.Hkv + g) * a.Nq + q_own) * a.nblk + jb] = own;
          }
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) run[nt] = -__builtin_huge_valf();
        }
      };
      {
      // Software pipeline over the four M-tiles: the products of M-tile mt+1
      // are issued before the max-pool of mt, so the VALU work of one tile
      // runs while the matrix core works on the next (two accumulator sets;
      // with the longest Top-k lists the second set would not fit in the
      // registers, and the tiles run one after the other).
      constexpr bool PIPE = KMAX <= 16;
      frag_t<T> A[2][KSTEPS];
      f32x16 acc[2][NT];
      auto products = [&](int mt) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[mt & 1][nt] = mma0(A[mt & 1][0], bq[nt][0]);
#pragma unroll
        for (int ks = 1; ks < KSTEPS; ++ks)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) mma(A[mt & 1][ks], bq[nt][ks], acc[mt & 1][nt]);
      };
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) A[0][ks] = frag(0, ks);
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) A[1][ks] = frag(1, ks);
      products(0);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        if constexpr (PIPE) {
          if (mt + 1 < 4) {
            products(mt + 1);
            if (mt + 2 < 4) {
#pragma unroll
              for (int ks = 0; ks < KSTEPS; ++ks) A[mt & 1][ks] = frag(mt + 2, ks);
            }
          }
        } else if (mt > 0) {
          products(mt);
          if (mt + 1 < 4) {
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) A[(mt + 1) & 1][ks] = frag(mt + 1, ks);
          }
        }
        pool(acc[mt & 1], mt);
      }
      }
      if constexpr (MX) {
        if (j + 1 < j_end) mx_lstore<T, MLOADS, MCPR, MCHUNKS, NTHR, PITCH>(mstage, mscl, lds[(j + 1) & 1], tid);
        __syncthreads();
      } else if constexpr (!DMA) {
        if (j + 1 < j_end) tile_lstore<LOADS, CPR, CHUNKS, NTHR, PITCH>(stage, lds[(j + 1) & 1], tid);
        __syncthreads();
      }
    }
  }
  if (TOPK && own_valid) {
    int cand[KMAX];
#pragma unroll
    for (int p = 0; p < KMAX; ++p) cand[p] = list.j[p];
    const int nsel = min(a.topk - 1, L_own);
    write_selection<KMAX>(cand, nsel, L_own, a.topk, a.ids + (((int64_t)b * a.Nq + q_own) * a.Hkv + g) * a.topk);
  }
}

struct ScanArgs {
  const void* iq;
  const void* ik;          // keys in the dtype, or MXFP8 codes
  const uint8_t* iks;      // MXFP8 scales, else null
  float* scores;
  int Nq, Nk, Hkv, nblk, blocks_per_wg, j_end, bk;  // j_end, blocks_per_wg: 128-token chunks
  int64_t q_offset;
};

constexpr int kScanThreads = 256;
constexpr int kScanUnroll = 8;

// One workgroup scores `blocks_per_wg` consecutive key blocks of one batch
// entry for every group and every query (Nq <= NQ).  MXFP8 keys: each lane
// takes a 16-byte chunk of codes (16 elements of one 32-element scale block),
// decodes it exactly, and scales its partial dot product by 2^(s-127).
template <typename T, int DI, int NQ, bool MX>
__global__ void __launch_bounds__(kScanThreads) k_index_scan(ScanArgs a) {
  constexpr int EPL = MX ? 16 : 8;               // key elements per lane
  constexpr int C = DI / EPL;                    // lanes per (token, group) row
  constexpr int ROWS_IT = kScanThreads / C;      // rows per sweep of the workgroup
  extern __shared__ __attribute__((aligned(16))) float smem[];
  float* qs = smem;                              // [NQ][Hkv][DI] index queries (fp32)
  float* dots = smem + NQ * a.Hkv * DI;          // [NQ][Hkv][128] token scores of one block
  uint8_t* sscl = reinterpret_cast<uint8_t*>(dots + NQ * a.Hkv * kChunk);  // MXFP8: the chunk's scale bytes

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.y;
  const int H = a.Hkv;
  const T* iq = static_cast<const T*>(a.iq);
  const T* ik = static_cast<const T*>(a.ik);
  for (int e = tid; e < a.Nq * H * DI; e += kScanThreads)
    qs[e] = to_f32(iq[(int64_t)b * a.Nq * H * DI + e]);
  __syncthreads();

  const int c = tid % C, rsub = tid / C;
  const int rows = kChunk * H;
  const int iters = rows / ROWS_IT;  // exact: 128 * H rows, ROWS_IT divides 128
  const int jb = blockIdx.x * a.blocks_per_wg;
  const int je = min(jb + a.blocks_per_wg, a.j_end);
  for (int j = jb; j < je; ++j) {
    // Chunk j: tokens [128 j, 128 j + ntok); tokens past n_k (possible in the last
    // chunk when blocks are smaller than a chunk) are skipped -- they belong to
    // the last, partial block, which is never a candidate.
    const int ntok = (int)min((int64_t)kChunk, (int64_t)a.Nk - (int64_t)j * kChunk);
    const int64_t row0 = ((int64_t)b * a.Nk + (int64_t)j * kChunk) * H;  // first (token, group) row of chunk j
    const T* blk = ik + row0 * DI;
    const uint8_t* blkc = static_cast<const uint8_t*>(a.ik) + row0 * DI;
    if constexpr (MX) {
      // The chunk's scale bytes (ntok * Hkv * DI/32, contiguous) go to LDS with
      // one 16-byte load per thread instead of a byte load per row and lane.
      const uint8_t* blks = a.iks + row0 * (DI / 32);
      const int nbytes = ntok * H * (DI / 32);
      if ((reinterpret_cast<uintptr_t>(blks) & 15) == 0 && (nbytes & 15) == 0) {
        for (int ch = tid; ch < nbytes / 16; ch += kScanThreads)
          reinterpret_cast<u32x4*>(sscl)[ch] = reinterpret_cast<const u32x4*>(blks)[ch];
      } else {  // scales not on a 16-byte boundary (odd Nk), or a partial chunk
        for (int i = tid; i < nbytes; i += kScanThreads) sscl[i] = blks[i];
      }
      __syncthreads();
    }
    // Full chunks (all but possibly the last) skip the per-row liveness test.
    auto sweep = [&](auto full_tag) {
    constexpr bool FULL = decltype(full_tag)::value;
    for (int it0 = 0; it0 < iters; it0 += kScanUnroll) {
      frag_t<T> x[kScanUnroll];
      u32x4 xc[kScanUnroll];
      uint32_t xs[kScanUnroll];
#pragma unroll
      for (int u = 0; u < kScanUnroll; ++u) {
        const int row = (it0 + u) * ROWS_IT + rsub;
        const bool live = it0 + u < iters && (FULL || row < ntok * H);
        if constexpr (MX) {
          xc[u] = u32x4{};
          xs[u] = 127;
          if (live) {
            xc[u] = *reinterpret_cast<const u32x4*>(blkc + (int64_t)row * DI + c * 16);
            xs[u] = sscl[row * (DI / 32) + c / 2];
          }
        } else {
          x[u] = live ? load8(blk + (int64_t)row * DI + c * 8) : zero_frag<T>();
        }
      }
#pragma unroll
      for (int u = 0; u < kScanUnroll; ++u) {
        const int row = (it0 + u) * ROWS_IT + rsub;
        const int tok = row / H, grp = row % H;
        float kf[EPL];
        if constexpr (MX) {
          float f[16];
          e4m3_decode16(xc[u], f);
#pragma unroll
          for (int e = 0; e < EPL; ++e) kf[e] = f[e];
        } else {
#pragma unroll
          for (int e = 0; e < EPL; ++e) kf[e] = to_f32(x[u][e]);
        }
#pragma unroll
        for (int qi = 0; qi < NQ; ++qi) {
          if (qi < a.Nq) {
            const float* qv = qs + (qi * H + grp) * DI + c * EPL;
            float acc = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc = fmaf(kf[e], qv[e], acc);
            if constexpr (MX) acc = __builtin_ldexpf(acc, (int)xs[u] - 127);
            acc = group_sum<C>(acc);
            if (c == 0 && it0 + u < iters) dots[(qi * H + grp) * kChunk + tok] = acc;
          }
        }
      }
    }
    };
    if (ntok == kChunk) sweep(std::true_type{});
    else sweep(std::false_type{});
    __syncthreads();
    // max over the Bk tokens of each block of chunk j, for every (query, group):
    // lane l holds tokens l and 64 + l; blocks of 128 / 64 / 32 tokens are
    // reduced over 64 / 64 / 32 lanes.
    for (int r = wave; r < a.Nq * H; r += kScanThreads / 64) {
      float m0 = dots[r * kChunk + lane], m1 = dots[r * kChunk + 64 + lane];
      if (a.bk == kChunk) m0 = m1 = fmaxf(m0, m1);
      const int span = a.bk == 32 ? 16 : 32;
#pragma unroll
      for (int s = 32; s >= 1; s >>= 1)
        if (s <= span) {
          m0 = fmaxf(m0, xor_shfl(m0, s));
          m1 = fmaxf(m1, xor_shfl(m1, s));
        }
      const int qi = r / H, grp = r % H;
      const int L = (int)((a.q_offset + qi) / a.bk);
      const int bpc = kChunk / a.bk;
      // lane 0 writes the first block of each half-chunk; for 32-token blocks
      // lane 32 writes the second one
      const int sub = a.bk == 32 ? (lane >> 5) : 0;
      if ((lane & 31) == 0 && (lane == 0 || a.bk == 32)) {
        float* out = a.scores + (((int64_t)b * H + grp) * a.Nq + qi) * a.nblk;
        const int jb0 = j * bpc + sub;              // block of tokens 0..63
        const int jb1 = j * bpc + bpc / 2 + sub;    // block of tokens 64..127
        if (a.bk == kChunk) {
          if (jb0 < L) out[jb0] = m0;
        } else {
          if (jb0 < L) out[jb0] = m0;
          if (jb1 < L) out[jb1] = m1;
        }
      }
    }
    __syncthreads();
  }
}

__global__ void k_fill_neg_inf(float* p, size_t n) {
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += (size_t)gridDim.x * blockDim.x)
    p[e] = -__builtin_huge_valf();
}

template <typename T, int DI, bool WRITE_S, bool TOPK, bool MX>
hipError_t tile_dispatch(const Shape& s, const TileArgs& a, dim3 grid, hipStream_t st) {
  constexpr int NT = (DI * (int)sizeof(T) <= 256) ? 2 : 1;
  const int kneed = s.topk - 1;
  if (!TOPK || kneed <= 8) {
    hipLaunchKernelGGL((k_index_tile<T, DI, NT, 8, WRITE_S, TOPK, MX, kTileWaves>), grid, dim3(kTileWaves * 64), 0, st, a);
  } else if (kneed <= 16) {
    hipLaunchKernelGGL((k_index_tile<T, DI, NT, 16, WRITE_S, TOPK, MX, kTileWaves>), grid, dim3(kTileWaves * 64), 0, st, a);
  } else {
    hipLaunchKernelGGL((k_index_tile<T, DI, NT, 32, WRITE_S, TOPK, MX, kTileWaves>), grid, dim3(kTileWaves * 64), 0, st, a);
  }
  return hipGetLastError();
}

template <typename T, bool WRITE_S, bool TOPK, bool MX>
hipError_t tile_dispatch_di(const Shape& s, const TileArgs& a, dim3 grid, hipStream_t st) {
  switch (s.DI) {
    case 32: return tile_dispatch<T, 32, WRITE_S, TOPK, MX>(s, a, grid, st);
    case 64: return tile_dispatch<T, 64, WRITE_S, TOPK, MX>(s, a, grid, st);
    default: return tile_dispatch<T, 128, WRITE_S, TOPK, MX>(s, a, grid, st);
  }
}

template <typename T, bool WRITE_S, bool TOPK>
hipError_t tile_dispatch_fmt(const Shape& s, const TileArgs& a, dim3 grid, hipStream_t st) {
  return s.idx_mx ? tile_dispatch_di<T, WRITE_S, TOPK, true>(s, a, grid, st)
                  : tile_dispatch_di<T, WRITE_S, TOPK, false>(s, a, grid, st);
}

template <typename T, int DI, bool MX>
hipError_t scan_dispatch(const Shape& s, const ScanArgs& a, dim3 grid, hipStream_t st) {
  const int nq = s.Nq <= 1 ? 1 : s.Nq <= 2 ? 2 : s.Nq <= 4 ? 4 : 8;
  const size_t shm_q = (size_t)nq * s.Hkv * (DI + kChunk) * sizeof(float) + (MX ? (size_t)kChunk * s.Hkv * (DI / 32) : 0);
  if (s.Nq <= 1) hipLaunchKernelGGL((k_index_scan<T, DI, 1, MX>), grid, dim3(kScanThreads), shm_q, st, a);
  else if (s.Nq <= 2) hipLaunchKernelGGL((k_index_scan<T, DI, 2, MX>), grid, dim3(kScanThreads), shm_q, st, a);
  else if (s.Nq <= 4) hipLaunchKernelGGL((k_index_scan<T, DI, 4, MX>), grid, dim3(kScanThreads), shm_q, st, a);
  else hipLaunchKernelGGL((k_index_scan<T, DI, 8, MX>), grid, dim3(kScanThreads), shm_q, st, a);
  return hipGetLastError();
}

template <typename T, bool MX>
hipError_t scan_dispatch_di(const Shape& s, const ScanArgs& a, dim3 grid, hipStream_t st) {
  switch (s.DI) {
    case 32: return scan_dispatch<T, 32, MX>(s, a, grid, st);
    case 64: return scan_dispatch<T, 64, MX>(s, a, grid, st);
    default: return scan_dispatch<T, 128, MX>(s, a, grid, st);
  }
}

template <typename T>
hipError_t scan_dispatch_fmt(const Shape& s, const ScanArgs& a, dim3 grid, hipStream_t st) {
  return s.idx_mx ? scan_dispatch_di<T, true>(s, a, grid, st) : scan_dispatch_di<T, false>(s, a, grid, st);
}

// Scale bytes of an MXFP8 idx_k cache: right after the B*Nk*Hkv*d_idx codes.
const uint8_t* mx_scales(const Shape& s, const void* ik) {
  return s.idx_mx ? static_cast<const uint8_t*>(ik) + (size_t)s.B * s.Nk * s.Hkv * s.DI : nullptr;
}

constexpr int kScanMaxQueries = 8;

}  // namespace

bool index_use_tile(const Shape& s) { return s.Nq > kScanMaxQueries; }

static int tile_queries(const Shape& s) {
  const int NT = (s.DI * (s.dtype == kBF16 ? 2 : 4) <= 256) ? 2 : 1;
  return kTileWaves * NT * 32;
}

hipError_t launch_index_tile(const Shape& s, const void* iq, const void* ik, int32_t* ids, float* scores,
                             hipStream_t st) {
  static const int kid_topk = prof_register("index_tile_topk");
  static const int kid_scores = prof_register("index_tile_scores");
  const int kid = ids ? kid_topk : kid_scores;
  TileArgs a;
  a.iq = iq;
  a.ik = ik;
  a.iks = mx_scales(s, ik);
  a.ids = ids;
  a.scores = scores;
  a.Nq = s.Nq;
  a.Nk = s.Nk;
  a.Hkv = s.Hkv;
  a.topk = s.topk;
  a.nblk = s.nblk;
  a.n_tiles = (s.Nq + tile_queries(s) - 1) / tile_queries(s);
  a.bk = s.Bk;
  a.q_offset = s.q_offset;
  const dim3 grid(a.n_tiles * s.Hkv, s.B);
  prof_begin(st, kid);
  hipError_t e;
  if (s.dtype == kBF16)
    e = ids ? tile_dispatch_fmt<bf16_t, false, true>(s, a, grid, st) : tile_dispatch_fmt<bf16_t, true, false>(s, a, grid, st);
  else
    e = ids ? tile_dispatch_fmt<float, false, true>(s, a, grid, st) : tile_dispatch_fmt<float, true, false>(s, a, grid, st);
  prof_end(st, kid);
  return e;
}

hipError_t launch_index_scan(const Shape& s, const void* iq, const void* ik, float* scores, hipStream_t st) {
  static const int kid = prof_register("index_scan");
  if (s.Nq > kScanMaxQueries) return hipErrorInvalidValue;
  ScanArgs a;
  a.iq = iq;
  a.ik = ik;
  a.iks = mx_scales(s, ik);
  a.scores = scores;
  a.Nq = s.Nq;
  a.Nk = s.Nk;
  a.Hkv = s.Hkv;
  a.nblk = s.nblk;
  a.q_offset = s.q_offset;
  a.bk = s.Bk;
  // chunks holding a candidate block of the last query
  a.j_end = (int)(((s.q_offset + s.Nq - 1) / s.Bk * s.Bk + kChunk - 1) / kChunk);
  if (a.j_end <= 0) return hipSuccess;
  a.blocks_per_wg = 2;
  const dim3 grid((a.j_end + a.blocks_per_wg - 1) / a.blocks_per_wg, s.B);
  prof_begin(st, kid);
  const hipError_t e = s.dtype == kBF16 ? scan_dispatch_fmt<bf16_t>(s, a, grid, st) : scan_dispatch_fmt<float>(s, a, grid, st);
  prof_end(st, kid);
  return e;
}

hipError_t launch_fill_neg_inf(float* p, size_t n, hipStream_t st) {
  static const int kid = prof_register("fill_neg_inf");
  if (n == 0) return hipSuccess;
  const size_t blocks = std::min<size_t>((n + 255) / 256, 65536);
  prof_begin(st, kid);
  hipLaunchKernelGGL(k_fill_neg_inf, dim3((unsigned)blocks), dim3(256), 0, st, p, n);
  const hipError_t e = hipGetLastError();
  prof_end(st, kid);
  return e;
}

}  // namespace msa
