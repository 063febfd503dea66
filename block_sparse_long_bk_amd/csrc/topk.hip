// topk.hip -- exp-free Top-k over rows of block scores (gfx950).
//
// Selection rule (paper summary page, "Method"; zhichai.net write-up,
// sections 2 and 4.1): the local block L(i) = floor((q_offset + i)/Bk) is
// always kept; the other k-1 slots go to the candidate blocks j < L(i) with the
// highest raw scores -- no exponential, since only the order matters.  Equal
// scores go to the lower block id.  The row is emitted ascending, -1 padded.
//
// Short rows: one wave per (b, g, i) row.  Lane l scans blocks l, l+64, ... in
// increasing order keeping its own best-KMAX list in registers; the 64 lists are
// then merged by k-1 rounds of a wave-wide arg-max on (score, -id), the winning
// lane popping its head.  Integer/compare work only; no LDS, no atomics.
#include "msa_device.h"
#include "msa_internal.h"

namespace msa {
namespace {

template <int KMAX>
__global__ void __launch_bounds__(256) k_topk_rows(const float* __restrict__ S, int32_t* __restrict__ ids, int Nq,
                                                   int Hkv, int nblk, int topk, int64_t q_offset, int bk,
                                                   int64_t nrows) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= nrows) return;  // whole wave leaves together
  const int i = (int)(row % Nq);
  const int64_t bg = row / Nq;
  const int g = (int)(bg % Hkv);
  const int64_t b = bg / Hkv;
  const int L = (int)((q_offset + i) / bk);
  const float* Sr = S + row * nblk;

  TopList<KMAX> list;
  list.init();
  for (int j = lane; j < L; j += 64) list.offer(Sr[j], j);

  const int nsel = min(topk - 1, L);
  int sel[KMAX];
#pragma unroll
  for (int r = 0; r < KMAX; ++r) {
    sel[r] = INT32_MAX;
    if (r < nsel) {
      float bs = list.s[0];
      int bj = list.j[0];
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) {
        const float os = xor_shfl(bs, m);
        const int oj = xor_shfl(bj, m);
        const bool take = (os > bs) || (os == bs && oj < bj);
        bs = take ? os : bs;
        bj = take ? oj : bj;
      }
      sel[r] = bj;
      if (list.j[0] == bj) list.pop();
    }
  }
  if (lane == 0) write_selection<KMAX>(sel, nsel, L, topk, ids + (((int64_t)b * Nq + i) * Hkv + g) * topk);
}

// Long rows (decode: thousands of candidates, few rows): one 1024-thread
// workgroup per row.  Each of the 16 waves reduces its stride-1024 share of the
// candidates to its best nsel (per-lane lists + arg-max rounds, as above) and
// leaves them in LDS; wave 0 then merges the 16 short lists the same way, now
// comparing (score desc, id asc) explicitly since the ids no longer arrive in
// order.  The best nsel of the row are among the union of the waves' best nsel.
constexpr int kTopkWgThreads = 1024;
template <int KMAX>
__global__ void __launch_bounds__(kTopkWgThreads) k_topk_wg(const float* __restrict__ S, int32_t* __restrict__ ids,
                                                             int Nq, int Hkv, int nblk, int topk, int64_t q_offset,
                                                             int bk) {
  constexpr int NW = kTopkWgThreads / 64;
  constexpr int CPL = (NW * KMAX + 63) / 64;  // merge candidates per lane of wave 0
  __shared__ float cs[NW * KMAX];
  __shared__ int cj[NW * KMAX];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row = blockIdx.x;
  const int i = (int)(row % Nq);
  const int64_t bg = row / Nq;
  const int g = (int)(bg % Hkv);
  const int64_t b = bg / Hkv;
  const int L = (int)((q_offset + i) / bk);
  const float* Sr = S + row * nblk;
  const int nsel = min(topk - 1, L);

  TopList<KMAX> list;
  list.init();
  for (int j = wave * 64 + lane; j < L; j += kTopkWgThreads) list.offer(Sr[j], j);
#pragma unroll
  for (int r = 0; r < KMAX; ++r) {
    if (r < nsel) {
      float bs = list.s[0];
      int bj = list.j[0];
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) {
        const float os = xor_shfl(bs, m);
        const int oj = xor_shfl(bj, m);
        const bool take = (os > bs) || (os == bs && oj < bj);
        bs = take ? os : bs;
        bj = take ? oj : bj;
      }
      if (list.j[0] == bj) list.pop();
      if (lane == 0) {
        cs[wave * KMAX + r] = bs;
        cj[wave * KMAX + r] = bj;
      }
    }
  }
  __syncthreads();
  if (wave != 0) return;
  // Wave 0: per-lane sorted lists of the waves' candidates, then nsel rounds.
  float ms[CPL];
  int mj[CPL];
#pragma unroll
  for (int p = 0; p < CPL; ++p) {
    ms[p] = -__builtin_huge_valf();
    mj[p] = INT32_MAX;
  }
#pragma unroll
  for (int u = 0; u < CPL; ++u) {
    const int c = lane + 64 * u;
    const int r = c % KMAX;
    if (c < NW * KMAX && r < nsel && cj[c] != INT32_MAX) {
      float x = cs[c];
      int id = cj[c];
      // insertion by (score desc, id asc)
#pragma unroll
      for (int p = 0; p < CPL; ++p) {
        const bool before = (x > ms[p]) || (x == ms[p] && id < mj[p]);
        const float ts = ms[p];
        const int tj = mj[p];
        ms[p] = before ? x : ts;
        mj[p] = before ? id : tj;
        x = before ? ts : x;
        id = before ? tj : id;
      }
    }
  }
  int sel[KMAX];
#pragma unroll
  for (int r = 0; r < KMAX; ++r) {
    sel[r] = INT32_MAX;
    if (r < nsel) {
      float bs = ms[0];
      int bj = mj[0];
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) {
        const float os = xor_shfl(bs, m);
        const int oj = xor_shfl(bj, m);
        const bool take = (os > bs) || (os == bs && oj < bj);
        bs = take ? os : bs;
        bj = take ? oj : bj;
      }
      sel[r] = bj;
      if (mj[0] == bj) {
#pragma unroll
        for (int p = 0; p < CPL - 1; ++p) {
          ms[p] = ms[p + 1];
          mj[p] = mj[p + 1];
        }
        ms[CPL - 1] = -__builtin_huge_valf();
        mj[CPL - 1] = INT32_MAX;
      }
    }
  }
  if (lane == 0) write_selection<KMAX>(sel, nsel, L, topk, ids + (((int64_t)b * Nq + i) * Hkv + g) * topk);
}

}  // namespace

hipError_t launch_topk_rows(const Shape& s, const float* scores, int32_t* ids, hipStream_t st) {
  static const int kid = prof_register("topk_rows");
  const int64_t nrows = (int64_t)s.B * s.Hkv * s.Nq;
  const dim3 grid((unsigned)((nrows + 3) / 4));
  const int kneed = s.topk - 1;
  prof_begin(st, kid);
  // Few long rows: a workgroup per row; otherwise a wave per row.
  if (nrows <= 4096 && s.nblk >= 2048) {
    const dim3 g1((unsigned)nrows);
    if (kneed <= 8)
      hipLaunchKernelGGL(k_topk_wg<8>, g1, dim3(kTopkWgThreads), 0, st, scores, ids, s.Nq, s.Hkv, s.nblk, s.topk, s.q_offset, s.Bk);
    else if (kneed <= 16)
      hipLaunchKernelGGL(k_topk_wg<16>, g1, dim3(kTopkWgThreads), 0, st, scores, ids, s.Nq, s.Hkv, s.nblk, s.topk, s.q_offset, s.Bk);
    else
      hipLaunchKernelGGL(k_topk_wg<32>, g1, dim3(kTopkWgThreads), 0, st, scores, ids, s.Nq, s.Hkv, s.nblk, s.topk, s.q_offset, s.Bk);
  } else if (kneed <= 8) {
    hipLaunchKernelGGL(k_topk_rows<8>, grid, dim3(256), 0, st, scores, ids, s.Nq, s.Hkv, s.nblk, s.topk, s.q_offset, s.Bk, nrows);
  } else if (kneed <= 16) {
    hipLaunchKernelGGL(k_topk_rows<16>, grid, dim3(256), 0, st, scores, ids, s.Nq, s.Hkv, s.nblk, s.topk, s.q_offset, s.Bk, nrows);
  } else {
    hipLaunchKernelGGL(k_topk_rows<32>, grid, dim3(256), 0, st, scores, ids, s.Nq, s.Hkv, s.nblk, s.topk, s.q_offset, s.Bk, nrows);
  }
  const hipError_t e = hipGetLastError();
  prof_end(st, kid);
  return e;
}

}  // namespace msa
