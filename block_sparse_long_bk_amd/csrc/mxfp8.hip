// mxfp8.hip -- MXFP8 index-key caches on gfx950.
//
// The MiniMax write-up pairs MSA with MXFP8 caches for long-context decode
// (zhichai.net, section 9).  The format is the OCP Microscaling one (MX v1.0):
// 32 consecutive elements of a row share an E8M0 scale byte s (2^(s-127));
// the elements are OCP FP8 E4M3 codes (bias 7, no infinities, largest finite
// 448).  Conversion of a block (spec section 6.3): shared exponent
// e = floor(log2(max |v|)) - 8, where 8 is E4M3's largest exponent, clamped to
// the E8M0 range; each element becomes E4M3(v / 2^e), rounded to nearest even
// and saturated at +-448.
//
// k_mxfp8_quantize: one thread per 32-element block.  The encoder is integer
// arithmetic on the fp32 bit pattern, so its rounding is exactly the round-
// half-to-even of the definition (no dependence on the conversion hardware).
#include "msa_device.h"
#include "msa_internal.h"

namespace msa {
namespace {

// E4M3 code of y (|y| < 2^9 by construction; larger magnitudes saturate).
__device__ __forceinline__ uint32_t e4m3_encode(float y) {
  const uint32_t bits = __float_as_uint(y);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const uint32_t a = bits & 0x7fffffffu;
  if (a >= 0x43E00000u) return sign | 0x7Eu;  // |y| >= 448 = 1.75 * 2^8
  if (a < 0x3C800000u) {                       // |y| < 2^-6: multiples of 2^-9
    const float m = __builtin_rintf(__uint_as_float(a) * 512.0f);  // exact scaling, half to even
    return sign | (uint32_t)m;                 // m == 8 is the code of 2^-6
  }
  const uint32_t e = (a >> 23) - 127u + 7u;    // biased E4M3 exponent, 1..15
  uint32_t q = (a >> 20) & 7u;                 // top three mantissa bits
  const uint32_t rem = a & 0xFFFFFu;
  q += (rem > 0x80000u || (rem == 0x80000u && (q & 1u))) ? 1u : 0u;
  return sign | ((e << 3) + q);                // q == 8 carries into the exponent
}

template <typename T>
__global__ void __launch_bounds__(256) k_mxfp8_quantize(const T* __restrict__ src, uint8_t* __restrict__ codes,
                                                        uint8_t* __restrict__ scales, int64_t nblocks) {
  const int64_t blk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (blk >= nblocks) return;
  float v[32];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const frag_t<T> f = load8(src + blk * 32 + 8 * u);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[8 * u + e] = to_f32(f[e]);
  }
  float amax = 0.f;
#pragma unroll
  for (int c = 0; c < 32; ++c) amax = fmaxf(amax, fabsf(v[c]));
  int e = -127;
  if (amax > 0.f) {
    const uint32_t ab = __float_as_uint(amax);
    const int fl = (ab >> 23) ? (int)(ab >> 23) - 127 : (31 - __clz((int)ab)) - 149;  // floor(log2 amax)
    e = min(127, max(-127, fl - 8));
  }
  u32x4 out[2];
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    uint32_t word = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) word |= e4m3_encode(__builtin_ldexpf(v[4 * w + k], -e)) << (8 * k);
    out[w / 4][w % 4] = word;
  }
  u32x4* dst = reinterpret_cast<u32x4*>(codes + blk * 32);
  dst[0] = out[0];
  dst[1] = out[1];
  scales[blk] = (uint8_t)(e + 127);
}

}  // namespace

hipError_t launch_mxfp8_quantize(const void* src, int dtype, int64_t n_rows, int row_len, uint8_t* codes,
                                 uint8_t* scales, hipStream_t st) {
  static const int kid = prof_register("mxfp8_quantize");
  const int64_t nblocks = n_rows * (row_len / 32);
  const dim3 grid((unsigned)((nblocks + 255) / 256));
  prof_begin(st, kid);
  if (dtype == kBF16)
    hipLaunchKernelGGL(k_mxfp8_quantize<bf16_t>, grid, dim3(256), 0, st, static_cast<const bf16_t*>(src), codes,
                       scales, nblocks);
  else
    hipLaunchKernelGGL(k_mxfp8_quantize<float>, grid, dim3(256), 0, st, static_cast<const float*>(src), codes,
                       scales, nblocks);
  const hipError_t e = hipGetLastError();
  prof_end(st, kid);
  return e;
}

}  // namespace msa
