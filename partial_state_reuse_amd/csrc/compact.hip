// Compact encoding of a cached bf16 attention state: int8 codes with one fp32
// scale per row, the LSE copied unchanged.
//
// The DiTango page leaves cache compression as future work for the memory
// that cached states hold (Significance and Claims, limitations).  Per row r
// (one query of one head):
//     a_r = max_d |O[r, d]|,   s_r = a_r / 127,
//     code[r, d] = round-half-even(O[r, d] * 127 / a_r)   in [-127, 127],
// and a row of zeros has s_r = 0 and zero codes.  A merge uses code * s_r.
// Every step is one fp32 operation with one rounding: O * 127 is exact for a
// bf16 value, both divisions are correctly rounded (HIP's fp32 division is),
// and round-half-even is v_rndne_f32, so the codes and scales are reproducible
// bit for bit.  136 bytes per row at D = 128 against 260 for the bf16 state.
//
// The pass is bound by HBM bandwidth: D/8 lanes per row, each reading one
// 16-byte chunk (8 values) and writing 8 code bytes; the row maximum is a
// shuffle reduction inside the row's lanes.

#include "dita_kernels.h"

namespace dita {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr float kCodeMax = 127.0f;

template <int D>
__global__ __launch_bounds__(kThreads) void compact_encode_kernel(
    const __bf16* __restrict__ o, const float* __restrict__ lse, int8_t* __restrict__ codes,
    float* __restrict__ scale, float* __restrict__ lse_out, int64_t rows) {
  constexpr int LPR = D / 8;           // lanes per row
  constexpr int RPB = kThreads / LPR;  // rows per block
  const int64_t row = int64_t(blockIdx.x) * RPB + threadIdx.x / LPR;
  const int c = threadIdx.x % LPR;
  if (row >= rows) return;             // whole rows leave together (LPR divides 64)
  const u32x4 r = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(o + row * D + c * 8));
  float x[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = r[i];
    x[2 * i] = __builtin_bit_cast(float, w << 16);
    x[2 * i + 1] = __builtin_bit_cast(float, w & 0xffff0000u);
  }
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(x[i]));
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) a = fmaxf(a, __shfl_xor(a, off));
  u32x2 packed = {0u, 0u};
  if (a > 0.0f) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float q = __builtin_rintf((x[i] * kCodeMax) / a);
      const uint32_t b = uint32_t(int32_t(q)) & 0xffu;
      packed[i / 4] |= b << (8 * (i % 4));
    }
  }
  *reinterpret_cast<u32x2*>(codes + row * D + c * 8) = packed;
  if (c == 0) {
    scale[row] = a > 0.0f ? a / kCodeMax : 0.0f;
    lse_out[row] = lse[row];
  }
}

}  // namespace

hipError_t launch_compact_encode(int D, const void* o, const float* lse, int8_t* codes,
                                 float* scale, float* lse_out, int64_t rows, hipStream_t stream) {
  const int lpr = D / 8;
  const int64_t blocks = (rows + kThreads / lpr - 1) / (kThreads / lpr);
  const __bf16* ob = static_cast<const __bf16*>(o);
  if (D == 128)
    compact_encode_kernel<128><<<dim3(unsigned(blocks)), kThreads, 0, stream>>>(ob, lse, codes, scale,
                                                                               lse_out, rows);
  else
    compact_encode_kernel<64><<<dim3(unsigned(blocks)), kThreads, 0, stream>>>(ob, lse, codes, scale,
                                                                              lse_out, rows);
  return hipGetLastError();
}

}  // namespace dita
