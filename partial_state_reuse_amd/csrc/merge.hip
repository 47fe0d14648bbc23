// Exact LSE-weighted merge of P attention states, and the state copy kernel.
//
// Merge (the state composition of the DiTango page, State-Centric Parallel
// Runtime > State Composition), per row:
//     M = max_p LSE_p,  w_p = exp(LSE_p - M),  L = sum_p w_p,
//     O = sum_p (w_p / L) O_p,  LSE = M + ln L
// States with LSE = -inf weigh 0; a row whose every LSE is -inf becomes
// (0, -inf).
//
// The pass is bound by HBM bandwidth: it reads P states and writes one,
// (P+1) * (D * sizeof(dtype) + 4) bytes per row, and does ~2*P*D flops per
// row.  A row is handled by D*sizeof(dtype)/16 lanes, each moving one
// 16-byte chunk of every O_p (fully coalesced: consecutive lanes, consecutive
// chunks, consecutive rows).  Each lane issues the loads of up to 16
// partitions (chunk and LSE) before it uses any, so P <= 16 costs one memory
// round trip; the weights use the hardware exp2 on a log2-scaled argument.
// The state chunks are read with nontemporal loads (each byte is read once;
// measured 5.2 -> 5.8 TB/s for the 16-way merge of 40 x 4725 rows of 128).
// Accumulation is fp32.

#include "dita_kernels.h"

#include <cmath>

namespace dita {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kChunk = 16;  // partitions whose loads are in flight together

template <typename T>
struct Vec;

template <>
struct Vec<float> {
  static constexpr int N = 4;
  __device__ static void unpack(u32x4 r, float* x) {
    // Element by value first: a bit_cast of a vector-element lvalue reads element 0.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t u = r[i];
      x[i] = __builtin_bit_cast(float, u);
    }
  }
  __device__ static u32x4 pack(const float* x) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = __builtin_bit_cast(uint32_t, x[i]);
    return r;
  }
};

template <>
struct Vec<__bf16> {
  static constexpr int N = 8;
  __device__ static void unpack(u32x4 r, float* x) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __builtin_bit_cast(float, r[i] << 16);
      x[2 * i + 1] = __builtin_bit_cast(float, r[i] & 0xffff0000u);
    }
  }
  __device__ static u32x4 pack(const float* x) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = __builtin_bit_cast(uint16_t, (__bf16)x[2 * i]);
      const uint32_t hi = __builtin_bit_cast(uint16_t, (__bf16)x[2 * i + 1]);
      r[i] = lo | (hi << 16);
    }
    return r;
  }
};

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// o and lse may be source 0 (in-place composition and the pre-merged two-stream
// step), so they are not declared __restrict__: every load of a lane's chunk
// (and of the row's LSE) feeds the lane's single store of that chunk.
//
// COMPACT (bf16 only): sources whose bit is set in `compact` are compact
// states -- src.o[j] holds int8 codes in the same [rows, D] layout and
// src.scale[j] one fp32 scale per row; their values are code * scale (one
// fp32 product, as the encoding defines).  The lane reads 8 code bytes and the
// row's scale instead of its 16-byte chunk.
//
// GROUP: the merge of sources [g.first, g.end) alone goes to (g.o, g.lse) as
// well, from the same loads, with the operations of a merge of those sources
// by themselves in the same order (the same bits as that merge).  g.o may be
// source g.first's output (in place, as above).
template <typename T, int D, bool COMPACT, bool GROUP>
__global__ __launch_bounds__(kThreads) void merge_kernel(MergeSrc src, int P, int64_t rows,
                                                         uint64_t compact, T* o, float* lse,
                                                         MergeGroup g) {
  constexpr int VN = Vec<T>::N;
  constexpr int LPR = D / VN;          // lanes per row
  constexpr int RPB = kThreads / LPR;  // rows per block
  const int64_t row = int64_t(blockIdx.x) * RPB + threadIdx.x / LPR;
  const int c = threadIdx.x % LPR;
  if (row >= rows) return;
  const int64_t off = row * D + c * VN;

  // Every load of the first kChunk states goes out before any result is used:
  // one memory round trip for P <= kChunk.
  u32x4 raw[kChunk];
  float lp[kChunk];
  float sc[kChunk];
  auto load_src = [&](int j, int p) {
    if (COMPACT && ((compact >> p) & 1)) {
      const u32x2 w = __builtin_nontemporal_load(
          reinterpret_cast<const u32x2*>(static_cast<const int8_t*>(src.o[p]) + off));
      raw[j][0] = w[0];
      raw[j][1] = w[1];
      sc[j] = src.scale[p][row];
    } else {
      raw[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(static_cast<const T*>(src.o[p]) + off));
    }
    lp[j] = src.lse[p][row];
  };
#pragma unroll
  for (int j = 0; j < kChunk; ++j) {
    if (j < P) load_src(j, j);
  }
  float M = -INFINITY;
#pragma unroll
  for (int j = 0; j < kChunk; ++j)
    if (j < P) M = fmaxf(M, lp[j]);
  for (int p = kChunk; p < P; ++p) M = fmaxf(M, src.lse[p][row]);
  auto in_group = [&](int p) { return GROUP && p >= g.first && p < g.end; };
  float M2 = -INFINITY;
  if constexpr (GROUP) {
#pragma unroll
    for (int j = 0; j < kChunk; ++j)
      if (j < P && in_group(j)) M2 = fmaxf(M2, lp[j]);
    for (int p = kChunk; p < P; ++p)
      if (in_group(p)) M2 = fmaxf(M2, src.lse[p][row]);
  }

  float acc[VN], acc2[VN];
#pragma unroll
  for (int i = 0; i < VN; ++i) acc[i] = acc2[i] = 0.0f;
  // The group's state, written after every load of the row (in place safe).
  auto store_group = [&](float L2) {
    if constexpr (GROUP) {
      if (M2 == -INFINITY) {
        *reinterpret_cast<u32x4*>(static_cast<T*>(g.o) + off) = Vec<T>::pack(acc2);
        if (c == 0) g.lse[row] = -INFINITY;
        return;
      }
      const float inv2 = 1.0f / L2;
#pragma unroll
      for (int i = 0; i < VN; ++i) acc2[i] *= inv2;
      *reinterpret_cast<u32x4*>(static_cast<T*>(g.o) + off) = Vec<T>::pack(acc2);
      if (c == 0) g.lse[row] = M2 + __builtin_amdgcn_logf(L2) * kLn2;
    }
  };
  if (M == -INFINITY) {
    *reinterpret_cast<u32x4*>(o + off) = Vec<T>::pack(acc);
    if (c == 0) lse[row] = -INFINITY;
    store_group(0.0f);  // M2 is -inf too
    return;
  }
  // w_p = exp(LSE_p - M) = exp2((LSE_p - M) log2 e); 0 for LSE_p = -inf.  The
  // difference is taken first, so the largest state weighs exactly 1 (a
  // one-state merge returns its input unchanged).
  float L = 0.0f, L2 = 0.0f;
  auto accumulate = [&](int j, int p) {
    const float w = __builtin_amdgcn_exp2f((lp[j] - M) * kLog2e);
    L += w;
    float x[VN];
    if (COMPACT && ((compact >> p) & 1)) {
#pragma unroll
      for (int i = 0; i < VN; ++i) {
        const int32_t code = int32_t(raw[j][i / 4] << (24 - 8 * (i % 4))) >> 24;
        x[i] = float(code) * sc[j];
      }
    } else {
      Vec<T>::unpack(raw[j], x);
    }
#pragma unroll
    for (int i = 0; i < VN; ++i) acc[i] = __builtin_fmaf(w, x[i], acc[i]);
    if (in_group(p)) {
      const float w2 = __builtin_amdgcn_exp2f((lp[j] - M2) * kLog2e);
      L2 += w2;
#pragma unroll
      for (int i = 0; i < VN; ++i) acc2[i] = __builtin_fmaf(w2, x[i], acc2[i]);
    }
  };
#pragma unroll
  for (int j = 0; j < kChunk; ++j)
    if (j < P) accumulate(j, j);
  for (int p0 = kChunk; p0 < P; p0 += kChunk) {
#pragma unroll
    for (int j = 0; j < kChunk; ++j) {
      if (p0 + j < P) load_src(j, p0 + j);
    }
#pragma unroll
    for (int j = 0; j < kChunk; ++j)
      if (p0 + j < P) accumulate(j, p0 + j);
  }
  const float inv = 1.0f / L;
#pragma unroll
  for (int i = 0; i < VN; ++i) acc[i] *= inv;
  *reinterpret_cast<u32x4*>(o + off) = Vec<T>::pack(acc);
  if (c == 0) lse[row] = M + __builtin_amdgcn_logf(L) * kLn2;  // hardware log2; L >= 1
  store_group(L2);
}

template <typename T, int D, bool GROUP>
hipError_t launch_merge_g(int64_t rows, int P, const MergeSrc& src, void* o, float* lse,
                          hipStream_t stream, const MergeGroup& g) {
  constexpr int LPR = D / Vec<T>::N;
  constexpr int RPB = kThreads / LPR;
  const int64_t blocks = (rows + RPB - 1) / RPB;
  uint64_t compact = 0;
  for (int p = 0; p < P; ++p)
    if (src.scale[p]) compact |= uint64_t(1) << p;
  if constexpr (sizeof(T) == 2) {
    if (compact) {
      merge_kernel<T, D, true, GROUP><<<dim3(unsigned(blocks)), kThreads, 0, stream>>>(
          src, P, rows, compact, static_cast<T*>(o), lse, g);
      return hipGetLastError();
    }
  }
  merge_kernel<T, D, false, GROUP><<<dim3(unsigned(blocks)), kThreads, 0, stream>>>(
      src, P, rows, 0, static_cast<T*>(o), lse, g);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_merge_t(int64_t rows, int P, const MergeSrc& src, void* o, float* lse,
                          hipStream_t stream, const MergeGroup& g) {
  if (g.end > g.first) return launch_merge_g<T, D, true>(rows, P, src, o, lse, stream, g);
  return launch_merge_g<T, D, false>(rows, P, src, o, lse, stream, g);
}

__global__ __launch_bounds__(kThreads) void copy_state_kernel(const u32x4* __restrict__ so,
                                                              u32x4* __restrict__ dO, int64_t n16,
                                                              const float* __restrict__ sl,
                                                              float* __restrict__ dl, int64_t n4) {
  const int64_t stride = int64_t(gridDim.x) * kThreads;
  for (int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x; i < n16; i += stride)
    dO[i] = __builtin_nontemporal_load(so + i);
  for (int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x; i < n4; i += stride) dl[i] = sl[i];
}

}  // namespace

hipError_t launch_merge(int dtype, int D, int64_t rows, int P, const MergeSrc& src, void* o,
                        float* lse, hipStream_t stream, const MergeGroup& group) {
  if (group.end > group.first &&
      (group.first < 0 || group.end > P || !group.o || !group.lse))
    return hipErrorInvalidValue;
  if (dtype == 1) {
    return D == 128 ? launch_merge_t<__bf16, 128>(rows, P, src, o, lse, stream, group)
                    : launch_merge_t<__bf16, 64>(rows, P, src, o, lse, stream, group);
  }
  return D == 128 ? launch_merge_t<float, 128>(rows, P, src, o, lse, stream, group)
                  : launch_merge_t<float, 64>(rows, P, src, o, lse, stream, group);
}

hipError_t launch_copy_state(const void* src_o, const float* src_lse, void* dst_o, float* dst_lse,
                             size_t o_bytes, size_t lse_bytes, hipStream_t stream) {
  const int64_t n16 = int64_t(o_bytes / 16);
  const int64_t n4 = int64_t(lse_bytes / 4);
  int64_t blocks = (n16 + kThreads - 1) / kThreads;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  copy_state_kernel<<<dim3(unsigned(blocks)), kThreads, 0, stream>>>(
      static_cast<const u32x4*>(src_o), static_cast<u32x4*>(dst_o), n16, src_lse, dst_lse, n4);
  return hipGetLastError();
}

}  // namespace dita
