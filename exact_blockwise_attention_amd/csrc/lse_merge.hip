// Log-sum-exp merge of two partial attention results computed over disjoint key sets.
//
// Method: "分布式注意力机制突破：长序列处理的全景技术架构与实践指南" §3.4 (align the parts to their common
// maximum, rescale and add the per-part sums, LSE = maximum + log of the sum) and §2.2 stage 3 (the pairwise
// form, read with the exponent sign corrected: log(e^a + e^b) = max(a,b) + log(1 + e^-|a-b|)). A partial
// stores (o_i, lse_i) with o_i already normalised by its own sum, so the merged output is the average of
// the o_i weighted by exp(lse_i - lse). lse = -inf marks a part with no visible key: it weighs zero, and two
// empty parts merge to (0, -inf).
//
// The kernel is HBM-bound: per row it reads two d-vectors and two scalars and writes one d-vector and one
// scalar, every byte once, so the d-vectors are read and written with non-temporal accesses (they are not
// kept in the caches). Each lane moves one 16-byte vector; a row is served by a power-of-two group of lanes inside one
// wave, so the scalar lse of a row is read by every lane of the group before any lane of the same wave
// stores (this keeps in-place merges, lse aliasing lse_a, race-free).
#include "internal.h"

namespace ebattn {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;

template <bool PF32>
struct PartVec;
template <>
struct PartVec<true> {
  static constexpr int N = 4;
  typedef f32x4 F;
  __device__ static F load(const void* p, int64_t off) {
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(p) + off));
  }
};
template <>
struct PartVec<false> {
  static constexpr int N = 8;
  typedef f32x8 F;
  __device__ static F load(const void* p, int64_t off) {
    return __builtin_convertvector(
        __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(reinterpret_cast<const __bf16*>(p) + off)), f32x8);
  }
};

template <bool PF32, bool OF32, int TPR>
__global__ __launch_bounds__(256) void lse_merge_kernel(MergeArgs a) {
  using P = PartVec<PF32>;
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = g / TPR;
  const int c0 = (int)(g % TPR) * P::N;
  if (row >= a.rows) return;
  const float la = a.lse_a[row];
  const float lb = a.lse_b[row];
  const float m = fmaxf(la, lb);
  const bool active = c0 < a.d;
  const int64_t off = row * a.d + c0;
  typename P::F y;
  float lse;
  if (m == -INFINITY) {
    y = typename P::F{};
    lse = -INFINITY;
  } else {
    const float wa = __builtin_amdgcn_exp2f((la - m) * kLog2e);
    const float wb = __builtin_amdgcn_exp2f((lb - m) * kLog2e);
    const float s = wa + wb;
    const float inv = 1.0f / s;
    lse = m + __builtin_amdgcn_logf(s) * kLn2;
    if (active) {
      const typename P::F xa = P::load(a.o_a, off);
      const typename P::F xb = P::load(a.o_b, off);
      y = xa * (wa * inv) + xb * (wb * inv);
    }
  }
  if (active) {
    if (OF32) {
      float* o = reinterpret_cast<float*>(a.o) + off;
#pragma unroll
      for (int q = 0; q < P::N; q += 4)
        __builtin_nontemporal_store(f32x4{y[q], y[q + 1], y[q + 2], y[q + 3]}, reinterpret_cast<f32x4*>(o + q));
    } else {
      __bf16* o = reinterpret_cast<__bf16*>(a.o) + off;
#pragma unroll
      for (int q = 0; q < P::N; q += 4)
        __builtin_nontemporal_store(__builtin_convertvector((f32x4{y[q], y[q + 1], y[q + 2], y[q + 3]}), bf16x4),
                                    reinterpret_cast<bf16x4*>(o + q));
    }
  }
  if (c0 == 0) a.lse[row] = lse;
}

template <bool PF32, bool OF32>
hipError_t launch_t(const MergeArgs& a, hipStream_t stream) {
  const int vec = PF32 ? 4 : 8;
  const int per_row = (a.d + vec - 1) / vec;
  int tpr = 1;
  while (tpr < per_row) tpr <<= 1;
  const int64_t threads = a.rows * tpr;
  const int64_t blocks = (threads + 255) / 256;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)blocks), block(256);
  switch (tpr) {
    case 1: hipLaunchKernelGGL((lse_merge_kernel<PF32, OF32, 1>), grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((lse_merge_kernel<PF32, OF32, 2>), grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL((lse_merge_kernel<PF32, OF32, 4>), grid, block, 0, stream, a); break;
    case 8: hipLaunchKernelGGL((lse_merge_kernel<PF32, OF32, 8>), grid, block, 0, stream, a); break;
    case 16: hipLaunchKernelGGL((lse_merge_kernel<PF32, OF32, 16>), grid, block, 0, stream, a); break;
    case 32: hipLaunchKernelGGL((lse_merge_kernel<PF32, OF32, 32>), grid, block, 0, stream, a); break;
    case 64: hipLaunchKernelGGL((lse_merge_kernel<PF32, OF32, 64>), grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Rows with no visible key at all: o = 0, lse = -inf.
template <bool OF32>
__global__ __launch_bounds__(256) void fill_empty_kernel(void* o, float* lse, int64_t rows, int d) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t n = rows * d;
  if (g < n) {
    if (OF32) reinterpret_cast<float*>(o)[g] = 0.0f;
    else reinterpret_cast<__bf16*>(o)[g] = __bf16(0.0f);
  }
  if (g < rows) lse[g] = -INFINITY;
}

}  // namespace

hipError_t launch_lse_merge(const MergeArgs& a, int part_f32, int o_f32, hipStream_t stream) {
  if (part_f32) return o_f32 ? launch_t<true, true>(a, stream) : launch_t<true, false>(a, stream);
  return o_f32 ? launch_t<false, true>(a, stream) : launch_t<false, false>(a, stream);
}

hipError_t launch_fill_empty(void* o, float* lse, int64_t rows, int d, int o_f32, hipStream_t stream) {
  const int64_t n = rows * (int64_t)d > rows ? rows * (int64_t)d : rows;
  const int64_t blocks = (n + 255) / 256;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (o_f32)
    hipLaunchKernelGGL((fill_empty_kernel<true>), dim3((unsigned)blocks), dim3(256), 0, stream, o, lse, rows, d);
  else
    hipLaunchKernelGGL((fill_empty_kernel<false>), dim3((unsigned)blocks), dim3(256), 0, stream, o, lse, rows, d);
  return hipGetLastError();
}

}  // namespace ebattn
