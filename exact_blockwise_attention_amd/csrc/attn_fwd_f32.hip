// Exact attention forward with fp32 operands and fp32 output, on the vector ALU.
//
// Same method as the MFMA kernel ("深度学习注意力机制优化与FlashAttention实践" §4.2, with the accumulator
// rescaled when the running maximum grows), kept simple: it serves fp32 workloads where accuracy, not
// throughput, is the point. One lane owns one query row (its q and its output accumulator stay in VGPRs);
// a wave streams 16-key K/V tiles through LDS, where every lane reads the same key row (LDS broadcast).
#include "internal.h"

namespace ebattn {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int kRows = 64;   // query rows per workgroup (one wave)
constexpr int kTk = 16;     // keys per tile

template <int D>
__global__ __launch_bounds__(kRows) void attn_fwd_f32_kernel(FwdArgs a, int n_qtiles) {
  __shared__ __attribute__((aligned(16))) float Ks[kTk * D];
  __shared__ __attribute__((aligned(16))) float Vs[kTk * D];
  const int tid = threadIdx.x;
  const int64_t w = blockIdx.x;
  const int64_t bh = w / n_qtiles;
  const int q0 = (int)(w % n_qtiles) * kRows;
  const int qi = q0 + tid;
  const float* Q = reinterpret_cast<const float*>(a.q) + bh * (int64_t)a.Nq * D;
  const int64_t kvbh = bh / a.kv_group;   // the key/value head this query head reads
  const float* K = reinterpret_cast<const float*>(a.k) + kvbh * (int64_t)a.Nk * D;
  const float* V = reinterpret_cast<const float*>(a.v) + kvbh * (int64_t)a.Nk * D;

  float q[D], acc[D];
#pragma unroll
  for (int c = 0; c < D; c += 4) {
    f32x4 x = {};
    if (qi < a.Nq) x = *reinterpret_cast<const f32x4*>(Q + (int64_t)qi * D + c);
    q[c] = x[0]; q[c + 1] = x[1]; q[c + 2] = x[2]; q[c + 3] = x[3];
    acc[c] = acc[c + 1] = acc[c + 2] = acc[c + 3] = 0.0f;
  }
  const int qlast = min(q0 + kRows, a.Nq) - 1;
  const int kend = a.causal ? min(a.Nk, qlast + a.diag + 1) : a.Nk;
  const int lim = a.causal ? min(qi + a.diag, a.Nk - 1) : a.Nk - 1;   // last visible key of this row
  const int low = a.causal ? qi + a.lo : 0;                            // first key of its sliding window
  const int first_key = a.causal ? q0 + a.lo : 0;                      // ... of the block's first row
  float m_run = -INFINITY, l_run = 0.0f;

  for (int j0 = first_key > 0 ? first_key / kTk * kTk : 0; j0 < kend; j0 += kTk) {
    __syncthreads();
    for (int e = tid * 4; e < kTk * D; e += kRows * 4) {
      const int j = j0 + e / D;
      f32x4 kx = {}, vx = {};
      if (j < a.Nk) {
        kx = *reinterpret_cast<const f32x4*>(K + (int64_t)j0 * D + e);
        vx = *reinterpret_cast<const f32x4*>(V + (int64_t)j0 * D + e);
      }
      *reinterpret_cast<f32x4*>(Ks + e) = kx;
      *reinterpret_cast<f32x4*>(Vs + e) = vx;
    }
    __syncthreads();
    float s[kTk];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < kTk; ++j) {
      float dot = 0.0f;
#pragma unroll
      for (int c = 0; c < D; ++c) dot = __builtin_fmaf(q[c], Ks[j * D + c], dot);
      s[j] = (j0 + j <= lim && j0 + j >= low) ? dot : -INFINITY;
      mx = fmaxf(mx, s[j]);
    }
    const float m_new = fmaxf(m_run, mx * a.scale_log2);
    const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int c = 0; c < D; ++c) acc[c] *= alpha;
#pragma unroll
    for (int j = 0; j < kTk; ++j) {
      const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[j], a.scale_log2, -m_use));
      l_run += p;
#pragma unroll
      for (int c = 0; c < D; ++c) acc[c] = __builtin_fmaf(p, Vs[j * D + c], acc[c]);
    }
  }
  if (qi >= a.Nq) return;
  const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
  a.lse[bh * (int64_t)a.Nq + qi] =
      l_run > 0.0f ? (m_run + __builtin_amdgcn_logf(l_run)) * 0.69314718055994531f : -INFINITY;
  float* O = reinterpret_cast<float*>(a.o) + (bh * (int64_t)a.Nq + qi) * D;
#pragma unroll
  for (int c = 0; c < D; c += 4)
    *reinterpret_cast<f32x4*>(O + c) = f32x4{acc[c] * inv, acc[c + 1] * inv, acc[c + 2] * inv, acc[c + 3] * inv};
}

template <int D>
hipError_t launch_d(const FwdArgs& a, hipStream_t stream) {
  const int n_qtiles = (a.Nq + kRows - 1) / kRows;
  const int64_t total = (int64_t)n_qtiles * a.BH;
  if (total > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((attn_fwd_f32_kernel<D>), dim3((unsigned)total), dim3(kRows), 0, stream, a, n_qtiles);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd_f32(const FwdArgs& a, int d, hipStream_t stream) {
  switch (d) {
    case 128: return launch_d<128>(a, stream);
    case 64: return launch_d<64>(a, stream);
    case 24: return launch_d<24>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ebattn
