// Exact attention backward with fp32 operands, on the vector ALU.
//
// The same gradient as the MFMA kernels ("深度学习注意力机制优化与FlashAttention实践" §4.1 item 3 and §3.3: the
// weights are recomputed from the saved lse), kept simple for fp32 workloads where accuracy is the point:
//   P_ij = exp(scale q_i.k_j - lse_i), delta_i = dO_i . O_i, dS_ij = P_ij (dO_i . V_j - delta_i),
//   dQ_i = scale sum_j dS_ij K_j, dK_j = scale sum_i dS_ij Q_i, dV_j = sum_i P_ij dO_i.
// Four lanes share one row and hold a quarter of its head dim each; a dot product is the four partial sums added
// across the lanes. The dq kernel (one row = one query, K and V tiles of 16 keys in LDS) runs first and writes
// delta; the dk/dv kernel (one row = one key, Q, dO, lse and delta tiles of 16 queries in LDS) follows and walks
// the query heads that share its key/value head.
#include "internal.h"

namespace ebattn {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
constexpr int kSplit = 4;                   // lanes per row
constexpr int kRows = 64;                   // rows per workgroup
constexpr int kThreads = kRows * kSplit;    // 256
constexpr int kT = 16;                      // rows per LDS tile of the other side
constexpr float kLog2e = 1.4426950408889634f;

// Sum over the four lanes of a row (lanes 4r .. 4r + 3).
__device__ __forceinline__ float row_sum(float x) {
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  return x;
}

// lse -> exp2-domain subtrahend; a row with no visible key (lse = -inf) gets +inf, so its weights are zero.
__device__ __forceinline__ float lse_to_sub(float lse) { return lse == -INFINITY ? INFINITY : lse * kLog2e; }

// Stores factor * x (this lane's DS columns starting at c0 of a row of length D) as fp32 (optionally added to
// the previous contents) or bf16.
template <int D, int DS, bool GF32>
__device__ __forceinline__ void store_part(void* out, int64_t row, int c0, const float (&x)[DS], float factor,
                                           bool accumulate) {
  if constexpr (GF32) {
    float* p = reinterpret_cast<float*>(out) + row * D + c0;
#pragma unroll
    for (int c = 0; c < DS; ++c) p[c] = accumulate ? p[c] + factor * x[c] : factor * x[c];
  } else {
    __bf16* p = reinterpret_cast<__bf16*>(out) + row * D + c0;
#pragma unroll
    for (int c = 0; c < DS; ++c) p[c] = (__bf16)(factor * x[c]);
  }
}

template <int D, bool GF32>
__global__ __launch_bounds__(kThreads) void attn_bwd_f32_dq_kernel(BwdArgs a, int n_qtiles) {
  constexpr int DS = D / kSplit;
  __shared__ __attribute__((aligned(16))) float Ks[kT * D];
  __shared__ __attribute__((aligned(16))) float Vs[kT * D];
  const int tid = threadIdx.x, r = tid / kSplit, c0 = (tid % kSplit) * DS;
  const int64_t bh = blockIdx.x / n_qtiles;
  const int q0 = (int)(blockIdx.x % n_qtiles) * kRows;
  const int qi = q0 + r;
  const int64_t kvbh = bh / a.kv_group;
  const float* K = reinterpret_cast<const float*>(a.k) + kvbh * (int64_t)a.Nk * D;
  const float* V = reinterpret_cast<const float*>(a.v) + kvbh * (int64_t)a.Nk * D;
  const int64_t row = bh * (int64_t)a.Nq + qi;

  float q[DS], g[DS], acc[DS];
  float dl = 0.0f;
#pragma unroll
  for (int c = 0; c < DS; ++c) {
    const bool in = qi < a.Nq;
    q[c] = in ? reinterpret_cast<const float*>(a.q)[row * D + c0 + c] : 0.0f;
    g[c] = in ? reinterpret_cast<const float*>(a.dout)[row * D + c0 + c] : 0.0f;
    const float o = in ? reinterpret_cast<const float*>(a.o)[row * D + c0 + c] : 0.0f;
    dl = __builtin_fmaf(g[c], o, dl);
    acc[c] = 0.0f;
  }
  dl = row_sum(dl);
  const float lsub = qi < a.Nq ? lse_to_sub(a.lse[row]) : INFINITY;
  if (qi < a.Nq && c0 == 0) a.delta[row] = dl;

  const int qlast = min(q0 + kRows, a.Nq) - 1;
  const int kend = a.causal ? min(a.Nk, qlast + a.diag + 1) : a.Nk;
  const int lim = a.causal ? min(qi + a.diag, a.Nk - 1) : a.Nk - 1;   // last key this row sees
  const int low = a.causal ? qi + a.lo : 0;                            // first key of its window
  const int first_key = a.causal ? q0 + a.lo : 0;

  for (int j0 = first_key > 0 ? first_key / kT * kT : 0; j0 < kend; j0 += kT) {
    __syncthreads();
    for (int e = tid * 4; e < kT * D; e += kThreads * 4) {
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
    for (int j = 0; j < kT; ++j) {
      float s = 0.0f, dp = 0.0f;
#pragma unroll
      for (int c = 0; c < DS; ++c) {
        s = __builtin_fmaf(q[c], Ks[j * D + c0 + c], s);
        dp = __builtin_fmaf(g[c], Vs[j * D + c0 + c], dp);
      }
      s = row_sum(s);
      dp = row_sum(dp);
      const bool vis = j0 + j <= lim && j0 + j >= low;
      const float p = vis ? __builtin_amdgcn_exp2f(__builtin_fmaf(s, a.scale_log2, -lsub)) : 0.0f;
      const float ds = p * (dp - dl);
#pragma unroll
      for (int c = 0; c < DS; ++c) acc[c] = __builtin_fmaf(ds, Ks[j * D + c0 + c], acc[c]);
    }
  }
  if (qi < a.Nq) store_part<D, DS, GF32>(a.dq, row, c0, acc, a.scale, a.accumulate != 0);
}

template <int D, bool GF32>
__global__ __launch_bounds__(kThreads) void attn_bwd_f32_dkdv_kernel(BwdArgs a, int n_ktiles) {
  constexpr int DS = D / kSplit;
  __shared__ __attribute__((aligned(16))) float Qs[kT * D];
  __shared__ __attribute__((aligned(16))) float Gs[kT * D];
  __shared__ float Ls[kT];
  __shared__ float Ds[kT];
  const int tid = threadIdx.x, r = tid / kSplit, c0 = (tid % kSplit) * DS;
  const int64_t kvbh = blockIdx.x / n_ktiles;
  const int k0 = (int)(blockIdx.x % n_ktiles) * kRows;
  const int kj = k0 + r;
  const int64_t krow = kvbh * (int64_t)a.Nk + kj;

  float k[DS], v[DS], dk[DS], dv[DS];
#pragma unroll
  for (int c = 0; c < DS; ++c) {
    const bool in = kj < a.Nk;
    k[c] = in ? reinterpret_cast<const float*>(a.k)[krow * D + c0 + c] : 0.0f;
    v[c] = in ? reinterpret_cast<const float*>(a.v)[krow * D + c0 + c] : 0.0f;
    dk[c] = dv[c] = 0.0f;
  }
  // query rows i that some key of the block sees: i + lo <= j <= i + diag
  int qbeg = 0, qend = a.Nq;
  if (a.causal) {
    qbeg = max(0, k0 - a.diag);
    if (a.lo != kNoWindow) qend = min(a.Nq, k0 + kRows - 1 - a.lo + 1);
  }
  for (int h = 0; h < a.kv_group; ++h) {
    const int64_t bh = kvbh * a.kv_group + h;
    const float* Q = reinterpret_cast<const float*>(a.q) + bh * (int64_t)a.Nq * D;
    const float* G = reinterpret_cast<const float*>(a.dout) + bh * (int64_t)a.Nq * D;
    for (int i0 = qbeg / kT * kT; i0 < qend; i0 += kT) {
      __syncthreads();
      for (int e = tid * 4; e < kT * D; e += kThreads * 4) {
        const int i = i0 + e / D;
        f32x4 qx = {}, gx = {};
        if (i < a.Nq) {
          qx = *reinterpret_cast<const f32x4*>(Q + (int64_t)i0 * D + e);
          gx = *reinterpret_cast<const f32x4*>(G + (int64_t)i0 * D + e);
        }
        *reinterpret_cast<f32x4*>(Qs + e) = qx;
        *reinterpret_cast<f32x4*>(Gs + e) = gx;
      }
      if (tid < kT) {
        const int i = i0 + tid;
        Ls[tid] = i < a.Nq ? lse_to_sub(a.lse[bh * (int64_t)a.Nq + i]) : INFINITY;
        Ds[tid] = i < a.Nq ? a.delta[bh * (int64_t)a.Nq + i] : 0.0f;
      }
      __syncthreads();
      for (int i = 0; i < kT; ++i) {
        float s = 0.0f, dp = 0.0f;
#pragma unroll
        for (int c = 0; c < DS; ++c) {
          s = __builtin_fmaf(Qs[i * D + c0 + c], k[c], s);
          dp = __builtin_fmaf(Gs[i * D + c0 + c], v[c], dp);
        }
        s = row_sum(s);
        dp = row_sum(dp);
        const int qi = i0 + i;
        const bool vis = !a.causal || (kj <= qi + a.diag && kj >= qi + a.lo);
        const float p = vis ? __builtin_amdgcn_exp2f(__builtin_fmaf(s, a.scale_log2, -Ls[i])) : 0.0f;
        const float ds = p * (dp - Ds[i]);
#pragma unroll
        for (int c = 0; c < DS; ++c) {
          dv[c] = __builtin_fmaf(p, Gs[i * D + c0 + c], dv[c]);
          dk[c] = __builtin_fmaf(ds, Qs[i * D + c0 + c], dk[c]);
        }
      }
    }
  }
  if (kj < a.Nk) {
    store_part<D, DS, GF32>(a.dk, krow, c0, dk, a.scale, a.accumulate != 0);
    store_part<D, DS, GF32>(a.dv, krow, c0, dv, 1.0f, a.accumulate != 0);
  }
}

template <int D, bool GF32>
hipError_t launch_d(const BwdArgs& a, hipStream_t stream) {
  if (a.BH > 0 && a.Nq > 0) {
    const int n = (a.Nq + kRows - 1) / kRows;
    const int64_t total = (int64_t)n * a.BH;
    if (total > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((attn_bwd_f32_dq_kernel<D, GF32>), dim3((unsigned)total), dim3(kThreads), 0, stream, a, n);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t BHkv = a.BH / a.kv_group;
  if (BHkv > 0 && a.Nk > 0) {
    const int n = (a.Nk + kRows - 1) / kRows;
    const int64_t total = (int64_t)n * BHkv;
    if (total > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((attn_bwd_f32_dkdv_kernel<D, GF32>), dim3((unsigned)total), dim3(kThreads), 0, stream, a, n);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_attn_bwd_f32(const BwdArgs& a, int d, int grad_f32, hipStream_t stream) {
  switch (d) {
    case 128: return grad_f32 ? launch_d<128, true>(a, stream) : launch_d<128, false>(a, stream);
    case 64: return grad_f32 ? launch_d<64, true>(a, stream) : launch_d<64, false>(a, stream);
    case 24: return grad_f32 ? launch_d<24, true>(a, stream) : launch_d<24, false>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ebattn
