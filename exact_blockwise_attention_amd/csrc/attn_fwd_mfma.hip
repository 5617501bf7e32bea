// Exact blockwise attention forward, bf16 operands on gfx950 MFMA, fp32 online softmax.
//
// Method: "深度学习注意力机制优化与FlashAttention实践" §4.2 (per query block, loop over key/value blocks, keep a
// running maximum and running sum, normalise at the end) with the accumulator rescaled whenever the running
// maximum grows -- the decomposition of "架构层解决方案 - Sparse Attention与Ring Attention", Ring Attention /
// 核心创新, applied one key tile at a time. Causal masking by global position ("深度学习注意力机制优化与
// FlashAttention实践" §5.1) arrives here as a diagonal offset: key j is visible to query i iff j <= i + diag.
// Only O and the per-row log-sum-exp are written to HBM ("注意力机制演进", section FlashAttention).
//
// Work decomposition (one workgroup = 4 waves = 128 query rows of one (batch, head)):
//   * each wave owns 32 query rows; its Q fragment stays in VGPRs for the whole key loop;
//   * key/value tiles of 64 rows are staged through LDS, shared by the 4 waves;
//   * the wave computes S^T = K . Q^T (32 keys x 32 queries per MFMA 32x32x16). In that orientation one lane
//     owns one query row (the MFMA output column), so the row max/sum are in-lane reductions plus one exchange
//     with the partner lane (lane ^ 32), and the rescale factor is a per-lane scalar;
//   * the keys of each 32-key chunk are placed in LDS with bits 2 and 3 of their index swapped. Read back in
//     natural order by the MFMA A operand, this makes lane l's 16 output registers hold, in order, 8
//     consecutive keys of each 16-key half -- exactly the B-operand layout of the next product
//     O^T = V^T . P^T, so P goes from the S accumulator to the P.V MFMA without leaving the registers;
//   * V is transposed while it is staged (each thread loads an 8x4 block, repacks it with v_perm) so the
//     V^T operand is a contiguous 16-byte LDS read; V^T rows are XOR-swizzled per 16-byte chunk so that both
//     the transposing stores and the operand reads spread over the LDS banks.
#include "internal.h"

namespace ebattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kBM = 128;       // query rows per workgroup (4 waves x 32)
constexpr int kBN = 64;        // keys per K/V tile
constexpr int kThreads = 256;

template <int D>
struct Geom {
  static constexpr int DP = (D + 31) / 32 * 32;  // head dim padded to the 32-row tiles of O^T
  static constexpr int KSTEPS = DP / 16;         // MFMA k-steps of S^T = K . Q^T
  static constexpr int CT = DP / 32;             // 32-row tiles of O^T
  static constexpr int CPR = D / 8;              // 16-byte chunks per global row
  static constexpr int KROW = DP + 8;            // LDS pitch (bf16) of a K row; +16 bytes spreads banks
  static constexpr int K_ELEMS = kBN * KROW;
  static constexpr int V_ELEMS = DP * kBN;       // V^T tile [DP][kBN]
  static constexpr int VCG = D / 4;              // 4-column groups per V row
  static constexpr int KLOADS = (kBN * CPR + kThreads - 1) / kThreads;
  static constexpr int VUNITS = (kBN / 8) * VCG; // 8-row x 4-column blocks per V tile
  static constexpr int VLOADS = (VUNITS + kThreads - 1) / kThreads;
};

// LDS row of key j (0..31) inside its 32-key chunk: bits 2 and 3 swapped (an involution).
__device__ __forceinline__ int key_slot(int j) { return (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1); }
// Swizzled 16-byte chunk index of V^T row c.
__device__ __forceinline__ int vt_chunk(int c, int chunk) { return chunk ^ ((c ^ (c >> 3)) & 7); }

__device__ __forceinline__ float wave_pair_max(float x) { return fmaxf(x, __shfl_xor(x, 32)); }
__device__ __forceinline__ float wave_pair_sum(float x) { return x + __shfl_xor(x, 32); }

template <int D>
struct TileRegs {
  u32x4 k[Geom<D>::KLOADS];
  u32x2 v[Geom<D>::VLOADS][8];
};

template <int D>
__device__ __forceinline__ void load_tile(TileRegs<D>& r, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
                                          int j0, int Nk, int tid) {
  using G = Geom<D>;
#pragma unroll
  for (int n = 0; n < G::KLOADS; ++n) {
    const int idx = tid + n * kThreads;
    u32x4 x = {0u, 0u, 0u, 0u};
    if (idx < kBN * G::CPR) {
      const int row = idx / G::CPR, ch = idx % G::CPR;
      const int j = j0 + row;
      if (j < Nk) x = *reinterpret_cast<const u32x4*>(K + (int64_t)j * D + ch * 8);
    }
    r.k[n] = x;
  }
#pragma unroll
  for (int n = 0; n < G::VLOADS; ++n) {
    const int u = tid + n * kThreads;
    const int cg = u % G::VCG, jg = u / G::VCG;
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
      u32x2 x = {0u, 0u};
      const int j = j0 + jg * 8 + rr;
      if (u < G::VUNITS && j < Nk) x = *reinterpret_cast<const u32x2*>(V + (int64_t)j * D + cg * 4);
      r.v[n][rr] = x;
    }
  }
}

template <int D>
__device__ __forceinline__ void store_tile(const TileRegs<D>& r, __bf16* Ks, __bf16* Vt, int tid) {
  using G = Geom<D>;
#pragma unroll
  for (int n = 0; n < G::KLOADS; ++n) {
    const int idx = tid + n * kThreads;
    if (idx < kBN * G::CPR) {
      const int row = idx / G::CPR, ch = idx % G::CPR;
      const int slot = (row & ~31) | key_slot(row & 31);
      *reinterpret_cast<u32x4*>(Ks + slot * G::KROW + ch * 8) = r.k[n];
    }
  }
#pragma unroll
  for (int n = 0; n < G::VLOADS; ++n) {
    const int u = tid + n * kThreads;
    if (u < G::VUNITS) {
      const int cg = u % G::VCG, jg = u / G::VCG;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c = cg * 4 + e;
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;  // high or low bf16 of each source dword
        u32x4 out;
#pragma unroll
        for (int m = 0; m < 4; ++m)
          out[m] = __builtin_amdgcn_perm(r.v[n][2 * m + 1][e >> 1], r.v[n][2 * m][e >> 1], sel);
        *reinterpret_cast<u32x4*>(Vt + c * kBN + 8 * vt_chunk(c, jg)) = out;
      }
    }
  }
}

template <int D, bool MASK>
__device__ __forceinline__ void compute_tile(const __bf16* Ks, const __bf16* Vt, const bf16x8 (&qf)[Geom<D>::KSTEPS],
                                             f32x16 (&acc)[Geom<D>::CT], float& m_run, float& l_run, int lim,
                                             float scale_log2, int l32, int hi) {
  using G = Geom<D>;
  f32x16 s0 = {}, s1 = {};
  const __bf16* k0 = Ks + l32 * G::KROW + 8 * hi;
  const __bf16* k1 = Ks + (32 + l32) * G::KROW + 8 * hi;
#pragma unroll
  for (int kc = 0; kc < G::KSTEPS; ++kc) {
    const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(k0 + kc * 16);
    const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(k1 + kc * 16);
    s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[kc], s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[kc], s1, 0, 0, 0);
  }
  // Register r of lane l holds key 16*(r/8) + 8*(l/32) + r%8 of its 32-key chunk, for query row l%32.
  if (MASK) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kr = 16 * (r >> 3) + (r & 7);
      if (kr > lim) s0[r] = -INFINITY;
      if (kr + 32 > lim) s1[r] = -INFINITY;
    }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int r = 0; r < 16; ++r) mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
  mx = wave_pair_max(mx);
  const float m_new = fmaxf(m_run, mx * scale_log2);
  const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
  const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
  m_run = m_new;
  float psum = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    s0[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[r], scale_log2, -m_use));
    s1[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[r], scale_log2, -m_use));
    psum += s0[r] + s1[r];
  }
  l_run = alpha * l_run + psum;
#pragma unroll
  for (int ct = 0; ct < G::CT; ++ct) acc[ct] *= alpha;

  bf16x8 pb[4];
  pb[0] = __builtin_convertvector(__builtin_shufflevector(s0, s0, 0, 1, 2, 3, 4, 5, 6, 7), bf16x8);
  pb[1] = __builtin_convertvector(__builtin_shufflevector(s0, s0, 8, 9, 10, 11, 12, 13, 14, 15), bf16x8);
  pb[2] = __builtin_convertvector(__builtin_shufflevector(s1, s1, 0, 1, 2, 3, 4, 5, 6, 7), bf16x8);
  pb[3] = __builtin_convertvector(__builtin_shufflevector(s1, s1, 8, 9, 10, 11, 12, 13, 14, 15), bf16x8);
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
    for (int ct = 0; ct < G::CT; ++ct) {
      const int c = ct * 32 + l32;
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(Vt + c * kBN + 8 * vt_chunk(c, 2 * kk + hi));
      acc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kk], acc[ct], 0, 0, 0);
    }
  }
}

template <int D, bool OF32>
__global__ __launch_bounds__(kThreads) void attn_fwd_kernel(FwdArgs a, int n_qtiles, int xcd_remap) {
  using G = Geom<D>;
  __shared__ __attribute__((aligned(16))) __bf16 Ks[G::K_ELEMS];
  __shared__ __attribute__((aligned(16))) __bf16 Vt[G::V_ELEMS];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;

  // Workgroups are dispatched round-robin over the 8 XCDs; give each XCD a contiguous range of (batch, head)
  // slices so that a slice's K/V tiles are re-read from one L2. Within a slice, the heaviest causal tile
  // (last query rows) goes first.
  int64_t w = blockIdx.x;
  if (xcd_remap) w = (w & 7) * ((int64_t)gridDim.x >> 3) + (w >> 3);
  const int64_t bh = w / n_qtiles;
  const int qt = n_qtiles - 1 - (int)(w % n_qtiles);
  const int q0 = qt * kBM;

  const __bf16* Q = reinterpret_cast<const __bf16*>(a.q) + bh * (int64_t)a.Nq * D;
  const __bf16* K = reinterpret_cast<const __bf16*>(a.k) + bh * (int64_t)a.Nk * D;
  const __bf16* V = reinterpret_cast<const __bf16*>(a.v) + bh * (int64_t)a.Nk * D;

  const int qlast = min(q0 + kBM, a.Nq) - 1;
  const int kend = a.causal ? min(a.Nk, qlast + a.diag + 1) : a.Nk;
  const int ntiles = kend > 0 ? (kend + kBN - 1) / kBN : 0;
  const int kfull = a.causal ? min(a.Nk, q0 + a.diag + 1) : a.Nk;   // keys visible to every row of the tile
  const int nfull = kfull > 0 ? kfull / kBN : 0;

  const int qi = q0 + wave * 32 + l32;     // this lane's query row
  bf16x8 qf[G::KSTEPS];
#pragma unroll
  for (int kc = 0; kc < G::KSTEPS; ++kc) {
    const int c = kc * 16 + 8 * hi;
    bf16x8 x = {};
    if (qi < a.Nq && c < D) x = *reinterpret_cast<const bf16x8*>(Q + (int64_t)qi * D + c);
    qf[kc] = x;
  }
  if (D < G::DP) {  // zero the padded head-dim columns once; tile stores never touch them
    for (int e = tid; e < kBN * (G::DP - D); e += kThreads)
      Ks[(e / (G::DP - D)) * G::KROW + D + e % (G::DP - D)] = __bf16(0.0f);
    for (int e = tid; e < (G::DP - D) * kBN; e += kThreads) Vt[D * kBN + e] = __bf16(0.0f);
  }

  f32x16 acc[G::CT];
#pragma unroll
  for (int ct = 0; ct < G::CT; ++ct) acc[ct] = f32x16{};
  float m_run = -INFINITY, l_run = 0.0f;
  const int row_lim = (a.causal ? min(qi + a.diag, a.Nk - 1) : a.Nk - 1) - 8 * hi;

  TileRegs<D> regs;
  if (ntiles > 0) load_tile<D>(regs, K, V, 0, a.Nk, tid);
  for (int t = 0; t < ntiles; ++t) {
    __syncthreads();
    store_tile<D>(regs, Ks, Vt, tid);
    __syncthreads();
    if (t + 1 < ntiles) load_tile<D>(regs, K, V, (t + 1) * kBN, a.Nk, tid);
    if (t < nfull)
      compute_tile<D, false>(Ks, Vt, qf, acc, m_run, l_run, 0, a.scale_log2, l32, hi);
    else
      compute_tile<D, true>(Ks, Vt, qf, acc, m_run, l_run, row_lim - t * kBN, a.scale_log2, l32, hi);
  }

  // Epilogue: O = acc / l, lse = ln2 * (m + log2 l); a row with no visible key gives (0, -inf).
  const float l_tot = wave_pair_sum(l_run);
  if (qi >= a.Nq) return;
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  if (hi == 0)
    a.lse[bh * (int64_t)a.Nq + qi] =
        l_tot > 0.0f ? (m_run + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f : -INFINITY;
  // Register r of O^T tile ct holds head-dim column 32*ct + 8*(r/4) + 4*hi + r%4 of row qi.
#pragma unroll
  for (int ct = 0; ct < G::CT; ++ct) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int c = ct * 32 + 8 * g + 4 * hi;
      if (c >= D) continue;
      f32x4 y = {acc[ct][4 * g] * inv, acc[ct][4 * g + 1] * inv, acc[ct][4 * g + 2] * inv, acc[ct][4 * g + 3] * inv};
      if (OF32) {
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.o) + (bh * (int64_t)a.Nq + qi) * D + c) = y;
      } else {
        *reinterpret_cast<bf16x4*>(reinterpret_cast<__bf16*>(a.o) + (bh * (int64_t)a.Nq + qi) * D + c) =
            __builtin_convertvector(y, bf16x4);
      }
    }
  }
}

template <int D, bool OF32>
hipError_t launch_d(const FwdArgs& a, hipStream_t stream) {
  const int n_qtiles = (a.Nq + kBM - 1) / kBM;
  const int64_t total = (int64_t)n_qtiles * a.BH;
  if (total > 0x7fffffff) return hipErrorInvalidConfiguration;
  const int remap = (total % 8 == 0) ? 1 : 0;
  hipLaunchKernelGGL((attn_fwd_kernel<D, OF32>), dim3((unsigned)total), dim3(kThreads), 0, stream, a, n_qtiles,
                     remap);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd_bf16(const FwdArgs& a, int d, int o_f32, hipStream_t stream) {
  switch (d) {
    case 128: return o_f32 ? launch_d<128, true>(a, stream) : launch_d<128, false>(a, stream);
    case 64: return o_f32 ? launch_d<64, true>(a, stream) : launch_d<64, false>(a, stream);
    case 24: return o_f32 ? launch_d<24, true>(a, stream) : launch_d<24, false>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ebattn
