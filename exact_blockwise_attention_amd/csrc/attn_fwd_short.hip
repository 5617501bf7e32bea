// Exact attention forward for short sequences (at most 16 queries and 16 keys per (batch, head) slice),
// bf16 operands, fp32 arithmetic.
//
// The multi-axis layout of "Mosaic多轴注意力分片：突破Transformer长序列处理瓶颈" §2.2/§3.1 attends over a small
// axis (a handful of features) for every row of a huge table: millions of independent tiny slices. Tiling
// one slice onto MFMA would waste almost all of it, and the job is HBM-bound anyway, so a workgroup takes
// many consecutive slices at once: it copies their K and V (contiguous in memory) into LDS with 16-byte
// coalesced loads, then every lane computes one query row exactly (all scores, max, exp, sum, weighted
// sum of V) with fp32 arithmetic; the scores take the bf16 products in pairs (packed dot, fp32 sum).
#include "internal.h"

namespace ebattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
constexpr int kThreads = 256;

template <int D, bool OF32>
__global__ __launch_bounds__(kThreads) void attn_fwd_short_kernel(FwdArgs a, int seqs_per_wg) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __bf16* Kl = reinterpret_cast<__bf16*>(smem);
  __bf16* Vl = Kl + (int64_t)seqs_per_wg * a.Nk * D;
  const int tid = threadIdx.x;
  const int64_t bh0 = (int64_t)blockIdx.x * seqs_per_wg;
  const int nseq = (int)min<int64_t>(seqs_per_wg, a.BH - bh0);

  // This lane's query row is loaded first, so that its latency overlaps the staging of K and V. K and V are
  // streamed once, with non-temporal loads (the 48-byte query and output rows of neighbouring lanes share cache
  // lines, so those accesses stay ordinary).
  const int s = tid / a.Nq, i = tid % a.Nq;
  const bool live = s < nseq;
  const int64_t bh = bh0 + (live ? s : 0);
  const __bf16* qrow = reinterpret_cast<const __bf16*>(a.q) + (bh * a.Nq + (live ? i : 0)) * D;
  bf16x8 qv[D / 8];
#pragma unroll
  for (int c = 0; c < D / 8; ++c) qv[c] = reinterpret_cast<const bf16x8*>(qrow)[c];

  // Stage K and V of this workgroup's slices in LDS (query slice bh reads key/value slice bh / kv_group; with
  // one key/value head per query head the slices are contiguous).
  const int per_slice = a.Nk * (D / 8);
  const int chunks = nseq * per_slice;
  const u32x4* Kg = reinterpret_cast<const u32x4*>(a.k);
  const u32x4* Vg = reinterpret_cast<const u32x4*>(a.v);
  for (int e = tid; e < chunks; e += kThreads) {
    const int se = e / per_slice;
    const int64_t src = ((bh0 + se) / a.kv_group) * (int64_t)per_slice + (e - se * per_slice);
    reinterpret_cast<u32x4*>(Kl)[e] = __builtin_nontemporal_load(Kg + src);
    reinterpret_cast<u32x4*>(Vl)[e] = __builtin_nontemporal_load(Vg + src);
  }
  __syncthreads();

  // The output rows (one per lane, D values) go out through LDS when the workgroup's rows fit in the K/V staging
  // area: they are one contiguous range in memory, which then leaves as full 16-byte vectors with non-temporal
  // stores instead of each lane's short row on its own. Otherwise each lane stores its row.
  constexpr int kOutBytes = D * (OF32 ? 4 : 2);
  const bool stage_out = (int64_t)a.Nq * kOutBytes <= 2LL * a.Nk * D * 2;
  float acc[D];
  float inv = 0.0f;
  if (live) {
    const __bf16* Ks = Kl + (int64_t)s * a.Nk * D;
    const __bf16* Vs = Vl + (int64_t)s * a.Nk * D;
    const int lim = a.causal ? min(i + a.diag, a.Nk - 1) : a.Nk - 1;   // last visible key of this row
    const int low = a.causal ? i + a.lo : 0;                            // first key of its sliding window

    // Scores with packed bf16 dot products (v_dot2_f32_bf16: two exact bf16 products added in fp32), two
    // accumulators per key for a shorter dependency chain.
    float sc[kShortMax];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < kShortMax; ++j) {
      sc[j] = -INFINITY;
      if (j <= lim && j >= low) {
        float d0 = 0.0f, d1 = 0.0f;
#pragma unroll
        for (int c = 0; c < D / 8; ++c) {
          const bf16x8 kx = *reinterpret_cast<const bf16x8*>(Ks + j * D + 8 * c);
          d0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(qv[c], qv[c], 0, 1),
                                               __builtin_shufflevector(kx, kx, 0, 1), d0, false);
          d1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(qv[c], qv[c], 2, 3),
                                               __builtin_shufflevector(kx, kx, 2, 3), d1, false);
          d0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(qv[c], qv[c], 4, 5),
                                               __builtin_shufflevector(kx, kx, 4, 5), d0, false);
          d1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(qv[c], qv[c], 6, 7),
                                               __builtin_shufflevector(kx, kx, 6, 7), d1, false);
        }
        sc[j] = (d0 + d1) * a.scale_log2;
        mx = fmaxf(mx, sc[j]);
      }
    }
#pragma unroll
    for (int c = 0; c < D; ++c) acc[c] = 0.0f;
    float l = 0.0f;
    if (mx != -INFINITY) {
#pragma unroll
      for (int j = 0; j < kShortMax; ++j) {
        if (j <= lim && j >= low) {
          const float p = __builtin_amdgcn_exp2f(sc[j] - mx);
          l += p;
#pragma unroll
          for (int c = 0; c < D; c += 8) {
            const f32x8 vx = __builtin_convertvector(*reinterpret_cast<const bf16x8*>(Vs + j * D + c), f32x8);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[c + e] = __builtin_fmaf(p, vx[e], acc[c + e]);
          }
        }
      }
    }
    inv = l > 0.0f ? 1.0f / l : 0.0f;
    a.lse[bh * a.Nq + i] = l > 0.0f ? (mx + __builtin_amdgcn_logf(l)) * 0.69314718055994531f : -INFINITY;
  }
  auto put = [&](unsigned char* row) {
#pragma unroll
    for (int c = 0; c < D; c += 4) {
      const f32x4 y = {acc[c] * inv, acc[c + 1] * inv, acc[c + 2] * inv, acc[c + 3] * inv};
      if (OF32)
        *reinterpret_cast<f32x4*>(row + c * 4) = y;
      else
        *reinterpret_cast<bf16x4*>(row + c * 2) = __builtin_convertvector(y, bf16x4);
    }
  };
  if (stage_out) {
    __syncthreads();   // every lane is done reading K and V: the staging area takes the output rows
    if (live) put(smem + (int64_t)(s * a.Nq + i) * kOutBytes);
    __syncthreads();
    const int nchunks = nseq * a.Nq * (kOutBytes / 16);
    u32x4* og = reinterpret_cast<u32x4*>(reinterpret_cast<unsigned char*>(a.o) + bh0 * a.Nq * kOutBytes);
    for (int e = tid; e < nchunks; e += kThreads)
      __builtin_nontemporal_store(reinterpret_cast<const u32x4*>(smem)[e], og + e);
  } else if (live) {
    put(reinterpret_cast<unsigned char*>(a.o) + (bh * a.Nq + i) * kOutBytes);
  }
}

template <int D, bool OF32>
hipError_t launch_d(const FwdArgs& a, hipStream_t stream) {
  constexpr int64_t kLdsBudget = 64 * 1024;
  int64_t spw = kThreads / a.Nq;
  const int64_t per_seq = 2LL * a.Nk * D * 2;   // K and V bytes of one slice
  if (spw * per_seq > kLdsBudget) spw = kLdsBudget / per_seq;
  if (spw < 1) return hipErrorInvalidValue;
  const int64_t blocks = (a.BH + spw - 1) / spw;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((attn_fwd_short_kernel<D, OF32>), dim3((unsigned)blocks), dim3(kThreads),
                     (size_t)(spw * per_seq), stream, a, (int)spw);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd_short(const FwdArgs& a, int d, int o_f32, hipStream_t stream) {
  if (a.Nq > kShortMax || a.Nk > kShortMax || a.Nq < 1 || a.Nk < 1) return hipErrorInvalidValue;
  switch (d) {
    case 128: return o_f32 ? launch_d<128, true>(a, stream) : launch_d<128, false>(a, stream);
    case 64: return o_f32 ? launch_d<64, true>(a, stream) : launch_d<64, false>(a, stream);
    case 24: return o_f32 ? launch_d<24, true>(a, stream) : launch_d<24, false>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ebattn
