// Exact blockwise attention forward, bf16 operands on gfx950 MFMA, fp32 online softmax.
//
// Method: "深度学习注意力机制优化与FlashAttention实践" §4.2 (per query block, loop over key/value blocks, keep a
// running maximum and running sum, normalise at the end) with the accumulator rescaled whenever the reference
// maximum moves -- the decomposition of "架构层解决方案 - Sparse Attention与Ring Attention", Ring Attention /
// 核心创新, applied one key tile at a time. Causal masking by global position ("深度学习注意力机制优化与
// FlashAttention实践" §5.1) arrives here as a diagonal offset: key j is visible to query i iff j <= i + diag.
// Only O and the per-row log-sum-exp are written to HBM ("注意力机制演进", section FlashAttention).
//
// Work decomposition (one workgroup = 4 waves = 128 query rows of one (batch, head)):
//   * each wave owns 32 query rows; its Q fragment stays in VGPRs for the whole key loop;
//   * 64-key K and V tiles are copied HBM -> LDS by the buffer unit itself (buffer_load ... lds, 16 bytes per
//     lane, out-of-range rows read as zero), double-buffered so that tile t+1 streams in while tile t is
//     consumed; one workgroup barrier per tile;
//   * the wave computes S^T = K . Q^T (32 keys x 32 queries per MFMA 32x32x16). In that orientation one lane
//     owns one query row (the MFMA output column): the row maximum and sum are in-lane reductions plus one
//     exchange with the partner lane (lane ^ 32), and the rescale factor is a per-lane scalar;
//   * the keys of each 32-key chunk sit in LDS with bits 2 and 3 of their index swapped. Read back in natural
//     order as the MFMA A operand, this leaves lane l's 16 output registers holding, in order, 8 consecutive
//     keys of each 16-key half -- the B-operand layout of the next product O^T = V^T . P^T, so P goes from the
//     S accumulator to the P.V MFMA without leaving the registers;
//   * V stays row-major in LDS; the V^T operand is gathered with the LDS transpose read ds_read_b64_tr_b16
//     (within each 16-lane group, lane i receives column i of a 4-row x 16-column block);
//   * K rows and V rows are XOR-swizzled per 16-byte chunk so that both the operand reads and the LDS writes
//     of the copy spread over all banks;
//   * O is normalised by the sum of the same bf16-rounded weights that enter P.V (packed bf16 dot with (1,1));
//     the log-sum-exp uses the sum of the fp32 weights;
//   * the reference maximum is only moved when a row's new maximum exceeds it by more than 8 (log2 units), so
//     most tiles skip the rescale of the accumulator; the weights stay below 2^8 and the result is unchanged
//     (the final normalisation uses the same reference).
#include <type_traits>

#include "internal.h"

namespace ebattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kBM = 128;       // query rows per workgroup (4 waves x 32)
constexpr int kBN = 64;        // keys per K/V tile
constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int32_t kRsrcWord3 = 0x00020000;     // raw buffer, 32-bit data format (gfx9 family)
constexpr uint32_t kOutOfRange = 0x7ffffff0u;  // a buffer offset past every num_records: the load returns 0
constexpr float kRescaleSlack = 8.0f;          // log2 units the running maximum may exceed the reference by

template <int D>
struct Geom {
  static constexpr int DP = (D + 31) / 32 * 32;   // head dim padded to the 32-row tiles of O^T
  static constexpr int KSTEPS = DP / 16;          // MFMA k-steps of S^T = K . Q^T
  static constexpr int CT = DP / 32;              // 32-row tiles of O^T
  static constexpr int ROW_BYTES = DP * 2;        // one K or V row in LDS
  static constexpr int CPR = DP / 8;              // 16-byte chunks per LDS row
  static constexpr int CPG = D / 8;               // 16-byte chunks per global row (the rest reads as zero)
  static constexpr int TILE_BYTES = kBN * ROW_BYTES;
  static constexpr int INSTR = TILE_BYTES / 1024; // wave-wide 16-byte-per-lane copies per tile
  static constexpr int ROWS_PER_INSTR = 1024 / ROW_BYTES;
  static_assert(INSTR % kWaves == 0, "tile copy must split evenly over the waves");
};

// Chunk swizzles (see the header comment). K: row p of the tile; V: row j of the tile.
template <int D>
__device__ __forceinline__ int k_swz(int p) { return D == 24 ? (p >> 1) & 3 : p & 7; }
template <int D>
__device__ __forceinline__ int v_swz(int j) { return D == 24 ? 2 * ((j >> 1) & 1) : 2 * (j & 3); }
// key held by LDS row p of a tile: bits 2 and 3 swapped inside each 32-key chunk (an involution)
__device__ __forceinline__ int key_of_row(int p) { return (p & ~12) | ((p & 4) << 1) | ((p & 8) >> 1); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int32_t n = (int32_t)(bytes < 0 ? 0 : (bytes > 0x7fffffff ? 0x7fffffff : bytes));
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, kRsrcWord3);
}

// Max / sum over the lane pair (l, l ^ 32) that shares a query row. After the swap one of the two results holds
// the partner's value and the other this lane's, whichever way the halves are exchanged.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Issue this wave's share of the HBM -> LDS copy of K and V tile rows [j0, j0 + kBN).
template <int D>
__device__ __forceinline__ void issue_tile_copy(const __bf16* K, const __bf16* V, int j0, int Nk, char* ks, char* vs,
                                                int wave, int lane) {
  using G = Geom<D>;
  const int rows_valid = min(kBN, Nk - j0);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(K + (int64_t)j0 * D, (int64_t)rows_valid * D * 2);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(V + (int64_t)j0 * D, (int64_t)rows_valid * D * 2);
  const int sub = lane / G::CPR, pos = lane % G::CPR;
#pragma unroll
  for (int i = 0; i < G::INSTR / kWaves; ++i) {
    const int instr = wave * (G::INSTR / kWaves) + i;
    const int row = instr * G::ROWS_PER_INSTR + sub;
    const int mk = pos ^ k_swz<D>(row);
    const int mv = pos ^ v_swz<D>(row);
    const uint32_t ok = mk < G::CPG ? (uint32_t)((key_of_row(row) * D + mk * 8) * 2) : kOutOfRange;
    const uint32_t ov = mv < G::CPG ? (uint32_t)((row * D + mv * 8) * 2) : kOutOfRange;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(ks + instr * 1024), 16, ok, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(vs + instr * 1024), 16, ov, 0, 0, 0);
  }
}

__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// One 64-key tile for this wave's 32 query rows. KB / VB: byte offsets of the tile's K and V buffers in LDS
// (compile-time, so they fold into the instructions' offset fields). `partial` tiles apply the mask.
template <int D, int KB, int VB>
__device__ __forceinline__ void compute_tile(const char* smem, const bf16x8 (&qf)[Geom<D>::KSTEPS],
                                             f32x16 (&acc)[Geom<D>::CT], float& m_ref, float& l_run, float& lq_run, bool partial,
                                             int lim, float scale_log2, int k_row, int k_xor, int hi,
                                             const int (&v_addr)[Geom<D>::CT]) {
  using G = Geom<D>;
  // S^T chunks: keys 0..31 (s0) and 32..63 (s1) of the tile against this wave's 32 query rows.
  f32x16 s0 = {}, s1 = {};
#pragma unroll
  for (int kc = 0; kc < G::KSTEPS; ++kc) {
    const char* p = smem + KB + k_row + 16 * ((2 * kc + hi) ^ k_xor);
    const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(p);
    const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(p + 32 * G::ROW_BYTES);
    s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[kc], s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[kc], s1, 0, 0, 0);
  }
  // Register r of lane l holds key 16*(r/8) + 8*(l/32) + r%8 of its 32-key chunk, for query row l%32.
  if (partial) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kr = 16 * (r >> 3) + (r & 7);
      if (kr > lim) s0[r] = -INFINITY;
      if (kr + 32 > lim) s1[r] = -INFINITY;
    }
  }
  // IEEE maximum (v_maximum3_f32): no NaN quieting of the MFMA results is needed before it.
  float mx = __builtin_elementwise_maximum(s0[0], s1[0]);
#pragma unroll
  for (int r = 1; r < 16; ++r) mx = __builtin_elementwise_maximum(mx, __builtin_elementwise_maximum(s0[r], s1[r]));
  const float mt = pair_max(mx) * scale_log2;
  const bool need = mt > m_ref + kRescaleSlack;
  const float m_new = need ? mt : m_ref;
  const float alpha = need ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.0f;
  m_ref = m_new;
  const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
  float psum = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    s0[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[r], scale_log2, -m_use));
    s1[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[r], scale_log2, -m_use));
    psum += s0[r] + s1[r];
  }
  l_run = __builtin_fmaf(alpha, l_run, psum);
  if (__builtin_amdgcn_ballot_w64(need)) {
#pragma unroll
    for (int ct = 0; ct < G::CT; ++ct) acc[ct] *= alpha;
  }

  bf16x8 pb[4];
  pb[0] = __builtin_convertvector(__builtin_shufflevector(s0, s0, 0, 1, 2, 3, 4, 5, 6, 7), bf16x8);
  pb[1] = __builtin_convertvector(__builtin_shufflevector(s0, s0, 8, 9, 10, 11, 12, 13, 14, 15), bf16x8);
  pb[2] = __builtin_convertvector(__builtin_shufflevector(s1, s1, 0, 1, 2, 3, 4, 5, 6, 7), bf16x8);
  pb[3] = __builtin_convertvector(__builtin_shufflevector(s1, s1, 8, 9, 10, 11, 12, 13, 14, 15), bf16x8);
  // Two row sums: l_run over the fp32 weights gives the log-sum-exp; lq_run over the bf16-rounded weights that
  // enter P.V (one packed dot with (1, 1) per pair) normalises O, so numerator and denominator use the same
  // weights and a constant V comes back exactly.
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  float psum0 = 0.0f, psum1 = 0.0f;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    psum0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[kk], pb[kk], 0, 1), ones, psum0, false);
    psum1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[kk], pb[kk], 2, 3), ones, psum1, false);
    psum0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[kk], pb[kk], 4, 5), ones, psum0, false);
    psum1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[kk], pb[kk], 6, 7), ones, psum1, false);
  }
  lq_run = __builtin_fmaf(alpha, lq_run, psum0 + psum1);
  // V^T operand via two transpose reads: slots 0-3 from key rows +0..3, slots 4-7 from +4..7 of the 8-key group.
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
    for (int ct = 0; ct < G::CT; ++ct) {
      const char* p = smem + VB + v_addr[ct] + kk * 16 * G::ROW_BYTES;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
      const i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 4 * G::ROW_BYTES));
      const bf16x8 av = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
      acc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[kk], acc[ct], 0, 0, 0);
    }
  }
}

template <int D, bool OF32>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_kernel(FwdArgs a, int n_qtiles, int xcd_remap) {
  using G = Geom<D>;
  __shared__ __attribute__((aligned(1024))) char smem[4 * G::TILE_BYTES];   // K0 V0 K1 V1

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;

  // Workgroups are dispatched round-robin over the 8 XCDs; give each XCD a contiguous range of (batch, head)
  // slices so that a slice's K/V tiles are re-read from one L2. Within a slice the heaviest causal tile (the
  // last query rows) goes first.
  int64_t w = blockIdx.x;
  if (xcd_remap) w = (w & 7) * ((int64_t)gridDim.x >> 3) + (w >> 3);
  const int64_t bh = w / n_qtiles;
  const int qt = n_qtiles - 1 - (int)(w % n_qtiles);
  const int q0 = qt * kBM;

  const __bf16* Q = reinterpret_cast<const __bf16*>(a.q) + (bh * (int64_t)a.Nq + q0) * D;
  const __bf16* K = reinterpret_cast<const __bf16*>(a.k) + bh * (int64_t)a.Nk * D;
  const __bf16* V = reinterpret_cast<const __bf16*>(a.v) + bh * (int64_t)a.Nk * D;

  const int qlast = min(q0 + kBM, a.Nq) - 1;
  const int kend = a.causal ? min(a.Nk, qlast + a.diag + 1) : a.Nk;
  const int ntiles = kend > 0 ? (kend + kBN - 1) / kBN : 0;
  const int kfull = a.causal ? min(a.Nk, q0 + a.diag + 1) : a.Nk;   // keys visible to every row of the tile
  const int nfull = kfull > 0 ? kfull / kBN : 0;
  // keys any row of this wave can see end here: this wave skips the compute of later tiles (it still copies)
  const int wave_kend = a.causal ? min(a.Nk, q0 + wave * 32 + 31 + a.diag + 1) : a.Nk;

  if (ntiles > 0) issue_tile_copy<D>(K, V, 0, a.Nk, smem, smem + G::TILE_BYTES, wave, lane);

  // Q^T fragment (B operand): lane holds query row 32*wave + l32, head-dim columns 16*kc + 8*hi .. +7.
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(Q, (int64_t)min(kBM, a.Nq - q0) * D * 2);
  bf16x8 qf[G::KSTEPS];
#pragma unroll
  for (int kc = 0; kc < G::KSTEPS; ++kc) {
    const int c = kc * 16 + 8 * hi;
    const uint32_t off = c < D ? (uint32_t)(((wave * 32 + l32) * D + c) * 2) : kOutOfRange;
    qf[kc] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0));
  }

  // Per-lane LDS addressing, fixed for the whole loop.
  const int k_row = l32 * G::ROW_BYTES;
  const int k_xor = k_swz<D>(l32);
  int v_addr[G::CT];
  {
    const int g2 = (lane >> 4) & 1, a4 = (lane & 15) >> 2, b4 = lane & 3;
    const int row = 8 * hi + a4;                      // key row of the first transpose read (kk = 0)
#pragma unroll
    for (int ct = 0; ct < G::CT; ++ct) {
      const int m = 4 * ct + 2 * g2 + (b4 >> 1);     // 16-byte chunk of columns 32*ct + 16*g2 + 4*b4 .. +3
      v_addr[ct] = row * G::ROW_BYTES + 16 * (m ^ v_swz<D>(row)) + 8 * (b4 & 1);
    }
  }

  f32x16 acc[G::CT];
#pragma unroll
  for (int ct = 0; ct < G::CT; ++ct) acc[ct] = f32x16{};
  float m_ref = -INFINITY, l_run = 0.0f, lq_run = 0.0f;
  const int qi = q0 + wave * 32 + l32;     // this lane's query row
  const int row_lim = (a.causal ? min(qi + a.diag, a.Nk - 1) : a.Nk - 1) - 8 * hi;

  // Tile t lives in buffer t & 1. Before tile t is read: this wave's copies have landed (vmcnt), then the
  // barrier guarantees every wave's copies have landed and every wave has finished tile t-1, whose buffer the
  // copy of tile t+1 then overwrites.
  auto step = [&](auto buf_tag, int t) {
    constexpr int B = decltype(buf_tag)::value;
    constexpr int KB = B ? 2 * G::TILE_BYTES : 0, VB = KB + G::TILE_BYTES;
    constexpr int KN = B ? 0 : 2 * G::TILE_BYTES, VN = KN + G::TILE_BYTES;
    wait_vmem_all();
    __syncthreads();
    if (t + 1 < ntiles) issue_tile_copy<D>(K, V, (t + 1) * kBN, a.Nk, smem + KN, smem + VN, wave, lane);
    if (t * kBN < wave_kend)
      compute_tile<D, KB, VB>(smem, qf, acc, m_ref, l_run, lq_run, t >= nfull, row_lim - t * kBN, a.scale_log2, k_row,
                              k_xor, hi, v_addr);
  };
  for (int t = 0; t < ntiles; t += 2) {
    step(std::integral_constant<int, 0>{}, t);
    if (t + 1 < ntiles) step(std::integral_constant<int, 1>{}, t + 1);
  }

  // Epilogue: O = acc / l, lse = ln2 * (m + log2 l); a row with no visible key gives (0, -inf).
  const float l_tot = pair_sum(l_run);
  const float lq_tot = pair_sum(lq_run);
  const float inv = lq_tot > 0.0f ? 1.0f / lq_tot : 0.0f;
  if (hi == 0 && qi < a.Nq)
    a.lse[bh * (int64_t)a.Nq + qi] =
        l_tot > 0.0f ? (m_ref + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f : -INFINITY;
  const int64_t o_rows = min(kBM, a.Nq - q0);
  const int local_row = wave * 32 + l32;
  // Register r of O^T tile ct holds head-dim column 32*ct + 8*(r/4) + 4*hi + r%4 of this lane's row; the
  // buffer range drops the stores of rows past Nq.
  if (OF32) {
    const __amdgpu_buffer_rsrc_t ro =
        make_rsrc(reinterpret_cast<float*>(a.o) + (bh * (int64_t)a.Nq + q0) * D, o_rows * D * 4);
#pragma unroll
    for (int ct = 0; ct < G::CT; ++ct)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = ct * 32 + 8 * g + 4 * hi;
        if (c >= D) continue;
        const f32x4 y = {acc[ct][4 * g] * inv, acc[ct][4 * g + 1] * inv, acc[ct][4 * g + 2] * inv,
                         acc[ct][4 * g + 3] * inv};
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, y), ro, (uint32_t)((local_row * D + c) * 4), 0, 0);
      }
  } else {
    const __amdgpu_buffer_rsrc_t ro =
        make_rsrc(reinterpret_cast<__bf16*>(a.o) + (bh * (int64_t)a.Nq + q0) * D, o_rows * D * 2);
#pragma unroll
    for (int ct = 0; ct < G::CT; ++ct)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = ct * 32 + 8 * g + 4 * hi;
        if (c >= D) continue;
        const f32x4 y = {acc[ct][4 * g] * inv, acc[ct][4 * g + 1] * inv, acc[ct][4 * g + 2] * inv,
                         acc[ct][4 * g + 3] * inv};
        const bf16x4 b = __builtin_convertvector(y, bf16x4);
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, b), ro, (uint32_t)((local_row * D + c) * 2), 0, 0);
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
