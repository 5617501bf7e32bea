// Exact attention backward, bf16 operands on gfx950 MFMA, fp32 accumulation.
//
// Method: "深度学习注意力机制优化与FlashAttention实践" §4.1 (item 3) and §3.3 -- the backward recomputes the
// attention weights tile by tile from the saved per-row log-sum-exp instead of storing them. With
// P_ij = exp(scale q_i.k_j - lse_i) and delta_i = dO_i . O_i (lse and O over the full key set), the gradient of
// exact attention is
//   dV_j = sum_i P_ij dO_i,  dS_ij = P_ij (dO_i . V_j - delta_i),  dQ_i = scale sum_j dS_ij K_j,
//   dK_j = scale sum_i dS_ij Q_i,
// a sum of independent (query tile, key tile) terms. That is also what lets one share of a ring run the
// backward block by block with the global lse and delta and add up the blocks' contributions.
//
// Two kernels, so that no gradient needs atomics:
//   * the dq kernel (runs first) owns 128 query rows per workgroup, 32 per wave with Q and dO held in VGPRs,
//     and walks the key tiles like the forward: S^T = K Q^T and dP^T = V dO^T put one query row in each lane
//     (its lse and delta are per-lane scalars), dS^T is formed in registers and dQ^T += K^T dS^T. Before the
//     loop it forms delta from O and dO and writes it out for the second kernel.
//   * the dk/dv kernel owns 128 keys of one key/value head, 32 per wave, and walks the query tiles of every
//     query head that reads that key/value head: S = Q K^T and dP = dO V^T put one key in each lane, and
//     dV^T += dO^T P, dK^T += Q^T dS. At d = 64 and 128 it runs eight waves with K and V in LDS, two waves per
//     key range splitting each tile's rows; at d = 24 four waves with K and V in VGPRs.
// Operand layout, shared by both kernels: the rows of the operand read from LDS by rows are taken in an order
// with bits 2 and 3 of the row index swapped, which leaves the 32x32 MFMA results in registers already laid out
// as the B operand of the next product (whose k index runs over those rows). The LDS tiles (64 rows of bf16)
// are read both by rows (16 bytes per lane, contraction over the head dim) and transposed
// (ds_read_b64_tr_b16, contraction over the rows); one XOR swizzle of the 16-byte chunks of a row keeps both
// patterns free of bank conflicts on the 64 four-byte banks. Tiles are copied HBM -> LDS by the buffer unit
// (buffer_load ... lds), double-buffered, one barrier per tile.
#include <type_traits>
#include <utility>

#include "internal.h"

namespace ebattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kBT = 64;                        // rows per LDS tile (keys in the dq kernel, queries in dk/dv)
constexpr int kWaves = 4;                      // waves per workgroup, 32 owned rows each
constexpr int kOwn = 32 * kWaves;              // owned rows per workgroup
constexpr int32_t kRsrcWord3 = 0x00020000;     // raw buffer, 32-bit data format (gfx9 family)
constexpr float kLog2e = 1.4426950408889634f;
constexpr uint32_t kOutOfRange = 0x7ffffff0u;  // a buffer offset past every num_records: the load returns 0

// Geometry of head dim D (24, 64 or 128). D = 24 runs padded to 32: its LDS rows, MFMA k-steps and result tiles
// have 32 columns, and the padding columns read as zero and are never stored.
template <int D>
struct BG {
  static_assert(D == 24 || D == 64 || D == 128, "head dim 24, 64 or 128");
  static constexpr int DP = (D + 31) / 32 * 32;    // padded head dim
  static constexpr int KSTEPS = DP / 16;           // MFMA k-steps over the head dim
  static constexpr int CT = DP / 32;               // 32-row tiles of a transposed (d x rows) result
  static constexpr int RB = DP * 2;                // bytes of one bf16 row in LDS
  static constexpr int CPR = DP / 8;               // 16-byte chunks per LDS row
  static constexpr int CPG = D / 8;                // 16-byte chunks per row in memory (the rest read as zero)
  static constexpr int TILE = kBT * RB;
  static constexpr int ROWS_PER_INSTR = 1024 / RB; // rows per wave-wide 16-byte-per-lane copy
};

// Chunk swizzle of LDS row `row` (XOR on the 16-byte chunk index). Row reads: 16 consecutive lanes read one chunk
// index of 16 rows that cover row & 15 = 0..15 -> the swizzle must be a bijection of those 16 rows onto distinct
// bank groups. Transposed reads: 32 lanes read 4 consecutive rows (an aligned group) x 4 chunks of an aligned
// group of 4 -> the 4 rows must land in 4 different 64-byte quarters of the 256-byte bank row.
// (Rows of 64 bytes, at D = 24: four rows share a bank row, so row & 3 already picks the quarter and the swizzle
// only has to separate the four rows of a 16-row group that share a quarter.)
template <int D>
__device__ __forceinline__ int swz(int row) {
  return D == 128 ? (((row & 3) << 2) | ((row >> 2) & 3))
       : D == 64  ? ((((row >> 1) & 1) << 2) | ((row >> 2) & 3))
                  : ((row >> 2) & 3);
}
// bits 2 and 3 swapped (an involution)
__device__ __forceinline__ int perm_row(int p) { return (p & ~12) | ((p & 4) << 1) | ((p & 8) >> 1); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int32_t n = (int32_t)(bytes < 0 ? 0 : (bytes > 0x7fffffff ? 0x7fffffff : bytes));
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, kRsrcWord3);
}

// min(max(x, 0), hi) for a wave-uniform x, kept in a scalar register: the vector ALU's med3 would otherwise take
// it, and a buffer resource built from a vector register costs a loop over the lanes at every use.
__device__ __forceinline__ int uniform_clamp(int x, int hi) {
  return __builtin_amdgcn_readfirstlane(x < 0 ? 0 : (x > hi ? hi : x));
}

__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// An empty asm statement that takes a value in and out of registers: the value counts as produced here, so the
// optimiser cannot move its computation into a later block (it emits no instruction).
__device__ __forceinline__ void pin(bf16x8& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(float& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(bf16x2& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(int& x) { asm volatile("" : "+v"(x)); }

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// This wave's share (of NW waves) of the HBM -> LDS copy of rows [r0, r0 + ROWS) of X (rows_total rows of D
// bf16): natural row order, chunks swizzled. Rows past rows_total read as zero (a tile wholly past the end touches
// no memory).
template <int D, int ROWS = kBT, int NW = kWaves>
__device__ __forceinline__ void copy_tile(const __bf16* X, int r0, int rows_total, char* dst, int wave, int lane) {
  using G = BG<D>;
  constexpr int INSTR = ROWS * G::RB / 1024;       // wave-wide 16-byte-per-lane copies
  static_assert(INSTR % NW == 0, "tile copy must split evenly over the waves");
  constexpr int PER_WAVE = INSTR / NW;
  const int valid = uniform_clamp(rows_total - r0, ROWS);
  // the range is in bytes of the rows in memory (D bf16 each), not of the padded LDS rows
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(X + (int64_t)r0 * D, (int64_t)valid * D * 2);
  const int sub = lane / G::CPR, pos = lane % G::CPR;
#pragma unroll
  for (int i = 0; i < PER_WAVE; ++i) {
    const int instr = wave * PER_WAVE + i;
    const int row = instr * G::ROWS_PER_INSTR + sub;
    const int m = pos ^ swz<D>(row);
    const uint32_t off = m < G::CPG ? (uint32_t)((row * D + m * 8) * 2) : kOutOfRange;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void*)(dst + instr * 1024), 16, off, 0, 0, 0);
  }
}

// Per-lane LDS addressing, fixed for the whole kernel.
template <int D>
struct Lanes {
  int hi;                       // lane / 32: which 8-wide half of each 16-wide k-step this lane supplies
  int row_off;                  // byte offset of this lane's row in a 32-row block: row perm_row(l % 32)
  int row_sw;                   // its chunk swizzle
  int tr[2][BG<D>::CT];         // transposed reads: rows 8*hi + (l%16)/4 and 4 rows further, per 32-column tile
  __device__ explicit Lanes(int lane) {
    using G = BG<D>;
    hi = lane >> 5;
    const int pr = perm_row(lane & 31);
    row_off = pr * G::RB;
    row_sw = swz<D>(pr);
    const int g2 = (lane >> 4) & 1, a4 = (lane & 15) >> 2, b4 = lane & 3;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int row = 8 * hi + 4 * half + a4;
#pragma unroll
      for (int ct = 0; ct < G::CT; ++ct) {
        const int m = 4 * ct + 2 * g2 + (b4 >> 1);   // chunk of columns 32*ct + 16*g2 + 4*b4 .. +3
        tr[half][ct] = row * G::RB + 16 * (m ^ swz<D>(row)) + 8 * (b4 & 1);
      }
    }
  }
};

// Row operand (A of a product contracting over the head dim) from an LDS tile: rows 32*blk + perm_row(l%32),
// head-dim columns 16*ks + 8*hi .. +7.
template <int D>
__device__ __forceinline__ bf16x8 row_frag(const char* t, const Lanes<D>& la, int blk, int ks) {
  const char* p = t + blk * 32 * BG<D>::RB + la.row_off + 16 * ((2 * ks + la.hi) ^ la.row_sw);
  return *reinterpret_cast<const bf16x8*>(p);
}

// Transposed operand (A of a product contracting over the tile rows): head-dim columns 32*ct + l%32, tile rows
// 16*kk + 8*hi .. +7 (two transpose reads of 4 rows each).
template <int D>
__device__ __forceinline__ bf16x8 tr_frag(const char* t, const Lanes<D>& la, int kk, int ct) {
  const char* p = t + kk * 16 * BG<D>::RB;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + la.tr[0][ct]));
  const i16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + la.tr[1][ct]));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7));
}

// B-operand fragments of 32 rows held in VGPRs: lane holds row row0 + l%32, head-dim columns 16*ks + 8*hi .. +7;
// rows past rows_total read as zero.
template <int D>
__device__ __forceinline__ void load_frags(const __bf16* X, int row0, int rows_total, int lane,
                                           bf16x8 (&f)[BG<D>::KSTEPS]) {
  const int valid = uniform_clamp(rows_total - row0, 32);
  const __amdgpu_buffer_rsrc_t r = make_rsrc(X + (int64_t)row0 * D, (int64_t)valid * D * 2);
  const int l32 = lane & 31, hi = lane >> 5;
#pragma unroll
  for (int ks = 0; ks < BG<D>::KSTEPS; ++ks) {
    const int c = 16 * ks + 8 * hi;
    const uint32_t off = c < D ? (uint32_t)((l32 * D + c) * 2) : kOutOfRange;
    f[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
  }
}

// Writes factor * acc for 32 rows (row0 + l%32) of a gradient [rows_total, D] at `out` (fp32 or bf16): register r
// of tile ct holds head-dim column 32*ct + 8*(r/4) + 4*hi + r%4. With `accumulate` (fp32 only) the previous
// contents are added. Rows past rows_total are dropped by the buffer range.
template <int D, bool GF32>
__device__ __forceinline__ void store_grad(void* out, int row0, int rows_total, int lane,
                                           const f32x16 (&acc)[BG<D>::CT], float factor, bool accumulate) {
  const int valid = uniform_clamp(rows_total - row0, 32);
  const int hi = lane >> 5, l32 = lane & 31;
  const __amdgpu_buffer_rsrc_t r =
      GF32 ? make_rsrc(reinterpret_cast<float*>(out) + (int64_t)row0 * D, (int64_t)valid * D * 4)
           : make_rsrc(reinterpret_cast<__bf16*>(out) + (int64_t)row0 * D, (int64_t)valid * D * 2);
#pragma unroll
  for (int ct = 0; ct < BG<D>::CT; ++ct)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int c = 32 * ct + 8 * g + 4 * hi;
      if (c >= D) continue;
      f32x4 y = {acc[ct][4 * g] * factor, acc[ct][4 * g + 1] * factor, acc[ct][4 * g + 2] * factor,
                 acc[ct][4 * g + 3] * factor};
      if constexpr (GF32) {
        const uint32_t off = (uint32_t)((l32 * D + c) * 4);
        if (accumulate) y += __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, y), r, off, 0, 0);
      } else {
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, __builtin_convertvector(y, bf16x4)), r,
                                              (uint32_t)((l32 * D + c) * 2), 0, 0);
      }
    }
}

// lse (natural log) -> the exp2-domain subtrahend of the weights; a row with no visible key (lse = -inf) gets
// +inf so that all of its weights are exactly zero.
__device__ __forceinline__ float lse_to_sub(float lse) { return lse == -INFINITY ? INFINITY : lse * kLog2e; }

// Workgroup -> (slice, tile). Workgroups are dispatched round-robin over the 8 XCDs; each XCD gets a contiguous
// range of slices so that the tiles one slice re-reads stay in one L2.
__device__ __forceinline__ void decode_block(int n_tiles, int xcd_remap, int64_t& slice, int& tile) {
  int64_t w = blockIdx.x;
  if (xcd_remap) w = (w & 7) * ((int64_t)gridDim.x >> 3) + (w >> 3);
  slice = w / n_tiles;
  tile = (int)(w % n_tiles);
}

// ------------------------------------------------------------------------------------------------------------
// dq kernel (and delta): 128 query rows per workgroup, key tiles of 64.

template <int D, bool GF32>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bwd_dq_kernel(BwdArgs a, int n_qtiles, int xcd_remap) {
  using G = BG<D>;
  __shared__ __attribute__((aligned(1024))) char k0[G::TILE];
  __shared__ __attribute__((aligned(1024))) char k1[G::TILE];
  __shared__ __attribute__((aligned(1024))) char v0[G::TILE];
  __shared__ __attribute__((aligned(1024))) char v1[G::TILE];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int64_t bh;
  int qt;
  decode_block(n_qtiles, xcd_remap, bh, qt);
  qt = n_qtiles - 1 - qt;    // the heaviest causal block (the last query rows) first
  const int q0 = qt * kOwn;
  const int64_t kvbh = bh / a.kv_group;
  const __bf16* K = reinterpret_cast<const __bf16*>(a.k) + kvbh * (int64_t)a.Nk * D;
  const __bf16* V = reinterpret_cast<const __bf16*>(a.v) + kvbh * (int64_t)a.Nk * D;
  const int64_t qbase = bh * (int64_t)a.Nq;   // first row of this query slice

  // key-tile range of the block and of this wave (as in the forward)
  const int qlast = min(q0 + kOwn, a.Nq) - 1;
  const int kend = a.causal ? min(a.Nk, qlast + a.diag + 1) : a.Nk;
  const int ntiles = kend > 0 ? (kend + kBT - 1) / kBT : 0;
  const int wrow0 = q0 + wave * 32;
  const int wkfull = a.causal ? min(a.Nk, wrow0 + a.diag + 1) : a.Nk;
  const int nfull = wkfull > 0 ? wkfull / kBT : 0;
  const int wkend = a.causal ? min(a.Nk, wrow0 + 31 + a.diag + 1) : a.Nk;
  const int nt_w = min(ntiles, wkend > 0 ? (wkend + kBT - 1) / kBT : 0);
  const int first_key = a.causal ? q0 + a.lo : 0;
  const int t0 = first_key > 0 ? first_key / kBT : 0;
  const int low_edge = a.causal ? wrow0 + 31 + a.lo : 0;
  const int nlow = low_edge > 0 ? (low_edge + kBT - 1) / kBT : 0;

  if (ntiles > t0) {
    copy_tile<D>(K, t0 * kBT, a.Nk, k0, wave, lane);
    copy_tile<D>(V, t0 * kBT, a.Nk, v0, wave, lane);
  }

  // Q and dO of this wave's rows as B operands; delta_i = dO_i . O_i over this lane's half of the head dim plus
  // its partner lane's half.
  bf16x8 qf[G::KSTEPS], df[G::KSTEPS];
  const __bf16* Qs = reinterpret_cast<const __bf16*>(a.q) + qbase * D;
  const __bf16* dOs = reinterpret_cast<const __bf16*>(a.dout) + qbase * D;
  load_frags<D>(Qs, wrow0, a.Nq, lane, qf);
  load_frags<D>(dOs, wrow0, a.Nq, lane, df);
  const int hi = lane >> 5;
  const int row = wrow0 + (lane & 31);
  float dl = 0.0f;
  {
    const int valid = uniform_clamp(a.Nq - wrow0, 32);
    if (a.o_f32) {
      const __amdgpu_buffer_rsrc_t r = make_rsrc(reinterpret_cast<const float*>(a.o) + (qbase + wrow0) * D,
                                                 (int64_t)valid * D * 4);
#pragma unroll
      for (int ks = 0; ks < G::KSTEPS; ++ks) {
        const int c = 16 * ks + 8 * hi;
        const uint32_t off = c < D ? (uint32_t)((((lane & 31) * D) + c) * 4) : kOutOfRange;
        const f32x4 x0 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
        const f32x4 x1 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, c < D ? off + 16 : off, 0, 0));
        const f32x8 g = __builtin_convertvector(df[ks], f32x8);
#pragma unroll
        for (int e = 0; e < 4; ++e) dl = __builtin_fmaf(g[e], x0[e], __builtin_fmaf(g[4 + e], x1[e], dl));
      }
    } else {
      bf16x8 of[G::KSTEPS];
      load_frags<D>(reinterpret_cast<const __bf16*>(a.o) + qbase * D, wrow0, a.Nq, lane, of);
#pragma unroll
      for (int ks = 0; ks < G::KSTEPS; ++ks) {
        const f32x8 x = __builtin_convertvector(of[ks], f32x8);
        const f32x8 g = __builtin_convertvector(df[ks], f32x8);
#pragma unroll
        for (int e = 0; e < 8; ++e) dl = __builtin_fmaf(g[e], x[e], dl);
      }
    }
  }
  dl = pair_sum(dl);
  const float lsub = row < a.Nq ? lse_to_sub(a.lse[qbase + row]) : INFINITY;
  if (hi == 0 && row < a.Nq) a.delta[qbase + row] = dl;

  const Lanes<D> la(lane);
  const int row_lim = (a.causal ? min(row + a.diag, a.Nk - 1) : a.Nk - 1) - 8 * hi;
  const int row_lo = (a.causal ? row + a.lo : kNoWindow) - 8 * hi;

  f32x16 acc[G::CT];
#pragma unroll
  for (int ct = 0; ct < G::CT; ++ct) acc[ct] = f32x16{};
  // -delta of the lane's row in every register: the dP products start from it, so they give dP - delta and the
  // score gradient needs one multiply per element
  f32x16 negd;
#pragma unroll
  for (int r = 0; r < 16; ++r) negd[r] = -dl;

  auto step = [&](int t, const char* kc, const char* vc, char* kn, char* vn) {
    wait_vmem_all();      // this wave's copies of tile t have landed
    __syncthreads();      // every wave's have; every wave is done with tile t-1
    if (t + 1 < ntiles) {
      copy_tile<D>(K, (t + 1) * kBT, a.Nk, kn, wave, lane);
      copy_tile<D>(V, (t + 1) * kBT, a.Nk, vn, wave, lane);
    }
    if (t >= nt_w) return;
    f32x16 s0 = f32x16{}, s1 = f32x16{}, p0, p1;
#pragma unroll
    for (int ks = 0; ks < G::KSTEPS; ++ks) {
      s0 = mfma(row_frag<D>(kc, la, 0, ks), qf[ks], s0);
      s1 = mfma(row_frag<D>(kc, la, 1, ks), qf[ks], s1);
      p0 = mfma(row_frag<D>(vc, la, 0, ks), df[ks], ks == 0 ? negd : p0);
      p1 = mfma(row_frag<D>(vc, la, 1, ks), df[ks], ks == 0 ? negd : p1);
    }
    // register r of s0/s1 holds key 32*h + 16*(r/8) + 8*hi + r%8 of the tile (h = 0/1)
    if (t >= nfull || t < nlow) {
      const int lim = row_lim - t * kBT, lo = row_lo - t * kBT;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kr = 16 * (r >> 3) + (r & 7);
        if (kr > lim || kr < lo) s0[r] = -INFINITY;
        if (kr + 32 > lim || kr + 32 < lo) s1[r] = -INFINITY;
      }
    }
    bf16x8 db[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      f32x8 x;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int r = 8 * (kk & 1) + e;
        const float sv = (kk >> 1) ? s1[r] : s0[r];
        const float pv = (kk >> 1) ? p1[r] : p0[r];
        const float pw = __builtin_amdgcn_exp2f(__builtin_fmaf(sv, a.scale_log2, -lsub));
        x[e] = pw * pv;   // pv is dP - delta
      }
      db[kk] = __builtin_convertvector(x, bf16x8);
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int ct = 0; ct < G::CT; ++ct) acc[ct] = mfma(tr_frag<D>(kc, la, kk, ct), db[kk], acc[ct]);
  };
  for (int t = t0; t < ntiles; t += 2) {
    step(t, k0, v0, k1, v1);
    if (t + 1 < ntiles) step(t + 1, k1, v1, k0, v0);
  }
  store_grad<D, GF32>(reinterpret_cast<char*>(a.dq) + qbase * D * (GF32 ? 4 : 2), wrow0, a.Nq, lane, acc, a.scale,
                      a.accumulate != 0);
}

// ------------------------------------------------------------------------------------------------------------
// The d = 24 dk/dv stage below is laid out slot by slot: one MFMA per slot, the LDS operand reads kLead slots
// ahead, and a scheduling fence after every slot so that the compiler keeps the order (its stage is too short
// for the other wave on the SIMD to hide the LDS latency and the vector-ALU work). Register r of the score and
// dP accumulators s_h / p_h
// (h = 0: tile rows 0..31, h = 1: rows 32..63) holds tile row 32*h + 16*(r/8) + 8*hi + r%8: operand group
// kk = 2*h + r/8 and element r%8 of the lane's 8 rows 16*kk + 8*hi .. +7 (whose lse and delta are read from LDS
// as two float4 each).
constexpr int kLead = 3;

// One query tile of the dk/dv kernel for one wave at d = 24 (padded to 32), in one stage. With NS = 2*KSTEPS and
// NP = 2*CT:
//   slots [0, NS)           S and dP of tile rows 0..31 (accumulators s0, p0)
//   slots [NS, 2NS)         S and dP of rows 32..63 (s1, p1), beside the weights and score gradients of rows
//                           0..31 (operand groups kk = 0, 1)
//   slots [2NS, 2NS + 2NP)  dV += dO^T P and dK += Q^T dS for kk = 0, 1, beside the weights and score gradients
//                           of rows 32..63 (kk = 2, 3)
//   slots [2NS + 2NP, ...)  dV and dK for kk = 2, 3.
// The stage is too short to spread the element steps: each operand group is formed in one or two slots, so that
// its last step lands before the first MFMA that takes it, and every element, bf16 pair and group row value has
// a register of its own.

template <int D>
struct DkdvStage {
  using G = BG<D>;
  static constexpr int NS = 2 * G::KSTEPS;
  static constexpr int NP = 2 * G::CT;
  static constexpr int NT = 2 * NS + 4 * NP;
  static_assert(NS < 8, "d = 64 and 128 take the pipelined stage");
  static constexpr int ED = 32;                   // per-element arrays, indexed E % ED
  static constexpr int GD = 4;                    // per-group arrays, indexed kk % GD
  // the slot at which element E (0..31: operand group E/8, element E%8) is formed
  static constexpr int elem_slot(int E) {
    const int kk = E >> 3, e = E & 7;
    return kk == 0 ? NS + 1 : kk == 1 ? NS + 2 + e / 4 : kk == 2 ? 2 * NS + e / 4 : 2 * NS + 2 + e / 4;
  }

  const char* qc;
  const char* oc;
  const float* lc;
  const float* dc;
  const bf16x8 (&kf)[G::KSTEPS];
  const bf16x8 (&vf)[G::KSTEPS];
  f32x16 (&dk)[G::CT];
  f32x16 (&dv)[G::CT];
  const Lanes<D>& la;
  float scale_log2;
  bool masked;
  int lo, up;

  f32x16 s0, s1, p0, p1;
  bf16x8 pb[4], sb[4];
  float x[ED], dd[ED], w[ED], g[ED];  // per element: exponent, dP - delta, weight, score gradient
  bf16x2 wp[GD][4], gp[GD][4];        // completed pairs of weights and score gradients (bf16) per group
  f32x4 lq[GD][2], dl[GD][2];         // lse (exp2 domain) and delta per group: the next group's are read while
                                      // the current group's last elements are still being formed
  bf16x8 ring[kLead + 1];

  // the A operand of slot I
  template <int I>
  __device__ __forceinline__ bf16x8 frag() const {
    if constexpr (I < 2 * NS) {
      constexpr int j = I % NS;
      return row_frag<D>((j & 1) ? oc : qc, la, I / NS, j >> 1);
    } else {
      constexpr int m = I - 2 * NS, j = m % NP;
      return tr_frag<D>((j & 1) ? qc : oc, la, m / NP, j >> 1);
    }
  }

  // Element E is formed in three steps on consecutive slots, so that no slot waits on its own results: (a) the
  // exponent and dP - delta, (b) the exponential, (c) the score gradient, and the bf16 rounding of the group's
  // eight weights and score gradients after its last element.
  template <int E>
  __device__ __forceinline__ void elem_a() {
    constexpr int kk = E >> 3, e = E & 7, r = 8 * (kk & 1) + e, i = E % ED;
    const float sv = (kk >> 1) ? s1[r] : s0[r];
    const float pv = (kk >> 1) ? p1[r] : p0[r];
    x[i] = __builtin_fmaf(sv, scale_log2, -lq[kk % GD][e >> 2][e & 3]);
    dd[i] = pv - dl[kk % GD][e >> 2][e & 3];
    // pinned in this slot: the optimiser would otherwise sink the work next to its first use, past the
    // scheduling fences and out of the MFMA shadow it is placed in
    pin(x[i]);
    pin(dd[i]);
  }
  template <int E>
  __device__ __forceinline__ void elem_b() {
    constexpr int i = E % ED;
    w[i] = __builtin_amdgcn_exp2f(x[i]);
    pin(w[i]);
  }
  template <int E>
  __device__ __forceinline__ void elem_c() {
    constexpr int kk = E >> 3, e = E & 7, i = E % ED, ip = (E + ED - 1) % ED;
    g[i] = w[i] * dd[i];
    if constexpr (e & 1) {
      // each completed pair is rounded to bf16 at once: the next group's elements reuse w and g before this
      // group's last pair is done
      const f32x2 xw = {w[ip], w[i]}, yg = {g[ip], g[i]};
      wp[kk % GD][e >> 1] = __builtin_convertvector(xw, bf16x2);
      gp[kk % GD][e >> 1] = __builtin_convertvector(yg, bf16x2);
      pin(wp[kk % GD][e >> 1]);
      pin(gp[kk % GD][e >> 1]);
    } else {
      pin(g[i]);
    }
    if constexpr (e == 7) {
      const bf16x2(&a)[4] = wp[kk % GD];
      const bf16x2(&b)[4] = gp[kk % GD];
      pb[kk] = __builtin_shufflevector(__builtin_shufflevector(a[0], a[1], 0, 1, 2, 3),
                                       __builtin_shufflevector(a[2], a[3], 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
      sb[kk] = __builtin_shufflevector(__builtin_shufflevector(b[0], b[1], 0, 1, 2, 3),
                                       __builtin_shufflevector(b[2], b[3], 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
    }
  }
  template <int I, int... Es>
  __device__ __forceinline__ void elems(std::integer_sequence<int, Es...>) {
    ((elem_slot(Es) + 2 == I ? elem_c<Es>() : void()), ...);
    ((elem_slot(Es) + 1 == I ? elem_b<Es>() : void()), ...);
    ((elem_slot(Es) == I ? elem_a<Es>() : void()), ...);
  }

  template <int KK>
  __device__ __forceinline__ void read_rows() {
    const int rb = 16 * KK + 8 * la.hi;
    lq[KK % GD][0] = *reinterpret_cast<const f32x4*>(lc + rb);
    lq[KK % GD][1] = *reinterpret_cast<const f32x4*>(lc + rb + 4);
    dl[KK % GD][0] = *reinterpret_cast<const f32x4*>(dc + rb);
    dl[KK % GD][1] = *reinterpret_cast<const f32x4*>(dc + rb + 4);
  }

  __device__ __forceinline__ void mask(f32x16& sm, int off) {
    if (masked) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qr = off + 16 * (r >> 3) + (r & 7);
        if (qr < lo || qr > up) sm[r] = -INFINITY;
      }
    }
  }

  template <int I>
  __device__ __forceinline__ void slot() {
    if constexpr (I + kLead < NT) ring[(I + kLead) % (kLead + 1)] = frag<I + kLead>();
    const bf16x8 A = ring[I % (kLead + 1)];
    if constexpr (I < 2 * NS) {
      constexpr int h = I / NS, j = I % NS, ks = j >> 1;
      f32x16& c = (j & 1) ? (h == 0 ? p0 : p1) : (h == 0 ? s0 : s1);
      c = mfma(A, (j & 1) ? vf[ks] : kf[ks], ks == 0 ? f32x16{} : c);
    } else {
      constexpr int m = I - 2 * NS, kk = m / NP, j = m % NP, ct = j >> 1;
      if constexpr (j & 1) dk[ct] = mfma(A, sb[kk], dk[ct]);
      else dv[ct] = mfma(A, pb[kk], dv[ct]);
    }
    // lse and delta of a group, three slots before its first element
    if constexpr (I == elem_slot(0) - 3) read_rows<0>();
    if constexpr (I == elem_slot(8) - 3) read_rows<1>();
    if constexpr (I == elem_slot(16) - 3) read_rows<2>();
    if constexpr (I == elem_slot(24) - 3) read_rows<3>();
    // the causal / window mask of a block of rows once its scores are complete (a uniform branch: only tiles
    // that straddle an edge of the mask need it)
    if constexpr (I == NS - 1) {
      __builtin_amdgcn_sched_barrier(0);
      mask(s0, 0);
    }
    if constexpr (I == 2 * NS - 1) {
      __builtin_amdgcn_sched_barrier(0);
      mask(s1, 32);
    }
    elems<I>(std::make_integer_sequence<int, 32>{});
    __builtin_amdgcn_sched_barrier(0);
  }

  template <int... Is>
  __device__ __forceinline__ void run(std::integer_sequence<int, Is...>) {
    ((ring[Is] = frag<Is>()), ...);
  }
  template <int... Is>
  __device__ __forceinline__ void slots(std::integer_sequence<int, Is...>) {
    (slot<Is>(), ...);
  }
  __device__ __forceinline__ void operator()() {
    run(std::make_integer_sequence<int, kLead>{});
    slots(std::make_integer_sequence<int, NT>{});
  }
};

// ------------------------------------------------------------------------------------------------------------
// dk/dv kernel at d = 24 (padded to 32): 128 keys of one key/value head per workgroup of four waves, 32 per wave
// with K and V held in VGPRs (two waves per SIMD fit); query tiles of 64 of every query head in its group, one
// DkdvStage per tile.
template <int D, bool GF32>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bwd_dkdv24_kernel(BwdArgs a, int n_ktiles, int xcd_remap) {
  static_assert(D == 24, "d = 64 and 128 take attn_bwd_dkdv_kernel");
  using G = BG<D>;
  __shared__ __attribute__((aligned(4096))) char qa[G::TILE];
  __shared__ __attribute__((aligned(4096))) char qb[G::TILE];
  __shared__ __attribute__((aligned(4096))) char oa[G::TILE];
  __shared__ __attribute__((aligned(4096))) char ob[G::TILE];
  __shared__ __attribute__((aligned(16))) float la_[kBT];   // exp2-domain lse of the tile rows, slot a
  __shared__ __attribute__((aligned(16))) float lb_[kBT];
  __shared__ __attribute__((aligned(16))) float da_[kBT];   // delta of the tile rows
  __shared__ __attribute__((aligned(16))) float db_[kBT];
  __shared__ __attribute__((aligned(16))) float rla[kBT];   // raw lse and delta as copied, slots a and b
  __shared__ __attribute__((aligned(16))) float rlb[kBT];
  __shared__ __attribute__((aligned(16))) float rda[kBT];
  __shared__ __attribute__((aligned(16))) float rdb[kBT];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int64_t kvbh;
  int kt;
  decode_block(n_ktiles, xcd_remap, kvbh, kt);   // ascending key tiles: under a causal mask the first see most
  const int k0 = kt * kOwn;
  const int kw0 = k0 + wave * 32;
  const int group = a.kv_group;
  const int64_t bh0 = kvbh * group;             // the first query slice that reads this key/value slice

  // query range of the block: rows i with i + lo <= j <= i + diag for some key j of the block
  int qbeg = 0, qend = a.Nq;
  if (a.causal) {
    qbeg = max(0, k0 - a.diag);
    if (a.lo != kNoWindow) qend = min(a.Nq, k0 + kOwn - 1 - a.lo + 1);
  }
  const int t0 = qbeg / kBT;
  const int nt = qend > qbeg ? (qend + kBT - 1) / kBT - t0 : 0;
  const int nstages = nt * group;

  const __bf16* Q = reinterpret_cast<const __bf16*>(a.q);
  const __bf16* dO = reinterpret_cast<const __bf16*>(a.dout);
  auto issue_stage = [&](int s, char* qd, char* od) {
    const int64_t bh = bh0 + s / nt;
    const int r0 = (t0 + s % nt) * kBT;
    copy_tile<D>(Q + bh * a.Nq * D, r0, a.Nq, qd, wave, lane);
    copy_tile<D>(dO + bh * a.Nq * D, r0, a.Nq, od, wave, lane);
  };
  // The per-row lse and delta of a stage's 64 rows reach LDS in two steps, both by wave 0 and off the critical
  // path: two stages ahead, a buffer-to-LDS copy of the raw values (issued with the tile copies); one stage ahead,
  // at the end of a stage, the conversion of lse to the exp2-domain subtrahend (+inf for rows with no visible key
  // and rows past Nq) into the slot the stage after next reads.
  auto issue_rows = [&](int s, float* rl, float* rd) {
    const int64_t bh = bh0 + s / nt;
    const int r0 = (t0 + s % nt) * kBT;
    const int valid = uniform_clamp(a.Nq - r0, kBT);
    const __amdgpu_buffer_rsrc_t r1 = make_rsrc(a.lse + bh * a.Nq + r0, (int64_t)valid * 4);
    const __amdgpu_buffer_rsrc_t r2 = make_rsrc(a.delta + bh * a.Nq + r0, (int64_t)valid * 4);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r1, (lds_void*)rl, 4, (uint32_t)(lane * 4), 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r2, (lds_void*)rd, 4, (uint32_t)(lane * 4), 0, 0, 0);
  };
  auto convert_rows = [&](int s, const float* rl, const float* rd, float* lq, float* dq) {
    const int i = (t0 + s % nt) * kBT + lane;
    lq[lane] = i < a.Nq ? lse_to_sub(rl[lane]) : INFINITY;
    dq[lane] = i < a.Nq ? rd[lane] : 0.0f;
  };

  if (nstages > 0) {
    issue_stage(0, qa, oa);
    if (wave == 0) {
      issue_rows(0, rla, rda);
      if (nstages > 1) issue_rows(1, rlb, rdb);
      wait_vmem_all();
      convert_rows(0, rla, rda, la_, da_);
    }
  }

  const __bf16* Ks = reinterpret_cast<const __bf16*>(a.k) + kvbh * (int64_t)a.Nk * D;
  const __bf16* Vs = reinterpret_cast<const __bf16*>(a.v) + kvbh * (int64_t)a.Nk * D;
  bf16x8 kf[G::KSTEPS], vf[G::KSTEPS];
  load_frags<D>(Ks, kw0, a.Nk, lane, kf);
  load_frags<D>(Vs, kw0, a.Nk, lane, vf);
  const Lanes<D> la(lane);
  const int hi = lane >> 5;
  const int key = kw0 + (lane & 31);
  // this lane's key is visible to query rows [key - diag, key - lo]; relative to register r's row offset
  // 16*(r/8) + 8*hi + r%8 within a 32-row block
  const int vis_lo = (a.causal ? key - a.diag : -(1 << 30)) - 8 * hi;
  const int vis_hi = (a.causal && a.lo != kNoWindow ? key - a.lo : (1 << 30)) - 8 * hi;
  // rows for which every key of this wave is visible: [kw0 + 31 - diag, kw0 - lo]; rows seen by some key of the
  // wave: [kw0 - diag, kw0 + 31 - lo]
  const int all_lo = a.causal ? kw0 + 31 - a.diag : -(1 << 30);
  const int all_hi = a.causal && a.lo != kNoWindow ? kw0 - a.lo : (1 << 30);
  const int any_lo = a.causal ? kw0 - a.diag : -(1 << 30);
  const int any_hi = a.causal && a.lo != kNoWindow ? kw0 + 31 - a.lo : (1 << 30);

  f32x16 dk[G::CT], dv[G::CT];
#pragma unroll
  for (int ct = 0; ct < G::CT; ++ct) {
    dk[ct] = f32x16{};
    dv[ct] = f32x16{};
  }

  // stage s: tiles in (qc, oc), converted rows in (lc, dc); the next stage's tiles go to (qn, on) and its rows
  // are converted from the raw slot (rn_l, rn_d) into (ln, dn); the raw rows of stage s + 2 go to (rs_l, rs_d),
  // the raw slot stage s used
  auto step = [&](int s, const char* qc, const char* oc, const float* lc, const float* dc, char* qn, char* on,
                  float* ln, float* dn, const float* rn_l, const float* rn_d, float* rs_l, float* rs_d) {
    wait_vmem_all();      // this wave's copies of stage s (tiles) and s + 1 (raw rows) have landed
    __syncthreads();      // every wave's have; every wave is done with stage s - 1
    const bool more = s + 1 < nstages;
    if (more) issue_stage(s + 1, qn, on);
    if (wave == 0 && s + 2 < nstages) issue_rows(s + 2, rs_l, rs_d);
    const int i0 = (t0 + s % nt) * kBT;
    if (i0 + kBT - 1 >= any_lo && i0 <= any_hi)
      DkdvStage<D>{qc, oc, lc, dc, kf, vf, dk, dv, la, a.scale_log2, !(i0 >= all_lo && i0 + kBT - 1 <= all_hi),
                   vis_lo - i0, vis_hi - i0}();
    if (more && wave == 0) convert_rows(s + 1, rn_l, rn_d, ln, dn);
  };
  for (int s = 0; s < nstages; s += 2) {
    step(s, qa, oa, la_, da_, qb, ob, lb_, db_, rlb, rdb, rla, rda);
    if (s + 1 < nstages) step(s + 1, qb, ob, lb_, db_, qa, oa, la_, da_, rla, rda, rlb, rdb);
  }
  const int64_t kvrow = kvbh * (int64_t)a.Nk;
  store_grad<D, GF32>(reinterpret_cast<char*>(a.dk) + kvrow * D * (GF32 ? 4 : 2), kw0, a.Nk, lane, dk, a.scale,
                      a.accumulate != 0);
  store_grad<D, GF32>(reinterpret_cast<char*>(a.dv) + kvrow * D * (GF32 ? 4 : 2), kw0, a.Nk, lane, dv, 1.0f,
                      a.accumulate != 0);
}

// ------------------------------------------------------------------------------------------------------------
// dk/dv kernel at d = 64 and 128, two waves per SIMD: 128 keys of one key/value head per workgroup of eight
// waves. K and V of the block sit in LDS for the whole kernel (their B-operand fragments are read from there at
// each use, which frees the 64 registers they would take); waves w and w + 4 own the same 32 keys and split each
// 64-row query tile, w taking rows 0..31 and w + 4 rows 32..63, each with its own dK and dV accumulators, which
// the pair adds up through LDS at the end. A wave's stage is 4*KSTEPS MFMAs: S and dP (2*KSTEPS, contraction over
// the head dim), then dV^T += dO^T P and dK^T += Q^T dS over its 32 rows (2*KSTEPS); the compiler schedules it,
// and the other wave on the SIMD fills the gaps of the element work between them. Register r of the score and dP
// accumulators holds row 16*(r/8) + 8*hi + r%8 of the wave's 32 (the row operand is read in perm_row order).
constexpr int kW2 = 8;   // waves per workgroup

template <int D, bool GF32>
__global__ __launch_bounds__(64 * kW2) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bwd_dkdv_kernel(BwdArgs a, int n_ktiles, int xcd_remap) {
  static_assert(D == 64 || D == 128, "d = 24 takes attn_bwd_dkdv24_kernel");
  using G = BG<D>;
  constexpr int KV = kOwn * G::RB;                // 128 key rows of K (or V)
  // Every LDS buffer is an array of its own: the compiler then knows which one a copy in flight writes, and does
  // not make the reads of the current stage's tiles wait for the copies of the next stage.
  // The tiles' larger alignment places them first in LDS, below 64 KB, where their addresses fit the offset field
  // of the LDS reads (only speed depends on it: elsewhere the compiler adds the address in a register).
  __shared__ __attribute__((aligned(4096))) char qa[G::TILE];
  __shared__ __attribute__((aligned(4096))) char qb[G::TILE];
  __shared__ __attribute__((aligned(4096))) char oa[G::TILE];
  __shared__ __attribute__((aligned(4096))) char ob[G::TILE];
  __shared__ __attribute__((aligned(1024))) char kb[KV];
  __shared__ __attribute__((aligned(1024))) char vb[KV];
  __shared__ __attribute__((aligned(16))) float la_[kBT];   // exp2-domain lse of the tile rows, slot a
  __shared__ __attribute__((aligned(16))) float lb_[kBT];
  __shared__ __attribute__((aligned(16))) float da_[kBT];   // -delta of the tile rows (0 past Nq)
  __shared__ __attribute__((aligned(16))) float db_[kBT];
  __shared__ __attribute__((aligned(16))) float rla[kBT];   // raw lse and delta as copied, slots a and b
  __shared__ __attribute__((aligned(16))) float rlb[kBT];
  __shared__ __attribute__((aligned(16))) float rda[kBT];
  __shared__ __attribute__((aligned(16))) float rdb[kBT];
  // the pair exchange at the end reuses K, V and the tiles: one fp32 gradient of 32 keys per slot
  constexpr int XCH = 32 * D * 4;
  static_assert(2 * XCH == KV && XCH == G::TILE, "exchange slots: two in K, two in V, one per tile");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kw = wave & 3, half = wave >> 2;     // owned keys 32*kw.., tile rows 32*half..
  int64_t kvbh;
  int kt;
  decode_block(n_ktiles, xcd_remap, kvbh, kt);   // ascending key tiles: under a causal mask the first see most
  const int k0 = kt * kOwn;
  const int kw0 = k0 + kw * 32;
  const int group = a.kv_group;
  const int64_t bh0 = kvbh * group;

  int qbeg = 0, qend = a.Nq;
  if (a.causal) {
    qbeg = max(0, k0 - a.diag);
    if (a.lo != kNoWindow) qend = min(a.Nq, k0 + kOwn - 1 - a.lo + 1);
  }
  const int t0 = qbeg / kBT;
  const int nt = qend > qbeg ? (qend + kBT - 1) / kBT - t0 : 0;
  const int nstages = nt * group;

  const __bf16* Q = reinterpret_cast<const __bf16*>(a.q);
  const __bf16* dO = reinterpret_cast<const __bf16*>(a.dout);
  auto issue_stage = [&](int s, char* qd, char* od) {
    const int64_t bh = bh0 + s / nt;
    const int r0 = (t0 + s % nt) * kBT;
    copy_tile<D, kBT, kW2>(Q + bh * a.Nq * D, r0, a.Nq, qd, wave, lane);
    copy_tile<D, kBT, kW2>(dO + bh * a.Nq * D, r0, a.Nq, od, wave, lane);
  };
  // lse and delta of a stage's rows: copied raw two stages ahead and converted one stage ahead, by wave 0 (lse
  // to the exp2-domain subtrahend, delta negated)
  auto issue_rows = [&](int s, float* rl, float* rd) {
    const int64_t bh = bh0 + s / nt;
    const int r0 = (t0 + s % nt) * kBT;
    const int valid = uniform_clamp(a.Nq - r0, kBT);
    const __amdgpu_buffer_rsrc_t r1 = make_rsrc(a.lse + bh * a.Nq + r0, (int64_t)valid * 4);
    const __amdgpu_buffer_rsrc_t r2 = make_rsrc(a.delta + bh * a.Nq + r0, (int64_t)valid * 4);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r1, (lds_void*)rl, 4, (uint32_t)(lane * 4), 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r2, (lds_void*)rd, 4, (uint32_t)(lane * 4), 0, 0, 0);
  };
  auto convert_rows = [&](int s, const float* rl, const float* rd, float* lq, float* dq) {
    const int i = (t0 + s % nt) * kBT + lane;
    lq[lane] = i < a.Nq ? lse_to_sub(rl[lane]) : INFINITY;
    dq[lane] = i < a.Nq ? -rd[lane] : 0.0f;
  };

  const __bf16* Ks = reinterpret_cast<const __bf16*>(a.k) + kvbh * (int64_t)a.Nk * D;
  const __bf16* Vs = reinterpret_cast<const __bf16*>(a.v) + kvbh * (int64_t)a.Nk * D;
  if (nstages > 0) {
    copy_tile<D, kOwn, kW2>(Ks, k0, a.Nk, kb, wave, lane);
    copy_tile<D, kOwn, kW2>(Vs, k0, a.Nk, vb, wave, lane);
    issue_stage(0, qa, oa);
    if (wave == 0) {
      issue_rows(0, rla, rda);
      if (nstages > 1) issue_rows(1, rlb, rdb);
      wait_vmem_all();
      convert_rows(0, rla, rda, la_, da_);
    }
  }

  const Lanes<D> la(lane);
  const int hi = lane >> 5;
  // B operand of this wave's keys (K or V in LDS): key 32*kw + l%32 (natural order), head-dim columns
  // 16*ks + 8*hi .. +7
  const int krow = 32 * kw + (lane & 31);
  const int koff = krow * G::RB, ksw = swz<D>(krow);
  // Per-lane byte offsets of every operand read of a stage, formed once and held in registers: each read is then a
  // named buffer plus one of them, which the compiler emits with the buffer's address (and any constant part) in
  // the instruction's offset field instead of adding addresses in the loop.
  int keyo[G::KSTEPS], rowo[G::KSTEPS], tro[2][G::CT];
#pragma unroll
  for (int ks = 0; ks < G::KSTEPS; ++ks) {
    keyo[ks] = koff + 16 * ((2 * ks + hi) ^ ksw);
    rowo[ks] = half * 32 * G::RB + la.row_off + 16 * ((2 * ks + la.hi) ^ la.row_sw);
    pin(keyo[ks]);
    pin(rowo[ks]);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int ct = 0; ct < G::CT; ++ct) {
      tro[j][ct] = 2 * half * 16 * G::RB + la.tr[j][ct];
      pin(tro[j][ct]);
    }
  auto key_frag = [&](const char* t, int ks) { return *reinterpret_cast<const bf16x8*>(t + keyo[ks]); };
  // rows 32*half + perm_row(l%32) of a tile, head-dim columns 16*ks + 8*hi .. +7
  auto own_rows = [&](const char* t, int ks) { return *reinterpret_cast<const bf16x8*>(t + rowo[ks]); };
  // head-dim columns 32*ct + l%32, tile rows 32*half + 16*g + 8*hi .. +7
  auto own_tr = [&](const char* t, int g, int ct) {
    const char* p = t + g * 16 * G::RB;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + tro[0][ct]));
    const i16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + tro[1][ct]));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  const int key = kw0 + (lane & 31);
  const int vis_lo = (a.causal ? key - a.diag : -(1 << 30)) - 8 * hi;
  const int vis_hi = (a.causal && a.lo != kNoWindow ? key - a.lo : (1 << 30)) - 8 * hi;
  const int all_lo = a.causal ? kw0 + 31 - a.diag : -(1 << 30);
  const int all_hi = a.causal && a.lo != kNoWindow ? kw0 - a.lo : (1 << 30);
  const int any_lo = a.causal ? kw0 - a.diag : -(1 << 30);
  const int any_hi = a.causal && a.lo != kNoWindow ? kw0 + 31 - a.lo : (1 << 30);

  f32x16 dk[G::CT], dv[G::CT];
#pragma unroll
  for (int ct = 0; ct < G::CT; ++ct) {
    dk[ct] = f32x16{};
    dv[ct] = f32x16{};
  }

  // stage s: tiles in (qc, oc), converted rows in (lc, dc); as in the one-stage kernel above
  auto step = [&](int s, const char* qc, const char* oc, const float* lc, const float* dc, char* qn, char* on,
                  float* ln, float* dn, const float* rn_l, const float* rn_d, float* rs_l, float* rs_d) {
    wait_vmem_all();      // this wave's copies of stage s (tiles) and s + 1 (raw rows) have landed
    __syncthreads();      // every wave's have; every wave is done with stage s - 1
    const bool more = s + 1 < nstages;
    if (more) issue_stage(s + 1, qn, on);
    if (wave == 0 && s + 2 < nstages) issue_rows(s + 2, rs_l, rs_d);
    const int r0 = (t0 + s % nt) * kBT + 32 * half;   // this wave's first row
    if (r0 + 31 >= any_lo && r0 <= any_hi && r0 < a.Nq) {
      // dP starts from -delta of its rows, so that it comes out of the MFMAs as dP - delta
      f32x16 sc = f32x16{}, dp;
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const int rb = 32 * half + 16 * g + 8 * hi;
        const f32x4 d0 = *reinterpret_cast<const f32x4*>(dc + rb), d1 = *reinterpret_cast<const f32x4*>(dc + rb + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dp[8 * g + e] = d0[e];
          dp[8 * g + 4 + e] = d1[e];
        }
      }
#pragma unroll
      for (int ks = 0; ks < G::KSTEPS; ++ks) {
        sc = mfma(own_rows(qc, ks), key_frag(kb, ks), sc);
        dp = mfma(own_rows(oc, ks), key_frag(vb, ks), dp);
      }
      // register r holds row r0 + 16*(r/8) + 8*hi + r%8 of this lane's key
      if (!(r0 >= all_lo && r0 + 31 <= all_hi)) {
        const int lo = vis_lo - r0, up = vis_hi - r0;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qr = 16 * (r >> 3) + (r & 7);
          if (qr < lo || qr > up) sc[r] = -INFINITY;
        }
      }
      bf16x8 pb[2], sb[2];
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const int rb = 32 * half + 16 * g + 8 * hi;
        const f32x4 l0 = *reinterpret_cast<const f32x4*>(lc + rb), l1 = *reinterpret_cast<const f32x4*>(lc + rb + 4);
        f32x8 w, gr;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float lq = e < 4 ? l0[e] : l1[e - 4];
          w[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[8 * g + e], a.scale_log2, -lq));
          gr[e] = w[e] * dp[8 * g + e];
        }
        pb[g] = __builtin_convertvector(w, bf16x8);
        sb[g] = __builtin_convertvector(gr, bf16x8);
      }
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int ct = 0; ct < G::CT; ++ct) {
          dv[ct] = mfma(own_tr(oc, g, ct), pb[g], dv[ct]);
          dk[ct] = mfma(own_tr(qc, g, ct), sb[g], dk[ct]);
        }
    }
    if (more && wave == 0) convert_rows(s + 1, rn_l, rn_d, ln, dn);
  };
  for (int s = 0; s < nstages; s += 2) {
    step(s, qa, oa, la_, da_, qb, ob, lb_, db_, rlb, rdb, rla, rda);
    if (s + 1 < nstages) step(s + 1, qb, ob, lb_, db_, qa, oa, la_, da_, rla, rda, rlb, rdb);
  }

  // Pair exchange: wave w + 4 hands its dV to wave w, wave w hands its dK to wave w + 4; each adds its partner's
  // part and stores one gradient. Register r of tile ct sits at float4 index (4*ct + r/4)*64 + lane of the slot.
  wait_vmem_all();        // no copy into LDS is still in flight (none is after a stage; this is for clarity)
  __syncthreads();        // every wave is done with the tiles (and K, V) the exchange overwrites
  float* xv = reinterpret_cast<float*>(kw < 2 ? kb + kw * XCH : vb + (kw - 2) * XCH);   // dV of pair kw
  float* xk = reinterpret_cast<float*>(kw == 0 ? qa : kw == 1 ? qb : kw == 2 ? oa : ob);  // dK of pair kw
  f32x16 (&mine)[G::CT] = half ? dv : dk;
  float* out_x = half ? xv : xk;
#pragma unroll
  for (int ct = 0; ct < G::CT; ++ct)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 y = {mine[ct][4 * g], mine[ct][4 * g + 1], mine[ct][4 * g + 2], mine[ct][4 * g + 3]};
      *reinterpret_cast<f32x4*>(out_x + ((4 * ct + g) * 64 + lane) * 4) = y;
    }
  __syncthreads();
  f32x16 (&keep)[G::CT] = half ? dk : dv;
  const float* in_x = half ? xk : xv;
#pragma unroll
  for (int ct = 0; ct < G::CT; ++ct)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 y = *reinterpret_cast<const f32x4*>(in_x + ((4 * ct + g) * 64 + lane) * 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) keep[ct][4 * g + e] += y[e];
    }
  const int64_t kvrow = kvbh * (int64_t)a.Nk;
  if (half)
    store_grad<D, GF32>(reinterpret_cast<char*>(a.dk) + kvrow * D * (GF32 ? 4 : 2), kw0, a.Nk, lane, dk, a.scale,
                        a.accumulate != 0);
  else
    store_grad<D, GF32>(reinterpret_cast<char*>(a.dv) + kvrow * D * (GF32 ? 4 : 2), kw0, a.Nk, lane, dv, 1.0f,
                        a.accumulate != 0);
}

template <int D, bool GF32>
hipError_t launch_d(const BwdArgs& a, hipStream_t stream) {
  if (a.BH > 0 && a.Nq > 0) {
    const int n_qtiles = (a.Nq + kOwn - 1) / kOwn;
    const int64_t total = (int64_t)n_qtiles * a.BH;
    if (total > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((attn_bwd_dq_kernel<D, GF32>), dim3((unsigned)total), dim3(64 * kWaves), 0, stream, a,
                       n_qtiles, total % 8 == 0 ? 1 : 0);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t BHkv = a.BH / a.kv_group;
  if (BHkv > 0 && a.Nk > 0) {
    const int n_ktiles = (a.Nk + kOwn - 1) / kOwn;
    const int64_t total = (int64_t)n_ktiles * BHkv;
    if (total > 0x7fffffff) return hipErrorInvalidConfiguration;
    if constexpr (D >= 64)
      hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, GF32>), dim3((unsigned)total), dim3(64 * kW2), 0, stream, a,
                         n_ktiles, total % 8 == 0 ? 1 : 0);
    else
      hipLaunchKernelGGL((attn_bwd_dkdv24_kernel<D, GF32>), dim3((unsigned)total), dim3(64 * kWaves), 0, stream, a,
                         n_ktiles, total % 8 == 0 ? 1 : 0);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_attn_bwd_bf16(const BwdArgs& a, int d, int grad_f32, hipStream_t stream) {
  switch (d) {
    case 128: return grad_f32 ? launch_d<128, true>(a, stream) : launch_d<128, false>(a, stream);
    case 64: return grad_f32 ? launch_d<64, true>(a, stream) : launch_d<64, false>(a, stream);
    case 24: return grad_f32 ? launch_d<24, true>(a, stream) : launch_d<24, false>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ebattn
