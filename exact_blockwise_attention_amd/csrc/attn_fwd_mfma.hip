// Exact blockwise attention forward, bf16 operands on gfx950 MFMA, fp32 online softmax.
//
// Method: "深度学习注意力机制优化与FlashAttention实践" §4.2 (per query block, loop over key/value blocks, keep a
// running maximum and running sum, normalise at the end) with the accumulator rescaled whenever the reference
// maximum moves -- the decomposition of "架构层解决方案 - Sparse Attention与Ring Attention", Ring Attention /
// 核心创新, applied one key tile at a time. Causal masking by global position ("深度学习注意力机制优化与
// FlashAttention实践" §5.1) arrives here as a diagonal offset: key j is visible to query i iff j <= i + diag.
// Only O and the per-row log-sum-exp are written to HBM ("注意力机制演进", section FlashAttention).
//
// Per wave (32 query rows, Q fragment held in VGPRs for the whole key loop):
//   * S^T = K . Q^T, 32 keys x 32 queries per MFMA 32x32x16. In that orientation one lane owns one query row
//     (the MFMA output column): the row maximum and sum are in-lane reductions plus one exchange with the
//     partner lane (lane ^ 32), and the rescale factor is a per-lane scalar;
//   * the keys of each 32-key chunk sit in LDS with bits 2 and 3 of their index swapped. Read back in natural
//     order as the MFMA A operand, this leaves lane l's 16 output registers holding, in order, 8 consecutive
//     keys of each 16-key half -- the B-operand layout of the next product O^T = V^T . P^T, so P goes from the
//     S accumulator to the P.V MFMA without leaving the registers;
//   * V stays row-major in LDS; the V^T operand is gathered with the LDS transpose read ds_read_b64_tr_b16
//     (within each 16-lane group, lane i receives column i of a 4-row x 16-column block);
//   * one running sum of the fp32 weights gives both the normaliser of O and the log-sum-exp; the weights enter
//     P.V rounded to bf16;
//   * the reference maximum only moves when a row's new maximum exceeds it by more than 8 (log2 units), so most
//     tiles skip the rescale of the accumulator; the weights stay below 2^8 and the result is unchanged (the
//     final normalisation uses the same reference).
//   * at d = 128 the key loop is software-pipelined: while the MFMAs of the next tile's scores run, the wave
//     forms the current tile's weights, and while the current tile's P.V MFMAs run, it finishes the weights and
//     the row sums (the stage functions below lay this out slot by slot).
// Per workgroup:
//   * 64-key K and V tiles are copied HBM -> LDS by the buffer unit itself (buffer_load ... lds, 16 bytes per
//     lane, rows past Nk read as zero), double-buffered in four separately named LDS arrays; K rows and V rows
//     are XOR-swizzled per 16-byte chunk so that the operand reads spread over all 64 LDS banks;
//   * 4 waves = 128 query rows per workgroup (8 waves = 256 rows for d = 128 calls without a mask, or with a
//     causal mask over 16K keys or more and no window), one barrier per tile; two waves share each SIMD, so one
//     wave's softmax can also overlap the other's MFMA work.
#include <type_traits>

#include "internal.h"

namespace ebattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kBN = 64;                        // keys per K/V tile
constexpr int32_t kRsrcWord3 = 0x00020000;     // raw buffer, 32-bit data format (gfx9 family)
constexpr uint32_t kOutOfRange = 0x7ffffff0u;  // a buffer offset past every num_records: the load returns 0
constexpr float kRescaleSlack = 8.0f;          // log2 units the running maximum may exceed the reference by
constexpr int kLead = 3;                       // LDS operand reads run this many MFMAs ahead (fenced loops)

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
};

// Chunk swizzles (XOR on the 16-byte chunk index within a row), chosen for 64 four-byte LDS banks (256 bytes
// per clock). K: row p of the tile, read 16 bytes per lane by 16 consecutive rows at one chunk index -> the 16
// rows must land on 16 different bank groups. V: row j of the tile, read 8 bytes per lane by the transpose
// reads, 32 lanes covering 4 consecutive rows x 64 bytes -> the 4 rows' 64-byte column groups must not overlap.
template <int D>
__device__ __forceinline__ int k_swz(int p) { return D == 128 ? p & 15 : D == 64 ? (p >> 1) & 7 : (p >> 2) & 3; }
template <int D>
__device__ __forceinline__ int v_swz(int j) { return D == 128 ? 4 * (j & 3) : D == 64 ? 4 * ((j >> 1) & 1) : 0; }
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

__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// This wave's share (of NW waves) of the HBM -> LDS copy of tile rows [j0, j0 + kBN) of K (IS_K: rows permuted,
// chunks K-swizzled) or of V (chunks V-swizzled): kPerWave wave-wide copy instructions of 16 bytes per lane. Rows
// past Nk read as zero (a tile wholly past Nk is all zeros and touches no memory).
template <int D, bool IS_K, int NW>
struct TileCopy {
  using G = Geom<D>;
  static_assert(G::INSTR % NW == 0, "tile copy must split evenly over the waves");
  static constexpr int kPerWave = G::INSTR / NW;
  __amdgpu_buffer_rsrc_t rx;
  char* dst;
  int wave, lane;
  __device__ __forceinline__ TileCopy(const __bf16* X, int j0, int Nk, char* dst_, int wave_, int lane_)
      : dst(dst_), wave(wave_), lane(lane_) {
    const int rows_valid = min(kBN, Nk - j0);
    rx = make_rsrc(X + (int64_t)j0 * D, (int64_t)rows_valid * D * 2);
  }
  __device__ __forceinline__ void issue(int i) const {
    const int sub = lane / G::CPR, pos = lane % G::CPR;
    const int instr = wave * kPerWave + i;
    const int row = instr * G::ROWS_PER_INSTR + sub;
    const int m = pos ^ (IS_K ? k_swz<D>(row) : v_swz<D>(row));
    const int src_row = IS_K ? key_of_row(row) : row;
    const uint32_t off = m < G::CPG ? (uint32_t)((src_row * D + m * 8) * 2) : kOutOfRange;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void*)(dst + instr * 1024), 16, off, 0, 0, 0);
  }
  __device__ __forceinline__ void issue_all() const {
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) issue(i);
  }
};

template <int D, bool IS_K, int NW>
__device__ __forceinline__ void issue_copy(const __bf16* X, int j0, int Nk, char* dst, int wave, int lane) {
  TileCopy<D, IS_K, NW>(X, j0, Nk, dst, wave, lane).issue_all();
}

// Per-lane pieces of the LDS addressing, fixed for the whole key loop.
template <int D>
struct LaneAddr {
  int k_row;                 // byte offset of this lane's K row (row l%32 of the first 32-key chunk)
  int k_xor;                 // its chunk swizzle
  int hi;                    // lane / 32: which 8-column half of each 16-wide k-step this lane supplies
  int v[Geom<D>::CT];        // byte offset of this lane's first transpose read, per 32-column tile of O^T
  __device__ LaneAddr(int lane) {
    using G = Geom<D>;
    const int l32 = lane & 31;
    hi = lane >> 5;
    k_row = l32 * G::ROW_BYTES;
    k_xor = k_swz<D>(l32);
    const int g2 = (lane >> 4) & 1, a4 = (lane & 15) >> 2, b4 = lane & 3;
    const int row = 8 * hi + a4;                      // key row of the first transpose read
#pragma unroll
    for (int ct = 0; ct < G::CT; ++ct) {
      const int m = 4 * ct + 2 * g2 + (b4 >> 1);     // 16-byte chunk of columns 32*ct + 16*g2 + 4*b4 .. +3
      v[ct] = row * G::ROW_BYTES + 16 * (m ^ v_swz<D>(row)) + 8 * (b4 & 1);
    }
  }
};

// K operand of MFMA i of S^T = K . Q^T over one 64-key tile (K tile at `kt` in LDS): k-step i/2, keys
// 32*(i%2) .. +31 (lane: key row l%32, head-dim columns 16*(i/2) + 8*(l/32) .. +7).
template <int D>
__device__ __forceinline__ bf16x8 k_frag(const char* kt, const LaneAddr<D>& la, int i) {
  const char* p = kt + la.k_row + 16 * ((2 * (i >> 1) + la.hi) ^ la.k_xor) + (i & 1) * 32 * Geom<D>::ROW_BYTES;
  return *reinterpret_cast<const bf16x8*>(p);
}

// V^T operand of MFMA j of O^T += V^T . P^T (V tile at `vt` in LDS): keys 16*(j/CT) .. +15, head-dim columns
// 32*(j%CT) .. +31, gathered by two transpose reads (slots 0-3 from key rows +0..3 and slots 4-7 from rows
// +4..7 of each 8-key group).
template <int D>
__device__ __forceinline__ bf16x8 v_frag(const char* vt, const LaneAddr<D>& la, int j) {
  using G = Geom<D>;
  const char* p = vt + la.v[j % G::CT] + (j / G::CT) * 16 * G::ROW_BYTES;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  const i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 4 * G::ROW_BYTES));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Marks a value as produced here: an empty asm statement that takes it in and out of registers, so that the
// optimiser cannot sink its computation into a later block (it emits no instruction).
__device__ __forceinline__ void pin(bf16x8& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(float& x) { asm volatile("" : "+v"(x)); }

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// S^T = K . Q^T for one 64-key tile and this wave's 32 query rows: keys 0..31 into s0, keys 32..63 into s1. With
// FENCED, the LDS reads run two MFMAs ahead in a ring of three registers and the order is fixed slot by slot
// (the pipelined kernel keeps two score tiles live and cannot afford the reads hoisted further).
template <int D, bool FENCED = false>
__device__ __forceinline__ void qk_tile(const char* kt, const bf16x8 (&qf)[Geom<D>::KSTEPS], f32x16& s0, f32x16& s1,
                                        const LaneAddr<D>& la) {
  using G = Geom<D>;
  if constexpr (FENCED) {
    constexpr int NM = 2 * G::KSTEPS;
    bf16x8 kf[kLead + 1];
#pragma unroll
    for (int i = 0; i < kLead; ++i) kf[i] = k_frag<D>(kt, la, i);
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      if (i + kLead < NM) kf[(i + kLead) % (kLead + 1)] = k_frag<D>(kt, la, i + kLead);
      if (i & 1)
        s1 = mfma(kf[i % (kLead + 1)], qf[i >> 1], i < 2 ? f32x16{} : s1);
      else
        s0 = mfma(kf[i % (kLead + 1)], qf[i >> 1], i < 2 ? f32x16{} : s0);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    s0 = f32x16{};
    s1 = f32x16{};
#pragma unroll
    for (int kc = 0; kc < G::KSTEPS; ++kc) {
      s0 = mfma(k_frag<D>(kt, la, 2 * kc), qf[kc], s0);
      s1 = mfma(k_frag<D>(kt, la, 2 * kc + 1), qf[kc], s1);
    }
  }
}

// The softmax works on one tile's 32 scores per lane as scalars, w[16*h + r] = register r of score accumulator h
// (h = 0: keys 0..31 of the tile, h = 1: keys 32..63): lane l holds key 32*h + 16*(r/8) + 8*(l/32) + r%8, for
// query row l%32. Scalars rather than in-place vector updates keep the register allocator from copying whole
// 16-register accumulators.
__device__ __forceinline__ void unpack_scores(const f32x16& s0, const f32x16& s1, float (&w)[32]) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    w[r] = s0[r];
    w[16 + r] = s1[r];
  }
}

// bf16 B operand of P.V for keys 16*kk .. +15 of the tile, from weights w[8*kk .. 8*kk + 7].
__device__ __forceinline__ bf16x8 pack_weights(const float (&w)[32], int kk) {
  const f32x8 v = {w[8 * kk], w[8 * kk + 1], w[8 * kk + 2], w[8 * kk + 3],
                   w[8 * kk + 4], w[8 * kk + 5], w[8 * kk + 6], w[8 * kk + 7]};
  return __builtin_convertvector(v, bf16x8);
}

// Hides the keys of a tile that straddles the causal diagonal or the lower edge of a sliding window, in the score
// accumulators themselves (masking the unpacked copy instead makes the allocator keep both): keys past `lim` or
// before `lo` (both relative to this lane's first key of the tile) are hidden.
__device__ __forceinline__ void mask_scores(f32x16& s0, f32x16& s1, int lim, int lo) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int kr = 16 * (r >> 3) + (r & 7);
    if (kr > lim || kr < lo) s0[r] = -INFINITY;
    if (kr + 32 > lim || kr + 32 < lo) s1[r] = -INFINITY;
  }
}

// Online softmax, first half (also the reference update of the pipelined stage): the tile's row maximum moves
// the reference maximum when it exceeds it by more than the slack; `alpha` is the factor that rescales everything
// accumulated so far (1 when the reference did not move); m_use is the reference the weights are taken against.
__device__ __forceinline__ void update_reference(float mx, float& m_ref, float& alpha, bool& need, float& m_use,
                                                 float scale_log2) {
  const float mt = pair_max(mx) * scale_log2;
  need = mt > m_ref + kRescaleSlack;
  const float m_new = need ? mt : m_ref;
  alpha = need ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.0f;
  m_ref = m_new;
  m_use = (m_new == -INFINITY) ? 0.0f : m_new;
}

__device__ __forceinline__ float weight(float s, float scale_log2, float m_use) {
  return __builtin_amdgcn_exp2f(__builtin_fmaf(s, scale_log2, -m_use));
}

// The scores become exp2 weights relative to the reference, in place (fp32, kept for the row sum) and rounded to
// bf16 in pb (the B operands of P.V, 16 keys each).
// With `skipmax` the reference stays as it is (finite in every lane: the caller checks).
__device__ __forceinline__ void weights_tile(float (&w)[32], bf16x8 (&pb)[4], float& m_ref, float& alpha, bool& need,
                                             float scale_log2, bool skipmax) {
  float m_use;
  if (!skipmax) {
    // IEEE maximum (v_maximum3_f32): no NaN quieting of the MFMA results is needed before it.
    float mx = __builtin_elementwise_maximum(w[0], w[1]);
#pragma unroll
    for (int e = 2; e < 32; e += 2)
      mx = __builtin_elementwise_maximum(__builtin_elementwise_maximum(mx, w[e]), w[e + 1]);
    update_reference(mx, m_ref, alpha, need, m_use, scale_log2);
  } else {
    alpha = 1.0f;
    need = false;
    m_use = m_ref;
  }
#pragma unroll
  for (int e = 0; e < 32; ++e) w[e] = weight(w[e], scale_log2, m_use);
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) pb[kk] = pack_weights(w, kk);
}

// Online softmax, second half: the running row sum of the fp32 weights (it normalises O and gives the
// log-sum-exp).
__device__ __forceinline__ void sums_tile(const float (&w)[32], float alpha, float& l_run) {
  float p[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int e = 0; e < 32; ++e) p[e & 3] += w[e];
  l_run = __builtin_fmaf(alpha, l_run, (p[0] + p[1]) + (p[2] + p[3]));
}

// Rescales the accumulator when any lane's reference maximum moved.
template <int D>
__device__ __forceinline__ void rescale_acc(f32x16 (&acc)[Geom<D>::CT], float alpha, bool need) {
  if (__builtin_amdgcn_ballot_w64(need)) {
#pragma unroll
    for (int ct = 0; ct < Geom<D>::CT; ++ct) acc[ct] *= alpha;
  }
}

// acc += P . V for one tile (V tile at `vt` in LDS); FENCED as for qk_tile.
template <int D, bool FENCED = false>
__device__ __forceinline__ void pv_tile(const char* vt, const bf16x8 (&pb)[4], f32x16 (&acc)[Geom<D>::CT],
                                        const LaneAddr<D>& la) {
  using G = Geom<D>;
  constexpr int NM = 4 * G::CT;
  if constexpr (FENCED) {
    bf16x8 vf[kLead + 1];
#pragma unroll
    for (int j = 0; j < kLead; ++j) vf[j] = v_frag<D>(vt, la, j);
#pragma unroll
    for (int j = 0; j < NM; ++j) {
      if (j + kLead < NM) vf[(j + kLead) % (kLead + 1)] = v_frag<D>(vt, la, j + kLead);
      acc[j % G::CT] = mfma(vf[j % (kLead + 1)], pb[j / G::CT], acc[j % G::CT]);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
#pragma unroll
    for (int j = 0; j < NM; ++j) acc[j % G::CT] = mfma(v_frag<D>(vt, la, j), pb[j / G::CT], acc[j % G::CT]);
  }
}

// ------------------------------------------------------------------------------------------------------------
// Software-pipelined stage (d = 128). A wave issues in order, and an MFMA keeps the matrix unit busy for 32
// cycles during which the same wave can issue vector-ALU work that does not depend on it. Each stage therefore
// lists its instructions slot by slot -- one MFMA, the LDS reads two MFMAs ahead, and a slice of the softmax work
// of the current tile -- with a scheduling fence after every slot so that the compiler keeps that order.
//
// Phase 1: the 16 MFMAs of the next tile's scores, beside the current tile's row maximum (slots 0-3) and reference
// update (slot 4) unless `skipmax` keeps the reference as it is, the weights of keys 0..31 (slots 5-12) and their
// bf16 rounding (slots 10, 14); the even slots also issue this wave's share of the copies of K tile t+2 and V
// tile t+1, and the last three slots, whose vector work is light, read phase 2's first V^T operands (the V tile
// is resident since the stage's barrier), so that phase 2 does not open with a wait on the LDS.
template <int D, class CopyK, class CopyV>
__device__ __forceinline__ void stage_phase1(const char* kn, const bf16x8 (&qf)[Geom<D>::KSTEPS], f32x16& n0,
                                             f32x16& n1, const LaneAddr<D>& la, float (&w)[32], bf16x8 (&pb)[4],
                                             float& m_ref, float& alpha, bool& need, float& m_use, float scale_log2,
                                             const CopyK& ck, const CopyV& cv, const char* vc, bf16x8 (&vpre)[kLead],
                                             bool skipmax) {
  constexpr int NM = 2 * Geom<D>::KSTEPS;
  static_assert(NM == 16, "the slot plan below is laid out for 16 MFMAs per phase");
  static_assert(CopyK::kPerWave <= 4 && CopyV::kPerWave <= 4, "one tile-copy instruction per even slot");
  bf16x8 kf[kLead + 1];
#pragma unroll
  for (int i = 0; i < kLead; ++i) kf[i] = k_frag<D>(kn, la, i);
  float mx = 0.0f;
#pragma unroll
  for (int i = 0; i < NM; ++i) {
    if (i + kLead < NM) kf[(i + kLead) % (kLead + 1)] = k_frag<D>(kn, la, i + kLead);
    if (i & 1)
      n1 = mfma(kf[i % (kLead + 1)], qf[i >> 1], i < 2 ? f32x16{} : n1);
    else
      n0 = mfma(kf[i % (kLead + 1)], qf[i >> 1], i < 2 ? f32x16{} : n0);
    // the copies for the next stages, spread out so that the memory pipeline never backs up into the wave
    if ((i & 1) == 0) {
      if (i < 2 * CopyK::kPerWave)
        ck.issue(i >> 1);
      else if (i >= 8 && i < 8 + 2 * CopyV::kPerWave)
        cv.issue((i - 8) >> 1);
    }
    if (i < 4) {
      // IEEE maximum (v_maximum3_f32): no NaN quieting of the MFMA results is needed before it. One chain over
      // the 32 scores, two more per instruction (16 instructions; a tree of pairs takes 23).
      if (!skipmax) {
        float m = i == 0 ? __builtin_elementwise_maximum(w[0], w[1])
                         : __builtin_elementwise_maximum(__builtin_elementwise_maximum(mx, w[8 * i]), w[8 * i + 1]);
#pragma unroll
        for (int e = 2; e < 8; e += 2)
          m = __builtin_elementwise_maximum(__builtin_elementwise_maximum(m, w[8 * i + e]), w[8 * i + e + 1]);
        mx = m;
      }
    } else if (i == 4) {
      if (!skipmax) {
        update_reference(mx, m_ref, alpha, need, m_use, scale_log2);
      } else {
        // the reference stays where it is (finite in every lane: the caller checks)
        alpha = 1.0f;
        need = false;
        m_use = m_ref;
      }
    } else if (i < 13) {
      const int e = 2 * (i - 5);
      w[e] = weight(w[e], scale_log2, m_use);
      w[e + 1] = weight(w[e + 1], scale_log2, m_use);
    }
    if (i == 10) {
      pb[0] = pack_weights(w, 0);
      pin(pb[0]);
    }
    if (i == 14) {
      pb[1] = pack_weights(w, 1);
      pin(pb[1]);
    }
    if (i >= NM - kLead) vpre[i - (NM - kLead)] = v_frag<D>(vc, la, i - (NM - kLead));
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Phase 2: the 16 MFMAs of P.V for the current tile (its first V^T operands read in phase 1), beside the weights
// of keys 32..63 (slots 0-7), their bf16 rounding (slots 5, 9; each needed three slots later) and the row sum of
// the fp32 weights (four partial sums, each started from its first pair).
template <int D>
__device__ __forceinline__ void stage_phase2(const char* vc, f32x16 (&acc)[Geom<D>::CT], const LaneAddr<D>& la,
                                             float (&w)[32], bf16x8 (&pb)[4], float alpha, float m_use,
                                             float scale_log2, float& l_run,
                                             const bf16x8 (&vpre)[kLead]) {
  using G = Geom<D>;
  constexpr int NM = 4 * G::CT;
  static_assert(NM == 16, "the slot plan below is laid out for 16 MFMAs per phase");
  bf16x8 vf[kLead + 1];
#pragma unroll
  for (int j = 0; j < kLead; ++j) vf[j] = vpre[j];
  float p[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int j = 0; j < NM; ++j) {
    if (j + kLead < NM) vf[(j + kLead) % (kLead + 1)] = v_frag<D>(vc, la, j + kLead);
    acc[j % G::CT] = mfma(vf[j % (kLead + 1)], pb[j / G::CT], acc[j % G::CT]);
    if (j < 8) {
      const int e = 16 + 2 * j;
      w[e] = weight(w[e], scale_log2, m_use);
      w[e + 1] = weight(w[e + 1], scale_log2, m_use);
      if (j < 4)
        p[j] = w[2 * j] + w[2 * j + 1];
      else
        p[j & 3] += w[2 * j] + w[2 * j + 1];
    } else {
      p[j & 3] += w[2 * j] + w[2 * j + 1];
    }
    if (j == 5) pb[2] = pack_weights(w, 2);
    if (j == 9) pb[3] = pack_weights(w, 3);
    pin(p[j & 3]);
    __builtin_amdgcn_sched_barrier(0);
  }
  l_run = __builtin_fmaf(alpha, l_run, (p[0] + p[1]) + (p[2] + p[3]));
}

// Q^T fragment (B operand) of this wave's 32 rows starting at `row0` of the workgroup's block: lane holds row
// row0 + l%32, head-dim columns 16*kc + 8*(l/32) .. +7; rows past the block read as zero.
template <int D>
__device__ __forceinline__ void load_q(const __bf16* Qblk, int rows_valid, int row0, int lane,
                                       bf16x8 (&qf)[Geom<D>::KSTEPS]) {
  using G = Geom<D>;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(Qblk, (int64_t)rows_valid * D * 2);
  const int l32 = lane & 31, hi = lane >> 5;
#pragma unroll
  for (int kc = 0; kc < G::KSTEPS; ++kc) {
    const int c = kc * 16 + 8 * hi;
    const uint32_t off = c < D ? (uint32_t)(((row0 + l32) * D + c) * 2) : kOutOfRange;
    qf[kc] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0));
  }
}

// Epilogue: O = acc / l, lse = ln2 * (m + log2 l); a row with no visible key gives (0, -inf). Register r of O^T
// tile ct holds head-dim column 32*ct + 8*(r/4) + 4*hi + r%4 of this lane's row; the buffer range of the
// workgroup's block drops the stores of rows past Nq.
// With MERGE the row is first merged with the running result (merge_o, merge_lse) by the log-sum-exp rule of
// "分布式注意力机制突破：长序列处理的全景技术架构与实践指南" §3.4 (common maximum, parts weighted by exp(lse_i - lse)):
// both lanes of the row read its running lse and their halves of its running o before either writes, so the
// output may alias the running result.
template <int D, bool OF32, bool MERGE>
__device__ __forceinline__ void store_out(const FwdArgs& a, int64_t bh, int q0, int block_rows, int local_row, int lane,
                                          const f32x16 (&acc)[Geom<D>::CT], float m_ref, float l_run) {
  using G = Geom<D>;
  const int hi = lane >> 5;
  const float l_tot = pair_sum(l_run);
  float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  const int qi = q0 + local_row;
  const int64_t o_rows = min(block_rows, a.Nq - q0);
  const int64_t base = (bh * (int64_t)a.Nq + q0) * D;
  float lse_out = l_tot > 0.0f ? (m_ref + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f : -INFINITY;
  float f_run = 0.0f;                    // weight of the running o in the merged row
  f32x4 run[G::CT][4];                   // this lane's half of the running o
  if constexpr (MERGE) {
    const __amdgpu_buffer_rsrc_t rr = make_rsrc(a.merge_o + base, o_rows * D * 4);
#pragma unroll
    for (int ct = 0; ct < G::CT; ++ct)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = ct * 32 + 8 * g + 4 * hi;
        run[ct][g] = c < D ? __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                       rr, (uint32_t)((local_row * D + c) * 4), 0, 0))
                           : f32x4{};
      }
    const float l_prev = qi < a.Nq ? a.merge_lse[bh * (int64_t)a.Nq + qi] : -INFINITY;
    // log2-domain merge of the two parts; an empty part (lse = -inf) weighs zero, two empty parts give (0, -inf)
    const float p2 = l_prev * 1.4426950408889634f;
    const float b2 = l_tot > 0.0f ? m_ref + __builtin_amdgcn_logf(l_tot) : -INFINITY;
    const float m2 = __builtin_fmaxf(p2, b2);
    if (m2 == -INFINITY) {
      lse_out = -INFINITY;
      inv = 0.0f;
    } else {
      const float wp = __builtin_amdgcn_exp2f(p2 - m2), wb = __builtin_amdgcn_exp2f(b2 - m2);
      const float rs = 1.0f / (wp + wb);
      lse_out = (m2 + __builtin_amdgcn_logf(wp + wb)) * 0.69314718055994531f;
      f_run = wp * rs;
      inv *= wb * rs;
    }
  }
  if (hi == 0 && qi < a.Nq) a.lse[bh * (int64_t)a.Nq + qi] = lse_out;
  const __amdgpu_buffer_rsrc_t ro = OF32 ? make_rsrc(reinterpret_cast<float*>(a.o) + base, o_rows * D * 4)
                                         : make_rsrc(reinterpret_cast<__bf16*>(a.o) + base, o_rows * D * 2);
#pragma unroll
  for (int ct = 0; ct < G::CT; ++ct)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int c = ct * 32 + 8 * g + 4 * hi;
      if (c >= D) continue;
      f32x4 y = {acc[ct][4 * g] * inv, acc[ct][4 * g + 1] * inv, acc[ct][4 * g + 2] * inv,
                 acc[ct][4 * g + 3] * inv};
      if constexpr (MERGE) y += f_run * run[ct][g];
      if (OF32)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, y), ro, (uint32_t)((local_row * D + c) * 4), 0, 0);
      else
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, __builtin_convertvector(y, bf16x4)), ro,
                                              (uint32_t)((local_row * D + c) * 2), 0, 0);
    }
}

// Workgroup -> the (batch*head slice, query block) pairs it computes, one after another. At d = 128 and 64 a
// launch has at most walk_rounds rounds of resident workgroups, so a workgroup's dispatch and wave launch are
// paid once per several blocks (each block still loads its own Q fragment and first K/V tiles). Workgroups are
// dispatched round-robin over the 8 XCDs; with the remap, workgroup b serves a contiguous range of blocks, range
// b mod 8, so that a slice's K/V tiles are re-read from one L2. A range lists its blocks slice by slice, the
// heaviest causal block (the last query rows) first, and deals them to its workgroups in snake order: in round r,
// slot s takes position r*S + s when r is even and r*S + S-1-s when r is odd (S workgroups per range), which
// pairs heavy blocks with light ones.
// At d = 24 the loop-carried state costs more scalar registers than the exponential-bound kernel can spare;
// there every workgroup computes one block.
template <int D>
constexpr bool walks_blocks() { return D >= 64; }
// Grid size in rounds of resident workgroups. Measured on causal 8k against one block per workgroup: d = 128 is
// fastest with one round (0.6-2 % faster), d = 64 with four (2-5 %); unmasked calls time the same either way.
template <int D>
constexpr int walk_rounds() { return D >= 128 ? 1 : 4; }

struct BlockWalk {
  int64_t per_range, base;
  int slots, slot;
  __device__ BlockWalk(int64_t total, int xcd_remap) {
    const int b = blockIdx.x, g = gridDim.x;
    per_range = xcd_remap ? total >> 3 : total;
    base = xcd_remap ? (int64_t)(b & 7) * per_range : 0;
    slots = xcd_remap ? g >> 3 : g;
    slot = xcd_remap ? b >> 3 : b;
  }
  // block of round r, false once the range is exhausted
  __device__ bool at(int r, int n_qtiles, int64_t& bh, int& qt) const {
    const int64_t pos = (int64_t)r * slots + ((r & 1) ? slots - 1 - slot : slot);
    if (pos >= per_range) return false;
    const int64_t w = base + pos;
    bh = w / n_qtiles;
    qt = n_qtiles - 1 - (int)(w % n_qtiles);
    return true;
  }
};

// ------------------------------------------------------------------------------------------------------------
// The kernel: 32 query rows per wave, one barrier per pipeline stage.

// Waves per SIMD the register budget allows (512 VGPRs per SIMD lane): d = 128 needs ~210 registers (two waves,
// two workgroups of 64 KB LDS per CU), d = 64 ~135 (three), d = 24 ~90 (four).
template <int D>
constexpr int waves_per_simd() { return D >= 128 ? 2 : D >= 64 ? 3 : 4; }
// The software pipeline keeps two score tiles live (32 more registers); it fits the d = 128 budget only.
template <int D>
constexpr bool pipelined() { return D == 128; }
// Waves per workgroup (32 query rows each): 4 (128 rows, two workgroups per CU) or, for the pipelined kernel
// without a causal mask, 8 (256 rows, one workgroup per CU: each K/V tile is copied into LDS once per 256 rows
// instead of once per 128). The larger block draws less power per FLOP, so the part holds a higher clock, but its
// eight waves share one barrier per tile, and under a causal mask the diagonal tiles leave some of them idle.
// Measured on three parts: with 16K keys or more per call (long rows, relatively few diagonal tiles) it is 0.4-2.6 %
// faster; at 8K keys and with a sliding window it is within -2 and +2.5 % by part, so those keep 4 waves.

template <int D, bool OF32, int NW, bool MERGE>
__global__ __launch_bounds__(64 * NW)
__attribute__((amdgpu_waves_per_eu(waves_per_simd<D>(), waves_per_simd<D>())))
void attn_fwd_kernel(FwdArgs a, int n_qtiles, int xcd_remap) {
  using G = Geom<D>;
  constexpr int T = G::TILE_BYTES;
  constexpr int kWaves = NW;
  constexpr int kRows = 32 * kWaves;
  // Four separate LDS arrays (K slots 0/1, V slots 0/1), always named at compile time: the compiler can then
  // tell that a tile copy in flight into one slot does not alias operand reads from another, and does not stall
  // those reads on the copy; the explicit vmcnt wait before each barrier orders the copies.
  __shared__ __attribute__((aligned(1024))) char k0[T];
  __shared__ __attribute__((aligned(1024))) char k1[T];
  __shared__ __attribute__((aligned(1024))) char v0[T];
  __shared__ __attribute__((aligned(1024))) char v1[T];
  __shared__ int redo_tag;   // the walk round of the last block a wave of this workgroup asked to redo
  if (threadIdx.x == 0) redo_tag = -1;   // read only after the barriers of the first block's first tile

  const int lane = threadIdx.x & 63;
  // the wave index is uniform across the wave; saying so keeps every per-wave bound (and the branches on them)
  // in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const BlockWalk walk((int64_t)n_qtiles * a.BH, xcd_remap);
  int64_t bh;
  int qt;
  for (int round = 0; walk.at(round, n_qtiles, bh, qt); ++round) {
    const int q0 = qt * kRows;
    const int64_t kvbh = bh / a.kv_group;   // the key/value head this query head reads
    const __bf16* K = reinterpret_cast<const __bf16*>(a.k) + kvbh * (int64_t)a.Nk * D;
    const __bf16* V = reinterpret_cast<const __bf16*>(a.v) + kvbh * (int64_t)a.Nk * D;

    const int qlast = min(q0 + kRows, a.Nq) - 1;
    const int kend = a.causal ? min(a.Nk, qlast + a.diag + 1) : a.Nk;
    const int ntiles = kend > 0 ? (kend + kBN - 1) / kBN : 0;
    const int wrow0 = q0 + wave * 32;
    const int wkfull = a.causal ? min(a.Nk, wrow0 + a.diag + 1) : a.Nk;
    const int nfull = wkfull > 0 ? wkfull / kBN : 0;
    const int wkend = a.causal ? min(a.Nk, wrow0 + 31 + a.diag + 1) : a.Nk;

    // tiles this wave has any visible key in (rows past Nq may see further; they are never stored)
    const int nt_w = min(ntiles, wkend > 0 ? (wkend + kBN - 1) / kBN : 0);
    // Sliding window: tiles before the first key the block's first row sees are skipped; tiles before `nlow`
    // hold keys below the window of some row of this wave and are masked.
    const int first_key = a.causal ? q0 + a.lo : 0;
    const int t0 = first_key > 0 ? first_key / kBN : 0;
    const int low_edge = a.causal ? wrow0 + 31 + a.lo : 0;
    const int nlow = low_edge > 0 ? (low_edge + kBN - 1) / kBN : 0;
    constexpr bool kPipe = pipelined<D>();

    auto first_copies = [&]() {
      if (ntiles > t0) {
        issue_copy<D, true, kWaves>(K, t0 * kBN, kend, k0, wave, lane);
        issue_copy<D, false, kWaves>(V, t0 * kBN, kend, v0, wave, lane);
        if (kPipe && ntiles > t0 + 1) issue_copy<D, true, kWaves>(K, (t0 + 1) * kBN, kend, k1, wave, lane);
      }
    };
    first_copies();
    bf16x8 qf[G::KSTEPS];
    load_q<D>(reinterpret_cast<const __bf16*>(a.q) + (bh * (int64_t)a.Nq + q0) * D, min(kRows, a.Nq - q0),
              wave * 32, lane, qf);
    const LaneAddr<D> la(lane);
    const int row_lim = (a.causal ? min(wrow0 + (lane & 31) + a.diag, a.Nk - 1) : a.Nk - 1) - 8 * la.hi;
    const int row_lo = (a.causal ? wrow0 + (lane & 31) + a.lo : kNoWindow) - 8 * la.hi;

    f32x16 acc[G::CT];
  #pragma unroll
    for (int ct = 0; ct < G::CT; ++ct) acc[ct] = f32x16{};
    float m_ref = -INFINITY, l_run = 0.0f;

    // Speculative reference: from the third tile of a block on, the row maximum is not formed and every lane's
    // weights are taken against the reference the first two tiles set (its rows' largest visible scores so far).
    // Weights then come out as large as 2^(row maximum - reference) instead of at most 2^slack; in fp32 and bf16
    // that changes no relative rounding, only the common scale of acc and l, which the epilogue divides out. Only
    // an overflow would do harm, so the block is redone with the row maximum formed at every tile (the exact lazy
    // rescaling above) when any wave's l or acc ends non-finite. A wave in which some lane has seen no visible
    // key yet keeps forming the maximum.
    bool spec = true;
    auto skip_max = [&](int t) { return spec && t >= t0 + 2 && !__builtin_amdgcn_ballot_w64(m_ref == -INFINITY); };
    // After a block's last tile, in every wave (it holds the workgroup's barrier, which also tells every wave that
    // no wave reads the LDS slots any more): true when this was the speculative pass and some wave ended it with
    // a non-finite l or acc. The verdict travels through an LDS word tagged with the walk round, so it needs no
    // reset; the barrier waits for LDS traffic only, not for the tile copies still in flight.
    auto end_of_pass = [&]() {
      const int round_tag = round;
      // Without a merge the block's result is stored first, so that the barrier below waits while the stores
      // drain; a redo stores it again. With a merge the running result it reads is the output, so nothing is
      // stored before the verdict.
      if constexpr (!MERGE) store_out<D, OF32, MERGE>(a, bh, q0, kRows, wave * 32 + (lane & 31), lane, acc, m_ref, l_run);
      // any inf or NaN in l or acc makes the sum non-finite (four chains, short latency)
      float part[4] = {l_run, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ct = 0; ct < G::CT; ++ct)
#pragma unroll
        for (int r = 0; r < 16; ++r) part[r & 3] += acc[ct][r];
      const float chk = (part[0] + part[1]) + (part[2] + part[3]);
      if (__builtin_amdgcn_ballot_w64(!__builtin_isfinite(chk)) != 0 && lane == 0) redo_tag = round_tag;
      // the wave's LDS reads and the tag write are complete, then the barrier; written out because a fence on LDS
      // would also wait for the tile copies into LDS still in flight, which nothing reads before the next wait
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      return spec && redo_tag == round_tag;
    };
    // A wave's copies land in issue order and each wave fills the same rows of a slot every time, so the unused
    // tiles the last steps copied cannot overwrite the tiles copied here.
    auto start_over = [&]() {
      spec = false;
#pragma unroll
      for (int ct = 0; ct < G::CT; ++ct) acc[ct] = f32x16{};
      m_ref = -INFINITY;
      l_run = 0.0f;
      first_copies();
    };

    // One tile at a time (every tile when d < 128): scores, mask, weights, rescale, P.V, sums.
    auto plain_tile = [&](f32x16& c0, f32x16& c1, bool partial, int t, const char* vc) {
      float w[32];
      bf16x8 pb[4];
      float alpha;
      bool need;
      if (partial) mask_scores(c0, c1, row_lim - t * kBN, row_lo - t * kBN);
      unpack_scores(c0, c1, w);
      weights_tile(w, pb, m_ref, alpha, need, a.scale_log2, skip_max(t));
      rescale_acc<D>(acc, alpha, need);
      __builtin_amdgcn_sched_barrier(0);
      pv_tile<D, kPipe>(vc, pb, acc, la);
      sums_tile(w, alpha, l_run);
    };

    if constexpr (kPipe) {
      // Software pipeline, one stage per tile t: the scores of tile t+1 (K tile t+1) are computed beside tile t's
      // weights, then P.V of tile t (V tile t) beside the rest of tile t's softmax. K tiles therefore arrive one
      // tile ahead of V tiles: after the barrier of stage t, K tile t+2 is copied into the slot of K tile t and V
      // tile t+1 into the slot of V tile t-1.
      f32x16 sa0, sa1, sb0, sb1;
      auto stage = [&](int t, f32x16& c0, f32x16& c1, f32x16& n0, f32x16& n1, const char* kn, char* kw,
                       const char* vc, char* vw) {
        wait_vmem_all();      // this wave's copies of K tile t+1 and V tile t have landed
        __syncthreads();      // so have every wave's; every wave is done with K tile t and V tile t-1
        // K tile t+2 goes to the slot of K tile t, V tile t+1 to the slot of V tile t-1 (tiles past the end are
        // copied as zeros, which keeps the stage free of branches; nothing reads them)
        const TileCopy<D, true, kWaves> ck(K, (t + 2) * kBN, kend, kw, wave, lane);
        const TileCopy<D, false, kWaves> cv(V, (t + 1) * kBN, kend, vw, wave, lane);
        // A wave past its last visible tile writes zeros to n0/n1: every path then writes them, so the scores of
        // tile t, which reach this stage in c0/c1, are dead once unpacked and are not kept beside their copy.
        if (t >= nt_w) {
          ck.issue_all();
          cv.issue_all();
          n0 = f32x16{};
          n1 = f32x16{};
          return;
        }
        float w[32];
        bf16x8 pb[4];
        float alpha, m_use;
        bool need;
        if (t >= nfull || t < nlow) mask_scores(c0, c1, row_lim - t * kBN, row_lo - t * kBN);
        unpack_scores(c0, c1, w);
        // The wave's last tile computes the scores of one more tile, which are never used (K slot `kn` then holds
        // an older tile): one branch-free stage shape keeps the register allocation of the loop tight.
        __builtin_amdgcn_sched_barrier(0);
        // Raised wave priority for phase 1: its chain (row maximum -> reference -> weights) gates the next phase,
        // so the issue arbiter favours it over the SIMD's other wave (measured: +2.5 % causal, +0.7 % unmasked).
        __builtin_amdgcn_s_setprio(1);
        bf16x8 vpre[kLead];
        stage_phase1<D>(kn, qf, n0, n1, la, w, pb, m_ref, alpha, need, m_use, a.scale_log2, ck, cv, vc, vpre,
                        skip_max(t));
        __builtin_amdgcn_s_setprio(0);
        rescale_acc<D>(acc, alpha, need);
        __builtin_amdgcn_sched_barrier(0);
        stage_phase2<D>(vc, acc, la, w, pb, alpha, m_use, a.scale_log2, l_run, vpre);
      };
      for (;;) {
        wait_vmem_all();
        __syncthreads();
        if (nt_w > t0) qk_tile<D, true>(k0, qf, sa0, sa1, la);
        for (int t = t0; t < ntiles; t += 2) {
          stage(t, sa0, sa1, sb0, sb1, k1, k0, v0, v1);
          if (t + 1 < ntiles) stage(t + 1, sb0, sb1, sa0, sa1, k0, k1, v1, v0);
        }
        if (!end_of_pass()) break;
        start_over();
      }
    } else {
      // One tile per step: after the barrier of tile t, tile t+1 is copied into the slots tile t-1 left.
      auto step = [&](int t, const char* kc, const char* vc, char* kn, char* vn) {
        wait_vmem_all();      // this wave's copies of tile t have landed
        __syncthreads();      // every wave's copies have landed; every wave is done with tile t-1
        if (t + 1 < ntiles) {
          issue_copy<D, true, kWaves>(K, (t + 1) * kBN, kend, kn, wave, lane);
          issue_copy<D, false, kWaves>(V, (t + 1) * kBN, kend, vn, wave, lane);
        }
        if (t >= nt_w) return;
        f32x16 s0, s1;
        qk_tile<D>(kc, qf, s0, s1, la);
        plain_tile(s0, s1, t >= nfull || t < nlow, t, vc);
      };
      for (;;) {
        for (int t = t0; t < ntiles; t += 2) {
          step(t, k0, v0, k1, v1);
          if (t + 1 < ntiles) step(t + 1, k1, v1, k0, v0);
        }
        if (!end_of_pass()) break;
        start_over();
      }
    }
    if constexpr (MERGE) store_out<D, OF32, MERGE>(a, bh, q0, kRows, wave * 32 + (lane & 31), lane, acc, m_ref, l_run);
    if constexpr (!walks_blocks<D>()) break;
    // The barrier at the end of the block's last pass has told every wave that no wave reads the LDS slots any
    // more, so the next block's first copies may go out now; as for a redo, the unused tiles the last steps copied
    // cannot overwrite them.
  }
}

template <int D, bool OF32, int NW>
hipError_t launch_d(const FwdArgs& a, hipStream_t stream) {
  constexpr int kRows = 32 * NW;
  const int n_qtiles = (a.Nq + kRows - 1) / kRows;
  const int64_t total = (int64_t)n_qtiles * a.BH;
  if (total > 0x7fffffff) return hipErrorInvalidConfiguration;
  // Workgroups resident at once on 256 CUs (register budget: waves_per_simd waves on each of 4 SIMDs), times
  // walk_rounds; the XCD remap needs the block count and the grid to be multiples of 8 (this cap is).
  constexpr int64_t kCap = (int64_t)256 * (4 * waves_per_simd<D>() / NW) * walk_rounds<D>();
  const int remap = (total % 8 == 0) ? 1 : 0;
  const unsigned grid = (unsigned)(walks_blocks<D>() && total > kCap ? kCap : total);
  if (a.merge_o)
    hipLaunchKernelGGL((attn_fwd_kernel<D, OF32, NW, true>), dim3(grid), dim3(64 * NW), 0, stream, a, n_qtiles,
                       remap);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<D, OF32, NW, false>), dim3(grid), dim3(64 * NW), 0, stream, a, n_qtiles,
                       remap);
  return hipGetLastError();
}

template <int D, bool OF32>
hipError_t launch_d(const FwdArgs& a, hipStream_t stream) {
  if constexpr (pipelined<D>()) {
    if (!a.causal || (a.lo == kNoWindow && a.Nk >= 16384)) return launch_d<D, OF32, 8>(a, stream);
  }
  return launch_d<D, OF32, 4>(a, stream);
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
