// LDS-tiled grouped GEMM for the QMoE expert FFN at larger token counts, on
// gfx950 matrix cores (v_mfma_f32_16x16x32_f16):
//
//   y[p, n] = sum_c a[p, c] * (q[e, n, c] - mid) * scale[e, n, c / bs]
//
// for the expert-sorted rows p of one 128-row tile of expert e (the
// GroupedMatMul of the ONNX GroupedMatMul-29 page, Summary, over weights
// dequantised as the QMoE WebGPU manifest's description and
// derive.quantMidpoint state).  Operand rows are f16 hi/lo of the row scaled
// by 2^e (see common.hpp); the epilogue multiplies each row's result by 2^-e.
// FC1 epilogue: ReLU, or interleaved SwiGLU g*sigmoid(alpha*g)*(u+beta) on
// row pairs (2j, 2j+1) (manifest attributeDescriptions.swiglu_fusion,
// activation_alpha, activation_beta), written as FC2's fp32 operand rows.
// FC2 epilogue: rows are written at their slot id, so the combine gathers
// them without atomics.
//
// Work decomposition: a workgroup of 8 wavefronts computes a 128 x 256 tile
// (2 x 4 wavefronts of 64 x 64).  Each 64-code K step's operands - the
// tile's activation slice (f16 hi/lo, 32 KB), packed weight slice (8 or
// 16 KB) and block scales - arrive in one of three LDS stage buffers by
// direct-to-LDS loads issued about two steps ahead.  The two rows of
// wavefronts alternate per half-step between reading fragments from LDS and
// running matrix instructions (a ping-pong on each SIMD, kept in step by
// workgroup barriers).  Packed weights are unpacked in registers to exact
// f16 (q - mid) between matrix instructions, and each fragment feeds 8
// instructions (4 row subtiles x hi/lo).
// Workgroups are ordered so that the ones resident on an XCD at the same time
// cover 8 row tiles x 4 column tiles: both operands are reused from that
// XCD's L2.
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "launch.h"

namespace qmoe {

namespace {

constexpr int kTM = 128;           // tile rows (expert-sorted activation rows)
constexpr int kTN = 256;           // tile columns (weight rows)
constexpr int kTK = 64;            // codes per K step
constexpr int kTWaves = 8;         // 2 (rows) x 4 (columns) wavefronts of 64 x 64
constexpr int kTThreads = 64 * kTWaves;
constexpr int kGroupM = 8;         // row tiles per tile group (L2 reuse)
constexpr int kABuf = kTM * kTK * 4;  // activation slice: 128 rows x 256 bytes

template <int BITS>
struct TiledLayout {
  static constexpr int kBRow = kTK * BITS / 8;      // packed bytes per weight row per step
  static constexpr int kGPR = kBRow / 16;           // 16-byte granules per weight row per step
  static constexpr int kBBuf = kTN * kBRow;
  static constexpr int kSBuf = 2 * kTN * 4;         // block scales of the step's two 32-code halves
  static constexpr int kStage = kABuf + kBBuf + kSBuf;
  static_assert(kStage >= 32 * kTN * 4, "a 32-row epilogue tile must fit one stage");
};

// Granule swizzle of a staged weight row (bank spread of the fragment reads):
// granule g of row n sits at g ^ swz(n).
template <int BITS>
__device__ __forceinline__ int bswz(int n) { return BITS == 4 ? (n >> 3) & 1 : (n >> 2) & 3; }

// Eight codes [32*j + 8*cg, +8) of staged weight row n: the packed word(s)
// (tile_raw), then exact f16 (q - mid) in A-row storage order (tile_unpack,
// see common.hpp).
template <int BITS>
struct BRaw {
  using type = typename std::conditional<BITS == 4, uint32_t, u32x2>::type;
};
template <int BITS>
__device__ __forceinline__ typename BRaw<BITS>::type tile_raw(const uint8_t* bbuf, int n, int j, int cg) {
  if constexpr (BITS == 4) return *(const uint32_t*)(bbuf + n * 32 + ((j ^ bswz<4>(n)) * 16) + 4 * cg);
  else return *(const u32x2*)(bbuf + n * 64 + (((2 * j + (cg >> 1)) ^ bswz<8>(n)) * 16) + (cg & 1) * 8);
}
template <int BITS>
__device__ __forceinline__ f16x8 tile_unpack(typename BRaw<BITS>::type v, const UnpackMasks& m) {
  if constexpr (BITS == 4) return unpack4(v, m);
  else return unpack8x2(v[0], v[1]);
}

// Wait until at most n vector-memory operations of this wavefront are in flight.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

}  // namespace

// Direct-to-LDS loads of one step: lane l of a load instruction fills the
// 16-byte LDS slot base + 16 * l (4 bytes for the scale loads).
#define QMOE_GLOBAL(p) ((const __attribute__((address_space(1))) void*)(p))
#define QMOE_LOCAL(p) ((__attribute__((address_space(3))) void*)(p))
// the kernel's helper lambdas are always inlined (arrays they capture stay in registers)
#define QMOE_INLINE __attribute__((always_inline))

// STEPFOLD: block sums are scaled every 32-code step (STEPFOLD_KT 0, 32-code
// blocks), every 64-code K step (1, 64-code blocks) or every two K steps (2,
// blocks of 128 codes and more).
// SEG (FC2): the operand rows carry one power-of-two scale per row tile and
// segment of 2^g.seg_shift codes (the FC1 epilogue's, see below) instead of
// one per row.  A span never straddles a segment, so the segment's factor
// g.seg_scale joins the span's block scales when the span closes (with
// column-wise scales the spans are two K steps, folded with that factor
// alone).  When FC1 raised *g.seg_flag the rows were taken back to one
// exponent each (g.a_exp): the factors are then 1 and the epilogue undoes
// the row exponents as without SEG.
// The work of one tile: 128 rows x 256 columns, or (HALF) 64 rows x 512
// columns, staged through the kernel's LDS arrays.
template <int BITS, int SCALE, int EPI, bool STEPFOLD, int STEPFOLD_KT, bool SEG, bool HALF>
__device__ __forceinline__ void tiled_tile(const GemmArgs& g, int ntn, int tile, int ntile, int kz, uint8_t* st0,
                                           uint8_t* st1, uint8_t* st2, long* s_arow, int* s_orow, int* s_rexp) {
  using L = TiledLayout<BITS>;
  constexpr bool half = HALF;
  const int e = g.tiles[4 * tile + 0];
  const int p0 = g.tiles[4 * tile + 1];
  const int rows = g.tiles[4 * tile + 2];
  const int n0 = ntile * kTN;

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  // this wavefront's first tile row and first column (half tiles: every
  // wavefront has rows 0..63, the second row of wavefronts the second 256
  // columns)
  const int rbase = half ? 0 : wm * 64;
  const int cbase = half ? wm * kTN : 0;
  const int col = lane & 15, grp = lane >> 4;
  const long ebase = (long)e * g.N;

  // SEG: rows back to one exponent each (segment factors 1), read before
  // the barrier so that its wait is not one for the first steps' loads
  const bool segrow = SEG && g.seg_flag[0] != 0;
  if (tid < kTM) {
    const int p = p0 + min(tid, rows - 1);
    const long ar = g.a_map ? (long)(g.a_map[p] / g.a_div) : (long)p;
    s_arow[tid] = ar * g.a_stride;
    s_orow[tid] = g.store_by_slot ? g.perm[p] : p;
    s_rexp[tid] = (SEG && !segrow) ? 0 : g.a_exp[ar];
  }
  __syncthreads();

  // Per-lane sources of the step's direct-to-LDS loads (rows past the tile
  // or past N re-read a valid row; every wavefront issues the same count).
  //  A: wavefront w fills rows 16w .. 16w + 15, four rows an instruction; the
  //     slot of row r holding piece q is q ^ (r & 15);
  //  B: the step's weight rows, GPR granules a row, granule g of row n in
  //     slot g ^ swz(n);
  //  S (block scales): wavefronts 0-3 the first 32-code half, 4-7 the second.
  //  Half tiles (column-wise scales only): wavefront w fills rows 8w ..
  //     8w + 7 (two instructions), and the weight rows of the second 256
  //     columns go to the second half of the activation buffer (kABuf / 2
  //     on; sources in asrc[2], asrc[3]).
  constexpr int BPW = L::kGPR * kTN / 64 / kTWaves;  // weight load instructions per wavefront
  static_assert(!HALF || (SCALE == SC_COL && BPW <= 2 && L::kBBuf <= kABuf / 2),
                "half tiles: column scales, second weight half in the activation buffer");
  constexpr int NV = HALF ? 2 + 2 * BPW : 4 + BPW + (SCALE == SC_BLOCK ? 1 : 0);
  const uint8_t* asrc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (!HALF || i < 2) {
      const int r = HALF ? (wave * 2 + i) * 4 + (lane >> 4) : (wave * 4 + i) * 4 + (lane >> 4);
      asrc[i] = g.a + s_arow[r] + (((lane & 15) ^ (r & 15)) * 16);
    } else {
      const int G = (wave * BPW + min(i - 2, BPW - 1)) * 64 + lane;
      const int n = G / L::kGPR, gs = G % L::kGPR;
      asrc[i] = g.wq + (ebase + min(n0 + kTN + n, g.N - 1)) * (long)g.kb + ((gs ^ bswz<BITS>(n)) * 16);
    }
  }
  const uint8_t* bsrc[BPW];
#pragma unroll
  for (int i = 0; i < BPW; ++i) {
    const int G = (wave * BPW + i) * 64 + lane;
    const int n = G / L::kGPR, gs = G % L::kGPR;
    bsrc[i] = g.wq + (ebase + min(n0 + n, g.N - 1)) * (long)g.kb + ((gs ^ bswz<BITS>(n)) * 16);
  }
  const float* ssrc = g.ws + (ebase + min(n0 + (wave & 3) * 64 + lane, g.N - 1)) * (long)g.nblk;
  const int shalf = (wave >> 2) * 32;
  // K range kz of g.ksplit (FC2): the sources start at its first step, kt
  // counts the range's steps (the range is a whole number of scale blocks,
  // segments and two-step spans)
  const int nk = g.K / kTK / g.ksplit;
  if (g.ksplit > 1) {
    const int kt0 = kz * nk;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (!HALF || i < 2) asrc[i] += (long)kt0 * (kTK * 4);
      else asrc[i] += (long)kt0 * L::kBRow;
#pragma unroll
    for (int i = 0; i < BPW; ++i) bsrc[i] += (long)kt0 * L::kBRow;
    if constexpr (SCALE == SC_BLOCK) ssrc += (kt0 * kTK) / g.bs;
  }
  auto issue = [&](uint8_t* sb, int kt) QMOE_INLINE {
    if constexpr (HALF) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
        __builtin_amdgcn_global_load_lds(QMOE_GLOBAL(asrc[i] + (long)kt * (kTK * 4)),
                                         QMOE_LOCAL(sb + (wave * 2 + i) * 1024), 16, 0, 0);
#pragma unroll
      for (int i = 0; i < BPW; ++i) {
        __builtin_amdgcn_global_load_lds(QMOE_GLOBAL(bsrc[i] + (long)kt * L::kBRow),
                                         QMOE_LOCAL(sb + kABuf + (wave * BPW + i) * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(QMOE_GLOBAL(asrc[2 + i] + (long)kt * L::kBRow),
                                         QMOE_LOCAL(sb + kABuf / 2 + (wave * BPW + i) * 1024), 16, 0, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_global_load_lds(QMOE_GLOBAL(asrc[i] + (long)kt * (kTK * 4)),
                                         QMOE_LOCAL(sb + (wave * 4 + i) * 1024), 16, 0, 0);
#pragma unroll
      for (int i = 0; i < BPW; ++i)
        __builtin_amdgcn_global_load_lds(QMOE_GLOBAL(bsrc[i] + (long)kt * L::kBRow),
                                         QMOE_LOCAL(sb + kABuf + (wave * BPW + i) * 1024), 16, 0, 0);
      if constexpr (SCALE == SC_BLOCK)
        __builtin_amdgcn_global_load_lds(QMOE_GLOBAL(ssrc + (kt * kTK + shalf) / g.bs),
                                         QMOE_LOCAL(sb + kABuf + L::kBBuf + (wave >> 2) * (kTN * 4) + (wave & 3) * 256),
                                         4, 0, 0);
    }
  };
  auto wait_loads = [&]() QMOE_INLINE { wait_vm<NV>(); };

  f32x4 acc[4][4];
  f32x4 blk[4][4];  // block-scale spans: the span's sum, folded into acc when it closes
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ms = 0; ms < 4; ++ms)
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) {
      acc[ms][ns] = zero4;
      blk[ms][ns] = zero4;
    }
  const UnpackMasks um = unpack_masks();
  const int cg = code_group_of_lane<BITS>(grp);

  // Schedule: the K loop runs in ticks separated by workgroup barriers.  Per
  // 32-code half-step a wavefront has a fragment tick (read the half's
  // operands from LDS into registers: the packed weight words of its four
  // column subtiles, A hi/lo of its four row subtiles, the closing span's
  // block scales; fold the span that closed before) and a matrix tick
  // (unpack the weights and run its 32 matrix instructions, no LDS access).
  // The second wavefront group (rows 64..127; one wavefront of each group on
  // every SIMD) meets one extra barrier before the loop, so it runs one tick
  // behind the first and on each SIMD one wavefront's matrix instructions
  // overlap the other's fragment work.  Both groups run the same code and
  // meet the same number of barriers (the first group's extra one comes
  // after the loop).  (One barrier per half-step, met by the two groups at
  // different points so that they alternate without a barrier between the
  // phases, measured 20 % slower: the groups drift into the same phase.)
  //
  // A K step (two halves) is four ticks, its barriers p0..p3.  Before p3 of
  // step kt a wavefront waits for its own loads of step kt + 1 (those of
  // kt + 2 stay in flight): the first group's fragment tick of step kt + 1
  // follows its p0 of kt + 1, which for the second group is p3 of step kt,
  // so every wavefront's loads of a step have landed before any wavefront
  // reads its buffer.  After p0 of step kt the loads of step kt + 2 go to the
  // buffer of step kt - 1, whose last reader (the second group's fragment
  // tick of half 1) ended at that barrier.
  f16x8 ah[4], al[4];
  typename BRaw<BITS>::type raw[4];
  float sc[4] = {0.f, 0.f, 0.f, 0.f};  // block scales of the span that closed last
  // nothing moves across a tick's barrier (LDS reads stay in their tick)
  auto bar = []() QMOE_INLINE {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
  };
  // fold the span that closed: acc += blk * its scales
  auto fold = [&]() QMOE_INLINE {
#pragma unroll
    for (int ms = 0; ms < 4; ++ms)
#pragma unroll
      for (int ns = 0; ns < 4; ++ns) acc[ms][ns] += blk[ms][ns] * sc[ns];
  };
  // SEG: the factor of the segment holding K step kt (a uniform load, read
  // through the scalar cache)
  const __attribute__((address_space(4))) float* segs =
      SEG ? (const __attribute__((address_space(4))) float*)(g.seg_scale + (long)tile * g.seg_n +
                                                             ((kz * nk * kTK) >> g.seg_shift))
          : nullptr;
  // this wavefront's weight rows of a stage (half tiles, second row of
  // wavefronts: the second column half, staged in the activation buffer)
  auto bsel = [&](const uint8_t* base) QMOE_INLINE { return (half && wm == 1) ? base + kABuf / 2 : base + kABuf; };
  // Fragment tick of half j of the step in buffer base: the packed weight
  // words of the wavefront's four column subtiles, the activation hi/lo
  // fragments of its four row subtiles and the closing span's scales come
  // into registers; the fold of the span that closed before runs while they
  // are in flight.  (The weights are unpacked in the matrix tick.)
  auto frag = [&](const uint8_t* base, int j, bool fold_first, bool close, int kt) QMOE_INLINE {
    const uint8_t* bbuf = base + kABuf;
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) raw[ns] = tile_raw<BITS>(bsel(base), wn * 64 + ns * 16 + col, j, cg);
#pragma unroll
    for (int ms = 0; ms < 4; ++ms) {
      const uint8_t* arow = base + (rbase + ms * 16 + col) * 256;  // row & 15 == col
      ah[ms] = *(const f16x8*)(arow + (((8 * j + 2 * grp) ^ col) * 16));
      al[ms] = *(const f16x8*)(arow + (((8 * j + 2 * grp + 1) ^ col) * 16));
    }
    float nsc[4] = {1.f, 1.f, 1.f, 1.f};
    float fseg = 1.f;
    if constexpr (SEG) {
      if (close) {
        const float f = segs[(kt * kTK) >> g.seg_shift];
        fseg = segrow ? 1.f : f;
      }
    }
    if constexpr (SCALE == SC_BLOCK) {
      if (close) {
        const float* srow = (const float*)(bbuf + L::kBBuf) + j * kTN + wn * 64 + col;
#pragma unroll
        for (int ns = 0; ns < 4; ++ns) nsc[ns] = srow[ns * 16];
      }
    }
    if constexpr (SCALE == SC_BLOCK || SEG) {
      if (fold_first) fold();
      if (close) {
#pragma unroll
        for (int ns = 0; ns < 4; ++ns) sc[ns] = SEG ? nsc[ns] * fseg : nsc[ns];
      }
    }
    // every fragment is in registers before the barrier that ends the tick
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  };
  // Matrix tick: column subtile by column subtile, hi parts then lo parts
  // of the four row subtiles (the two instructions on one accumulator are 4
  // apart; a span's first instruction starts from zero).  Each weight
  // fragment is unpacked to exact f16 (q - mid) while the previous
  // subtile's instructions run: the unpack instructions are interleaved
  // one or two per matrix instruction.
  auto mma = [&](bool start) QMOE_INLINE {
    __builtin_amdgcn_s_setprio(1);
    f16x8 bcur = tile_unpack<BITS>(raw[0], um);
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) {
      f16x8 bnext = bcur;
      if (ns < 3) bnext = tile_unpack<BITS>(raw[ns + 1], um);
#pragma unroll
      for (int hl = 0; hl < 2; ++hl)
#pragma unroll
        for (int ms = 0; ms < 4; ++ms) {
          const f16x8& av = hl ? al[ms] : ah[ms];
          if constexpr (SCALE == SC_COL && !SEG) acc[ms][ns] = mfma16(av, bcur, acc[ms][ns]);
          else blk[ms][ns] = mfma16(av, bcur, (hl == 0 && start) ? zero4 : blk[ms][ns]);
        }
      bcur = bnext;
    }
    // order: the first fragment's unpack, then per subtile 8 matrix
    // instructions each followed by unpack instructions of the next one
    constexpr int kU0 = BITS == 4 ? 2 : 1;  // int4 unpack: 9 instructions, int8: 8
    __builtin_amdgcn_sched_group_barrier(0x002, kU0 + 7, 0);
#define QMOE_MFMA_VALU(n)                                \
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    \
  __builtin_amdgcn_sched_group_barrier(0x002, n, 0);
#define QMOE_SUBTILE() \
  QMOE_MFMA_VALU(kU0) QMOE_MFMA_VALU(1) QMOE_MFMA_VALU(1) QMOE_MFMA_VALU(1) \
  QMOE_MFMA_VALU(1) QMOE_MFMA_VALU(1) QMOE_MFMA_VALU(1) QMOE_MFMA_VALU(1)
    QMOE_SUBTILE() QMOE_SUBTILE() QMOE_SUBTILE()
#undef QMOE_SUBTILE
#undef QMOE_MFMA_VALU
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    __builtin_amdgcn_s_setprio(0);
  };
  // Spans of the block-scale sums: one half (STEPFOLD_KT 0, 32-code blocks),
  // one K step (1, 64-code blocks) or two K steps (2, blocks of 128 codes and
  // more; a span never straddles blocks).  Whether half j of a K step of
  // parity odd starts (closing false) or closes (closing true) a span:
  auto span = [](bool odd, int j, bool closing) QMOE_INLINE {
    if (STEPFOLD_KT == 0) return true;
    if (STEPFOLD_KT == 1) return closing ? j == 1 : j == 0;
    return closing ? (j == 1 && odd) : (j == 0 && !odd);
  };
  const bool trail = wm == 1;  // wave-uniform
  uint8_t* const sts[3] = {st0, st1, st2};
  issue(st0, 0);
  issue(st1, min(1, nk - 1));
  wait_loads();
  if (trail) bar();
  // one K step; D = kt modulo the unroll, so buffers and span parity are static
  auto step_d = [&](int kt, auto d_tag) QMOE_INLINE {
    constexpr int D = decltype(d_tag)::value;
    constexpr bool ODD = (D & 1) == 1;
    const uint8_t* base = sts[D % 3];
    bar();  // p0
    issue(sts[(D + 2) % 3], min(kt + 2, nk - 1));
    // fold the span that closed at half 1 of the previous step (before kt 0
    // blk and sc are zero and the fold adds nothing)
    frag(base, 0, span(!ODD, 1, true), span(ODD, 0, true), kt);
    bar();  // p1
    mma(span(ODD, 0, false));
    bar();  // p2
    frag(base, 1, span(ODD, 0, true), span(ODD, 1, true), kt);
    wait_loads();
    bar();  // p3
    mma(span(ODD, 1, false));
  };
  constexpr int U = STEPFOLD_KT == 2 ? 6 : 3;
  int kt = 0;
  for (; kt + U - 1 < nk; kt += U) {
    step_d(kt, std::integral_constant<int, 0>{});
    step_d(kt + 1, std::integral_constant<int, 1>{});
    step_d(kt + 2, std::integral_constant<int, 2>{});
    if constexpr (U == 6) {
      step_d(kt + 3, std::integral_constant<int, 3>{});
      step_d(kt + 4, std::integral_constant<int, 4>{});
      step_d(kt + 5, std::integral_constant<int, 5>{});
    }
  }
  if (kt < nk) step_d(kt, std::integral_constant<int, 0>{});
  if (kt + 1 < nk) step_d(kt + 1, std::integral_constant<int, 1>{});
  if constexpr (U == 6) {
    if (kt + 2 < nk) step_d(kt + 2, std::integral_constant<int, 2>{});
    if (kt + 3 < nk) step_d(kt + 3, std::integral_constant<int, 3>{});
    if (kt + 4 < nk) step_d(kt + 4, std::integral_constant<int, 4>{});
  }
  if (!trail) bar();
  // the last span's fold: K is a whole number of spans
  if constexpr (SCALE == SC_BLOCK || SEG) fold();
  if constexpr (SCALE == SC_COL) {
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) {
      const float sc = g.ws[ebase + min(n0 + cbase + wn * 64 + ns * 16 + col, g.N - 1)];
#pragma unroll
      for (int ms = 0; ms < 4; ++ms) acc[ms][ns] *= sc;
    }
  }

  // FC1 with segment scales: one exponent e for the whole tile (a segment of
  // FC2's reduction), from a bound B of its activated values' magnitudes so
  // that B * 2^e < 2^kRowTop: with ReLU B is their largest value; with SwiGLU
  // (|gate * sigmoid(alpha * gate)| <= |gate|) the largest gate magnitude
  // times the largest linear magnitude plus |beta|, each rounded up to a
  // power of two (a negative limit clamps to -limit).  The factor 2^-e goes
  // to seg_scale, with e clamped to [-100, 64] so that it is a normal float
  // (below -100, for magnitudes from 2^113 on, every row takes its own
  // exponent; above 64 the rows that need more do, see the epilogue).
  // Each wavefront's maxima cross the barrier below (the one that ends the
  // K loop) in s_red.
  constexpr bool seg1 = EPI != EPI_STORE;
  __shared__ float s_red[seg1 ? 2 * kTWaves : 1];
  if constexpr (seg1) {
    if (g.seg_scale != nullptr) {
      // per lane: its rows' largest magnitude (row scales undone); the lanes
      // of even columns hold gates, of odd columns linear parts (SwiGLU)
      float m = 0.f;
#pragma unroll
      for (int ms = 0; ms < 4; ++ms)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float r = 0.f;
#pragma unroll
          for (int ns = 0; ns < 4; ++ns) r = fmaxf(r, EPI == EPI_RELU ? acc[ms][ns][i] : fabsf(acc[ms][ns][i]));
          m = fmaxf(m, __builtin_ldexpf(r, -s_rexp[rbase + ms * 16 + 4 * grp + i]));
        }
#pragma unroll
      for (int o = EPI == EPI_SWIGLU ? 2 : 1; o < 64; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
      if (lane < 2) s_red[wave * 2 + lane] = m;
    }
  }
  // every load has landed and every wavefront is done with the stages
  wait_vm<0>();
  __syncthreads();
  // (half tiles: one exponent per column half, from its row of wavefronts)
  int tile_e[2] = {0, 0};
  bool tile_own[2] = {false, false};  // every nonzero row takes its own exponent
  if constexpr (seg1) {
    if (g.seg_scale != nullptr) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float G = 0.f, Lm = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < kTWaves; ++w2)
          if (!half || (w2 >> 2) == h) {
            G = fmaxf(G, s_red[2 * w2]);
            Lm = fmaxf(Lm, s_red[2 * w2 + 1]);
          }
        int e = 0;
        if constexpr (EPI == EPI_SWIGLU) {
          if (g.limit < 0.f) {
            G = fmaxf(G, -g.limit);
            Lm = fmaxf(Lm, -g.limit);
          }
          const float Lb = Lm + fabsf(g.beta);
          if (G > 0.f && Lb > 0.f && G <= 3.4028235e38f && Lb <= 3.4028235e38f)
            e = kRowTop - (__builtin_amdgcn_frexp_expf(G) + __builtin_amdgcn_frexp_expf(Lb));
        } else {
          e = row_exp(G);
        }
        tile_own[h] = e < -100;
        tile_e[h] = max(min(e, 64), -100);
      }
      if (tid < (half ? 2 : 1) && ntile + tid < ntn)
        g.seg_scale[(long)tile * g.seg_n + ntile + tid] = __builtin_ldexpf(1.f, -(tid == 0 ? tile_e[0] : tile_e[1]));
    }
  }

  // Epilogue in four rounds of 32 rows: the wavefronts holding those rows put
  // them (row scales undone) in an fp32 LDS tile [32][256] (columns
  // XOR-swizzled by 16 * ((row / 4) % 4)), then the workgroup writes whole
  // rows.  (Half tiles: rows 0-31 and 32-63 of the first column half, then
  // of the second.)
  float* otile = reinterpret_cast<float*>(st0);
  auto tix = [](int rr, int c) { return rr * kTN + (c ^ (16 * ((rr >> 2) & 3))); };
#pragma unroll
  for (int round = 0; round < 4; ++round) {  // unrolled: acc is indexed by round
    if (wm == round >> 1) {
#pragma unroll
      for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
        for (int ns = 0; ns < 4; ++ns)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int ms = (round & 1) * 2 + m2;
            const int rr = m2 * 16 + 4 * grp + i;
            otile[tix(rr, wn * 64 + ns * 16 + col)] =
                __builtin_ldexpf(acc[ms][ns][i], -s_rexp[(half ? (round & 1) * 32 : round * 32) + rr]);
          }
    }
    __syncthreads();
    const int r0 = half ? (round & 1) * 32 : round * 32;
    const int ch = half ? round >> 1 : 0;  // column half
    const int nc0 = n0 + ch * kTN;         // first column of this round
    const int rlim = min(32, rows - r0);   // valid rows of this round
    if constexpr (EPI == EPI_STORE) {
      for (int idx = tid; idx < rlim * (kTN / 4); idx += kTThreads) {
        const int rr = idx / (kTN / 4), c = 4 * (idx % (kTN / 4));
        if (nc0 + c < g.N)
          *(f32x4*)(g.slot_out + ((long)kz * g.S + s_orow[r0 + rr]) * g.N + nc0 + c) = *(const f32x4*)(otile + tix(rr, c));
      }
    } else if (g.seg_scale != nullptr) {
      // FC2 operand rows as f16 hi/lo groups of v * 2^e (the layout of the
      // operand split): this tile's codes are one segment of FC2's
      // reduction.  A thread takes one 8-code group; the groups of a row are
      // consecutive lanes.  e = tile_e unless the row's largest magnitude m
      // in the segment is nonzero and more than 2^12 below the tile's bound
      // (row_exp(m) - tile_e > 12, i.e. 0 < m < 2^(1 - tile_e)), or nonzero
      // in a tile of magnitudes from 2^113 on: then e = row_exp(m), the
      // row's own, and the flag goes up, so that FC2 takes the rows back to
      // one exponent each.  Lane masks decide it; only a wavefront holding
      // such a row reduces m across lanes.
      constexpr bool swiglu = EPI == EPI_SWIGLU;
      const int I = swiglu ? g.N / 2 : g.N;
      constexpr int jw = swiglu ? kTN / 2 : kTN;  // codes of this tile
      constexpr int GR = jw / 8;                  // 8-code groups a row
      static_assert(GR <= 64 && (64 % GR) == 0, "a row's groups lie in one wavefront");
      const int jbase = swiglu ? nc0 / 2 : nc0;
      const int te = ch ? tile_e[1] : tile_e[0];
      const bool town = ch ? tile_own[1] : tile_own[0];
      const float thr = __builtin_ldexpf(1.f, 1 - te);
#pragma unroll
      for (int b = 0; b < 32 * GR; b += kTThreads) {
        const int idx = b + tid;
        const int rr = idx / GR, gq = idx % GR;
        const int j0 = jbase + 8 * gq;
        float v[8];
        if constexpr (swiglu) {
          const int t0 = 2 * (j0 - jbase);
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            const f32x4 u = *(const f32x4*)(otile + tix(rr, t0 + 4 * h));
            v[2 * h] = swiglu_act(u[0], u[1], g.alpha, g.beta, g.limit);
            v[2 * h + 1] = swiglu_act(u[2], u[3], g.alpha, g.beta, g.limit);
          }
        } else {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const f32x4 u = *(const f32x4*)(otile + tix(rr, j0 - jbase + 4 * h));
#pragma unroll
            for (int c = 0; c < 4; ++c) v[4 * h + c] = fmaxf(u[c], 0.f);
          }
        }
        float m = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          if (j0 + c >= I) v[c] = 0.f;
          m = fmaxf(m, fabsf(v[c]));
        }
        const unsigned long long rowm = (GR == 64 ? ~0ull : ((1ull << GR) - 1)) << (lane & (64 - GR));
        const unsigned long long big = __ballot(m >= thr), nz = __ballot(m > 0.f);
        const bool own = (nz & rowm) != 0 && (town || (big & rowm) == 0);
        int e = te;
        if (__ballot(own) != 0) {
          const float mr = seg_max<GR>(m);
          if (own) e = row_exp(mr);
        }
        if (rr < rlim) {
          const long prow = (long)(p0 + r0 + rr);
          if (j0 < I) {
            f16x8 hi, lo;
            split_group<BITS>(v, e, hi, lo);
            const int q = j0 / 8;  // code group; 8-bit rows keep group sigma(q % 4) of a 32-code block
            const int sgrp = BITS == 4 ? q : ((q & ~3) | sigma8(q & 3));
            uint8_t* dst = g.act + prow * g.act_stride + (long)sgrp * 32;
            *(f16x8*)dst = hi;
            *(f16x8*)(dst + 16) = lo;
          }
          if (gq == 0) {
            if (ntile + ch < ntn) g.seg_rows[(long)(ntile + ch) * g.S + prow] = e;
            if (own) *g.seg_flag = 1;
          }
        }
      }
    } else {
      // fp32 FC2 operand rows (natural code order) for this tile's codes,
      // four a thread: ReLU code j = column n; SwiGLU code j = columns 2j
      // (gate) and 2j + 1 (linear).
      constexpr bool swiglu = EPI == EPI_SWIGLU;
      const int I = swiglu ? g.N / 2 : g.N;
      constexpr int jw = swiglu ? kTN / 2 : kTN;  // codes of this tile
      const int jbase = swiglu ? nc0 / 2 : nc0;
      for (int idx = tid; idx < rlim * (jw / 4); idx += kTThreads) {
        const int rr = idx / (jw / 4);
        const int j0 = jbase + 4 * (idx % (jw / 4));
        if (j0 >= I) continue;
        f32x4 a;
        if constexpr (swiglu) {
          const int t0 = 2 * (j0 - jbase);
          const f32x4 v0 = *(const f32x4*)(otile + tix(rr, t0)), v1 = *(const f32x4*)(otile + tix(rr, t0 + 4));
          a[0] = swiglu_act(v0[0], v0[1], g.alpha, g.beta, g.limit);
          a[1] = swiglu_act(v0[2], v0[3], g.alpha, g.beta, g.limit);
          a[2] = swiglu_act(v1[0], v1[1], g.alpha, g.beta, g.limit);
          a[3] = swiglu_act(v1[2], v1[3], g.alpha, g.beta, g.limit);
        } else {
          const f32x4 v = *(const f32x4*)(otile + tix(rr, j0 - jbase));
#pragma unroll
          for (int c = 0; c < 4; ++c) a[c] = fmaxf(v[c], 0.f);
        }
        *(f32x4*)(g.act + (long)(p0 + r0 + rr) * g.act_stride + (long)j0 * 4) = a;
      }
    }
    __syncthreads();
  }
}

template <int BITS, int SCALE, int EPI, bool STEPFOLD, int STEPFOLD_KT, bool SEG = false>
__global__ void __launch_bounds__(kTThreads) qmoe_tiled(GemmArgs g, int ntn) {
  static_assert(!SEG || (EPI == EPI_STORE && STEPFOLD && (SCALE == SC_BLOCK || STEPFOLD_KT == 2)),
                "segment scales: FC2, folded spans");
  using L = TiledLayout<BITS>;
  // Three stage buffers: a step's operands arrive by direct-to-LDS loads two
  // steps ahead of their use.
  __shared__ __align__(16) uint8_t st0[L::kStage];
  __shared__ __align__(16) uint8_t st1[L::kStage];
  __shared__ __align__(16) uint8_t st2[L::kStage];
  __shared__ long s_arow[kTM];
  __shared__ int s_orow[kTM];
  __shared__ int s_rexp[kTM];  // row scale exponent of each tile row

  // Tile order: each XCD (workgroups are dealt round robin by linear id)
  // takes a contiguous run of work ids; work ids run over groups of kGroupM
  // row tiles, column tile by column tile, row tile fastest.  The grid is
  // sized for the most tiles routing can produce; only the first linear ids
  // carry work, and they are the ones dealt out, so every XCD gets its share
  // of the real tiles.  With g.split_small the table ends with the experts'
  // last tiles of at most 64 rows (ntiles[1] tiles before them): each of
  // those is a half tile, 64 rows x 512 columns, whose second wavefront row
  // takes the second 256 columns (work ids after the full tiles').  With
  // g.ksplit K ranges (FC2) the whole order repeats once per range.
  const int mtiles = g.ntiles[0];
  const int nfull = g.split_small ? g.ntiles[1] : mtiles;
  const int ntn2 = (ntn + 1) >> 1;
  const int totf = nfull * ntn;
  const int tot1 = totf + (mtiles - nfull) * ntn2;  // tiles of one K range
  const int total = tot1 * g.ksplit;
  const int lin = blockIdx.x;
  if (lin >= total) return;
  const int xcd = lin & 7, per = total >> 3, extra = total & 7;
  const int wk = xcd * per + min(xcd, extra) + (lin >> 3);
  const int kz = wk / tot1;  // K range (the slowest index)
  const int w = wk - kz * tot1;
  const bool half = w >= totf;  // workgroup-uniform
  const int wh = half ? w - totf : w;
  const int nt_ = half ? ntn2 : ntn, t0_ = half ? nfull : 0, nm_ = half ? mtiles - nfull : nfull;
  const int grp0 = (wh / (kGroupM * nt_)) * kGroupM;
  const int gsize = min(kGroupM, nm_ - grp0);
  const int wr = wh % (kGroupM * nt_);
  const int tile = t0_ + grp0 + wr % gsize;
  const int ntile = half ? 2 * (wr / gsize) : wr / gsize;  // first 256-column tile
  // the two kinds of tile are separate instantiations of the tile's code
  // (a mode known only at run time inside the K loop makes the compiler
  // wait for every load before LDS reads it cannot separate from them)
  if (half) {
    // (the host sets split_small only with column-wise scales)
    if constexpr (SCALE == SC_COL)
      tiled_tile<BITS, SCALE, EPI, STEPFOLD, STEPFOLD_KT, SEG, true>(g, ntn, tile, ntile, kz, st0, st1, st2, s_arow,
                                                                     s_orow, s_rexp);
  } else
    tiled_tile<BITS, SCALE, EPI, STEPFOLD, STEPFOLD_KT, SEG, false>(g, ntn, tile, ntile, kz, st0, st1, st2, s_arow,
                                                                    s_orow, s_rexp);
}

#undef QMOE_GLOBAL
#undef QMOE_LOCAL
#undef QMOE_INLINE

namespace {

template <int BITS, int SCALE, int EPI, bool STEPFOLD, int STEPFOLD_KT, bool SEG = false>
hipError_t go_tiled(const GemmArgs& g, int max_tiles, int ntn, hipStream_t st) {
  auto kern = qmoe_tiled<BITS, SCALE, EPI, STEPFOLD, STEPFOLD_KT, SEG>;
  hipLaunchKernelGGL(kern, dim3(max_tiles * ntn * g.ksplit), dim3(kTThreads), 0, st, g, ntn);
  return hipGetLastError();
}

// Block sums are folded once per span of one 32-code step (32-code
// blocks), one K step (64) or two K steps (128 and more): fewer multiply-adds
// than folding every step, and no pipeline drain of a fold at block ends.
template <int BITS, int EPI>
hipError_t pick_tiled(const GemmArgs& g, int max_tiles, int ntn, hipStream_t st) {
  if (g.seg_scale != nullptr) {
    if constexpr (EPI == EPI_STORE) {
      // FC2: whole spans (two K steps with column scales), each within one
      // segment of at least 128 codes
      if (g.seg_shift < 7 || (g.bs == 0 && g.K % (2 * kTK) != 0) || g.seg_flag == nullptr || g.a_exp == nullptr)
        return hipErrorInvalidValue;
      if (g.bs == 0) return go_tiled<BITS, SC_COL, EPI, true, 2, true>(g, max_tiles, ntn, st);
      if (g.bs == 32) return go_tiled<BITS, SC_BLOCK, EPI, true, 0, true>(g, max_tiles, ntn, st);
      if (g.bs == 64) return go_tiled<BITS, SC_BLOCK, EPI, true, 1, true>(g, max_tiles, ntn, st);
      return go_tiled<BITS, SC_BLOCK, EPI, true, 2, true>(g, max_tiles, ntn, st);
    } else {
      // FC1: a segment is the codes of one column tile, seg_n of them a row
      const int codes = EPI == EPI_SWIGLU ? kTN / 2 : kTN;
      if ((1 << g.seg_shift) != codes || g.seg_n != ntn || g.seg_rows == nullptr || g.seg_flag == nullptr)
        return hipErrorInvalidValue;
    }
  }
  if (g.bs == 0) return go_tiled<BITS, SC_COL, EPI, false, 0>(g, max_tiles, ntn, st);
  if (g.bs == 32) return go_tiled<BITS, SC_BLOCK, EPI, true, 0>(g, max_tiles, ntn, st);
  if (g.bs == 64) return go_tiled<BITS, SC_BLOCK, EPI, true, 1>(g, max_tiles, ntn, st);
  return go_tiled<BITS, SC_BLOCK, EPI, true, 2>(g, max_tiles, ntn, st);
}

}  // namespace

int tiled_rows() { return kTM; }

bool tiled_ok(int64_t K, int64_t bs, bool aligned) { return aligned && K > 0 && K % kTK == 0 && (bs == 0 || bs >= 32); }

bool tiled_ksplit_ok(int64_t K, int64_t bs, int ksplit, bool store) {
  if (ksplit == 1) return true;
  if (!store || ksplit < 1 || K % ksplit != 0) return false;
  const int64_t kr = K / ksplit;
  return kr % 256 == 0 && (bs == 0 || kr % bs == 0);
}

hipError_t launch_tiled(int bits, int epi, const GemmArgs& g_in, int max_tiles, hipStream_t st) {
  if (!tiled_ok(g_in.K, g_in.bs, true) || (g_in.N & 3) != 0) return hipErrorInvalidValue;
  GemmArgs g = g_in;
  if (g.ksplit < 1) g.ksplit = 1;
  if (g.ksplit > 1 && !tiled_ksplit_ok(g.K, g.bs, g.ksplit, epi == EPI_STORE)) return hipErrorInvalidValue;
  const int ntn = (g.N + kTN - 1) / kTN;
  if (bits == 4) {
    if (epi == EPI_RELU) return pick_tiled<4, EPI_RELU>(g, max_tiles, ntn, st);
    if (epi == EPI_SWIGLU) return pick_tiled<4, EPI_SWIGLU>(g, max_tiles, ntn, st);
    return pick_tiled<4, EPI_STORE>(g, max_tiles, ntn, st);
  }
  if (epi == EPI_RELU) return pick_tiled<8, EPI_RELU>(g, max_tiles, ntn, st);
  if (epi == EPI_SWIGLU) return pick_tiled<8, EPI_SWIGLU>(g, max_tiles, ntn, st);
  return pick_tiled<8, EPI_STORE>(g, max_tiles, ntn, st);
}

}  // namespace qmoe
