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
// direct-to-LDS loads issued two steps ahead, so two steps of loads are in
// flight while a step runs on the matrix cores.  Weights are unpacked from
// LDS straight into matrix-core operands (exact f16 q - mid) and each
// fragment feeds 8 instructions (4 row subtiles x hi/lo).
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

// Eight codes [32*j + 8*cg, +8) of staged weight row n as exact f16 (q - mid)
// in A-row storage order (see common.hpp).
template <int BITS>
__device__ __forceinline__ f16x8 tile_operand(const uint8_t* bbuf, int n, int j, int cg, const UnpackMasks& m) {
  if constexpr (BITS == 4) {
    return unpack4(*(const uint32_t*)(bbuf + n * 32 + ((j ^ bswz<4>(n)) * 16) + 4 * cg), m);
  } else {
    const u32x2 v = *(const u32x2*)(bbuf + n * 64 + (((2 * j + (cg >> 1)) ^ bswz<8>(n)) * 16) + (cg & 1) * 8);
    return unpack8x2(v[0], v[1]);
  }
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

// STEPFOLD: block sums are scaled every 32-code step (STEPFOLD_KT 0, 32-code
// blocks), every 64-code K step (1, 64-code blocks) or every two K steps (2,
// blocks of 128 codes and more).
template <int BITS, int SCALE, int EPI, bool STEPFOLD, int STEPFOLD_KT>
__global__ void __launch_bounds__(kTThreads) qmoe_tiled(GemmArgs g, int ntn) {
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
  // sized for the most tiles routing can produce; only the first
  // ntiles * ntn linear ids carry work, and they are the ones dealt out, so
  // every XCD gets its share of the real tiles.
  const int mtiles = g.ntiles[0];
  const int total = mtiles * ntn;
  const int lin = blockIdx.x;
  if (lin >= total) return;
  const int xcd = lin & 7, per = total >> 3, extra = total & 7;
  const int w = xcd * per + min(xcd, extra) + (lin >> 3);
  const int grp0 = (w / (kGroupM * ntn)) * kGroupM;
  const int gsize = min(kGroupM, mtiles - grp0);
  const int wr = w % (kGroupM * ntn);
  const int tile = grp0 + wr % gsize;
  const int ntile = wr / gsize;
  const int e = g.tiles[4 * tile + 0];
  const int p0 = g.tiles[4 * tile + 1];
  const int rows = g.tiles[4 * tile + 2];
  const int n0 = ntile * kTN;

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int col = lane & 15, grp = lane >> 4;
  const long ebase = (long)e * g.N;

  if (tid < kTM) {
    const int p = p0 + min(tid, rows - 1);
    const long ar = g.a_map ? (long)(g.a_map[p] / g.a_div) : (long)p;
    s_arow[tid] = ar * g.a_stride;
    s_orow[tid] = g.store_by_slot ? g.perm[p] : p;
    s_rexp[tid] = g.a_exp[ar];
  }
  __syncthreads();

  // Per-lane sources of the step's direct-to-LDS loads (rows past the tile
  // or past N re-read a valid row; every wavefront issues the same count).
  //  A: wavefront w fills rows 16w .. 16w + 15, four rows an instruction; the
  //     slot of row r holding piece q is q ^ (r & 15);
  //  B: the step's weight rows, GPR granules a row, granule g of row n in
  //     slot g ^ swz(n);
  //  S (block scales): wavefronts 0-3 the first 32-code half, 4-7 the second.
  constexpr int BPW = L::kGPR * kTN / 64 / kTWaves;  // weight load instructions per wavefront
  constexpr int NV = 4 + BPW + (SCALE == SC_BLOCK ? 1 : 0);
  const uint8_t* asrc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (wave * 4 + i) * 4 + (lane >> 4);
    asrc[i] = g.a + s_arow[r] + (((lane & 15) ^ (r & 15)) * 16);
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
  const int nk = g.K / kTK;
  auto issue = [&](uint8_t* sb, int kt) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_global_load_lds(QMOE_GLOBAL(asrc[i] + (long)kt * (kTK * 4)), QMOE_LOCAL(sb + (wave * 4 + i) * 1024),
                                       16, 0, 0);
#pragma unroll
    for (int i = 0; i < BPW; ++i)
      __builtin_amdgcn_global_load_lds(QMOE_GLOBAL(bsrc[i] + (long)kt * L::kBRow),
                                       QMOE_LOCAL(sb + kABuf + (wave * BPW + i) * 1024), 16, 0, 0);
    if constexpr (SCALE == SC_BLOCK)
      __builtin_amdgcn_global_load_lds(QMOE_GLOBAL(ssrc + (kt * kTK + shalf) / g.bs),
                                       QMOE_LOCAL(sb + kABuf + L::kBBuf + (wave >> 2) * (kTN * 4) + (wave & 3) * 256),
                                       4, 0, 0);
  };

  f32x4 acc[4][4];
  f32x4 blk[4][4];
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

  // Step kt reads stage buffer kt % 3.  Its loads were issued two steps
  // earlier: wait for them (the next step's may stay in flight), then the
  // barrier makes every wavefront's loads visible and frees buffer
  // (kt + 2) % 3 (last read in step kt - 1) for the loads of step kt + 2.
  auto kstep = [&](int kt, uint8_t* base, uint8_t* next2, auto odd_tag) {
    constexpr bool ODD = decltype(odd_tag)::value;  // second K step of a 128-code span
    wait_vm<NV>();
    __builtin_amdgcn_s_barrier();
    // nothing moves across the barrier: reads of buffer kt % 3 stay after it,
    // the refill of buffer (kt + 2) % 3 stays after every wavefront's reads
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    issue(next2, min(kt + 2, nk - 1));
    const uint8_t* bbuf = base + kABuf;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      // weight fragments of the step, then the four row subtiles with their
      // activation fragments loaded one subtile ahead; hi parts then lo
      // parts, so the two instructions on one accumulator are 4 apart
      f16x8 bf[4], ah[2], al[2];
#pragma unroll
      for (int ns = 0; ns < 4; ++ns) bf[ns] = tile_operand<BITS>(bbuf, wn * 64 + ns * 16 + col, j, cg, um);
      auto aload = [&](int ms, f16x8& h, f16x8& l) {
        const uint8_t* arow = base + (wm * 64 + ms * 16 + col) * 256;  // row & 15 == col
        h = *(const f16x8*)(arow + (((8 * j + 2 * grp) ^ col) * 16));
        l = *(const f16x8*)(arow + (((8 * j + 2 * grp + 1) ^ col) * 16));
      };
      if constexpr (SCALE == SC_BLOCK && STEPFOLD) {
        // Scale blocks folded per 32-code step (32-code blocks), per K step
        // (64-code blocks) or per two K steps (blocks of 128 codes and more;
        // a span never straddles blocks): the first instruction of a span starts
        // from zero (no zeroing moves), and each row subtile is folded right
        // after the next subtile's instructions are issued, so no fold waits
        // on the matrix pipeline.
        // STEPFOLD_KT 0: every 32-code half starts and closes a span; 1: the
        // K step is the span; 2: two K steps (128 codes) are the span
        const bool start = STEPFOLD_KT == 0 ? true : STEPFOLD_KT == 1 ? j == 0 : (j == 0 && !ODD);
        const bool close = STEPFOLD_KT == 0 ? true : STEPFOLD_KT == 1 ? j == 1 : (j == 1 && ODD);
        const float* srow = (const float*)(base + kABuf + L::kBBuf) + j * kTN + wn * 64 + col;
        float sc[4];
        if (close) {
#pragma unroll
          for (int ns = 0; ns < 4; ++ns) sc[ns] = srow[ns * 16];
        }
        auto fold = [&](int ms) {
#pragma unroll
          for (int ns = 0; ns < 4; ++ns) acc[ms][ns] += blk[ms][ns] * sc[ns];
        };
        aload(0, ah[0], al[0]);
#pragma unroll
        for (int ms = 0; ms < 4; ++ms) {
          if (ms < 3) aload(ms + 1, ah[(ms + 1) & 1], al[(ms + 1) & 1]);
#pragma unroll
          for (int hl = 0; hl < 2; ++hl)
#pragma unroll
            for (int ns = 0; ns < 4; ++ns)
              blk[ms][ns] = mfma16(hl ? al[ms & 1] : ah[ms & 1], bf[ns], (hl == 0 && start) ? zero4 : blk[ms][ns]);
          if (close && ms > 0) fold(ms - 1);
        }
        if (close) fold(3);
      } else {
        aload(0, ah[0], al[0]);
#pragma unroll
        for (int ms = 0; ms < 4; ++ms) {
          if (ms < 3) aload(ms + 1, ah[(ms + 1) & 1], al[(ms + 1) & 1]);
#pragma unroll
          for (int hl = 0; hl < 2; ++hl)
#pragma unroll
            for (int ns = 0; ns < 4; ++ns) {
              const f16x8& av = hl ? al[ms & 1] : ah[ms & 1];
              if constexpr (SCALE == SC_COL) acc[ms][ns] = mfma16(av, bf[ns], acc[ms][ns]);
              else blk[ms][ns] = mfma16(av, bf[ns], blk[ms][ns]);
            }
        }
        if constexpr (SCALE == SC_BLOCK) {
          // blocks of 64 codes and more: scale the block's sum when it closes
          const int ks = 2 * kt + j;  // 32-code step
          if (((ks + 1) * 32) % g.bs == 0) {
            const float* srow = (const float*)(base + kABuf + L::kBBuf) + j * kTN;
#pragma unroll
            for (int ns = 0; ns < 4; ++ns) {
              const float sc = srow[wn * 64 + ns * 16 + col];
#pragma unroll
              for (int ms = 0; ms < 4; ++ms) {
                acc[ms][ns] += blk[ms][ns] * sc;
                blk[ms][ns] = zero4;
              }
            }
          }
        }
      }
    }
  };
  issue(st0, 0);
  issue(st1, min(1, nk - 1));
  // Step kt uses buffer kt % 3 and refills (kt + 2) % 3; with two-step
  // folds the parity of kt must be static too, so that mode unrolls six.
  uint8_t* const sts[3] = {st0, st1, st2};
  auto step_d = [&](int kt, auto d_tag) {
    constexpr int D = decltype(d_tag)::value;
    kstep(kt, sts[D % 3], sts[(D + 2) % 3], std::integral_constant<bool, (D & 1) == 1>{});
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
  // every load has landed and every wavefront is done with the stages
  wait_vm<0>();
  __syncthreads();

  if constexpr (SCALE == SC_COL) {
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) {
      const float sc = g.ws[ebase + min(n0 + wn * 64 + ns * 16 + col, g.N - 1)];
#pragma unroll
      for (int ms = 0; ms < 4; ++ms) acc[ms][ns] *= sc;
    }
  }

  // Epilogue in four rounds of 32 rows: the wavefronts holding those rows put
  // them (row scales undone) in an fp32 LDS tile [32][256] (columns
  // XOR-swizzled by 16 * ((row / 4) % 4)), then the workgroup writes whole
  // rows.
  float* otile = reinterpret_cast<float*>(st0);
  auto tix = [](int rr, int c) { return rr * kTN + (c ^ (16 * ((rr >> 2) & 3))); };
  for (int round = 0; round < 4; ++round) {
    if (wm == round >> 1) {
#pragma unroll
      for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
        for (int ns = 0; ns < 4; ++ns)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int ms = (round & 1) * 2 + m2;
            const int rr = m2 * 16 + 4 * grp + i;
            otile[tix(rr, wn * 64 + ns * 16 + col)] = __builtin_ldexpf(acc[ms][ns][i], -s_rexp[round * 32 + rr]);
          }
    }
    __syncthreads();
    const int r0 = round * 32;
    const int rlim = min(32, rows - r0);  // valid rows of this round
    if constexpr (EPI == EPI_STORE) {
      for (int idx = tid; idx < rlim * (kTN / 4); idx += kTThreads) {
        const int rr = idx / (kTN / 4), c = 4 * (idx % (kTN / 4));
        if (n0 + c < g.N)
          *(f32x4*)(g.slot_out + (long)s_orow[r0 + rr] * g.N + n0 + c) = *(const f32x4*)(otile + tix(rr, c));
      }
    } else {
      // fp32 FC2 operand rows (natural code order) for this tile's codes,
      // four a thread: ReLU code j = column n; SwiGLU code j = columns 2j
      // (gate) and 2j + 1 (linear).
      constexpr bool swiglu = EPI == EPI_SWIGLU;
      const int I = swiglu ? g.N / 2 : g.N;
      constexpr int jw = swiglu ? kTN / 2 : kTN;  // codes of this tile
      const int jbase = swiglu ? n0 / 2 : n0;
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

#undef QMOE_GLOBAL
#undef QMOE_LOCAL

namespace {

template <int BITS, int SCALE, int EPI, bool STEPFOLD, int STEPFOLD_KT>
hipError_t go_tiled(const GemmArgs& g, int max_tiles, int ntn, hipStream_t st) {
  auto kern = qmoe_tiled<BITS, SCALE, EPI, STEPFOLD, STEPFOLD_KT>;
  hipLaunchKernelGGL(kern, dim3(max_tiles * ntn), dim3(kTThreads), 0, st, g, ntn);
  return hipGetLastError();
}

// Block sums are folded once per span of one 32-code step (32-code
// blocks), one K step (64) or two K steps (128 and more): fewer multiply-adds
// than folding every step, and no pipeline drain of a fold at block ends.
template <int BITS, int EPI>
hipError_t pick_tiled(const GemmArgs& g, int max_tiles, int ntn, hipStream_t st) {
  if (g.bs == 0) return go_tiled<BITS, SC_COL, EPI, false, 0>(g, max_tiles, ntn, st);
  if (g.bs == 32) return go_tiled<BITS, SC_BLOCK, EPI, true, 0>(g, max_tiles, ntn, st);
  if (g.bs == 64) return go_tiled<BITS, SC_BLOCK, EPI, true, 1>(g, max_tiles, ntn, st);
  return go_tiled<BITS, SC_BLOCK, EPI, true, 2>(g, max_tiles, ntn, st);
}

}  // namespace

int tiled_rows() { return kTM; }

bool tiled_ok(int64_t K, int64_t bs, bool aligned) { return aligned && K > 0 && K % kTK == 0 && (bs == 0 || bs >= 32); }

hipError_t launch_tiled(int bits, int epi, const GemmArgs& g, int max_tiles, hipStream_t st) {
  if (!tiled_ok(g.K, g.bs, true) || (g.N & 3) != 0) return hipErrorInvalidValue;
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
