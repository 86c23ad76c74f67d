// Weight-streaming grouped GEMM for small token counts (every expert's rows fit
// one M tile of at most 64 rows): the same product as gemm.hip,
//
//   part[z, p, n] = sum_{c in K-range z} a[p, c] * (q[e, n, c] - mid) * scale[e, n, c / bs]
//
// (ONNX GroupedMatMul-29, Summary, over weights dequantised as the QMoE
// WebGPU manifest's description and derive.quantMidpoint state), organised so
// that packed weights leave HBM exactly once, in long coalesced runs:
//
//  * a workgroup owns one K range (blockIdx.x), one expert tile (blockIdx.y)
//    and RBW blocks of 32 weight rows per wavefront (blockIdx.z); it stages
//    the tile's activation rows for that K range in LDS once and streams its
//    row blocks one after another;
//  * each wavefront streams ITEMS items of 16*NT weight rows x 128 bytes
//    (whole cache lines), lane (n, g) loading 16 bytes of row n from each
//    64-byte half; the item loop is fully unrolled and the next kP items'
//    loads are in flight while one item is consumed, so every wait is exact;
//  * a cross-lane exchange (v_permlane32/16_swap) puts each lane's bytes in
//    the matrix-core operand position; bytes are unpacked to exact f16
//    (q - mid) in registers and multiplied by the f16 hi and lo parts of the
//    activations on v_mfma_f32_16x16x32_f16 (fp32 accumulation);
//  * block scales travel in the ring with the weights and are applied in fp32
//    at the end of each scale block;
//  * fp32 partial rows of all row blocks are stored once, after the stream
//    (no stores interleave with the weight loads); qmoe_act (FC1) and the
//    combine (FC2) sum the K ranges in a fixed order (no atomics).
#include <algorithm>
#include <atomic>

#include "common.hpp"
#include "launch.h"

namespace qmoe {

namespace {

// Tunables (compile-time).
#ifndef QMOE_STREAM_INFLIGHT
#define QMOE_STREAM_INFLIGHT 2
#endif
#ifndef QMOE_STREAM_NT_LOADS
#define QMOE_STREAM_NT_LOADS 0
#endif
constexpr int kSWaves = 8;  // wavefronts per workgroup
constexpr int kCPI = 2;     // 64-byte chunks per item (one 128-byte line per row)
constexpr int kP = QMOE_STREAM_INFLIGHT;  // items of loads in flight per wavefront while one is consumed

// Packed weights are read exactly once: optionally mark the loads streaming.
__device__ __forceinline__ u32x4 load_weights(const uint8_t* p) {
#if QMOE_STREAM_NT_LOADS
  return __builtin_nontemporal_load((const u32x4*)p);
#else
  return *(const u32x4*)p;
#endif
}

template <int BITS>
__device__ __forceinline__ f16x8 chunk_operand(const u32x4& v, int j, const UnpackMasks& m) {
  if constexpr (BITS == 4) return unpack4(v[j], m);
  else return unpack8x2(v[2 * j], v[2 * j + 1]);
}

// Keep a scale-block flush where it is written: without this the compiler may
// sink every "acc += blk * scale" to the end and keep all block partials live.
__device__ __forceinline__ void pin(f32x4& v) { asm volatile("" : "+v"(v)); }

template <int BITS>
__device__ __forceinline__ void exchange(u32x4& v) {
  if constexpr (BITS == 4) transpose4x4(v);
  else swap_pairs(v);
}

}  // namespace

// SPB: MFMA steps per scale block when blocks end inside a chunk; 0 when the
// scales are column-wise or a block spans whole chunks.  RBW: row blocks of
// kSWaves*16*NT rows that the workgroup streams one after another (the staged
// activations are reused for all of them).
template <int BITS, int MT, int NT, int ITEMS, int SCALE, int SPB, int RBW>
__global__ void __launch_bounds__(64 * kSWaves) __attribute__((amdgpu_waves_per_eu(MT == 1 ? 4 : 2, MT == 1 ? 4 : 2)))
qmoe_stream(GemmArgs g) {
  constexpr int CC = BITS == 4 ? 128 : 64;      // codes per 64-byte chunk
  constexpr int NS = CC / 32;                   // MFMA steps per chunk
  constexpr int ROWS = 16 * MT;
  constexpr int NCHR = ITEMS * kCPI;            // chunks in the K range
  constexpr int LSTRIDE = NCHR * CC * 4;        // LDS bytes per activation row
  constexpr int PIECES = LSTRIDE / 16;          // 16-byte pieces per row
  constexpr int PPT = ROWS * PIECES / (64 * kSWaves);  // pieces per thread
  static_assert(ROWS * PIECES % (64 * kSWaves) == 0, "staging must divide evenly");
  constexpr int WROWS = kSWaves * 16 * NT;      // weight rows of one row block
  constexpr int NITEMS = RBW * ITEMS;           // items streamed by each wavefront
  extern __shared__ __align__(16) uint8_t lds[];  // [ROWS][LSTRIDE] activations
  __shared__ long s_rowbase[ROWS];

  // Block scales of the K range per weight row when blocks end inside a chunk
  // (SPB > 0): NBR of them, Q per lane group.
  constexpr int NBR = SPB > 0 ? NCHR * CC / (SPB * 32) : 4;
  constexpr int Q = NBR / 4;
  static_assert(SPB == 0 || (NBR % 4 == 0 && Q <= 8), "scale blocks per K range");

  // Work w = (K range, expert tile, group of RBW row blocks), K range fastest.
  // Workgroups are dealt to the 8 XCDs round robin by linear id; each XCD is
  // given a contiguous run of work ids, so the K ranges of the same weight
  // rows run side by side on one XCD and share its L2 (scale rows and
  // activation slices are fetched from HBM once).
  const int gx = gridDim.x, gy = gridDim.y;
  const int total = gx * gy * gridDim.z;
  const int lin = blockIdx.x + gx * (blockIdx.y + gy * blockIdx.z);
  const int xcd = lin & 7, per = total >> 3, extra = total & 7;
  const int w = xcd * per + min(xcd, extra) + (lin >> 3);
  const int split = w % gx;
  const int tile = (w / gx) % gy;
  const int rgroup = w / (gx * gy);
  if (tile >= g.ntiles[0]) return;
  const int e = g.tiles[4 * tile + 0];
  const int p0 = g.tiles[4 * tile + 1];
  const int rows = g.tiles[4 * tile + 2];
  const int c0 = split * NCHR;

  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int grp = lane >> 4;
  // This wavefront's rows in row block r: rb0 + r * WROWS + nt * 16 + col.
  const int rb0 = rgroup * RBW * WROWS + wave * 16 * NT;
  const bool active = rb0 < g.N;  // all waves take part in the staging below
  const long ebase = (long)e * g.N;
  const long kb_bytes = g.kb;

  // Per-subtile base pointers for row block 0; row block r adds r * WROWS rows
  // (with RBW > 1 the rows of every block are in range: N is a multiple of
  // RBW * WROWS).
  const uint8_t* bbase[NT];
  const float* sbase[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const long row = ebase + min(rb0 + nt * 16 + col, g.N - 1);
    bbase[nt] = g.wq + row * kb_bytes + grp * 16 + (long)c0 * 64;
    sbase[nt] = g.ws + row * g.nblk;
    if constexpr (SPB > 0) sbase[nt] += (c0 * CC) / (SPB * 32) + grp * Q;  // this lane group's blocks
  }
  const long bstep = (long)WROWS * kb_bytes;  // bytes between row blocks
  const long sstep = (long)WROWS * g.nblk;    // scales between row blocks

  // Ring of kP items in flight: packed weights, plus the scales of blocks
  // that span whole chunks.
  u32x4 bq[kP][NT][kCPI];
  float sq[kP][NT][kCPI];
  auto issue = [&](int slot, int it) {  // it is a compile-time constant after unrolling
    const int r = it / ITEMS, il = it % ITEMS;
    const int c = c0 + il * kCPI;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const uint8_t* src = bbase[nt] + r * bstep + il * kCPI * 64;
#pragma unroll
      for (int h = 0; h < kCPI; ++h) bq[slot][nt][h] = load_weights(src + h * 64);
      if constexpr (SCALE != SC_COL && SPB == 0) {
        const float* sr = sbase[nt] + r * sstep;
#pragma unroll
        for (int h = 0; h < kCPI; ++h) sq[slot][nt][h] = sr[((c + h) * CC) / g.bs];
      }
    }
  };
  // Blocks that end inside chunks: each lane group loads Q consecutive block
  // scales of its row once per row block (one coalesced 16-byte-class load);
  // a block's scale is then fetched from the owning lane group by ds_bpermute.
  float sreg[2][NT][Q];
  auto issue_scales = [&](int r) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const float* sp = sbase[nt] + r * sstep;
#pragma unroll
      for (int q4 = 0; q4 < Q; q4 += 4) {
        if constexpr (Q >= 4) {
          const f32x4 v = *(const f32x4*)(sp + q4);
#pragma unroll
          for (int i = 0; i < 4; ++i) sreg[r & 1][nt][q4 + i] = v[i];
        }
      }
      if constexpr (Q == 2) {
        const float2 v = *(const float2*)sp;
        sreg[r & 1][nt][0] = v.x;
        sreg[r & 1][nt][1] = v.y;
      } else if constexpr (Q == 1) {
        sreg[r & 1][nt][0] = sp[0];
      }
    }
  };

  // Start the weight stream before the activation staging so that its latency
  // overlaps the staging's dependent loads.
  if (active) {
    if constexpr (SCALE == SC_BLOCK && SPB > 0) issue_scales(0);
#pragma unroll
    for (int u = 0; u < kP && u < NITEMS; ++u) issue(u, u);
  }
  // Output rows (slot ids or sorted positions) for the epilogue.
  int orow[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = min(mt * 16 + 4 * grp + i, rows - 1);
      orow[mt][i] = g.store_by_slot ? g.perm[p0 + rr] : p0 + rr;
    }

  // Stage activation rows [p0, p0 + ROWS) (clamped to valid rows) for the K
  // range into LDS.  Row r keeps its 16-byte pieces with the piece index XOR-ed
  // by (r & 15), so the 16 rows read by one instruction hit distinct banks.
  if (threadIdx.x < ROWS) {
    const int p = p0 + min((int)threadIdx.x, rows - 1);
    const long ar = g.a_map ? (long)(g.a_map[p] / g.a_div) : (long)p;
    s_rowbase[threadIdx.x] = ar * g.a_stride + (long)c0 * CC * 4;
  }
  __syncthreads();
  // Only the tile's valid rows are staged; matrix rows beyond them read the
  // last valid row (their results are discarded).
  if (g.a_f32) {
    // fp32 rows (the layer input): each thread converts groups of 8 codes,
    // 32 bytes of floats, into their 16-byte hi and lo pieces.
    constexpr int GR = PIECES / 2;                                // groups per row
    constexpr int GPT = (ROWS * GR + 64 * kSWaves - 1) / (64 * kSWaves);
    f32x4 v[GPT][2];
#pragma unroll
    for (int i = 0; i < GPT; ++i) {
      const int idx = threadIdx.x + i * 64 * kSWaves;
      const int r = idx / GR, gq = idx % GR;
      // first code of storage group gq (see common.hpp): 4-bit groups hold
      // their own 8 codes, 8-bit groups those of code group sigma(gq % 4)
      const int j0 = BITS == 4 ? 8 * gq : ((8 * gq) & ~31) | (sigma8(gq & 3) << 3);
      if (idx < ROWS * GR && r < rows) {
        const float* src = (const float*)(g.a + s_rowbase[r]) + j0;
        v[i][0] = *(const f32x4*)src;
        v[i][1] = *(const f32x4*)(src + 4);
      }
    }
#pragma unroll
    for (int i = 0; i < GPT; ++i) {
      const int idx = threadIdx.x + i * 64 * kSWaves;
      const int r = idx / GR, gq = idx % GR;
      if (idx < ROWS * GR && r < rows) {
        f16x8 hi, lo;
#pragma unroll
        for (int sl = 0; sl < 8; ++sl) {
          const int c = BITS == 4 ? perm4_of_slot(sl) : sl;  // code inside the group at storage slot sl
          _Float16 h, l;
          split_f16(v[i][c >> 2][c & 3], h, l);
          hi[sl] = h;
          lo[sl] = l;
        }
        uint8_t* row = lds + r * LSTRIDE;
        *(f16x8*)(row + (((2 * gq) ^ (r & 15)) * 16)) = hi;
        *(f16x8*)(row + (((2 * gq + 1) ^ (r & 15)) * 16)) = lo;
      }
    }
  } else {
    u32x4 v[PPT];
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int idx = threadIdx.x + i * 64 * kSWaves;
      const int r = idx / PIECES, q = idx % PIECES;
      if (r < rows) v[i] = *(const u32x4*)(g.a + s_rowbase[r] + q * 16);
    }
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int idx = threadIdx.x + i * 64 * kSWaves;
      const int r = idx / PIECES, q = idx % PIECES;
      if (r < rows) *(u32x4*)(lds + r * LSTRIDE + ((q ^ (r & 15)) * 16)) = v[i];
    }
  }
  __syncthreads();
  if (!active) return;

  f32x4 acc[MT][NT];
  f32x4 blk[MT][NT];
  f32x4 res[RBW][MT][NT];  // finished row blocks, stored after the stream
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      acc[mt][nt] = zero4;
      blk[mt][nt] = zero4;
    }

  const int cpb = (SCALE != SC_COL && SPB == 0) ? g.bs / CC : 1;  // chunks per scale block
  // Swizzled piece q of row r sits at ((q & ~15) | ((q & 15) ^ (r & 15))) * 16.
  // The low four bits of q here are 8*(step parity) + 2*grp + (0 hi | 1 lo),
  // so the runtime part of every activation address is one of four per-lane
  // offsets per row subtile.
  const uint8_t* lrow[MT];
  int aoff[MT][2][2];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int ar = min(mt * 16 + col, rows - 1);
    lrow[mt] = lds + ar * LSTRIDE;
#pragma unroll
    for (int jp = 0; jp < 2; ++jp)
#pragma unroll
      for (int hl = 0; hl < 2; ++hl) aoff[mt][jp][hl] = (((jp * 8 + grp * 2 + hl) ^ (ar & 15)) * 16);
  }

  const UnpackMasks um = unpack_masks();

#pragma unroll
  for (int it = 0; it < NITEMS; ++it) {
    // keep each item's work in its own scheduling region (bounded live ranges)
    __builtin_amdgcn_sched_barrier(0);
    const int u = it % kP;
    const int r = it / ITEMS, il = it % ITEMS;
    u32x4 cur[NT][kCPI];
    float scur[NT][kCPI];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
      for (int h = 0; h < kCPI; ++h) {
        cur[nt][h] = bq[u][nt][h];
        scur[nt][h] = sq[u][nt][h];
      }
    }
    if constexpr (SCALE == SC_BLOCK && SPB > 0)
      if (il == 0 && r + 1 < RBW) issue_scales(r + 1);  // next row block's scales
    if (it + kP < NITEMS) issue(u, it + kP);
#pragma unroll
    for (int h = 0; h < kCPI; ++h) {
      const int cl = il * kCPI + h;  // chunk index inside the K range
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) exchange<BITS>(cur[nt][h]);
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        __builtin_amdgcn_sched_barrier(0);  // one step at a time: bounded live operands
        f16x8 ahi[MT], alo[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const int qhigh = ((cl * NS + j) * 8) & ~15;  // compile-time part of the piece index
          ahi[mt] = *(const f16x8*)(lrow[mt] + qhigh * 16 + aoff[mt][j & 1][0]);
          alo[mt] = *(const f16x8*)(lrow[mt] + qhigh * 16 + aoff[mt][j & 1][1]);
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const f16x8 b = chunk_operand<BITS>(cur[nt][h], j, um);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            if constexpr (SCALE == SC_COL) {
              acc[mt][nt] = mfma16(ahi[mt], b, acc[mt][nt]);
              acc[mt][nt] = mfma16(alo[mt], b, acc[mt][nt]);
            } else if constexpr (SPB > 0) {
              if (j % SPB == 0) blk[mt][nt] = mfma16(ahi[mt], b, zero4);
              else blk[mt][nt] = mfma16(ahi[mt], b, blk[mt][nt]);
              blk[mt][nt] = mfma16(alo[mt], b, blk[mt][nt]);
              if (j % SPB == SPB - 1) {
                // block of SPB*32 codes ends inside the chunk: apply its scale
                const int b = (cl * CC + j * 32) / (SPB * 32);  // block inside the K range
                const float sc = __shfl(sreg[r & 1][nt][b % Q], col + 16 * (b / Q));
                acc[mt][nt] += blk[mt][nt] * sc;
                pin(acc[mt][nt]);
              }
            } else {
              blk[mt][nt] = mfma16(ahi[mt], b, blk[mt][nt]);
              blk[mt][nt] = mfma16(alo[mt], b, blk[mt][nt]);
            }
          }
        }
      }
      if constexpr (SCALE != SC_COL && SPB == 0) {
        // end of a scale block, or end of this K range's share of one
        if ((c0 + cl + 1) % cpb == 0 || cl == NCHR - 1) {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
              acc[mt][nt] += blk[mt][nt] * scur[nt][h];
              pin(acc[mt][nt]);
              blk[mt][nt] = zero4;
            }
        }
      }
    }
    if (il == ITEMS - 1) {
      // row block r finished: keep it until the stream ends
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          res[r][mt][nt] = acc[mt][nt];
          acc[mt][nt] = zero4;
        }
    }
  }

  // Column scales, then the fp32 partial rows of every row block.
#pragma unroll
  for (int r = 0; r < RBW; ++r)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int n = rb0 + r * WROWS + nt * 16 + col;
      float sc = 1.f;
      if constexpr (SCALE == SC_COL) sc = g.ws[ebase + min(n, g.N - 1)];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rr = mt * 16 + 4 * grp + i;
          if (rr < rows && n < g.N)
            g.slot_out[((long)split * g.S + orow[mt][i]) * g.N + n] = res[r][mt][nt][i] * sc;
        }
    }
}

// FC1 epilogue for the streamed path: sum the K-range partials of each
// expert-sorted row p in range order, apply ReLU or interleaved SwiGLU
// (g * sigmoid(alpha * g) * (u + beta), g = h[2j], u = h[2j+1]) and write the
// f16 hi/lo operand rows of FC2.  One thread per 8-code storage group: its 8
// codes are consecutive (see common.hpp), so it reads 8 (ReLU) or 16 (SwiGLU)
// consecutive fp32 values of every partial row with 16-byte loads, all
// partials of a batch of four ranges in flight at once.  Groups beyond I are
// zero padding.
template <int BITS, int EPI>
__global__ void __launch_bounds__(256) qmoe_act(const float* __restrict__ part, int splits, int S, int F, int I,
                                                int kp2, float alpha, float beta, uint8_t* __restrict__ act) {
  constexpr int W = EPI == EPI_SWIGLU ? 16 : 8;  // FC1 values per group
  const long gid = (long)blockIdx.x * 256 + threadIdx.x;
  const int groups = kp2 / 8;
  if (gid >= (long)S * groups) return;
  const int p = gid / groups;
  const int gq = gid % groups;
  const int j0 = BITS == 4 ? 8 * gq : ((8 * gq) & ~31) | (sigma8(gq & 3) << 3);  // first code of the group
  const long zstride = (long)S * F;
  float h[W];
  if (j0 + 8 <= I && (F & 3) == 0) {
    const float* base = part + (long)p * F + (W / 8) * j0;
    for (int z0 = 0; z0 < splits; z0 += 4) {
      f32x4 v[4][W / 4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (z0 + i < splits)
#pragma unroll
          for (int m = 0; m < W / 4; ++m) v[i][m] = *(const f32x4*)(base + (z0 + i) * zstride + 4 * m);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (z0 + i < splits)
#pragma unroll
          for (int m = 0; m < W / 4; ++m)
#pragma unroll
            for (int c = 0; c < 4; ++c) h[4 * m + c] = (z0 + i == 0) ? v[i][m][c] : h[4 * m + c] + v[i][m][c];
    }
  } else {
#pragma unroll
    for (int c = 0; c < W; ++c) {
      const int f = (W / 8) * j0 + c;  // FC1 row of value c
      float a = 0.f;
      if (f < (W / 8) * I)
        for (int z = 0; z < splits; ++z) a = (z == 0) ? part[(long)p * F + f] : a + part[z * zstride + (long)p * F + f];
      h[c] = a;
    }
  }
  f16x8 hi, lo;
#pragma unroll
  for (int sl = 0; sl < 8; ++sl) {
    const int c = BITS == 4 ? perm4_of_slot(sl) : sl;  // code j0 + c sits at storage slot sl
    float a = 0.f;
    if (j0 + c < I) {
      if constexpr (EPI == EPI_SWIGLU) {
        const float gv = h[2 * c], uv = h[2 * c + 1];
        a = gv / (1.f + expf(-alpha * gv)) * (uv + beta);
      } else {
        a = fmaxf(h[c], 0.f);
      }
    }
    _Float16 hh, ll;
    split_f16(a, hh, ll);
    hi[sl] = hh;
    lo[sl] = ll;
  }
  uint8_t* dst = act + (long)p * kp2 * 4 + (long)gq * 32;
  *(f16x8*)dst = hi;
  *(f16x8*)(dst + 16) = lo;
}

namespace {

template <int BITS, int MT, int NT, int ITEMS, int SCALE, int SPB, int RBW>
hipError_t go(const GemmArgs& g, dim3 grid, size_t lds, hipStream_t st) {
  auto kern = qmoe_stream<BITS, MT, NT, ITEMS, SCALE, SPB, RBW>;
  // Dynamic LDS above the 64 KB default needs a per-kernel opt-in (host-side,
  // no synchronisation); remember the largest size granted so far.
  static std::atomic<size_t> granted{64 * 1024};
  if (lds > granted.load()) {
    const hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    granted.store(lds);
  }
  hipLaunchKernelGGL(kern, grid, dim3(64 * kSWaves), lds, st, g);
  return hipGetLastError();
}

template <int BITS, int MT, int NT, int ITEMS, int RBW>
hipError_t pick_scale(const GemmArgs& g, dim3 grid, size_t lds, hipStream_t st) {
  constexpr int CC = BITS == 4 ? 128 : 64;
  if (g.bs == 0) return go<BITS, MT, NT, ITEMS, SC_COL, 0, RBW>(g, grid, lds, st);
  if (g.bs >= CC) return go<BITS, MT, NT, ITEMS, SC_BLOCK, 0, RBW>(g, grid, lds, st);
  if (g.bs == 32) return go<BITS, MT, NT, ITEMS, SC_BLOCK, 1, RBW>(g, grid, lds, st);
  if constexpr (BITS == 4) {
    if (g.bs == 64) return go<BITS, MT, NT, ITEMS, SC_BLOCK, 2, RBW>(g, grid, lds, st);
  }
  return hipErrorInvalidValue;  // scale layouts the planner never routes here
}

// Item counts per K range allowed by the 64 KB activation slice (16*MT rows,
// 4 bytes a code, 256 or 128 codes an item).
template <int BITS, int MT>
constexpr int max_items() { return 65536 / (64 * MT * (BITS == 4 ? 256 : 128)); }

template <int BITS, int MT, int RBW>
hipError_t pick_items(int items, const GemmArgs& g, dim3 grid, size_t lds, hipStream_t st) {
  constexpr int MX = max_items<BITS, MT>();
  if (items == 1) return pick_scale<BITS, MT, 2, 1, RBW>(g, grid, lds, st);
  if constexpr (MX >= 2) if (items == 2) return pick_scale<BITS, MT, 2, 2, RBW>(g, grid, lds, st);
  if constexpr (MX >= 4) if (items == 4) return pick_scale<BITS, MT, 2, 4, RBW>(g, grid, lds, st);
  if constexpr (MX >= 8) if (items == 8) return pick_scale<BITS, MT, 2, 8, RBW>(g, grid, lds, st);
  return hipErrorInvalidValue;
}

template <int BITS, int MT>
hipError_t pick_rbw(int rbw, int items, const GemmArgs& g, dim3 grid, size_t lds, hipStream_t st) {
  if (rbw == 2) return pick_items<BITS, MT, 2>(items, g, grid, lds, st);
  return pick_items<BITS, MT, 1>(items, g, grid, lds, st);
}

template <int BITS>
hipError_t pick_mt(int mt, int rbw, int items, const GemmArgs& g, dim3 grid, size_t lds, hipStream_t st) {
  switch (mt) {
    case 1: return pick_rbw<BITS, 1>(rbw, items, g, grid, lds, st);
    case 2: return pick_rbw<BITS, 2>(1, items, g, grid, lds, st);
    case 3: return pick_rbw<BITS, 3>(1, items, g, grid, lds, st);
    default: return pick_rbw<BITS, 4>(1, items, g, grid, lds, st);
  }
}

}  // namespace

hipError_t launch_stream(int bits, int mt, int items, int rbw, int splits, const GemmArgs& g, int max_tiles,
                         hipStream_t st) {
  const int cc = bits == 4 ? 128 : 64;
  const int rows_per_wg = kSWaves * 16 * 2 * (mt == 1 ? rbw : 1);
  const size_t lds = (size_t)16 * mt * items * kCPI * cc * 4;
  const dim3 grid(splits, max_tiles, (g.N + rows_per_wg - 1) / rows_per_wg);
  return bits == 4 ? pick_mt<4>(mt, rbw, items, g, grid, lds, st) : pick_mt<8>(mt, rbw, items, g, grid, lds, st);
}

hipError_t launch_act(int bits, int epi, const float* part, int splits, int S, int F, int I, int kp2, float alpha,
                      float beta, uint8_t* act, hipStream_t st) {
  const long n = (long)S * (kp2 / 8);
  const dim3 grid((n + 255) / 256), block(256);
  if (bits == 4) {
    if (epi == EPI_SWIGLU) hipLaunchKernelGGL((qmoe_act<4, EPI_SWIGLU>), grid, block, 0, st, part, splits, S, F, I, kp2, alpha, beta, act);
    else hipLaunchKernelGGL((qmoe_act<4, EPI_RELU>), grid, block, 0, st, part, splits, S, F, I, kp2, alpha, beta, act);
  } else {
    if (epi == EPI_SWIGLU) hipLaunchKernelGGL((qmoe_act<8, EPI_SWIGLU>), grid, block, 0, st, part, splits, S, F, I, kp2, alpha, beta, act);
    else hipLaunchKernelGGL((qmoe_act<8, EPI_RELU>), grid, block, 0, st, part, splits, S, F, I, kp2, alpha, beta, act);
  }
  return hipGetLastError();
}

}  // namespace qmoe
