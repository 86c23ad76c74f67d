// Weight-streaming grouped GEMM for small token counts (tiles of 8 or 16 * mt
// expert-sorted rows; an expert with more rows takes several tiles): the same
// product as gemm.hip,
//
//   y[p, n] = sum_{c in K range z} a[p, c] * (q[e, n, c] - mid) * scale[e, n, c / bs]
//
// (ONNX GroupedMatMul-29, Summary, over weights dequantised as the QMoE
// WebGPU manifest's description and derive.quantMidpoint state), organised so
// that packed weights leave HBM exactly once, in long coalesced runs:
//
//  * a workgroup owns one expert tile (blockIdx.z), 256 weight rows
//    (blockIdx.y, 32 per wavefront) and one K range (blockIdx.x; the whole of
//    K unless there are too few workgroups to fill the chip).  It walks the
//    range in stages; the tile's activation slice of the next stage is
//    fetched while the current one is used (two LDS buffers, one barrier a
//    stage), so each weight row is read front to back in one pass;
//  * each wavefront streams items of 32 weight rows x 128 bytes (whole cache
//    lines), lane (n, g) loading 16 bytes of row n from each 64-byte half; kP
//    items are in flight while one is consumed, and only loads are in flight
//    during the stream, so every wait is exact;
//  * a cross-lane exchange (v_permlane32/16_swap) puts each lane's bytes in
//    the matrix-core operand position; bytes are unpacked to exact f16
//    (q - mid) in registers and multiplied by the f16 hi and lo parts of the
//    activations on v_mfma_f32_16x16x32_f16 (fp32 accumulation).  Operand
//    rows are fp32 (the layer input for FC1, the activation rows for FC2) and
//    are split into hi/lo while staged, after scaling by a power of two per
//    row: a single-stage workgroup takes its own per K range, a
//    double-buffered one the whole row's (see common.hpp);
//  * block scales are loaded one stage ahead, shared across lanes with
//    ds_bpermute, and applied in fp32 as each block closes;
//  * results go through an LDS tile and leave as contiguous 16-byte stores:
//    FC1 over the whole of K applies ReLU or interleaved SwiGLU there and
//    writes FC2's fp32 operand rows directly; otherwise fp32 partial rows per
//    K range are written, and qmoe_act (FC1) or the combine (FC2) sum the
//    ranges in a fixed order (no atomics).
#pragma once

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "common.hpp"
#include "launch.h"
#include "qmoe_plan.h"

namespace qmoe {

namespace {

// Tunables (compile-time).
#ifndef QMOE_STREAM_INFLIGHT
#define QMOE_STREAM_INFLIGHT 2
#endif
#ifndef QMOE_STREAM_XCD_ORDER
#define QMOE_STREAM_XCD_ORDER 0
#endif
#ifndef QMOE_STREAM_NT_LOADS
#define QMOE_STREAM_NT_LOADS 0
#endif
#ifndef QMOE_STREAM_ROTATE
#define QMOE_STREAM_ROTATE 0
#endif
constexpr int kSWaves = 8;  // wavefronts per workgroup
constexpr int kCPI = 2;     // 64-byte chunks per item (one 128-byte line per row)
// Items of loads in flight per wavefront while one is consumed: double-buffered
// stages / single stage.
constexpr int kPStaged = QMOE_STREAM_INFLIGHT;
#ifndef QMOE_STREAM_INFLIGHT_ONE
#define QMOE_STREAM_INFLIGHT_ONE 2
#endif
constexpr int kPOne = QMOE_STREAM_INFLIGHT_ONE;
#ifndef QMOE_STREAM_NT
#define QMOE_STREAM_NT 2
#endif
constexpr int kNT = QMOE_STREAM_NT;  // 16-row weight subtiles per wavefront
constexpr int kWGRows = kSWaves * 16 * kNT;  // weight rows per workgroup

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

// Template parameters: STG items per stage; SCALE mode; SPB = MFMA steps per
// scale block when blocks end inside a chunk (0 when scales are column-wise or
// a block spans whole chunks); FC1 = the A rows are the layer's fp32 input
// rows (token of each slot) and the epilogue may apply the activation;
// otherwise A rows are the fp32 FC2 operand rows in sorted order.  Either way
// rows are split into f16 hi/lo while staging.
// ONE: the K range is a single stage, staged once (no barriers in the
// stream); otherwise stages are double buffered.  RB: row blocks of
// kWGRows weight rows streamed one after the other against the one stage
// (ONE only), amortising the staging.  HS > 0 (ONE, MT == 1 only): tiles of
// 8 rows, whose single stage holds HS items (the matrix instructions still
// cover 16 rows; rows past the tile's read its last row and are dropped).
template <int BITS, int MT, int SCALE, int SPB, bool FC1, bool ONE, int RB, int HS>
__global__ void __launch_bounds__(64 * kSWaves) __attribute__((amdgpu_waves_per_eu(MT == 1 ? 4 : 2, MT == 1 ? 4 : 2)))
qmoe_stream(GemmArgs g) {
  static_assert(HS == 0 || (ONE && MT == 1), "8-row tiles: single stage, one row subtile");
  constexpr int STG = HS > 0 ? HS : stream_stage_items(MT, ONE);  // items per stage
  // Row blocks: ONE streams them one after the other against its one stage;
  // double-buffered mode walks the whole K range once per row block.
  constexpr int WGR = kWGRows * RB;                 // weight rows of the workgroup
  constexpr int RBI = ONE ? RB : 1;                 // row blocks inside one stage
  // With one stage there is no next stage to stage, so registers allow the
  // ring to be copied out and refilled before each item is consumed.
#ifndef QMOE_STREAM_ONE_LATE
#define QMOE_STREAM_ONE_LATE 0
#endif
  constexpr bool LATE = !ONE || QMOE_STREAM_ONE_LATE;
  constexpr int CC = BITS == 4 ? 128 : 64;      // codes per 64-byte chunk
  constexpr int NS = CC / 32;                   // MFMA steps per chunk
  constexpr int ROWS = HS > 0 ? 8 : 16 * MT;     // tile rows (staged in LDS)
  constexpr int NT = kNT;
  constexpr int SCH = STG * kCPI;               // chunks per stage
  constexpr int SCODES = SCH * CC;              // codes per stage
  constexpr int LSTRIDE = SCODES * 4;           // LDS bytes per activation row of a stage
  constexpr int BUF = ROWS * LSTRIDE;           // bytes of one stage buffer
  constexpr int PIECES = LSTRIDE / 16;          // 16-byte pieces per row
  constexpr int GR = PIECES / 2;                // 8-code groups per row
  constexpr int NTH = 64 * kSWaves;
  constexpr int GPT = (ROWS * GR + NTH - 1) / NTH;      // staged groups per thread (fp32 rows)
  // stages per loop trip: a whole number of ring turns, so ring slots are
  // compile-time constants
  constexpr int KP = ONE ? kPOne : kPStaged;      // ring depth
  constexpr int SPT = (ONE || STG % KP == 0) ? 1 : KP / STG;
  static_assert(ONE || STG % KP == 0 || KP % STG == 0, "ring and stage sizes must nest");
  static_assert(ONE || RB == 1 || SPT == 1, "row blocks of a walk start on ring slot 0");
  extern __shared__ __align__(16) uint8_t lds[];  // 2 stage buffers, then the output tile
  __shared__ long s_rowbase[ROWS];
  __shared__ int s_orow[ROWS];
  __shared__ int s_rexp[ROWS];  // row scale exponent of each tile row (results are multiplied by 2^-e)

  // Block scales of one stage per weight row when blocks end inside a chunk
  // (SPB > 0): NBS of them, Q per lane group.
  constexpr int NBS = SPB > 0 ? SCODES / (SPB * 32) : 4;
  constexpr int Q = NBS / 4;
  static_assert(SPB == 0 || (NBS % 4 == 0 && (Q == 1 || Q == 2 || Q == 4 || Q == 8)), "scale blocks per stage");

#if QMOE_STREAM_XCD_ORDER
  // Workgroups are dealt to the 8 XCDs round robin by linear id; give each
  // XCD a contiguous run of work ids (K ranges of the same rows side by side).
  const int gx = gridDim.x, gy = gridDim.y;
  const int total = gx * gy * gridDim.z;
  const int lin = blockIdx.x + gx * (blockIdx.y + gy * blockIdx.z);
  const int xcd = lin & 7, per = total >> 3, extra = total & 7;
  const int w = xcd * per + min(xcd, extra) + (lin >> 3);
  const int split = w % gx;
  const int tile = (w / gx) % gy;
  const int rgroup = w / (gx * gy);
#else
  // Tile-major order: the grid is sized for the most tiles routing can
  // produce, and the slots past the real tile count (which exit at once)
  // are dispatched last instead of between the real workgroups.
  const int split = blockIdx.x;
  const int rgroup = blockIdx.y;
  const int tile = blockIdx.z;
#endif
  // The tile record is read together with the tile count (the record of a
  // tile past the count is never used): one round trip, not two.
  const int ntl = g.ntiles[0];
  const int e = g.tiles[4 * tile + 0];
  const int p0 = g.tiles[4 * tile + 1];
  const int rows = g.tiles[4 * tile + 2];
  const int* trow = g.trows + tile * ROWS;  // slot id of each tile row (rows past the count: the last row)
  // Single stage, FC1: the fp32 input row of each tile row this wavefront
  // stages (rows wv + 8i), from the same round trip.
  constexpr int RPW = ROWS / kSWaves;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int rslot[RPW];
#pragma unroll
  for (int i = 0; i < RPW; ++i) rslot[i] = (ONE && FC1) ? trow[wv + kSWaves * i] : 0;
#pragma unroll
  for (int i = 0; i < RPW; ++i) asm volatile("" ::"s"(rslot[i]));
  asm volatile("" ::"s"(ntl), "s"(e), "s"(p0), "s"(rows));
  if (tile >= ntl) return;
  const int nst = g.nst;                 // stages in this K range
  const int nit = nst * STG;             // items in this K range
  const int c0 = split * nst * SCH;      // first chunk of the K range
  const int nstt = ONE ? 1 : RB * nst;   // stages of the whole walk
  // Double-buffered mode starts its walk of the K range at stage rot (then
  // wraps), so that concurrent workgroups read different columns of their rows.
#if QMOE_STREAM_ROTATE
  const int rot = ONE ? 0 : (int)((blockIdx.z * 5u + blockIdx.y * 3u + blockIdx.x) % (unsigned)nst);
#else
  const int rot = 0;
#endif
  auto kpos = [&](int kst) { return kst + rot < nst ? kst + rot : kst + rot - nst; };  // stage -> K stage

  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int grp = lane >> 4;
  // Rows of the workgroup: WGR, or in double-buffered mode g.wg_rows (up to
  // RB row blocks; waves whose rows of a row block lie past them re-read one
  // cached line instead and their results are dropped).
  const int R = ONE ? WGR : g.wg_rows;
  const int n0 = rgroup * R;             // first weight row of the workgroup
  const long ebase = (long)e * g.N;
  const long kb_bytes = g.kb;

  // Rows past N (last row group) stream a clamped row; their results are
  // dropped.  Row block rb adds rb * kWGRows rows.
  const long bstep = (long)kWGRows * kb_bytes;
  const long sstep = (long)kWGRows * g.nblk;
  const uint8_t* bbase[NT];
  const float* sbase[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const long row = ebase + min(n0 + wave * 16 * NT + nt * 16 + col, g.N - 1);
    bbase[nt] = g.wq + row * kb_bytes + grp * 16 + (long)c0 * 64;
    sbase[nt] = g.ws + row * g.nblk;
    if constexpr (SPB > 0) sbase[nt] += (c0 * CC) / (SPB * 32) + grp * Q;  // this lane group's blocks
  }

  // Ring of KP items: packed weights, plus the scales of blocks that span
  // whole chunks.  Item indices past the range re-read its last item (kept
  // unconditional so that the waits stay exact).
  u32x4 bq[KP][NT][kCPI];
  float sq[KP][NT][kCPI];
  // K item of walk item i of a row block
  auto kitem = [&](int i) { return kpos(i / STG) * STG + i % STG; };
  auto issue = [&](int slot, int it) {
    // ONE: item it is piece it % STG of row block it / STG (compile-time);
    // otherwise walk item it % nit of row block it / nit, past the end the
    // last item again
    int rb, itc;
    bool live = true;  // this wave has rows in the row block
    if constexpr (ONE) {
      rb = it / STG;
      itc = it % STG;
    } else {
      const int itw = min(it, RB * nit - 1);
      rb = RB > 1 && itw >= nit ? itw / nit : 0;
      itc = kitem(itw - rb * nit);
      if constexpr (RB > 1) live = rb * kWGRows + wv * 16 * NT < R;
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      // (a wave without rows here re-reads its first line: a cache hit)
      const uint8_t* src;
      if constexpr (!ONE && RB > 1) src = bbase[nt] + (live ? (int)(rb * bstep) + itc * (kCPI * 64) : 0);
      else src = bbase[nt] + rb * bstep + (long)itc * (kCPI * 64);
#pragma unroll
      for (int h = 0; h < kCPI; ++h) bq[slot][nt][h] = load_weights(src + h * 64);
      if constexpr (SCALE != SC_COL && SPB == 0) {
#pragma unroll
        for (int h = 0; h < kCPI; ++h)
          sq[slot][nt][h] = sbase[nt][(!ONE && RB > 1) ? (live ? (int)(rb * sstep) + ((c0 + itc * kCPI + h) * CC) / g.bs : 0)
                                                       : rb * sstep + ((c0 + itc * kCPI + h) * CC) / g.bs];
      }
    }
  };
  // Blocks that end inside chunks: each lane group loads its Q consecutive
  // block scales of the stage (one 4- to 16-byte load), one stage ahead; a
  // block's scale is then fetched from the owning lane group by ds_bpermute.
  float snext[NT][Q], scur[NT][Q];
  auto issue_scales = [&](int st) {  // ONE: st is the row block
    long off;
    if constexpr (ONE) {
      off = st * sstep;
    } else {
      const int stw = min(st, nstt - 1);
      int rb = RB > 1 && stw >= nst ? stw / nst : 0;
      const int kst = stw - rb * nst;
      if (RB > 1 && rb * kWGRows + wv * 16 * NT >= R) rb = 0;  // no rows there: row block 0's scales
      off = rb * sstep + (long)kpos(kst) * NBS;
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const float* sp = sbase[nt] + off;
      if constexpr (Q == 8) {
        const f32x4 v0 = *(const f32x4*)sp, v1 = *(const f32x4*)(sp + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          snext[nt][i] = v0[i];
          snext[nt][4 + i] = v1[i];
        }
      } else if constexpr (Q == 4) {
        const f32x4 v = *(const f32x4*)sp;
#pragma unroll
        for (int i = 0; i < 4; ++i) snext[nt][i] = v[i];
      } else if constexpr (Q == 2) {
        const float2 v = *(const float2*)sp;
        snext[nt][0] = v.x;
        snext[nt][1] = v.y;
      } else {
        snext[nt][0] = sp[0];
      }
    }
  };

  // Start the weight stream: its addresses depend only on the tile.
  auto start_stream = [&]() {
    if constexpr (SCALE == SC_BLOCK && SPB > 0) issue_scales(0);
#pragma unroll
    for (int u = 0; u < KP; ++u)
      if (!ONE || u < RB * STG) issue(u, u);
  };
  if constexpr (!ONE) {
    start_stream();
    // Activation row of every tile row (clamped to valid rows) and its output row.
    if (threadIdx.x < ROWS) {
      const int p = p0 + min((int)threadIdx.x, rows - 1);
      const int slot = trow[threadIdx.x];
      const long ar = FC1 ? (long)(slot / g.a_div) : (long)p;
      s_rowbase[threadIdx.x] = ar * g.a_stride + (long)c0 * CC * 4;
      s_orow[threadIdx.x] = g.store_by_slot ? slot : p;
      s_rexp[threadIdx.x] = g.a_exp ? g.a_exp[ar] : 0;  // the whole row's: the walk spans the K range
    }
    __syncthreads();
  }

  // Activation staging of one stage: loads into registers, then LDS writes.
  // Row r keeps its 16-byte pieces with the piece index XOR-ed by (r & 15), so
  // the 16 rows read by one instruction hit distinct banks.  Invalid rows
  // (>= rows) re-read the last valid row; loads are unconditional.
  // The next stage's slice is fetched in NPART parts at the start of a stage
  // (before that stage's ring refills, so that waiting for it never waits
  // for them) and written to LDS one part after each item.
  constexpr int NPART = GPT % STG == 0 ? STG : 1;
  constexpr int GPP = GPT / NPART;   // fp32 groups per thread per part
  f32x4 areg32[NPART][GPP][2];
  auto stage_load = [&](int st, int part) {
    const int stw = min(st, nstt - 1);
    const long off = (long)kpos(stw % nst) * SCODES * 4;
#pragma unroll
    for (int ii = 0; ii < GPP; ++ii) {
      const int i = part * GPP + ii;
      const int idx = min((int)threadIdx.x + i * NTH, ROWS * GR - 1);
      const int r = idx / GR, gq = idx % GR;
      // first code of storage group gq (see common.hpp): 4-bit groups hold
      // their own 8 codes, 8-bit groups those of code group sigma(gq % 4)
      const int j0 = BITS == 4 ? 8 * gq : ((8 * gq) & ~31) | (sigma8(gq & 3) << 3);
      const float* src = (const float*)(g.a + s_rowbase[min(r, rows - 1)] + off) + j0;
      areg32[part][ii][0] = *(const f32x4*)src;
      areg32[part][ii][1] = *(const f32x4*)(src + 4);
    }
  };
  auto stage_store = [&](int buf, int part) {
    uint8_t* base = lds + buf * BUF;
#pragma unroll
    for (int ii = 0; ii < GPP; ++ii) {
      const int idx = threadIdx.x + (part * GPP + ii) * NTH;
      const int r = idx / GR, gq = idx % GR;
      if (idx < ROWS * GR) {
        float v[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) v[c] = areg32[part][ii][c >> 2][c & 3];
        f16x8 hi, lo;
        split_group<BITS>(v, s_rexp[r], hi, lo);
        uint8_t* row = base + r * LSTRIDE;
        *(f16x8*)(row + (((2 * gq) ^ (r & 15)) * 16)) = hi;
        *(f16x8*)(row + (((2 * gq + 1) ^ (r & 15)) * 16)) = lo;
      }
    }
  };
  if constexpr (ONE) {
    // The only stage, staged once: wavefront w stages tile rows w + 8i (valid
    // rows only; the matrix rows past them read the last valid row), with
    // loads issued before the weight stream, so that waiting for them never
    // waits for it (loads complete in issue order).  The fp32 rows are held
    // in registers until the stream is issued; then each row's largest
    // magnitude over this K range gives its scale exponent, and the rows go
    // into LDS as f16 hi/lo of the scaled values.
    constexpr int UPR = GR;                          // load units (fp32 8-code groups) per row
    constexpr int RPI = UPR >= 64 ? 1 : 64 / UPR;    // rows per load instruction
    constexpr int MPW = RPI > 1 ? (RPW + RPI - 1) / RPI : RPW * UPR / 64;  // units per lane
    constexpr int SEG = UPR >= 64 ? 64 : UPR;        // lanes holding one row of one instruction
    static_assert(UPR % 64 == 0 || 64 % UPR == 0, "staging units");
    long rbase[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const int r = wv + kSWaves * i;
      const long ar = FC1 ? (long)(rslot[i] / g.a_div) : (long)(p0 + min(r, rows - 1));
      rbase[i] = ar * g.a_stride + (long)c0 * CC * 4;
    }
    // unit m of this lane: tile row r (r >= ROWS: none), load unit q, row base
    auto unit = [&](int m, int& r, int& q, long& base) {
      const int i0 = RPI > 1 ? m * RPI : (64 * m) / UPR;
      const int i = RPI > 1 ? i0 + lane / UPR : i0;
      r = i < RPW ? wv + kSWaves * i : ROWS;
      q = RPI > 1 ? lane % UPR : (64 * m + lane) % UPR;
      base = rbase[min(i0, RPW - 1)];
#pragma unroll
      for (int k = 1; k < RPI; ++k) {
        long v = rbase[min(i0 + k, RPW - 1)];
        asm volatile("" : "+s"(v));  // a plain select, not an indexed private array
        if (lane / UPR == k) base = v;
      }
    };
    f32x4 sv[MPW][2];
#pragma unroll
    for (int m = 0; m < MPW; ++m) {
      int r, q;
      long base;
      unit(m, r, q, base);
      sv[m][0] = f32x4{0.f, 0.f, 0.f, 0.f};
      sv[m][1] = sv[m][0];
      if (r < rows) {
        const int j0 = BITS == 4 ? 8 * q : ((8 * q) & ~31) | (sigma8(q & 3) << 3);
        const float* src = (const float*)(g.a + base) + j0;
        sv[m][0] = *(const f32x4*)src;
        sv[m][1] = *(const f32x4*)(src + 4);
      }
    }
    start_stream();
    // Largest magnitude of each row over this K range: a row of one unit is
    // held by SEG lanes; with whole-wavefront units a row spans UPR / 64
    // consecutive units.
    float um[MPW];
#pragma unroll
    for (int m = 0; m < MPW; ++m) {
      float v = 0.f;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int c = 0; c < 4; ++c) v = fmaxf(v, fabsf(sv[m][h][c]));
      um[m] = seg_max<SEG>(v);
    }
    if constexpr (RPI == 1) {
      constexpr int UW = UPR / 64;  // units per row
#pragma unroll
      for (int i = 0; i < MPW / UW; ++i) {
        float rm = 0.f;
#pragma unroll
        for (int u = 0; u < UW; ++u) rm = fmaxf(rm, um[i * UW + u]);
#pragma unroll
        for (int u = 0; u < UW; ++u) um[i * UW + u] = rm;
      }
    }
#pragma unroll
    for (int m = 0; m < MPW; ++m) {
      int r, q;
      long base;
      unit(m, r, q, base);
      const int e = row_exp(um[m]);
      const bool first = RPI > 1 ? lane % UPR == 0 : (lane == 0 && m % (UPR / 64) == 0);
      if (first && r < ROWS) s_rexp[r] = e;
      if (r < rows) {
        float v[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) v[c] = sv[m][c >> 2][c & 3];
        f16x8 hi, lo;
        split_group<BITS>(v, e, hi, lo);
        uint8_t* row = lds + r * LSTRIDE;
        *(f16x8*)(row + (((2 * q) ^ (r & 15)) * 16)) = hi;
        *(f16x8*)(row + (((2 * q + 1) ^ (r & 15)) * 16)) = lo;
      }
    }
  } else {
#pragma unroll
    for (int part = 0; part < NPART; ++part) {
      stage_load(0, part);
      stage_store(0, part);
    }
  }

  __syncthreads();

  f32x4 acc[MT][NT];
  f32x4 blk[MT][NT];
  f32x4 res[RB > 1 ? MT : 1][NT];  // first row block's results (RB == 2)
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
  int lrow[MT];
  int aoff[MT][2][2];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int ar = min(mt * 16 + col, rows - 1);
    lrow[mt] = ar * LSTRIDE;
#pragma unroll
    for (int jp = 0; jp < 2; ++jp)
#pragma unroll
      for (int hl = 0; hl < 2; ++hl) aoff[mt][jp][hl] = (((jp * 8 + grp * 2 + hl) ^ (ar & 15)) * 16);
  }

  const UnpackMasks um = unpack_masks();

  // Output of TW weight rows from n0e: every wavefront puts its rows
  // (column scales applied, row scales undone; val(row block, mt, nt, i)
  // gives the results) into the LDS tile [ROWS][TW]; tile columns are
  // XOR-swizzled by 16 * ((row / 4) % 4), so the four row groups of one
  // write hit distinct banks.  Then FC1 with one K range applies the
  // activation and writes fp32 FC2 operand rows; otherwise fp32 partial rows
  // of this K range are written.
  auto emit = [&](float* otile, auto twc, const int n0e, const int ncols, auto val) {
  constexpr int TW = decltype(twc)::value;
  auto tix = [](int rr, int c) { return rr * TW + (c ^ (16 * ((rr >> 2) & 3))); };
#pragma unroll
  for (int cb = 0; cb < TW / kWGRows; ++cb)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int c = cb * kWGRows + wave * 16 * NT + nt * 16 + col;  // tile column
      float sc = 1.f;
      if constexpr (SCALE == SC_COL) sc = g.ws[ebase + min(n0e + c, g.N - 1)];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rr = mt * 16 + 4 * grp + i;
          if (rr < rows) otile[tix(rr, c)] = __builtin_ldexpf(val(cb, mt, nt, i) * sc, -s_rexp[rr]);
        }
    }
  __syncthreads();

  if (FC1 && g.act != nullptr) {
    // Whole of K: apply the activation and write fp32 FC2 operand rows
    // (natural code order) for this workgroup's codes, four a thread.
    // ReLU: code j = row n.  Interleaved SwiGLU: code j takes rows 2j (gate)
    // and 2j + 1 (linear): g * sigmoid(alpha * g) * (u + beta).
    const bool swiglu = g.act_swiglu != 0;
    const int I = swiglu ? g.N / 2 : g.N;
    const int jbase = swiglu ? n0e / 2 : n0e;
    const int jw = swiglu ? ncols / 2 : ncols;  // codes of this tile
    for (int idx = threadIdx.x; idx < rows * (jw / 4); idx += NTH) {
      const int rr = idx / (jw / 4);
      const int j0 = jbase + 4 * (idx % (jw / 4));
      if (j0 >= I) continue;
      f32x4 a;
      if (swiglu) {
        const int t0 = 2 * (j0 - jbase);  // tile column of row 2*j0 (8 consecutive columns)
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
      // the row is padded to a multiple of 128 codes: lanes past I write zeros there
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (j0 + c >= I) a[c] = 0.f;
      *(f32x4*)(g.act + (long)(p0 + rr) * g.act_stride + (long)j0 * 4) = a;
    }
  } else if ((g.N & 3) == 0) {
    for (int idx = threadIdx.x; idx < rows * (TW / 4); idx += NTH) {
      const int rr = idx / (TW / 4), c = 4 * (idx % (TW / 4));
      if (c < ncols && n0e + c < g.N)
        *(f32x4*)(g.slot_out + ((long)split * g.S + s_orow[rr]) * g.N + n0e + c) = *(const f32x4*)(otile + tix(rr, c));
    }
  } else {
    for (int idx = threadIdx.x; idx < rows * TW; idx += NTH) {
      const int rr = idx / TW, c = idx % TW;
      if (c < ncols && n0e + c < g.N) g.slot_out[((long)split * g.S + s_orow[rr]) * g.N + n0e + c] = otile[tix(rr, c)];
    }
  }
  };

  // One stage: its STG items from LDS buffer (st & 1), with the next stage's
  // scales and activation slice fetched during the last item (issued before
  // that item's ring refill, so waiting for them never waits for the refill).
  // Q0 = position of the stage in the loop trip (compile-time), so ring slots
  // are constants.
  auto stage = [&](int st, auto q0c) {
    constexpr int Q0 = decltype(q0c)::value;
    const uint8_t* abuf = lds + (st & 1) * BUF;
    const int kst = ONE ? 0 : st % nst;    // walk stage inside the row block
#pragma unroll
    for (int il = 0; il < RBI * STG; ++il) {
      // keep each item's work in its own scheduling region (bounded live ranges)
      __builtin_amdgcn_sched_barrier(0);
      const int u = (Q0 * STG + il) % KP;
      const int it = st * STG + il;          // ONE: st == 0
      const int ii = il % STG;               // item inside the stage
      const int rb = il / STG;               // row block (ONE)
      const int itc = kst * STG + ii;        // walk item inside the row block (double-buffered)
      if constexpr (SCALE == SC_BLOCK && SPB > 0)
        if (ii == 0) {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int i = 0; i < Q; ++i) scur[nt][i] = snext[nt][i];
        }
      // LATE: consume the ring slot in place and refill it after the item;
      // otherwise copy it out and refill it first.
      u32x4 cur_copy[LATE ? 1 : NT][kCPI];
      float sc1_copy[LATE ? 1 : NT][kCPI];
      if constexpr (!LATE) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int h = 0; h < kCPI; ++h) {
            cur_copy[nt][h] = bq[u][nt][h];
            sc1_copy[nt][h] = sq[u][nt][h];
          }
      }
      u32x4 (&cur)[NT][kCPI] = *(LATE ? &bq[u] : reinterpret_cast<u32x4(*)[NT][kCPI]>(&cur_copy));
      float (&sc1)[NT][kCPI] = *(LATE ? &sq[u] : reinterpret_cast<float(*)[NT][kCPI]>(&sc1_copy));
      if constexpr (!ONE) {
        if (il == STG - 1)
          if constexpr (SCALE == SC_BLOCK && SPB > 0) issue_scales(st + 1);
        if (il == 0)
#pragma unroll
          for (int part = 0; part < NPART; ++part) stage_load(st + 1, part);
      } else if constexpr (SCALE == SC_BLOCK && SPB > 0) {
        if (ii == STG - 1 && rb + 1 < RB) issue_scales(rb + 1);  // next row block's scales
      }
      // (with one stage the items past the range are known at compile time
      // and are not fetched)
      if constexpr (!LATE)
        if (!ONE || il + KP < RBI * STG) issue(u, it + KP);
#pragma unroll
      for (int h = 0; h < kCPI; ++h) {
        const int cl = ii * kCPI + h;  // chunk index inside the stage
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) exchange<BITS>(cur[nt][h]);
#pragma unroll
        for (int j = 0; j < NS; ++j) {
          __builtin_amdgcn_sched_barrier(0);  // one step at a time: bounded live operands
          f16x8 ahi[MT], alo[MT];
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            const int qhigh = ((cl * NS + j) * 8) & ~15;  // compile-time part of the piece index
            ahi[mt] = *(const f16x8*)(abuf + lrow[mt] + qhigh * 16 + aoff[mt][j & 1][0]);
            alo[mt] = *(const f16x8*)(abuf + lrow[mt] + qhigh * 16 + aoff[mt][j & 1][1]);
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
                  const int bk = (cl * CC + j * 32) / (SPB * 32);  // block inside the stage
                  const float sc = __shfl(scur[nt][bk % Q], col + 16 * (bk / Q));
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
          const int chunk = c0 + (ONE ? ii : kitem(itc)) * kCPI + h;
          if ((chunk + 1) % cpb == 0 || ((ONE ? ii == STG - 1 : itc == nit - 1) && h == kCPI - 1)) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
              for (int mt = 0; mt < MT; ++mt) {
                acc[mt][nt] += blk[mt][nt] * sc1[nt][h];
                pin(acc[mt][nt]);
                blk[mt][nt] = zero4;
              }
          }
        }
      }
      if constexpr (LATE)
        if (!ONE || il + KP < RBI * STG) issue(u, it + KP);
      if constexpr (ONE && RB > 1)
        if (ii == STG - 1 && rb + 1 < RB) {
          // row block done: keep it until the stream ends
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
              res[mt][nt] = acc[mt][nt];
              acc[mt][nt] = zero4;
            }
        }
      // Publish this part of the next stage's activations: its buffer was last
      // read in the previous stage, which every wavefront finished before the
      // last barrier.
      if constexpr (!ONE)
        if (NPART == STG || il == STG - 1)
          if (st + 1 < nstt) stage_store((st + 1) & 1, NPART == STG ? il : 0);
    }
    __syncthreads();
  };

  // Row block rb is complete: its results leave through the stage buffer just
  // read (free after the barrier; the next write to it follows the next
  // stage) or, after the last stage, through the whole allocation; then the
  // accumulators restart.
  auto close_block = [&](int rb) {
    const int st = (rb + 1) * nst - 1;  // its last stage
    emit(reinterpret_cast<float*>(lds + (st + 1 < nstt ? (st & 1) * BUF : 0)), std::integral_constant<int, kWGRows>{},
         n0 + rb * kWGRows, min(kWGRows, R - rb * kWGRows), [&](int, int mt, int nt, int i) { return acc[mt][nt][i]; });
    if (rb + 1 < RB) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = zero4;
      __syncthreads();
    }
  };

  const int nmain = nst - nst % SPT;  // stages of one row block's walk in whole loop trips
#pragma unroll
  for (int rb = 0; rb < (ONE ? 1 : RB); ++rb) {
    const int sb = rb * nst;
    for (int s0 = 0; s0 < nmain; s0 += SPT) {
      stage(sb + s0, std::integral_constant<int, 0>{});
      if constexpr (SPT > 1) stage(sb + s0 + 1, std::integral_constant<int, 1>{});
    }
    if constexpr (SPT > 1)
      if (nmain < nst) stage(sb + nmain, std::integral_constant<int, 0>{});
    if constexpr (!ONE) close_block(rb);
  }

  if constexpr (ONE) {
    // Output: the stage buffer is free after the last barrier.  Output row
    // ids are read now (the stream is drained, so this load waits for
    // nothing else).
    if (threadIdx.x < ROWS) s_orow[threadIdx.x] = g.store_by_slot ? trow[threadIdx.x] : p0 + min((int)threadIdx.x, rows - 1);
    emit(reinterpret_cast<float*>(lds), std::integral_constant<int, WGR>{}, n0, WGR, [&](int cb, int mt, int nt, int i) {
      return (RB > 1 && cb < RB - 1) ? res[RB > 1 ? mt : 0][nt][i] : acc[mt][nt][i];
    });
  }
}


namespace {

template <int BITS, int MT, int SCALE, int SPB, bool FC1, bool ONE, int RB, int HS>
hipError_t go(const GemmArgs& g, dim3 grid, size_t lds, hipStream_t st) {
  auto kern = qmoe_stream<BITS, MT, SCALE, SPB, FC1, ONE, RB, HS>;
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

template <int BITS, int MT, bool FC1, bool ONE, int RB, int HS = 0>
hipError_t pick_scale(const GemmArgs& g, dim3 grid, size_t lds, hipStream_t st) {
  constexpr int CC = BITS == 4 ? 128 : 64;
  constexpr int SCODES = (HS > 0 ? HS : stream_stage_items(MT, ONE)) * (BITS == 4 ? 256 : 128);
  if (g.bs == 0) return go<BITS, MT, SC_COL, 0, FC1, ONE, RB, HS>(g, grid, lds, st);
  if (g.bs >= CC) return go<BITS, MT, SC_BLOCK, 0, FC1, ONE, RB, HS>(g, grid, lds, st);
  if (g.bs == 32) {
    // 32-code blocks: at most 32 a stage
    if constexpr (SCODES / 32 <= 32) return go<BITS, MT, SC_BLOCK, 1, FC1, ONE, RB, HS>(g, grid, lds, st);
    return hipErrorInvalidValue;
  }
  if constexpr (BITS == 4) {
    if (g.bs == 64) return go<BITS, MT, SC_BLOCK, 2, FC1, ONE, RB, HS>(g, grid, lds, st);
  }
  return hipErrorInvalidValue;  // scale layouts the planner never routes here
}

}  // namespace

// 8-row tiles (stream_half.hip): one-stage launches of hs items a stage.
hipError_t launch_stream_half(int bits, bool fc1, int rb, int hs, const GemmArgs& g, dim3 grid, size_t lds,
                              hipStream_t st);

}  // namespace qmoe
