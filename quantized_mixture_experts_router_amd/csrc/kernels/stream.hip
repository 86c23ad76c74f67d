// Weight-streaming grouped GEMM for small token counts (every expert's rows fit
// one M tile of at most 64 rows): the same product as gemm.hip,
//
//   part[z, p, n] = sum_{c in K-range z} a[p, c] * (q[e, n, c] - mid) * scale[e, n, c / bs]
//
// (ONNX GroupedMatMul-29, Summary, over weights dequantised as the QMoE
// WebGPU manifest's description and derive.quantMidpoint state), organised so
// that packed weights leave HBM exactly once, in long coalesced runs:
//
//  * a workgroup owns one expert tile, one K range (blockIdx.z) and a group of
//    row blocks (blockIdx.y); it stages the tile's activation rows for its K
//    range in LDS once;
//  * each wavefront streams (row block, CPI 64-byte chunks) items: 16*NT
//    weight rows, lane (n, g) loading 16 contiguous bytes of row n per chunk,
//    so an item covers whole 128-byte lines; P items of loads are in flight in
//    a register ring that runs across row blocks;
//  * a cross-lane exchange (v_permlane32/16_swap) puts each lane's bytes in
//    the matrix-core operand position; bytes are unpacked to exact f16
//    (q - mid) in registers and multiplied by the f16 hi and lo parts of the
//    activations on v_mfma_f32_16x16x32_f16 (fp32 accumulation);
//  * scales travel in the same ring and are applied in fp32 at the end of each
//    scale block;
//  * fp32 partial rows go to part[z]; qmoe_act (FC1) and the combine (FC2)
//    sum the K ranges in a fixed order, so nothing uses atomics.
#include "common.hpp"
#include "launch.h"

namespace qmoe {

namespace {

constexpr int kSWaves = 8;  // wavefronts per workgroup

template <int BITS>
__device__ __forceinline__ f16x8 chunk_operand(const u32x4& v, int j) {
  if constexpr (BITS == 4) return unpack4(v[j]);
  else return unpack8x2(v[2 * j], v[2 * j + 1]);
}

template <int BITS>
__device__ __forceinline__ void exchange(u32x4& v) {
  if constexpr (BITS == 4) transpose4x4(v);
  else swap_pairs(v);
}

}  // namespace

// SPB: MFMA steps per scale block when blocks end inside a chunk; 0 when the
// scales are column-wise or a block spans whole chunks.
// CPI: 64-byte chunks per streamed item (2 = whole 128-byte lines per row).
template <int BITS, int MT, int NT, int P, int SCALE, int SPB, int CPI>
__global__ void __launch_bounds__(64 * kSWaves, 2) qmoe_stream(GemmArgs g) {
  constexpr int CC = BITS == 4 ? 128 : 64;     // codes per 64-byte chunk
  constexpr int NS = CC / 32;                  // MFMA steps per chunk
  constexpr int NSC = SPB > 0 ? NS / SPB : 1;  // scale blocks ending per chunk
  constexpr int NSI = NSC * CPI;               // scales per item and row
  constexpr int ROWS = 16 * MT;
  extern __shared__ __align__(16) uint8_t lds[];

  const int tile = blockIdx.x;
  if (tile >= g.ntiles[0]) return;
  const int e = g.tiles[4 * tile + 0];
  const int p0 = g.tiles[4 * tile + 1];
  const int rows = g.tiles[4 * tile + 2];
  const int nch = g.K / CC;
  const int c0 = blockIdx.z * g.chunks_per_split;
  const int c1 = min(nch, c0 + g.chunks_per_split);
  if (c0 >= c1) return;
  const int nchr = c1 - c0;
  // LDS row r holds the K range's 16-byte pieces with the piece index XOR-ed
  // by (r & 15), so the 16 rows read by one instruction hit distinct banks.
  const int lstride = nchr * CC * 4;

  // Stage activation rows [p0, p0 + ROWS) (clamped to valid rows) for codes of
  // chunks [c0, c1) into LDS, 16 bytes per thread per pass.
  {
    const int pieces = nchr * CC * 4 / 16;  // 16-byte pieces per row
    for (int i = threadIdx.x; i < ROWS * pieces; i += 64 * kSWaves) {
      const int r = i / pieces;
      const int q = i - r * pieces;
      const int p = p0 + min(r, rows - 1);
      const long ar = g.a_map ? (long)(g.a_map[p] / g.a_div) : (long)p;
      const u32x4 v = *(const u32x4*)(g.a + ar * g.a_stride + (long)c0 * CC * 4 + q * 16);
      *(u32x4*)(lds + r * lstride + ((q ^ (r & 15)) * 16)) = v;
    }
  }
  __syncthreads();

  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int rb_rows = kSWaves * 16 * NT;              // rows per row block
  const int rg0 = blockIdx.y * g.rb_per_group;        // first row block of this group
  // row blocks of this wave that start inside N form a prefix
  int nrb = 0;
  for (int rb = 0; rb < g.rb_per_group; ++rb)
    if ((rg0 + rb) * rb_rows + wave * 16 * NT < g.N) nrb = rb + 1;
  const int ipr = nchr / CPI;  // items per row block (K ranges are whole items)
  const int items = nrb * ipr;
  if (items == 0) return;

  const long ebase = (long)e * g.N;
  auto row_of = [&](int rb, int nt) { return min((rg0 + rb) * rb_rows + wave * 16 * NT + nt * 16 + col, g.N - 1); };

  f32x4 acc[MT][NT];
  f32x4 blk[MT][NT];
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      acc[mt][nt] = zero4;
      blk[mt][nt] = zero4;
    }

  u32x4 bq[P][NT][CPI];
  float sq[P][NT][NSI];
  auto issue = [&](int slot, int it) {
    const int rb = it / ipr;
    const int c = c0 + (it - rb * ipr) * CPI;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const long row = ebase + row_of(rb, nt);
      const uint8_t* src = g.wq + row * g.kb + grp * 16 + (long)c * 64;
#pragma unroll
      for (int h = 0; h < CPI; ++h) bq[slot][nt][h] = *(const u32x4*)(src + h * 64);
      if constexpr (SCALE != SC_COL) {
        const float* sr = g.ws + row * g.nblk;
        if constexpr (SPB > 0) {
          // NSI consecutive block scales starting at this item's first block
          const float* sp = sr + (c * CC) / g.bs;
          if constexpr (NSI == 4) {
            const f32x4 v = *(const f32x4*)sp;
#pragma unroll
            for (int i = 0; i < 4; ++i) sq[slot][nt][i] = v[i];
          } else if constexpr (NSI == 2) {
            const float2 v = *(const float2*)sp;
            sq[slot][nt][0] = v.x;
            sq[slot][nt][1] = v.y;
          } else {
#pragma unroll
            for (int i = 0; i < NSI; ++i) sq[slot][nt][i] = sp[i];
          }
        } else {
          // blocks of whole chunks: the block scale of each chunk of the item
#pragma unroll
          for (int h = 0; h < CPI; ++h) sq[slot][nt][h] = sr[((c + h) * CC) / g.bs];
        }
      }
    }
  };
#pragma unroll
  for (int u = 0; u < P; ++u)
    if (u < items) issue(u, u);

  const int cpb = (SCALE != SC_COL && SPB == 0) ? g.bs / CC : 1;  // chunks per scale block
  const uint8_t* lrow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) lrow[mt] = lds + (mt * 16 + col) * lstride;
  const int swz = col;  // (row & 15) of every row this lane reads

  for (int i0 = 0; i0 < items; i0 += P) {
#pragma unroll
    for (int u = 0; u < P; ++u) {
      const int it = i0 + u;
      if (it < items) {
        const int rb = it / ipr;
        const int il = it - rb * ipr;  // item index inside the K range
        u32x4 cur[NT][CPI];
        float scur[NT][NSI];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
          for (int h = 0; h < CPI; ++h) cur[nt][h] = bq[u][nt][h];
#pragma unroll
          for (int i = 0; i < NSI; ++i) scur[nt][i] = sq[u][nt][i];
        }
        if (it + P < items) issue(u, it + P);
#pragma unroll
        for (int h = 0; h < CPI; ++h) {
          const int cl = il * CPI + h;  // chunk index inside the K range
          const int c = c0 + cl;
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) exchange<BITS>(cur[nt][h]);
#pragma unroll
          for (int j = 0; j < NS; ++j) {
            f16x8 ahi[MT], alo[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
              const int q = (cl * NS + j) * 8 + grp * 2;  // 16-byte piece of the hi half
              ahi[mt] = *(const f16x8*)(lrow[mt] + ((q ^ swz) * 16));
              alo[mt] = *(const f16x8*)(lrow[mt] + (((q + 1) ^ swz) * 16));
            }
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
              const f16x8 b = chunk_operand<BITS>(cur[nt][h], j);
#pragma unroll
              for (int mt = 0; mt < MT; ++mt) {
                if constexpr (SCALE == SC_COL) {
                  acc[mt][nt] = mfma16(ahi[mt], b, acc[mt][nt]);
                  acc[mt][nt] = mfma16(alo[mt], b, acc[mt][nt]);
                } else if constexpr (SPB > 0) {
                  f32x4 t = mfma16(ahi[mt], b, (j % SPB == 0) ? zero4 : blk[mt][nt]);
                  t = mfma16(alo[mt], b, t);
                  if (j % SPB == SPB - 1) acc[mt][nt] += t * scur[nt][h * NSC + j / SPB];
                  else blk[mt][nt] = t;
                } else {
                  blk[mt][nt] = mfma16(ahi[mt], b, blk[mt][nt]);
                  blk[mt][nt] = mfma16(alo[mt], b, blk[mt][nt]);
                }
              }
            }
          }
          if constexpr (SCALE != SC_COL && SPB == 0) {
            // end of a scale block, or end of this K range's share of one
            if ((c + 1) % cpb == 0 || cl == nchr - 1) {
#pragma unroll
              for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                  acc[mt][nt] += blk[mt][nt] * scur[nt][h];
                  blk[mt][nt] = zero4;
                }
            }
          }
        }
        if (il == ipr - 1) {
          // row block done: column scales, then fp32 partial rows
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            const int n = (rg0 + rb) * rb_rows + wave * 16 * NT + nt * 16 + col;
            float sc = 1.f;
            if constexpr (SCALE == SC_COL) sc = g.ws[ebase + min(n, g.N - 1)];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
              for (int i2 = 0; i2 < 4; ++i2) {
                const int r = mt * 16 + 4 * grp + i2;
                if (r < rows && n < g.N) {
                  const long prow = g.store_by_slot ? (long)g.perm[p0 + r] : (long)(p0 + r);
                  g.slot_out[((long)blockIdx.z * g.S + prow) * g.N + n] = acc[mt][nt][i2] * sc;
                }
              }
              acc[mt][nt] = zero4;
            }
          }
        }
      }
    }
  }
}

// FC1 epilogue for the streamed path: sum the K-range partials of each
// expert-sorted row p in range order, apply ReLU or interleaved SwiGLU
// (g * sigmoid(alpha * g) * (u + beta), g = h[2j], u = h[2j+1]) and write the
// f16 hi/lo operand rows of FC2.  One thread per 8-code storage group; groups
// beyond I are zero padding.
template <int BITS, int EPI>
__global__ void __launch_bounds__(256) qmoe_act(const float* __restrict__ part, int splits, int S, int F, int I,
                                                int kp2, float alpha, float beta, uint8_t* __restrict__ act) {
  const long gid = (long)blockIdx.x * 256 + threadIdx.x;
  const int groups = kp2 / 8;
  if (gid >= (long)S * groups) return;
  const int p = gid / groups;
  const int q0 = (gid % groups) * 8;
  f16x8 hi, lo;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int j = code_of_storage<BITS>(q0 + i);
    float a = 0.f;
    if (j < I) {
      if constexpr (EPI == EPI_SWIGLU) {
        float gv = 0.f, uv = 0.f;
        for (int z = 0; z < splits; ++z) {
          const float* row = part + ((long)z * S + p) * F;
          gv += row[2 * j];
          uv += row[2 * j + 1];
        }
        a = gv / (1.f + expf(-alpha * gv)) * (uv + beta);
      } else {
        float hv = 0.f;
        for (int z = 0; z < splits; ++z) hv += part[((long)z * S + p) * F + j];
        a = fmaxf(hv, 0.f);
      }
    }
    _Float16 h, l;
    split_f16(a, h, l);
    hi[i] = h;
    lo[i] = l;
  }
  uint8_t* dst = act + (long)p * kp2 * 4 + (long)q0 * 4;
  *(f16x8*)dst = hi;
  *(f16x8*)(dst + 16) = lo;
}

namespace {

template <int BITS, int MT, int NT, int SCALE, int SPB>
void go(int cpi, const GemmArgs& g, dim3 grid, size_t lds, hipStream_t st) {
  if (cpi == 2)
    hipLaunchKernelGGL((qmoe_stream<BITS, MT, NT, 2, SCALE, SPB, 2>), grid, dim3(64 * kSWaves), lds, st, g);
  else
    hipLaunchKernelGGL((qmoe_stream<BITS, MT, NT, 3, SCALE, SPB, 1>), grid, dim3(64 * kSWaves), lds, st, g);
}

template <int BITS, int MT, int NT>
void pick_scale(int cpi, const GemmArgs& g, dim3 grid, size_t lds, hipStream_t st) {
  constexpr int CC = BITS == 4 ? 128 : 64;
  if (g.bs == 0) return go<BITS, MT, NT, SC_COL, 0>(cpi, g, grid, lds, st);
  if (g.bs >= CC) return go<BITS, MT, NT, SC_BLOCK, 0>(cpi, g, grid, lds, st);
  if (g.bs == 32) return go<BITS, MT, NT, SC_BLOCK, 1>(cpi, g, grid, lds, st);
  if constexpr (BITS == 4) {
    if (g.bs == 64) return go<BITS, MT, NT, SC_BLOCK, 2>(cpi, g, grid, lds, st);
  }
}

template <int BITS, int NT>
void pick_mt(int mt, int cpi, const GemmArgs& g, dim3 grid, size_t lds, hipStream_t st) {
  switch (mt) {
    case 1: return pick_scale<BITS, 1, NT>(cpi, g, grid, lds, st);
    case 2: return pick_scale<BITS, 2, NT>(cpi, g, grid, lds, st);
    case 3: return pick_scale<BITS, 3, NT>(cpi, g, grid, lds, st);
    default: return pick_scale<BITS, 4, NT>(cpi, g, grid, lds, st);
  }
}

}  // namespace

hipError_t launch_stream(int bits, int mt, int nt, int cpi, int splits, int rb_groups, const GemmArgs& g,
                         int max_tiles, hipStream_t st) {
  const int cc = bits == 4 ? 128 : 64;
  const size_t lds = (size_t)16 * mt * g.chunks_per_split * cc * 4;
  const dim3 grid(max_tiles, rb_groups, splits);
  if (bits == 4) {
    if (nt == 2) pick_mt<4, 2>(mt, cpi, g, grid, lds, st);
    else pick_mt<4, 4>(mt, cpi, g, grid, lds, st);
  } else {
    if (nt == 2) pick_mt<8, 2>(mt, cpi, g, grid, lds, st);
    else pick_mt<8, 4>(mt, cpi, g, grid, lds, st);
  }
  return hipGetLastError();
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
