// Grouped quantised GEMM for the QMoE expert FFN, with fused dequantisation
// and fused epilogues, on gfx950 matrix cores (v_mfma_f32_16x16x32_f16).
//
// out[p, n] = sum_c a[p, c] * (q[e, n, c] - mid) * scale[e, n, c / bs]
//
// for every expert-sorted row p of an M tile that belongs to expert e (the
// GroupedMatMul of the ONNX GroupedMatMul-29 page, Summary, over weights
// dequantised as the QMoE WebGPU manifest's description and derive.quantMidpoint
// state).  FC1 epilogue: ReLU, or interleaved SwiGLU g*sigmoid(alpha*g)*(u+beta)
// on row pairs (2j, 2j+1) (manifest attributeDescriptions.swiglu_fusion,
// activation_alpha, activation_beta), written as the next GEMM's fp32
// operand rows.  FC2 epilogue: rows are written back to their slot id, so the
// combine can gather them without atomics.
//
// Work decomposition: a workgroup (blockIdx.x = M tile, blockIdx.y = weight
// row block) owns one M tile (expert, <= 16*MT rows) and 64*WAVES weight rows; each wavefront owns 16*NT weight rows, streams them
// from HBM once, unpacks them in registers straight into the matrix-core B
// operand, and reuses each unpacked fragment for all MT row subtiles.
//
// Operand precision: weights are exact integers in f16; activation rows are
// scaled by 2^e (one e per row, see common.hpp), split into f16 hi + lo and
// multiplied twice into fp32 accumulators; each row's result is multiplied
// by 2^-e in the epilogue.  Blockwise scales are applied in fp32 when a scale
// block ends.
#include "common.hpp"
#include "launch.h"

namespace qmoe {

constexpr int kNT = 4;     // 16-row weight subtiles per wavefront
constexpr int kWaves = 4;  // wavefronts per workgroup

// Eight codes of weight row `row` starting at code c0 = 32*s + 8*group, as
// exact f16 (q - mid) in A-row storage order.  Codes at or beyond K read as 0
// (their activation partner is zero padding).
template <int BITS, bool ALIGNED>
__device__ __forceinline__ f16x8 load_b(const uint8_t* __restrict__ row, int c0, int K) {
  if constexpr (BITS == 4) {
    uint32_t d = 0;
    if constexpr (ALIGNED) {
      if (c0 < K) d = *(const uint32_t*)(row + c0 / 2);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (c0 + 2 * j < K) d |= uint32_t(row[c0 / 2 + j]) << (8 * j);
    }
    return unpack4(d);
  } else {
    uint32_t d0 = 0, d1 = 0;
    if constexpr (ALIGNED) {
      if (c0 < K) {
        const u32x2 v = *(const u32x2*)(row + c0);
        d0 = v[0];
        d1 = v[1];
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (c0 + j < K) d0 |= uint32_t(row[c0 + j]) << (8 * j);
        if (c0 + 4 + j < K) d1 |= uint32_t(row[c0 + 4 + j]) << (8 * j);
      }
    }
    return unpack8x2(d0, d1);
  }
}

template <int BITS, int MT, int EPI, int SCALE, bool ALIGNED>
__global__ void __launch_bounds__(64 * kWaves) qmoe_gemm(GemmArgs g) {
  const int tile = blockIdx.x;
  if (tile >= g.ntiles[0]) return;
  const int e = g.tiles[4 * tile + 0];
  const int p0 = g.tiles[4 * tile + 1];
  const int rows = g.tiles[4 * tile + 2];
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int nb = (blockIdx.y * kWaves + wave) * (16 * kNT);
  if (nb >= g.N) return;
  const int col = lane & 15;  // B column / A row owned by this lane
  const int grp = lane >> 4;  // code group inside a 32-code step

  const uint8_t* arow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int r = min(mt * 16 + col, rows - 1);
    const int p = p0 + r;
    const long ar = g.a_map ? (long)(g.a_map[p] / g.a_div) : (long)p;
    arow[mt] = g.a + ar * g.a_stride + grp * 32;
  }
  const uint8_t* brow[kNT];
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) {
    const int n = min(nb + nt * 16 + col, g.N - 1);
    brow[nt] = g.wq + ((long)e * g.N + n) * g.kb;
  }

  f32x4 acc[MT][kNT];
  f32x4 blk[MT][kNT];
  f32x4 blk2[MT][kNT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
      acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
      blk[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
      blk2[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

  const int nsteps = (g.K + 31) / 32;
  const f16x8 zero8 = {};
  for (int s = 0; s < nsteps; ++s) {
    f16x8 ahi[MT], alo[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const uint8_t* ap = arow[mt] + (long)s * 128;
      ahi[mt] = *(const f16x8*)ap;
      alo[mt] = *(const f16x8*)(ap + 16);
    }
    const int c0 = s * 32 + code_group_of_lane<BITS>(grp) * 8;
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
      const f16x8 b = load_b<BITS, ALIGNED>(brow[nt], c0, g.K);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if constexpr (SCALE == SC_COL) {
          acc[mt][nt] = mfma16(ahi[mt], b, acc[mt][nt]);
          acc[mt][nt] = mfma16(alo[mt], b, acc[mt][nt]);
        } else if constexpr (SCALE == SC_BLOCK) {
          blk[mt][nt] = mfma16(ahi[mt], b, blk[mt][nt]);
          blk[mt][nt] = mfma16(alo[mt], b, blk[mt][nt]);
        } else {
          // 16-code scale blocks: code groups 0,1 and 2,3 of a step belong to
          // different blocks; split the step by masking the activation side.
          const bool first = code_group_of_lane<BITS>(grp) < 2;
          const f16x8 h0 = first ? ahi[mt] : zero8, l0 = first ? alo[mt] : zero8;
          const f16x8 h1 = first ? zero8 : ahi[mt], l1 = first ? zero8 : alo[mt];
          blk[mt][nt] = mfma16(h0, b, blk[mt][nt]);
          blk[mt][nt] = mfma16(l0, b, blk[mt][nt]);
          blk2[mt][nt] = mfma16(h1, b, blk2[mt][nt]);
          blk2[mt][nt] = mfma16(l1, b, blk2[mt][nt]);
        }
      }
    }
    if constexpr (SCALE == SC_BLOCK) {
      if (((s + 1) * 32) % g.bs == 0 || s == nsteps - 1) {
        const int kbi = (s * 32) / g.bs;
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
          const int n = min(nb + nt * 16 + col, g.N - 1);
          const float sc = g.ws[((long)e * g.N + n) * g.nblk + kbi];
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            acc[mt][nt] += blk[mt][nt] * sc;
            blk[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
        }
      }
    } else if constexpr (SCALE == SC_BLOCK16) {
      const int kb0 = 2 * s;
      const int kb1 = min(2 * s + 1, g.nblk - 1);
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) {
        const int n = min(nb + nt * 16 + col, g.N - 1);
        const float s0 = g.ws[((long)e * g.N + n) * g.nblk + kb0];
        const float s1 = g.ws[((long)e * g.N + n) * g.nblk + kb1];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          acc[mt][nt] += blk[mt][nt] * s0 + blk2[mt][nt] * s1;
          blk[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
          blk2[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
    }
  }
  if constexpr (SCALE == SC_COL) {
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
      const int n = min(nb + nt * 16 + col, g.N - 1);
      const float sc = g.ws[(long)e * g.N + n];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt][nt] *= sc;
    }
  }

  // Epilogue.  acc[mt][nt][i] is row mt*16 + 4*grp + i, column nb + nt*16 + col.
  int nexp[MT][4];  // -e of each row this lane holds
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = p0 + min(mt * 16 + 4 * grp + i, rows - 1);
      const long ar = g.a_map ? (long)(g.a_map[p] / g.a_div) : (long)p;
      nexp[mt][i] = -g.a_exp[ar];
    }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
      const int n = nb + nt * 16 + col;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = mt * 16 + 4 * grp + i;
        const float v = __builtin_ldexpf(acc[mt][nt][i], nexp[mt][i]);
        if constexpr (EPI == EPI_STORE) {
          if (r < rows && n < g.N) g.slot_out[(long)g.perm[p0 + r] * g.N + n] = v;
        } else {
          float a;
          int j;
          bool writer;
          if constexpr (EPI == EPI_SWIGLU) {
            const float u = __shfl_xor(v, 1);
            a = swiglu_act(v, u, g.alpha, g.beta, g.limit);
            j = n >> 1;
            writer = (col & 1) == 0;
          } else {
            a = fmaxf(v, 0.f);
            j = n;
            writer = true;
          }
          if (writer && r < rows && n < g.N) *(float*)(g.act + (long)(p0 + r) * g.act_stride + (long)j * 4) = a;
        }
      }
    }
  }
}

template <int BITS, int EPI, int SCALE, bool AL>
static void launch_mt(int mt, const GemmArgs& g, dim3 grid, hipStream_t st) {
  const dim3 block(64 * kWaves);
  switch (mt) {
    case 1: hipLaunchKernelGGL((qmoe_gemm<BITS, 1, EPI, SCALE, AL>), grid, block, 0, st, g); break;
    case 2: hipLaunchKernelGGL((qmoe_gemm<BITS, 2, EPI, SCALE, AL>), grid, block, 0, st, g); break;
    case 3: hipLaunchKernelGGL((qmoe_gemm<BITS, 3, EPI, SCALE, AL>), grid, block, 0, st, g); break;
    default: hipLaunchKernelGGL((qmoe_gemm<BITS, 4, EPI, SCALE, AL>), grid, block, 0, st, g); break;
  }
}

template <int BITS, int EPI>
static void launch_scale(int mt, bool aligned, const GemmArgs& g, dim3 grid, hipStream_t st) {
  const int sc = g.bs == 0 ? SC_COL : (g.bs == 16 ? SC_BLOCK16 : SC_BLOCK);
  if (aligned) {
    if (sc == SC_COL) launch_mt<BITS, EPI, SC_COL, true>(mt, g, grid, st);
    else if (sc == SC_BLOCK) launch_mt<BITS, EPI, SC_BLOCK, true>(mt, g, grid, st);
    else launch_mt<BITS, EPI, SC_BLOCK16, true>(mt, g, grid, st);
  } else {
    if (sc == SC_COL) launch_mt<BITS, EPI, SC_COL, false>(mt, g, grid, st);
    else if (sc == SC_BLOCK) launch_mt<BITS, EPI, SC_BLOCK, false>(mt, g, grid, st);
    else launch_mt<BITS, EPI, SC_BLOCK16, false>(mt, g, grid, st);
  }
}

hipError_t launch_gemm(int bits, int epi, int mt, bool aligned, const GemmArgs& g, int max_tiles, hipStream_t st) {
  const int rows_per_wg = 16 * kNT * kWaves;
  const dim3 grid(max_tiles, (g.N + rows_per_wg - 1) / rows_per_wg);
  if (bits == 4) {
    if (epi == EPI_RELU) launch_scale<4, EPI_RELU>(mt, aligned, g, grid, st);
    else if (epi == EPI_SWIGLU) launch_scale<4, EPI_SWIGLU>(mt, aligned, g, grid, st);
    else launch_scale<4, EPI_STORE>(mt, aligned, g, grid, st);
  } else {
    if (epi == EPI_RELU) launch_scale<8, EPI_RELU>(mt, aligned, g, grid, st);
    else if (epi == EPI_SWIGLU) launch_scale<8, EPI_SWIGLU>(mt, aligned, g, grid, st);
    else launch_scale<8, EPI_STORE>(mt, aligned, g, grid, st);
  }
  return hipGetLastError();
}

// out[t, h] = sum_s w[t, s] * (sum_z slot_out[z][t*k + s, h]); z then s
// ascending, fp32.  One writer per output element, no atomics.  SHARE (a
// share of the experts): slots with local[t*k + s] >= El have no row and are
// skipped.
template <bool SHARE>
__global__ void __launch_bounds__(256) qmoe_combine(const float* __restrict__ slot_out,
                                                    const float* __restrict__ topk_w, int T, int k, int H,
                                                    int splits, float* __restrict__ out,
                                                    const int* __restrict__ local, int El) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  const long S = (long)T * k;
  if ((H & 3) == 0) {
    const long n4 = (long)T * H / 4;
    if (i >= n4) return;
    const long t = (i * 4) / H;
    const int h = (int)((i * 4) % H);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (splits == 1 && SHARE) {
      // one partial row per slot, held slots only (a share holds a few of
      // each token's slots), in slot order
      for (int s = 0; s < k; ++s)
        if (local[t * k + s] < El) acc += topk_w[t * k + s] * *(const f32x4*)(slot_out + (t * k + s) * H + h);
      *(f32x4*)(out + t * H + h) = acc;
      return;
    }
    if (splits == 1) {
      // one partial row per slot: eight slots' rows in flight at a time,
      // weighted and summed in slot order
      for (int s0 = 0; s0 < k; s0 += 8) {
        f32x4 v[8];
        float wv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (s0 + i < k) {
            wv[i] = topk_w[t * k + s0 + i];
            v[i] = *(const f32x4*)(slot_out + (t * k + s0 + i) * H + h);
          }
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (s0 + i < k) acc += wv[i] * v[i];
      }
      *(f32x4*)(out + t * H + h) = acc;
      return;
    }
    for (int s = 0; s < k; ++s) {
      if (SHARE && local[t * k + s] >= El) continue;
      const float w = topk_w[t * k + s];
      const float* src = slot_out + (t * k + s) * H + h;
      f32x4 y;
      // sixteen partial rows in flight at a time, summed in range order
      for (int z0 = 0; z0 < splits; z0 += 16) {
        f32x4 v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (z0 + i < splits) v[i] = *(const f32x4*)(src + (long)(z0 + i) * S * H);
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (z0 + i < splits) y = (z0 + i == 0) ? v[i] : y + v[i];
      }
      acc += w * y;
    }
    *(f32x4*)(out + t * H + h) = acc;
  } else {
    if (i >= (long)T * H) return;
    const long t = i / H;
    const int h = (int)(i % H);
    float acc = 0.f;
    for (int s = 0; s < k; ++s) {
      if (SHARE && local[t * k + s] >= El) continue;
      float y = slot_out[(t * k + s) * H + h];
      for (int z = 1; z < splits; ++z) y += slot_out[((long)z * S + t * k + s) * H + h];
      acc += topk_w[t * k + s] * y;
    }
    out[t * H + h] = acc;
  }
}

hipError_t launch_combine(const float* slot_out, const float* topk_w, int T, int k, int H, int splits, float* out,
                          hipStream_t st, const int* local, int El) {
  const long n = (H & 3) == 0 ? (long)T * H / 4 : (long)T * H;
  if (local)
    hipLaunchKernelGGL(qmoe_combine<true>, dim3((n + 255) / 256), dim3(256), 0, st, slot_out, topk_w, T, k, H, splits,
                       out, local, El);
  else
    hipLaunchKernelGGL(qmoe_combine<false>, dim3((n + 255) / 256), dim3(256), 0, st, slot_out, topk_w, T, k, H, splits,
                       out, local, El);
  return hipGetLastError();
}

__global__ void qmoe_fill_zero(float* __restrict__ out, long n) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i < n) out[i] = 0.f;
}

hipError_t launch_fill_zero(float* out, long n, hipStream_t st) {
  if (n > 0) hipLaunchKernelGGL(qmoe_fill_zero, dim3((n + 255) / 256), dim3(256), 0, st, out, n);
  return hipGetLastError();
}

template <typename V>
__global__ void qmoe_copy(const V* __restrict__ src, V* __restrict__ dst, long n) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i < n) dst[i] = src[i];
}

hipError_t launch_copy_i32(const int* src, int* dst, long n, hipStream_t st) {
  if (n > 0) hipLaunchKernelGGL(qmoe_copy<int>, dim3((n + 255) / 256), dim3(256), 0, st, src, dst, n);
  return hipGetLastError();
}

hipError_t launch_copy_f32(const float* src, float* dst, long n, hipStream_t st) {
  if (n > 0) hipLaunchKernelGGL(qmoe_copy<float>, dim3((n + 255) / 256), dim3(256), 0, st, src, dst, n);
  return hipGetLastError();
}

}  // namespace qmoe
