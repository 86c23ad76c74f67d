// Launchers of the weight-streaming grouped GEMM (stream_kernel.hpp) for
// 16 * mt-row tiles, and the FC1 activation pass over its K-range partials.
#include "stream_kernel.hpp"

namespace qmoe {

// FC1 epilogue for the streamed path: sum the K-range partials of each
// expert-sorted row p in range order, apply ReLU or interleaved SwiGLU
// (g * sigmoid(alpha * g) * (u + beta), g = h[2j], u = h[2j+1]) and write the
// fp32 operand rows of FC2 (natural code order, row stride kp2 codes).  One
// thread per 8 consecutive codes: it reads 8 (ReLU) or 16 (SwiGLU)
// consecutive fp32 values of every partial row with 16-byte loads, all
// partials of a batch of four ranges in flight at once.
template <int EPI>
__global__ void __launch_bounds__(256) qmoe_act(const float* __restrict__ part, int splits, int S, int F, int I,
                                                int kp2, float alpha, float beta, float limit,
                                                uint8_t* __restrict__ act) {
  constexpr int W = EPI == EPI_SWIGLU ? 16 : 8;  // FC1 values per thread
  const long gid = (long)blockIdx.x * 256 + threadIdx.x;
  const int groups = (I + 7) / 8;
  if (gid >= (long)S * groups) return;
  const int p = gid / groups;
  const int j0 = 8 * (int)(gid % groups);  // first code of the thread
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
  float a[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    a[c] = 0.f;
    if (j0 + c < I) {
      if constexpr (EPI == EPI_SWIGLU) a[c] = swiglu_act(h[2 * c], h[2 * c + 1], alpha, beta, limit);
      else a[c] = fmaxf(h[c], 0.f);
    }
  }
  // rows are padded to kp2 >= roundup(I, 8) codes: the tail group writes zeros there
  float* dst = (float*)(act + (long)p * kp2 * 4) + j0;
  *(f32x4*)dst = f32x4{a[0], a[1], a[2], a[3]};
  *(f32x4*)(dst + 4) = f32x4{a[4], a[5], a[6], a[7]};
}

namespace {

template <int BITS, bool FC1, bool ONE>
hipError_t pick_mt(int mt, int rb, const GemmArgs& g, dim3 grid, size_t lds, hipStream_t st) {
  switch (mt) {
    case 1:
      if (rb == 2) return pick_scale<BITS, 1, FC1, ONE, 2>(g, grid, lds, st);
      return pick_scale<BITS, 1, FC1, ONE, 1>(g, grid, lds, st);
    case 2: return pick_scale<BITS, 2, FC1, ONE, 1>(g, grid, lds, st);
    case 3: return pick_scale<BITS, 3, FC1, ONE, 1>(g, grid, lds, st);
    default: return pick_scale<BITS, 4, FC1, ONE, 1>(g, grid, lds, st);
  }
}

template <int BITS>
hipError_t pick_mode(bool fc1, bool one, int mt, int rb, const GemmArgs& g, dim3 grid, size_t lds, hipStream_t st) {
  if (fc1) return one ? pick_mt<BITS, true, true>(mt, rb, g, grid, lds, st) : pick_mt<BITS, true, false>(mt, rb, g, grid, lds, st);
  return one ? pick_mt<BITS, false, true>(mt, rb, g, grid, lds, st) : pick_mt<BITS, false, false>(mt, rb, g, grid, lds, st);
}

}  // namespace

// Row blocks per workgroup: two for one-stage launches at mt == 1 when they
// tile N exactly and the grid still holds at least three rounds of
// workgroups (two resident on each of 256 compute units); with fewer rounds
// the idle share of the last round costs more than the shared staging saves
// (the decode FC2: 896 workgroups of two row blocks, 62 us, against 1792 of
// one, 60 us; its FC1: 1792 of two, 110 us, against 3584 of one, 112 us).
static int stream_row_blocks(int mt, bool one, int N, int splits, int max_tiles) {
  if (!(one && mt == 1 && N % (2 * kWGRows) == 0)) return 1;
  const long wgs = (long)splits * max_tiles * (N / (2 * kWGRows));
  return wgs >= 3 * 512 ? 2 : 1;
}

size_t stream_lds_bytes(int bits, int mt, bool one, int rb, int hs) {
  const int item_codes = bits == 4 ? 256 : 128;
  const int rows = hs > 0 ? 8 : 16 * mt;
  const size_t stage = (size_t)rows * (hs > 0 ? hs : stream_stage_items(mt, one)) * item_codes * 4;
  // output tile: the workgroup's rows (one stage) or one row block
  const int tile_rb = one ? rb : 1;
  return std::max((one ? 1 : 2) * stage, (size_t)rows * kWGRows * tile_rb * 4);
}

hipError_t launch_stream(int bits, int mt, bool one, int splits, int wg_rows, int half_stg, const GemmArgs& g_in,
                         int max_tiles, hipStream_t st) {
  if (mt < 1 || mt > 4 || (one && g_in.nst != 1) || g_in.trows == nullptr) return hipErrorInvalidValue;
  if (half_stg != 0 && ((half_stg != 8 && half_stg != 4 && half_stg != 1) || !one || mt != 1)) return hipErrorInvalidValue;
  GemmArgs g = g_in;
  int rb = stream_row_blocks(mt, one, g.N, splits, max_tiles);
  if (!one) {
    if (wg_rows == 0) wg_rows = kWGRows;
    if (wg_rows % 64 != 0 || wg_rows > 2 * kWGRows || (wg_rows > kWGRows && mt != 1)) return hipErrorInvalidValue;
    rb = wg_rows > kWGRows ? 2 : 1;
  } else {
    wg_rows = kWGRows * rb;
  }
  g.wg_rows = wg_rows;
  const size_t lds = stream_lds_bytes(bits, mt, one, one ? rb : 1, half_stg);
#if QMOE_STREAM_XCD_ORDER
  const dim3 grid(splits, max_tiles, (g.N + wg_rows - 1) / wg_rows);
#else
  const dim3 grid(splits, (g.N + wg_rows - 1) / wg_rows, max_tiles);
#endif
  // operand rows are fp32 in both GEMMs; FC1 gathers them through the slot map
  if (!g.a_f32) return hipErrorInvalidValue;
  const bool fc1 = g.a_map != nullptr;
  if (half_stg != 0) return launch_stream_half(bits, fc1, rb, half_stg, g, grid, lds, st);
  return bits == 4 ? pick_mode<4>(fc1, one, mt, rb, g, grid, lds, st) : pick_mode<8>(fc1, one, mt, rb, g, grid, lds, st);
}

hipError_t launch_act(int bits, int epi, const float* part, int splits, int S, int F, int I, int kp2, float alpha,
                      float beta, float limit, uint8_t* act, hipStream_t st) {
  (void)bits;
  if (kp2 < (I + 7) / 8 * 8 || kp2 % 4 != 0) return hipErrorInvalidValue;
  const long n = (long)S * ((I + 7) / 8);
  const dim3 grid((n + 255) / 256), block(256);
  if (epi == EPI_SWIGLU) hipLaunchKernelGGL((qmoe_act<EPI_SWIGLU>), grid, block, 0, st, part, splits, S, F, I, kp2, alpha, beta, limit, act);
  else hipLaunchKernelGGL((qmoe_act<EPI_RELU>), grid, block, 0, st, part, splits, S, F, I, kp2, alpha, beta, limit, act);
  return hipGetLastError();
}

}  // namespace qmoe
