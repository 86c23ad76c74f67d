// Routing front end of the QMoE operator:
//   qmoe_router        top-k selection and routing weights, one wavefront per token
//   qmoe_hist          per-chunk expert histogram of the selected slots
//   qmoe_scan          per-expert counts, exclusive offsets, chunk bases, M-tile table
//   qmoe_scatter       stable expert-sorted slot order (perm)
//   qmoe_route_small   all of the above in one workgroup (<= 1024 slots)
//   qmoe_route_wave    all of the above in one wavefront (<= 64 tokens, E * k <= 64)
//
// Routing follows the QMoE WebGPU manifest (description: softmax over the
// selected top-k logits; attributeDescriptions.normalize_routing_weights) and
// the float MoE README (Description: softmax over all logits before top-k,
// optional renormalisation).  The permutation is the manifest's group stage
// (variants quant_grouped_routed, pass group_stage: expert-grouped slot list
// and M-tile metadata), made stable so that it is deterministic.
#include <math.h>

#include "common.hpp"
#include "launch.h"

namespace qmoe {

// Total order used for selection: larger logit first, then lower index.
// NaN is mapped to -inf so that every token still selects k experts.
__device__ __forceinline__ bool key_before(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// Routing of token t by one wavefront; each lane holds logits e = lane + 64 * j.
// Lane 0 writes the selected experts (also to s_idx when given, for kernels
// that keep working on them in LDS).
template <int V>
__device__ __forceinline__ void route_token(const float* __restrict__ logits, int t, int E, int k, int routing,
                                            int normalize, int* __restrict__ topk_idx, float* __restrict__ topk_w,
                                            int* s_idx) {
  const int lane = lane_id();
  const float* row = logits + (size_t)t * E;
  float v[V];
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const int e = lane + 64 * j;
    float x = e < E ? row[e] : -INFINITY;
    v[j] = (x != x) ? -INFINITY : x;
  }
  // k rounds: each picks the best key strictly after the previous pick.
  float pv = INFINITY;
  int pi = -1;
  float my_val = 0.f;  // lane r keeps pick number r (k <= 64 * V handled below)
  float v0 = 0.f;
  float sum_sel = 0.f;
  for (int r = 0; r < k; ++r) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int e = lane + 64 * j;
      if (e < E && key_before(pv, pi, v[j], e) && key_before(v[j], e, bv, bi)) {
        bv = v[j];
        bi = e;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (key_before(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    bi = min(max(bi, 0), E - 1);  // always a valid expert index
    pv = bv;
    pi = bi;
    if (r == 0) v0 = bv;
    const float ex = expf(bv - v0);  // identical in every lane
    sum_sel += ex;
    if (lane == 0) {
      topk_idx[(size_t)t * k + r] = bi;
      if (s_idx) s_idx[t * k + r] = bi;
    }
    if (lane == (r & 63)) {
      if (r < 64) my_val = ex;
      else topk_w[(size_t)t * k + r] = ex;  // picks beyond 64 wait in the output buffer
    }
  }
  float denom = sum_sel;
  if (routing == 1 && !normalize) {
    // Full softmax over all experts, taken at the selection.
    float part = 0.f;
#pragma unroll
    for (int j = 0; j < V; ++j)
      if (lane + 64 * j < E) part += expf(v[j] - v0);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off);
    denom = part;
  }
  // MoE with normalisation reduces to the selected-logit softmax.
  if (lane < k) topk_w[(size_t)t * k + lane] = my_val / denom;
  for (int r = 64 + lane; r < k; r += 64) {
    const float ex = topk_w[(size_t)t * k + r];
    topk_w[(size_t)t * k + r] = ex / denom;
  }
}

// One wavefront per token.
template <int V>
__global__ void __launch_bounds__(256) qmoe_router(const float* __restrict__ logits, int T, int E, int k,
                                                   int routing, int normalize, int* __restrict__ topk_idx,
                                                   float* __restrict__ topk_w) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  route_token<V>(logits, t, E, k, routing, normalize, topk_idx, topk_w, nullptr);
}

// Histogram of selected experts over chunks of `chunk` consecutive slots.
__global__ void __launch_bounds__(256) qmoe_hist(const int* __restrict__ topk_idx, int S, int E, int chunk,
                                                 int* __restrict__ hist) {
  extern __shared__ int cnt[];
  for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
  __syncthreads();
  const int s0 = blockIdx.x * chunk;
  const int s1 = min(S, s0 + chunk);
  for (int s = s0 + threadIdx.x; s < s1; s += blockDim.x) atomicAdd(&cnt[topk_idx[s]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[(size_t)blockIdx.x * E + e] = cnt[e];
}

// Tile split (the LDS-tiled GEMMs): an expert's last tile with at most
// bm / 2 rows is small.  Small tiles go after all the others, in expert
// order, and ntiles[1] = the count of the others.
__device__ __forceinline__ int small_tile(int c, int nt, int bm, int split) {
  return (split && nt > 0 && c - (nt - 1) * bm <= bm / 2) ? 1 : 0;
}

// Tile i (< nt) of expert e with first sorted position off_e: written at its
// place in the table (big tiles from tileb0, the small one at small_at).
__device__ __forceinline__ void write_expert_tiles(int e, int c, int nt, int small, int bm, int off_e, int tileb0,
                                                   int small_at, int* __restrict__ tiles) {
  for (int i = 0; i < nt; ++i) {
    int* tp = tiles + 4 * (small && i == nt - 1 ? small_at : tileb0 + i);
    tp[0] = e;
    tp[1] = off_e + i * bm;
    tp[2] = min(bm, c - i * bm);
    tp[3] = 0;
  }
}

// Block-wide (1024 threads, thread e = expert e < E <= 1024): given each
// expert's slot count c, write counts, exclusive offsets and the M-tile table
//   tiles[4*i .. 4*i+3] = (expert, first sorted position, rows, 0), ntiles[0] = count
// (with split, small tiles last and ntiles[1] = the count of the others);
// returns the expert's first sorted position (and in *first_tile its first
// tile; without split).  Only the first tile_groups groups get tiles (a share
// of the experts: the last group holds the slots of experts the weights do
// not hold).
__device__ __forceinline__ int scan_experts(int c, int E, int S, int bm, int* __restrict__ counts,
                                            int* __restrict__ offsets, int* __restrict__ tiles,
                                            int* __restrict__ ntiles, int* first_tile = nullptr,
                                            int tile_groups = 1 << 30, int split = 0) {
  __shared__ int s_warp[16];
  __shared__ int s_warp2[16];
  __shared__ int s_warp3[16];
  __shared__ int s_tot[2];
  const int e = threadIdx.x;
  if (e < E) counts[e] = c;
  const int nt = threadIdx.x < tile_groups ? (c + bm - 1) / bm : 0;
  const int sm = small_tile(c, nt, bm, split);
  // Inclusive scans of counts, big-tile counts and small-tile counts (wave
  // scan, then wave totals).
  int inc = c, inct = nt - sm, incs = sm;
  const int lane = lane_id(), w = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int a = __shfl_up(inc, off);
    const int b = __shfl_up(inct, off);
    const int d = __shfl_up(incs, off);
    if (lane >= off) {
      inc += a;
      inct += b;
      incs += d;
    }
  }
  if (lane == 63) {
    s_warp[w] = inc;
    s_warp2[w] = inct;
    s_warp3[w] = incs;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int a = 0, b = 0, d = 0;
    for (int i = 0; i < 16; ++i) {
      const int x = s_warp[i], y = s_warp2[i], z = s_warp3[i];
      s_warp[i] = a;
      s_warp2[i] = b;
      s_warp3[i] = d;
      a += x;
      b += y;
      d += z;
    }
    s_tot[0] = b;
    s_tot[1] = d;
  }
  __syncthreads();
  const int off_e = inc - c + s_warp[w];
  const int tile0 = inct - (nt - sm) + s_warp2[w];
  const int nbig = s_tot[0];
  if (e < E) {
    offsets[e] = off_e;
    write_expert_tiles(e, c, nt, sm, bm, off_e, tile0, nbig + incs - sm + s_warp3[w], tiles);
  }
  if (e == E - 1) {
    offsets[E] = S;
    ntiles[0] = nbig + s_tot[1];
    if (split) ntiles[1] = nbig;
  }
  if (first_tile) *first_tile = tile0;
  return off_e;
}

// Slot id of every row of tile t: trows[t * bm + r] = perm[first + min(r, rows - 1)]
// (rows past the tile's count repeat its last row), for the tiles of expert e
// (nt tiles from tile0, sorted positions from off_e).  perm may be LDS.
__device__ __forceinline__ void write_tile_rows(const int* perm, int off_e, int c, int tile0, int bm,
                                                int* __restrict__ trows) {
  const int nt = (c + bm - 1) / bm;
  for (int i = 0; i < nt; ++i) {
    const int rows = min(bm, c - i * bm);
    for (int r = 0; r < bm; ++r) trows[(tile0 + i) * bm + r] = perm[off_e + i * bm + min(r, rows - 1)];
  }
}

// Single block: counts from the chunk histograms (which become per-chunk
// bases for the scatter), offsets and the M-tile table.
__global__ void __launch_bounds__(1024) qmoe_scan(int* __restrict__ hist, int nchunks, int E, int S, int bm,
                                                  int* __restrict__ counts, int* __restrict__ offsets,
                                                  int* __restrict__ tiles, int* __restrict__ ntiles,
                                                  int tile_groups, int split) {
  const int e = threadIdx.x;
  int c = 0;
  // eight chunks' counts in flight at a time (one round trip per eight)
  if (e < E) {
    for (int ch0 = 0; ch0 < nchunks; ch0 += 8) {
      int v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = ch0 + i < nchunks ? hist[(size_t)(ch0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (ch0 + i < nchunks) {
          hist[(size_t)(ch0 + i) * E + e] = c;  // exclusive prefix over chunks
          c += v[i];
        }
    }
  }
  const int off_e = scan_experts(c, E, S, bm, counts, offsets, tiles, ntiles, nullptr, tile_groups, split);
  if (e < E)
    for (int ch0 = 0; ch0 < nchunks; ch0 += 8) {
      int v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = ch0 + i < nchunks ? hist[(size_t)(ch0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (ch0 + i < nchunks) hist[(size_t)(ch0 + i) * E + e] = v[i] + off_e;
    }
}

// Stable scatter: slot s (expert e) goes to base[chunk][e] + (number of slots
// of the same chunk with expert e and a smaller slot id).  A workgroup of
// kScatterWaves wavefronts takes 64 * kScatterWaves slots a round.
constexpr int kScatterWaves = 8;
__global__ void __launch_bounds__(64 * kScatterWaves) qmoe_scatter(const int* __restrict__ topk_idx,
                                                                   const int* __restrict__ hist, int S, int E,
                                                                   int chunk, int* __restrict__ perm) {
  constexpr int NT = 64 * kScatterWaves;
  extern __shared__ int sm[];
  int* base = sm;          // [E]
  int* wcnt = sm + E;      // [kScatterWaves][E]
  const int lane = lane_id(), w = threadIdx.x >> 6;
  for (int e = threadIdx.x; e < E; e += NT) base[e] = hist[(size_t)blockIdx.x * E + e];
  const int s0 = blockIdx.x * chunk;
  const int s1 = min(S, s0 + chunk);
  for (int r0 = s0; r0 < s1; r0 += NT) {
    for (int i = threadIdx.x; i < kScatterWaves * E; i += NT) wcnt[i] = 0;
    __syncthreads();
    const int s = r0 + threadIdx.x;
    const bool valid = s < s1;
    const int e = valid ? topk_idx[s] : -1;
    // rank among lower lanes of this wave with the same expert
    unsigned long long todo = __ballot(valid);
    int rank = 0;
    while (todo) {
      const int leader = __ffsll((long long)todo) - 1;
      const int le = __shfl(e, leader);
      const unsigned long long m = __ballot(valid && e == le);
      if (e == le) rank = __popcll(m & ((1ull << lane) - 1ull));
      if (lane == leader) wcnt[w * E + le] = __popcll(m);
      todo &= ~m;
    }
    __syncthreads();
    if (valid) {
      int pos = base[e] + rank;
      for (int ww = 0; ww < w; ++ww) pos += wcnt[ww * E + e];
      perm[pos] = s;
    }
    __syncthreads();
    for (int ee = threadIdx.x; ee < E; ee += NT) {
      int add = 0;
#pragma unroll
      for (int ww = 0; ww < kScatterWaves; ++ww) add += wcnt[ww * E + ee];
      base[ee] += add;
    }
    __syncthreads();
  }
}

// The whole front end in one workgroup of 1024 threads, for up to 1024 slots
// and 1024 experts: routing (16 tokens at a time, one per wavefront), counts
// in LDS, the scan and tile table, then the stable scatter.  The scatter runs
// wavefront by wavefront in slot order: a wavefront ranks its 64 slots among
// equal experts with ballots and advances each expert's cursor, so slot ids
// stay ascending within every expert.
template <int V>
__global__ void __launch_bounds__(1024) qmoe_route_small(const float* __restrict__ logits, int T, int E, int k,
                                                         int routing, int normalize, int bm,
                                                         int* __restrict__ topk_idx, float* __restrict__ topk_w,
                                                         int* __restrict__ counts, int* __restrict__ offsets,
                                                         int* __restrict__ perm, int* __restrict__ tiles,
                                                         int* __restrict__ ntiles, int* __restrict__ trows,
                                                         int split) {
  __shared__ int s_idx[1024];
  __shared__ int s_cnt[1024];  // counts, then each expert's next sorted position
  __shared__ int s_perm[1024];
  const int S = T * k;
  const int lane = lane_id(), w = threadIdx.x >> 6;
  if (threadIdx.x < E) s_cnt[threadIdx.x] = 0;
  for (int t = w; t < T; t += 16) route_token<V>(logits, t, E, k, routing, normalize, topk_idx, topk_w, s_idx);
  __syncthreads();
  if (threadIdx.x < S) atomicAdd(&s_cnt[s_idx[threadIdx.x]], 1);
  __syncthreads();
  const int c = threadIdx.x < E ? s_cnt[threadIdx.x] : 0;
  int tile0 = 0;
  const int off_e = scan_experts(c, E, S, bm, counts, offsets, tiles, ntiles, &tile0, 1 << 30, split);  // synchronises
  if (threadIdx.x < E) s_cnt[threadIdx.x] = off_e;
  __syncthreads();
  const int nw = (S + 63) / 64;
  for (int ww = 0; ww < nw; ++ww) {
    if (w == ww) {
      const int s = threadIdx.x;
      const bool valid = s < S;
      const int e = valid ? s_idx[s] : -1;
      unsigned long long todo = __ballot(valid);
      while (todo) {
        const int leader = __ffsll((long long)todo) - 1;
        const int le = __shfl(e, leader);
        const unsigned long long m = __ballot(valid && e == le);
        const int base = s_cnt[le];
        if (valid && e == le) {
          const int pos = base + __popcll(m & ((1ull << lane) - 1ull));
          perm[pos] = s;
          s_perm[pos] = s;
        }
        if (lane == leader) s_cnt[le] = base + __popcll(m);
        todo &= ~m;
      }
    }
    __syncthreads();
  }
  if (trows && !split && threadIdx.x < E) write_tile_rows(s_perm, off_e, c, tile0, bm, trows);
}

// The whole front end in one wavefront when every token fits a lane and the
// selection is short (T <= 64, E <= EV <= 64, E * k <= 64, tiles of at least
// 8 rows): lane t routes
// token t from its logits in registers (the key order of route_token, k
// passes over the E keys), experts are counted with LDS atomics, lane e
// scans expert e's count and tile count, and the stable scatter places the
// slots of each expert in token order with one ballot per expert (a
// token's k experts are distinct, so its slots of one expert are at most
// one).  No barrier spans more than one wavefront.
template <int EV>
__global__ void __launch_bounds__(64) qmoe_route_wave(const float* __restrict__ logits, int T, int E, int k,
                                                      int routing, int normalize, int bm,
                                                      int* __restrict__ topk_idx, float* __restrict__ topk_w,
                                                      int* __restrict__ counts, int* __restrict__ offsets,
                                                      int* __restrict__ perm, int* __restrict__ tiles,
                                                      int* __restrict__ ntiles, int* __restrict__ trows, int split) {
  // k <= min(E, 64 / E) <= 8, so S <= 512 slots; with tiles of at least 8
  // rows at most S / 8 + E <= 64 + 64 tiles
  __shared__ int s_cnt[64];
  __shared__ int s_perm[1024];
  __shared__ int s_tile[2 * 128];  // (first sorted position, rows) of each tile
  const int lane = threadIdx.x;
  const int S = T * k;
  const bool tok = lane < T;
  s_cnt[lane] = 0;
  float v[EV];
#pragma unroll
  for (int e = 0; e < EV; ++e) {
    const float x = (tok && e < E) ? logits[(size_t)lane * E + e] : -INFINITY;
    v[e] = (x != x) ? -INFINITY : x;
  }
  __syncthreads();
  // Selection: pass r takes the best key strictly after pass r - 1's.
  int sel[EV];
  float pv = INFINITY, v0 = 0.f, sum_sel = 0.f;
  int pi = -1;
  float ex[EV];
  for (int r = 0; r < k; ++r) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int e = 0; e < EV; ++e)
      if (e < E && key_before(pv, pi, v[e], e) && key_before(v[e], e, bv, bi)) {
        bv = v[e];
        bi = e;
      }
    bi = min(max(bi, 0), E - 1);
    pv = bv;
    pi = bi;
    if (r == 0) v0 = bv;
    const float x = expf(bv - v0);
    sum_sel += x;
#pragma unroll
    for (int q = 0; q < EV; ++q)
      if (q == r) {
        sel[q] = bi;
        ex[q] = x;
      }
  }
  float denom = sum_sel;
  if (routing == 1 && !normalize) {
    // Full softmax over all experts, taken at the selection.
    float part = 0.f;
#pragma unroll
    for (int e = 0; e < EV; ++e)
      if (e < E) part += expf(v[e] - v0);
    denom = part;
  }
  if (tok) {
#pragma unroll
    for (int q = 0; q < EV; ++q)
      if (q < k) {
        topk_idx[lane * k + q] = sel[q];
        topk_w[lane * k + q] = ex[q] / denom;
        atomicAdd(&s_cnt[sel[q]], 1);
      }
  }
  __syncthreads();
  // Counts, exclusive offsets and tile counts of expert e in lane e.
  const int c = lane < E ? s_cnt[lane] : 0;
  const int nt = (c + bm - 1) / bm;
  const int sm = small_tile(c, nt, bm, split);
  int inc = c, inct = nt - sm, incs = sm;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int a = __shfl_up(inc, off);
    const int b = __shfl_up(inct, off);
    const int d = __shfl_up(incs, off);
    if (lane >= off) {
      inc += a;
      inct += b;
      incs += d;
    }
  }
  const int off_e = inc - c, tile0 = inct - (nt - sm);
  const int nbig = __shfl(inct, 63);
  const int ntot = nbig + __shfl(incs, 63);
  if (lane < E) {
    counts[lane] = c;
    offsets[lane] = off_e;
    write_expert_tiles(lane, c, nt, sm, bm, off_e, tile0, nbig + incs - sm, tiles);
    if (!split)
      for (int i = 0; i < nt; ++i) {
        s_tile[2 * (tile0 + i)] = off_e + i * bm;
        s_tile[2 * (tile0 + i) + 1] = min(bm, c - i * bm);
      }
  }
  if (lane == 0) {
    offsets[E] = S;
    ntiles[0] = ntot;
    if (split) ntiles[1] = nbig;
  }
  // Stable scatter: slots of expert e in token order.
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int e = 0; e < E; ++e) {
    int slot = -1;
#pragma unroll
    for (int q = 0; q < EV; ++q)
      if (q < k && sel[q] == e) slot = lane * k + q;
    const bool has = tok && slot >= 0;
    const unsigned long long m = __ballot(has);
    const int base = __shfl(off_e, e);
    if (has) {
      const int pos = base + __popcll(m & below);
      perm[pos] = slot;
      s_perm[pos] = slot;
    }
  }
  __syncthreads();
  // Tile rows: rows past a tile's count repeat its last row.
  if (trows && !split)
    for (int j = lane; j < ntot * bm; j += 64) {
      const int t = j / bm, r = j - t * bm;
      trows[j] = s_perm[s_tile[2 * t] + min(r, s_tile[2 * t + 1] - 1)];
    }
}

// Tile-row table after the multi-kernel permutation: one thread per
// (tile, row) entry; entries of unused tiles are left alone.
__global__ void __launch_bounds__(256) qmoe_tile_rows(const int* __restrict__ perm, const int* __restrict__ tiles,
                                                      const int* __restrict__ ntiles, int max_tiles, int bm,
                                                      int* __restrict__ trows) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= max_tiles * bm) return;
  const int t = i / bm, r = i % bm;
  if (t >= ntiles[0]) return;
  const int p0 = tiles[4 * t + 1], rows = tiles[4 * t + 2];
  trows[i] = perm[p0 + min(r, rows - 1)];
}

// A share of the experts: local[s] = topk_idx[s] - first when the weights
// hold that expert (first <= e < first + El), else El (one more group, given
// no tiles, whose slots the combine skips).
__global__ void __launch_bounds__(256) qmoe_local_index(const int* __restrict__ topk_idx, int S, int first, int El,
                                                        int* __restrict__ local) {
  const int s = blockIdx.x * 256 + threadIdx.x;
  if (s >= S) return;
  const int e = topk_idx[s] - first;
  local[s] = (e >= 0 && e < El) ? e : El;
}

// ---------------------------------------------------------------- launchers
hipError_t launch_router(const float* logits, int T, int E, int k, int routing, int normalize, int* topk_idx,
                         float* topk_w, hipStream_t st) {
  const dim3 grid((T + 3) / 4), block(256);
  const int V = (E + 63) / 64;
  if (V <= 1) hipLaunchKernelGGL(qmoe_router<1>, grid, block, 0, st, logits, T, E, k, routing, normalize, topk_idx, topk_w);
  else if (V <= 2) hipLaunchKernelGGL(qmoe_router<2>, grid, block, 0, st, logits, T, E, k, routing, normalize, topk_idx, topk_w);
  else if (V <= 4) hipLaunchKernelGGL(qmoe_router<4>, grid, block, 0, st, logits, T, E, k, routing, normalize, topk_idx, topk_w);
  else if (V <= 8) hipLaunchKernelGGL(qmoe_router<8>, grid, block, 0, st, logits, T, E, k, routing, normalize, topk_idx, topk_w);
  else hipLaunchKernelGGL(qmoe_router<16>, grid, block, 0, st, logits, T, E, k, routing, normalize, topk_idx, topk_w);
  return hipGetLastError();
}

hipError_t launch_route_small(const float* logits, int T, int E, int k, int routing, int normalize, int bm,
                              int* topk_idx, float* topk_w, int* counts, int* offsets, int* perm, int* tiles,
                              int* ntiles, int* trows, hipStream_t st, int split) {
  if (T * k > 1024 || E > 1024) return hipErrorInvalidValue;
  if (T <= 64 && E <= 64 && E * k <= 64 && bm >= 8) {
#define QMOE_ROUTE_WAVE(EVV)                                                                                      \
  hipLaunchKernelGGL(qmoe_route_wave<EVV>, dim3(1), dim3(64), 0, st, logits, T, E, k, routing, normalize, bm,     \
                     topk_idx, topk_w, counts, offsets, perm, tiles, ntiles, trows, split)
    if (E <= 8) QMOE_ROUTE_WAVE(8);
    else if (E <= 16) QMOE_ROUTE_WAVE(16);
    else if (E <= 32) QMOE_ROUTE_WAVE(32);
    else QMOE_ROUTE_WAVE(64);
#undef QMOE_ROUTE_WAVE
    return hipGetLastError();
  }
  const int V = (E + 63) / 64;
#define QMOE_ROUTE_SMALL(VV)                                                                                       \
  hipLaunchKernelGGL(qmoe_route_small<VV>, dim3(1), dim3(1024), 0, st, logits, T, E, k, routing, normalize, bm,  \
                     topk_idx, topk_w, counts, offsets, perm, tiles, ntiles, trows, split)
  if (V <= 1) QMOE_ROUTE_SMALL(1);
  else if (V <= 2) QMOE_ROUTE_SMALL(2);
  else if (V <= 4) QMOE_ROUTE_SMALL(4);
  else if (V <= 8) QMOE_ROUTE_SMALL(8);
  else QMOE_ROUTE_SMALL(16);
#undef QMOE_ROUTE_SMALL
  return hipGetLastError();
}

hipError_t launch_permute(const int* topk_idx, int S, int E, int chunk, int nchunks, int bm, int* hist,
                          int* counts, int* offsets, int* perm, int* tiles, int* ntiles, hipStream_t st,
                          int tile_groups, int split) {
  hipLaunchKernelGGL(qmoe_hist, dim3(nchunks), dim3(256), E * sizeof(int), st, topk_idx, S, E, chunk, hist);
  hipLaunchKernelGGL(qmoe_scan, dim3(1), dim3(1024), 0, st, hist, nchunks, E, S, bm, counts, offsets, tiles, ntiles,
                     tile_groups < 0 ? E : tile_groups, split);
  hipLaunchKernelGGL(qmoe_scatter, dim3(nchunks), dim3(64 * kScatterWaves), (1 + kScatterWaves) * E * sizeof(int), st,
                     topk_idx, hist, S, E, chunk, perm);
  return hipGetLastError();
}

hipError_t launch_local_index(const int* topk_idx, int S, int first, int El, int* local, hipStream_t st) {
  if (S > 0) hipLaunchKernelGGL(qmoe_local_index, dim3((S + 255) / 256), dim3(256), 0, st, topk_idx, S, first, El, local);
  return hipGetLastError();
}

hipError_t launch_tile_rows(const int* perm, const int* tiles, const int* ntiles, int max_tiles, int bm, int* trows,
                            hipStream_t st) {
  const int n = max_tiles * bm;
  hipLaunchKernelGGL(qmoe_tile_rows, dim3((n + 255) / 256), dim3(256), 0, st, perm, tiles, ntiles, max_tiles, bm, trows);
  return hipGetLastError();
}

}  // namespace qmoe
