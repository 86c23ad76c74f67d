// Launch functions of the QMoE kernels (host side; enqueue only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmoe {

hipError_t launch_router(const float* logits, int T, int E, int k, int routing, int normalize, int* topk_idx,
                         float* topk_w, hipStream_t st);

// Router, counts, offsets, tile table and stable permutation in one launch
// (T * k <= 1024 and E <= 1024); with trows given, also the tile-row table
// (see launch_tile_rows).  split (the LDS-tiled GEMMs): each expert's last
// tile of at most bm / 2 rows goes after all the other tiles, and
// ntiles[1] = the count of the others (no tile-row table then).
hipError_t launch_route_small(const float* logits, int T, int E, int k, int routing, int normalize, int bm,
                              int* topk_idx, float* topk_w, int* counts, int* offsets, int* perm, int* tiles,
                              int* ntiles, int* trows, hipStream_t st, int split = 0);

// Counts, offsets, stable permutation and M-tile table over E groups; only
// the first tile_groups groups (all when negative) get tiles; split as above.
hipError_t launch_permute(const int* topk_idx, int S, int E, int chunk, int nchunks, int bm, int* hist,
                          int* counts, int* offsets, int* perm, int* tiles, int* ntiles, hipStream_t st,
                          int tile_groups = -1, int split = 0);

// A share of the experts: local[s] = topk_idx[s] - first for the experts
// [first, first + El) the weights hold, else El.
hipError_t launch_local_index(const int* topk_idx, int S, int first, int El, int* local, hipStream_t st);

// Tile-row table of the streaming kernels: trows[t * bm + r] = slot id of row
// r of tile t (rows past the tile's count repeat its last row), t < ntiles.
hipError_t launch_tile_rows(const int* perm, const int* tiles, const int* ntiles, int max_tiles, int bm, int* trows,
                            hipStream_t st);

// Operand rows of the f16 GEMMs (see operand.hip): rows of n fp32 codes at
// src + r * sstride (floats) -> kp hi/lo codes of v * 2^e at dst + r * dstride
// (bytes), exps[r] = e; src and dst may be the same rows of 4-byte codes.
// live (device, optional): only rows below live[0] are in use.
// zero_flag (device, optional): set to 0 by the launch.
hipError_t launch_split_rows(int bits, const float* src, long sstride, int n, uint8_t* dst, long dstride, int kp,
                             long rows, int* exps, hipStream_t st, const int* live = nullptr,
                             int* zero_flag = nullptr);
// exps[r] = e of the n fp32 codes at src + r * stride, r < rows.
hipError_t launch_row_exp(const float* src, long stride, long rows, int n, int* exps, hipStream_t st);
// FC2 operand rows that the tiled FC1 wrote with segment exponents, back to
// one exponent per row, in place, when flag[0] != 0 (else every workgroup
// exits at once): row r < rows holds n hi/lo codes at d + r * stride
// (bytes), code c written with exponent seg_rows[(c >> seg_shift) * rows +
// r]; exps[r] = the row's new exponent.  live as above.
hipError_t launch_resplit_rows(int bits, uint8_t* d, long stride, int n, long rows, const int* seg_rows, int seg_shift,
                               int* exps, const int* flag, hipStream_t st, const int* live = nullptr);

// Grouped quantised GEMM over expert-sorted rows.
//   FC1: rows are tokens (via perm / k), weights fc1 [E][F][K/pack], output act rows.
//   FC2: rows are act rows in sorted order, weights fc2 [E][H][I/pack], output slot rows.
struct GemmArgs {
  const uint8_t* wq;    // packed weights [E][N][kb]
  const float* ws;      // scales [E][N] or [E][N][nblk]
  const uint8_t* a;     // operand rows (f16 hi/lo groups), row stride a_stride bytes
  int a_f32;            // stream kernel: a holds fp32 rows (4 bytes a code) to split while staging
  const int* a_exp;     // row scale exponent of every operand row (indexed like a), or nullptr: the
                        // single-stage streaming kernel takes one per K range of its own
  const int* a_map;     // FC1: perm (sorted position -> slot); FC2: nullptr (row = position)
  int a_div;            // FC1: k (slot -> token)
  long a_stride;
  const int* tiles;     // [max_tiles][4] = expert, first position, rows, 0
  const int* ntiles;    // [0] = tiles; [1] (split_small) = tiles before the small ones
  int split_small;      // tiled GEMMs: the table ends with tiles of at most 64 rows (half tiles)
  int N, K, kb, nblk, bs;
  int store_by_slot;     // stream kernel: partial rows by slot id (1) or by sorted position (0)
  int S;                 // slots (stride between split partials, in rows)
  // epilogue
  uint8_t* act;         // FC1 output rows (fp32 after the activation), stride act_stride bytes
  // Segment scales between the tiled GEMMs [max_tiles][seg_n]: when set, the
  // FC1 epilogue writes FC2's operand rows as f16 hi/lo groups of v * 2^e
  // with one e per row tile and FC1 column tile (2^seg_shift codes, a
  // segment of FC2's reduction) and stores 2^-e in seg_scale; FC2 multiplies
  // the sums of each segment by it (a_exp unused).  nullptr: FC1 writes fp32
  // rows, split per row afterwards.
  float* seg_scale;
  int seg_shift, seg_n;
  // FC1 with segment scales: a row whose largest magnitude in the segment is
  // more than 2^12 below the tile's bound keeps its own exponent instead
  // (and sets *seg_flag); seg_rows [seg_n][S] gets the exponent each row
  // segment was written with.  FC2 with segment scales reads *seg_flag: when
  // set, its rows carry one exponent each again (a_exp) and the segment
  // factors are not applied.
  int* seg_rows;
  int* seg_flag;
  long act_stride;
  float* slot_out;      // FC2 output [splits][S][N] by slot id
  int ksplit;           // tiled FC2: K ranges, range z's sums in slot_out[z] (0 or 1: one)
  const int* perm;      // FC2: sorted position -> slot
  float alpha, beta;
  float limit;          // SwiGLU clamp limit (+inf: none); set it, zero clamps everything
  // stream kernel
  int nst;              // stages per K range
  int act_swiglu;       // FC1 over the whole of K: activation written by the kernel (act != nullptr)
  const int* trows;     // stream kernel: slot id of every tile row, [max_tiles][16 * mt] (see launch_tile_rows)
  int wg_rows;          // stream kernel, double-buffered: weight rows per workgroup (set by launch_stream)
};

enum { EPI_RELU = 0, EPI_SWIGLU = 1, EPI_STORE = 2 };

// Scale modes: column-wise, blocks of >= 32 codes, blocks of 16 codes.
enum { SC_COL = 0, SC_BLOCK = 1, SC_BLOCK16 = 2 };

hipError_t launch_gemm(int bits, int epi, int mt, bool aligned, const GemmArgs& g, int max_tiles, hipStream_t st);

// LDS-tiled variant (see tiled.hip): 128-row tiles, K a multiple of 64,
// column-wise or >= 32-code block scales, 8-code-aligned rows, N % 4 == 0.
// FC2 (EPI_STORE) may take g.ksplit K ranges of a multiple of 256 codes and
// of the block size each.
hipError_t launch_tiled(int bits, int epi, const GemmArgs& g, int max_tiles, hipStream_t st);

// Weight-streaming variant for small token counts (see stream.hip).  A rows
// are fp32 (g.a_f32 must be set).  FC1 (g.a_map set): A rows are the input's
// token rows; with g.act set (one K range) the kernel writes fp32 FC2 operand
// rows after the activation, else fp32 partial rows part[z][p][N].  FC2: A
// rows are the fp32 operand rows in sorted order; partial rows by slot id,
// slot_out[z][slot][N].
// z < splits K ranges of g.nst stages each.
// wg_rows: double-buffered mode, weight rows per workgroup (a multiple of 64
// up to 512, above 256 only for mt == 1; 0 = 256).
// half_stg: 0, or 1, 4 or 8 for tiles of 8 rows (g.trows holds 8 rows a
// tile) whose single stage (one, mt == 1) holds that many items.
size_t stream_lds_bytes(int bits, int mt, bool one, int rb, int half_stg);  // rb: row blocks per one-stage workgroup
hipError_t launch_stream(int bits, int mt, bool one, int splits, int wg_rows, int half_stg, const GemmArgs& g,
                         int max_tiles, hipStream_t st);

// Sum FC1 partials over K ranges, apply the activation, write fp32 FC2 operand rows.
hipError_t launch_act(int bits, int epi, const float* part, int splits, int S, int F, int I, int kp2, float alpha,
                      float beta, float limit, uint8_t* act, hipStream_t st);

// out[t, h] = sum_s w[t, s] * sum_z slot_out[z][t*k + s][h]  (fixed order);
// with local given, slots with local[t*k + s] >= El are skipped (no row).
hipError_t launch_combine(const float* slot_out, const float* topk_w, int T, int k, int H, int splits, float* out,
                          hipStream_t st, const int* local = nullptr, int El = 0);

// Float32 grouped GEMM over group-sorted rows (see gmm.hip), shared by
// GroupedMatMul and the float MoE projections.
struct F32Gemm {
  const float* a;       // operand rows, K floats each
  const int* a_perm;    // operand row of sorted position p: a_perm[p] / a_div; nullptr: row p
  int a_div;
  const float* w;       // KN layout [G][K][N] or NK layout [G][N][K]
  const float* bias;    // [G][N] or nullptr
  const int* perm;      // sorted position -> slot id
  int out_by_slot;      // output row perm[p] (1) or p (0)
  const int* tiles;     // [max_tiles][4] = group, first position, rows, 0
  const int* ntiles;
  int K, N, G;          // tiles of group >= G write zero rows
  float* out;           // N floats per row
};

// Index conversion: out[j] = idx[j] when in [0, G), else G.
hipError_t launch_gmm_index(const void* idx, bool idx64, long n, int G, int* out, hipStream_t st);
// LDS-tiled kernel: tiles of at most gmm_tile_rows() rows, any K / N; vec:
// K % 4 == 0, a and w 16-byte aligned (KN: also N % 4 == 0).
int gmm_tile_rows();
hipError_t launch_gmm_f32(const F32Gemm& g, bool nk, bool vec, int max_tiles, hipStream_t st);
// Weight-streaming kernel: tiles of at most gmm_rows16_tile_rows() rows;
// K % 4 == 0, a and w 16-byte aligned (KN: also N % 4 == 0 and 16-byte
// aligned bias and out).
// ksplit 1 or 4: wavefronts of a workgroup on four column strips or on four
// K ranges of one strip; gmm_rows16_ksplit picks it from an estimate of the
// tiles in use.
int gmm_rows16_tile_rows();
int gmm_rows16_ksplit(long est_tiles, int N);
hipError_t launch_gmm_rows16(const F32Gemm& g, bool nk, int ksplit, int max_tiles, hipStream_t st);

// GroupedMatMul in float16, bfloat16 and double (see gmm_typed.hip): the
// rows of F32Gemm's GroupedMatMul use (a_perm / a_div gathers token rows,
// output rows by slot id through perm), weights [G][K][N] of the element
// type, optional bias [G][N]; 64-row tiles (gmm_tile_rows()).  vec: x and w
// 16-byte aligned and rows of K and N elements whole 16-byte runs.
enum { GMM_F16 = 0, GMM_BF16 = 1, GMM_F64 = 2 };
struct TypedGemm {
  const void* a;
  const int* a_perm;
  int a_div;
  const void* w;
  const void* bias;     // or nullptr
  const int* perm;
  const int* tiles;
  const int* ntiles;
  int K, N, G;          // tiles of group >= G write zero rows
  void* out;
};
// tile_rows: most rows a tile of the table holds, at most 64, or 128 for
// float16 / bfloat16 with vec, K % 8 == 0 and N % 8 == 0 (gmm16_tile_rows()).
hipError_t launch_gmm_typed(int type, const TypedGemm& g, bool vec, int max_tiles, hipStream_t st, int tile_rows = 64);
// Rows per tile for the float16 / bfloat16 tile kernel on R rows over
// `spread` groups.
int gmm16_tile_rows(long R, long spread);
// float16 / bfloat16 on 16-row tiles, weight streaming (gmm_typed.hip): K %
// 4 == 0, N % 4 == 0, 8-byte aligned input, weights, bias and output; ksplit
// 1 or 4 (K ranges of one workgroup's four wavefronts).
hipError_t launch_gmm16_rows16(int type, const TypedGemm& g, int ksplit, int max_tiles, hipStream_t st);
// float16 / bfloat16 on 16-row tiles, weight streaming on the 16-bit matrix
// instruction (gmm_typed.hip): K % 8 == 0, N % 8 == 0, 16-byte aligned input,
// weights, bias and output; est_tiles as below.
hipError_t launch_gmm16_stream(int type, const TypedGemm& g, long est_tiles, int max_tiles, hipStream_t st);
// double on 16-row tiles, weight streaming (gmm_typed.hip): K % 4 == 0,
// N % 2 == 0, 16-byte aligned input, weights, bias and output; est_tiles:
// the tiles to expect (groups in use) for the K-range choice.
hipError_t launch_gmm64_rows16(const TypedGemm& g, long est_tiles, int max_tiles, hipStream_t st);

// Float MoE activation pass (see moe.hip): act[p][j], p < S, j < I, from
// FC1 rows h (F floats) and FC3 rows u3 (I floats, or nullptr).  Codes
// match qmoe_activation.
enum { MOE_ACT_RELU = 0, MOE_ACT_SWIGLU = 1, MOE_ACT_GELU = 2, MOE_ACT_SILU = 3, MOE_ACT_IDENTITY = 4 };
hipError_t launch_moe_act(int act_type, const float* h, const float* u3, long S, int I, int F, int fusion,
                          float alpha, float beta, float limit, float* act, hipStream_t st);

hipError_t launch_fill_zero(float* out, long n, hipStream_t st);

hipError_t launch_copy_i32(const int* src, int* dst, long n, hipStream_t st);
hipError_t launch_copy_f32(const float* src, float* dst, long n, hipStream_t st);

}  // namespace qmoe
