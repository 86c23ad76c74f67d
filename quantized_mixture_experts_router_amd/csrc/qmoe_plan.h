// Host-side contract check and launch plan for the QMoE operator.
// Pure C++ (no HIP types), so the contract logic runs and is tested on any CPU.
#pragma once
#include <cstddef>
#include <cstdint>

#include "qmoe.h"

namespace qmoe {

// Sizes derived from the tensors (QMoE WebGPU manifest, `derive`:
// hiddenSize, numTokens, fusionSize, interSize, packSize, quantMidpoint,
// colWiseScales, fc1ScaleBlocks, fc2ScaleBlocks).
struct Dims {
  int64_t T = 0;   // tokens = numel(input) / H
  int64_t H = 0;   // hidden size
  int64_t E = 0;   // experts (router logits per token)
  int64_t El = 0;  // experts held by the weights: global experts [first, first + El)
  int64_t first = 0;
  int64_t I = 0;   // inter size
  int64_t F = 0;   // FC1 rows = fusion * I
  int64_t k = 0;
  int bits = 4, pack = 2, mid = 8, fusion = 1;
  int64_t bs = 0;            // 0 = column-wise
  int64_t nb1 = 1, nb2 = 1;  // scale blocks per FC1 / FC2 row
  int act = QMOE_ACT_RELU;
  int routing = QMOE_ROUTE_QMOE;
  int normalize = 0;
  float alpha = 1.f, beta = 0.f;
  float limit = __builtin_inff();  // SwiGLU clamp (+inf: none)
};

// Largest expert count the routing kernels hold in registers / LDS.
constexpr int64_t kMaxExperts = 1024;

// Token counts up to which the weight-streaming GEMMs run (measured
// crossovers; see make_plan): when both GEMMs stream, and when only FC1
// streams (then also at most kStreamMixedMaxExperts experts held).
constexpr int64_t kStreamMaxTokens = 224;
constexpr int64_t kStreamMixedMaxTokens = 64;
constexpr int64_t kStreamMixedMaxExperts = 16;

qmoe_status validate(const qmoe_tensor* input, const qmoe_tensor* router, const qmoe_tensor* fc1w,
                     const qmoe_tensor* fc1s, const qmoe_tensor* fc2w, const qmoe_tensor* fc2s,
                     const qmoe_tensor* output, const qmoe_attrs* attrs, Dims* d);

// Items (128-byte weight-row pieces) per activation stage of the streaming
// kernel: one stage holding the whole K range (one = true, a single 64 KB LDS
// buffer of 16*mt rows), or double-buffered stages.
constexpr int stream_stage_items(int mt, bool one) {
  return one ? (mt == 1 ? 4 : mt == 2 ? 2 : 1) : (mt == 1 ? 2 : 1);
}

// Which kernels run, with what tiles, and where each intermediate lives in the
// caller's workspace.  Offsets are bytes from the workspace base, 256-aligned.
struct Plan {
  Dims d;
  int64_t S = 0;         // slots = T * k
  bool decode = false;   // weight-streaming path (every expert's rows fit one M tile)
  bool tiled = false;    // LDS-tiled GEMMs (128-row tiles) for both FC1 and FC2
  // tiled, segment scales: the FC1 epilogue writes FC2's hi/lo operand rows
  // itself, one power-of-two scale per row tile and FC1 column tile
  // (2^seg_shift codes), seg_n segments a row; 0: fp32 rows split per row
  // afterwards
  int seg_n = 0, seg_shift = 0;
  // tiled, column-wise scales: each expert's last tile of at most 64 rows
  // runs as a half tile (64 rows x 512 columns; the tile table lists those
  // tiles last)
  int half_tiles = 0;
  int mt = 1;            // 16-row M subtiles per tile
  int64_t bm = 16;       // rows per M tile
  int64_t max_tiles = 0; // ceil(S / bm) + E
  int64_t kp1 = 0, kp2 = 0;  // padded reduction lengths of the A operands (codes)
  bool aligned = true;   // packed rows allow vector loads
  // weight-streaming kernels (decode): used per GEMM when its shapes allow
  struct Stream {
    bool on = false;
    bool one = false;    // the K range is one stage (staged once, no barriers)
    int stg = 2;         // 128-byte row items per stage (activation slice per LDS buffer)
    int nst = 1;         // stages per K range
    int splits = 1;      // K ranges (fp32 partials summed afterwards, in order)
    int wg_rows = 0;     // double-buffered mode: weight rows per workgroup (0 = one row block of 256)
  } s1, s2;
  bool half = false;     // streaming tiles of 8 rows (each K range one stage of s.stg items), else 16 * mt rows
  int splits2 = 1;       // FC2 partial sets the combine sums (1 off the stream path)
  int ksplit2 = 1;       // tiled FC2: K ranges (each writes its own partial set)
  size_t off_part1 = 0;  // FC1 fp32 partials [s1.splits][S][F] (stream path with K ranges)
  size_t off_trows = 0;  // streaming kernels: slot id of every tile row [max_tiles][bm]
  bool small_front = false;  // router + permutation in one workgroup (S, E <= 1024)
  bool share = false;    // the weights hold only some of the experts (El < E)
  int64_t chunk = 1024;  // slots per permutation block
  int64_t nchunks = 0;
  // workspace layout
  size_t off_topk_idx = 0, off_topk_w = 0, off_counts = 0, off_offsets = 0, off_perm = 0;
  size_t off_tiles = 0, off_ntiles = 0, off_hist = 0, off_xa = 0, off_act = 0, off_slot = 0;
  size_t off_exp1 = 0, off_exp2 = 0;  // row scale exponents of the FC1 [T] and FC2 [S] operand rows
  // segment scales: f32 [max_tiles][seg_n] (2^-e of each row tile and
  // segment), i32 [seg_n][S] (the exponent each row segment was written
  // with), i32 flag (a row kept its own exponent: FC2 rows go back to one
  // exponent a row)
  size_t off_seg = 0, off_segrows = 0, off_segflag = 0;
  size_t off_local = 0;  // share: local expert of every slot [S] (El = not held)
  size_t bytes = 0;
};

// Fill *p from validated dims.  Never fails.
void make_plan(const Dims& d, Plan* p);

}  // namespace qmoe
