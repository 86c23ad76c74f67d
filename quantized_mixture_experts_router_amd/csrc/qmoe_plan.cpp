// Contract validation and workspace planning for the QMoE operator.
//
// Every clause follows the QMoE WebGPU manifest: `attributeConstraints`,
// `typeConstraints`, and the `derive` booleans activationSupported,
// routingModeSupported, rawWeightLayout, inputOutputShapeOk,
// quantBlockSizeOk, quantScalesOk, quantShapeOk and quantContract.
#include "qmoe_plan.h"

#include <algorithm>
#include <cstdlib>
#include <string>

// Workgroups the streaming kernels aim for before splitting K (two per
// compute unit on 256 compute units).
#ifndef QMOE_STREAM_NT
#define QMOE_STREAM_NT 2
#endif
#ifndef QMOE_STREAM_MAX_ONE_SPLITS
#define QMOE_STREAM_MAX_ONE_SPLITS 16
#endif
#ifndef QMOE_STREAM_MIN_WORKGROUPS
#define QMOE_STREAM_MIN_WORKGROUPS 512
#endif

namespace qmoe {
namespace {

bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// The streaming kernel needs whole 128-byte row items and scale blocks of at
// least one 32-code matrix step.
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Most K ranges a single-stage streaming launch may take; the environment
// variable QMOE_STREAM_SINGLE_STAGE_MAX_SPLITS (a non-negative integer)
// overrides it, e.g. 0 to run every streaming GEMM double-buffered.
int64_t max_one_splits() {
  if (const char* v = std::getenv("QMOE_STREAM_SINGLE_STAGE_MAX_SPLITS")) {
    char* end = nullptr;
    const long x = std::strtol(v, &end, 10);
    if (end != v && *end == 0 && x >= 0) return x;
  }
  return QMOE_STREAM_MAX_ONE_SPLITS;
}

bool rank_ok(const qmoe_tensor* t, int r) { return t->rank == r; }

// Extents the kernels index with 32-bit integers, and the largest element
// count of any intermediate (2^40 four-byte elements, beyond any GPU's
// memory): past these a call is UNSUPPORTED, never computed with wrapped
// sizes.
constexpr int64_t kMaxExtent = (int64_t(1) << 31) - 1;
// Largest second and third grid dimension of a launch.
constexpr int64_t kMaxGridYZ = 65535;
constexpr int64_t kMaxElements = int64_t(1) << 40;

// Rank 1..3 with every used extent in [0, kMaxExtent]: QMOE_OK, or SHAPE
// (bad rank, negative extent) or UNSUPPORTED (an extent past kMaxExtent).
qmoe_status extents_ok(const qmoe_tensor* t) {
  if (t->rank < 1 || t->rank > 3) return QMOE_ERR_SHAPE;
  for (int i = 0; i < t->rank; ++i) {
    if (t->dims[i] < 0) return QMOE_ERR_SHAPE;
    if (t->dims[i] > kMaxExtent) return QMOE_ERR_UNSUPPORTED;
  }
  return QMOE_OK;
}

// GEMM path override, for measuring the paths against each other: the
// environment variable QMOE_PATH = "stream" (weight streaming, 64-row tiles
// past 64 tokens), "tiled" (LDS-tiled where the shapes allow, else
// register-tiled) or "gemm" (register-tiled); unset or anything else: the
// plan's own choice.
enum { PATH_AUTO = 0, PATH_STREAM = 1, PATH_TILED = 2, PATH_GEMM = 3 };
// Rows per streaming tile, for measurement: QMOE_STREAM_TILE_ROWS = 8 (when
// both GEMMs allow it), 16, 32, 48 or 64 (at most the token count rounded up
// to 16); anything else: the plan's own.
int stream_rows_override() {
  const char* v = std::getenv("QMOE_STREAM_TILE_ROWS");
  if (!v) return 0;
  const std::string s(v);
  return (s == "8" || s == "16" || s == "32" || s == "48" || s == "64") ? std::stoi(s) : 0;
}

// Items per single stage of 8-row streaming tiles, for measurement and
// tests: QMOE_STREAM_STAGE_ITEMS = n (both GEMMs) or "n1,n2" (FC1, FC2) with
// n in {1, 4, 8}, where the shapes allow it; anything else: the plan's own.
int stream_items_override(int gemm) {
  const char* v = std::getenv("QMOE_STREAM_STAGE_ITEMS");
  if (!v) return 0;
  std::string s(v);
  const size_t comma = s.find(',');
  if (comma != std::string::npos) s = gemm == 0 ? s.substr(0, comma) : s.substr(comma + 1);
  return s == "1" ? 1 : s == "4" ? 4 : s == "8" ? 8 : 0;
}

// QMOE_TILED_HALF=0 runs every tiled GEMM tile at 128 rows (for measurement
// and tests); anything else: the plan's own choice.
bool half_tiles_off() {
  const char* v = std::getenv("QMOE_TILED_HALF");
  return v && std::string(v) == "0";
}

// QMOE_TILED_SEGMENTS=0 keeps the per-row operand split between the tiled
// GEMMs (for measurement and tests); anything else: the plan's own choice.
bool segments_off() {
  const char* v = std::getenv("QMOE_TILED_SEGMENTS");
  return v && std::string(v) == "0";
}

// QMOE_TILED_KSPLIT=1, 2 or 4 sets the K ranges of the tiled FC2 (for
// measurement and tests; a count the shape does not allow gives one range);
// anything else: the plan's own choice.
int tiled_ksplit_override() {
  const char* v = std::getenv("QMOE_TILED_KSPLIT");
  if (!v) return 0;
  const std::string s(v);
  return s == "1" ? 1 : s == "2" ? 2 : s == "4" ? 4 : 0;
}

int path_override() {
  const char* v = std::getenv("QMOE_PATH");
  if (!v) return PATH_AUTO;
  const std::string s(v);
  if (s == "stream") return PATH_STREAM;
  if (s == "tiled") return PATH_TILED;
  if (s == "gemm") return PATH_GEMM;
  return PATH_AUTO;
}

}  // namespace

qmoe_status validate(const qmoe_tensor* input, const qmoe_tensor* router, const qmoe_tensor* fc1w,
                     const qmoe_tensor* fc1s, const qmoe_tensor* fc2w, const qmoe_tensor* fc2s,
                     const qmoe_tensor* output, const qmoe_attrs* a, Dims* d) {
  if (!input || !router || !fc1w || !fc1s || !fc2w || !fc2s || !a || !d) return QMOE_ERR_NULL;

  // Standard attribute values this library does not implement.
  if (a->quant_type != 0) return QMOE_ERR_UNSUPPORTED;
  if (a->use_sparse_mixer == 1) return QMOE_ERR_UNSUPPORTED;
  if (a->use_sparse_mixer != 0) return QMOE_ERR_ATTR;
  if (a->weights_prepacked == 1) return QMOE_ERR_UNSUPPORTED;
  if (a->weights_prepacked != -1 && a->weights_prepacked != 0) return QMOE_ERR_ATTR;
  if (a->swiglu_fusion == 2) return QMOE_ERR_UNSUPPORTED;
  // attributeConstraints
  if (a->expert_weight_bits != 4 && a->expert_weight_bits != 8) return QMOE_ERR_ATTR;
  if (a->normalize_routing_weights != 0 && a->normalize_routing_weights != 1) return QMOE_ERR_ATTR;
  if (a->routing != QMOE_ROUTE_QMOE && a->routing != QMOE_ROUTE_MOE) return QMOE_ERR_ATTR;
  // activationSupported
  const bool relu = a->activation_type == QMOE_ACT_RELU && a->swiglu_fusion == 0;
  const bool swiglu = a->activation_type == QMOE_ACT_SWIGLU && a->swiglu_fusion == 1;
  if (!relu && !swiglu) return QMOE_ERR_ATTR;
  // swiglu_limit: optional, > 0 when given
  if (a->has_swiglu_limit != 0 && a->has_swiglu_limit != 1) return QMOE_ERR_ATTR;
  if (a->has_swiglu_limit == 1 && !(a->swiglu_limit > 0.f)) return QMOE_ERR_ATTR;
  // quantBlockSizeOk, attribute part
  const int64_t bs = a->block_size;
  if (bs < 0 || (bs != 0 && (bs < 16 || !is_pow2(bs)))) return QMOE_ERR_ATTR;

  // typeConstraints: T = float32, T1 = uint8, T2 = float32
  if (input->dtype != QMOE_F32 || router->dtype != QMOE_F32 || fc1w->dtype != QMOE_U8 ||
      fc2w->dtype != QMOE_U8 || fc1s->dtype != QMOE_F32 || fc2s->dtype != QMOE_F32)
    return QMOE_ERR_DTYPE;
  if (output && output->dtype != QMOE_F32) return QMOE_ERR_DTYPE;

  // inputOutputShapeOk
  if (input->rank != 2 && input->rank != 3) return QMOE_ERR_SHAPE;
  for (const qmoe_tensor* t : {input, router, fc1w, fc1s, fc2w, fc2s, output}) {
    if (!t) continue;
    const qmoe_status st = extents_ok(t);
    if (st != QMOE_OK) return st;
  }
  const int64_t H = input->dims[input->rank - 1];
  if (H <= 0) return QMOE_ERR_SHAPE;
  int64_t T = 1;  // each factor < 2^31: the product of two fits int64
  for (int i = 0; i < input->rank - 1; ++i) T *= input->dims[i];
  if (T > kMaxExtent) return QMOE_ERR_UNSUPPORTED;
  if (output) {
    if (output->rank != input->rank) return QMOE_ERR_SHAPE;
    for (int i = 0; i < input->rank; ++i)
      if (output->dims[i] != input->dims[i]) return QMOE_ERR_SHAPE;
  }

  const int bits = a->expert_weight_bits;
  const int pack = bits == 4 ? 2 : 1;
  const int fusion = swiglu ? 2 : 1;

  // quantShapeOk
  if (!rank_ok(router, 2) || !rank_ok(fc1w, 3) || !rank_ok(fc2w, 3)) return QMOE_ERR_SHAPE;
  const int64_t E = router->dims[1];
  if (router->dims[0] != T || E < 0) return QMOE_ERR_SHAPE;
  // The weights hold El consecutive experts from first_expert (all E by default).
  const int64_t El = fc1w->dims[0];
  if (El < 0 || El > E || fc2w->dims[0] != El) return QMOE_ERR_SHAPE;
  if (a->first_expert < 0 || a->first_expert + El > E) return QMOE_ERR_ATTR;
  const int64_t F = fc1w->dims[1];
  if (F < 0 || F % fusion != 0) return QMOE_ERR_SHAPE;
  const int64_t I = F / fusion;
  if (fc2w->dims[1] != H) return QMOE_ERR_SHAPE;
  if (H % pack != 0 || I % pack != 0 || fc1w->dims[2] != H / pack || fc2w->dims[2] != I / pack)
    return QMOE_ERR_SHAPE;
  // quantBlockSizeOk, shape part
  if (bs != 0 && (H % bs != 0 || I % bs != 0)) return QMOE_ERR_SHAPE;
  // quantScalesOk
  if (fc1s->rank < 2 || fc2s->rank < 2) return QMOE_ERR_SHAPE;
  if (fc1s->dims[0] != El || fc2s->dims[0] != El || fc1s->dims[1] != F || fc2s->dims[1] != H)
    return QMOE_ERR_SHAPE;
  if (bs == 0) {
    if (fc1s->rank != 2 || fc2s->rank != 2) return QMOE_ERR_SHAPE;
  } else {
    if (fc1s->rank != 3 || fc2s->rank != 3 || fc1s->dims[2] != H / bs || fc2s->dims[2] != I / bs)
      return QMOE_ERR_SHAPE;
  }
  // quantContract: 1 <= k <= num_experts
  if (a->k < 1 || a->k > E) return QMOE_ERR_ATTR;
  // slot count and intermediates within the kernels' index ranges
  if (T * a->k > kMaxExtent) return QMOE_ERR_UNSUPPORTED;
  if (T * H > kMaxElements || T * a->k * (F + 128) > kMaxElements || T * a->k * H > kMaxElements)
    return QMOE_ERR_UNSUPPORTED;
  // The routing kernels hold one row of logits per wavefront in registers.
  if (E > kMaxExperts) return QMOE_ERR_UNSUPPORTED;

  d->T = T; d->H = H; d->E = E; d->I = I; d->F = F; d->k = a->k;
  d->El = El; d->first = a->first_expert;
  d->bits = bits; d->pack = pack; d->mid = bits == 4 ? 8 : 128; d->fusion = fusion;
  d->bs = bs; d->nb1 = bs ? H / bs : 1; d->nb2 = bs ? I / bs : 1;
  d->act = swiglu ? QMOE_ACT_SWIGLU : QMOE_ACT_RELU;
  d->routing = a->routing; d->normalize = a->normalize_routing_weights;
  d->alpha = a->activation_alpha; d->beta = a->activation_beta;
  d->limit = a->has_swiglu_limit ? a->swiglu_limit : __builtin_inff();
  return QMOE_OK;
}

namespace {

// Tiles of 8 rows: each K range is one stage, staged once, of 8, 4 or 1
// items (2048, 1024 or 256 codes at 4 bits; half that at 8; 8 items take the
// LDS of a 16-row tile's 4-item stage).  Preference, measured on the decode
// layer at 8 and 16 tokens, the large-E layer at 8 and 16 tokens and the
// decode inter share: FC1 (gemm 0) 8, 4, then 1 items (8 items faster by
// 2-5 % even in as few as 224 workgroups); FC2 (gemm 1) 4, 8, then 1 (4
// items faster by 0-5 %; single items 20-25 % slower where 4 fit, but they
// stream the inter share's 1792-code FC2 in 17 us against 70 us on the
// register-tiled GEMM).  st->on is false when no stage tiles K.
void stream_shape_half(const Dims& d, int64_t K, int64_t N, int gemm, Plan::Stream* st) {
  *st = Plan::Stream();
  const int64_t item_codes = d.bits == 4 ? 256 : 128;
  if (ceil_div(N, 128 * QMOE_STREAM_NT) > kMaxGridYZ) return;
  const int force = stream_items_override(gemm);
  int best = 0;
  const int order[2][3] = {{8, 4, 1}, {4, 8, 1}};
  for (int items : order[gemm]) {
    const int64_t scodes = items * item_codes;
    if (!(K > 0 && K % scodes == 0 && (d.bs == 0 || d.bs >= 32))) continue;
    if (d.bs > 0 && d.bs < item_codes / 2) {
      const int64_t nbs = scodes / d.bs;  // blocks ending inside 64-byte chunks, per stage
      if (nbs % 4 != 0 || nbs > 32) continue;
    }
    if (K / scodes > max_one_splits()) continue;
    if (force != 0 && items != force) continue;
    best = items;
    break;
  }
  if (best == 0) return;
  st->on = true;
  st->one = true;
  st->stg = best;
  st->splits = (int)(K / (best * item_codes));
  st->nst = 1;
}

// Split of one streaming GEMM (reduction length K, N weight rows) into K
// ranges of stages of 128-byte row items, for tiles of 16 * mt rows; st->on
// is false when the stages cannot tile K.
void stream_shape(const Dims& d, int mt, int64_t K, int64_t N, Plan::Stream* st) {
  *st = Plan::Stream();
  // Stages of stg items (256 codes an item at 4 bits, 128 at 8) must tile
  // K.  Scale blocks that end inside a 64-byte chunk (bs < codes per chunk)
  // must come 4 to 16 to a stage.
  const int64_t item_codes = d.bits == 4 ? 256 : 128;
  const int64_t chunk_codes = item_codes / 2;
  const int64_t units = d.El * ceil_div(N, 128 * QMOE_STREAM_NT);
  if (ceil_div(N, 128 * QMOE_STREAM_NT) > kMaxGridYZ) return;  // row groups are a grid dimension
  auto fits = [&](int64_t scodes) {
    if (!(K > 0 && K % scodes == 0 && (d.bs == 0 || d.bs >= 32))) return false;
    if (d.bs > 0 && d.bs < chunk_codes) {
      const int64_t nbs = scodes / d.bs;  // blocks ending inside chunks, per stage
      return nbs % 4 == 0 && nbs <= 16;
    }
    return true;
  };
  // One stage per K range (staged once) when that takes at most
  // QMOE_STREAM_MAX_ONE_SPLITS ranges; else double-buffered stages over the
  // whole of K, split only as far as needed to fill the chip.
  const int64_t one_codes = stream_stage_items(mt, true) * item_codes;
  if (fits(one_codes) && K / one_codes <= max_one_splits()) {
    st->on = true;
    st->one = true;
    st->stg = stream_stage_items(mt, true);
    st->splits = (int)(K / one_codes);
    st->nst = 1;
    return;
  }
  st->one = false;
  st->stg = stream_stage_items(mt, false);
  const int64_t scodes = st->stg * item_codes;
  st->on = fits(scodes);
  if (!st->on) return;
  const int64_t nst_total = K / scodes;
  int64_t splits = nst_total;
  for (int64_t z = 1; z <= nst_total; ++z)
    if (nst_total % z == 0 && units * z >= QMOE_STREAM_MIN_WORKGROUPS) {
      splits = z;
      break;
    }
  st->splits = (int)splits;
  st->nst = (int)(nst_total / splits);
  // With one K range and one tile row of 16, size the workgroups so that the
  // grid is one round of QMOE_STREAM_MIN_WORKGROUPS equal workgroups when
  // that takes 256 to 512 rows each (whole 64-row pieces): every compute
  // unit then streams the same share to the end.
  st->wg_rows = 0;
  const int64_t rbrows = 128 * QMOE_STREAM_NT;
  if (mt == 1 && splits == 1 && units > QMOE_STREAM_MIN_WORKGROUPS) {
    const int64_t r = round_up(ceil_div(d.El * N, QMOE_STREAM_MIN_WORKGROUPS), 64);
    st->wg_rows = (int)std::min(r, 2 * rbrows);
  }
}

}  // namespace

void make_plan(const Dims& d, Plan* p) {
  *p = Plan();
  p->d = d;
  p->S = d.T * d.k;
  if (d.T == 0) return;  // nothing to enqueue
  p->share = d.El < d.E;
  // GEMM path.  The weight-streaming kernels read every weight row once per
  // M tile of 16 rows (an expert with more rows takes several tiles); the
  // LDS-tiled kernels use 128-row tiles.  Measured on the decode (8 large
  // experts), large-E (128 int8 experts), fine-grained (64 small experts) and
  // decode inter-share layers (bench.py --crossover): where both GEMMs
  // stream, streaming is faster up to about 240 tokens on the decode layer
  // and 100 to 160 on the large-E one (whose tiled GEMMs run the experts'
  // few rows as 64-row half tiles), within 3 to 5 % between them; the switch
  // is at 224 tokens.  Where only FC1 streams (FC2's reduction is not a
  // whole number of stages) streaming is faster up to 64 tokens with 8
  // experts and slower at every size with 64.  Taller streaming tiles (each weight fragment
  // feeding 2 to 4 row subtiles) made the kernel bound by matrix-core and LDS
  // work instead of HBM: 0.36 / 0.63 / 0.72 ms at 32 / 64 / 96 decode tokens
  // against 0.20 / 0.30 / 0.35 ms with 16-row tiles.
  const int force = path_override();
  // (the streaming grid's third dimension is the tile count: a forced
  // streaming plan needs it within the grid limit)
  bool stream = force == PATH_STREAM && (p->S + 15) / 16 + d.El <= kMaxGridYZ;
  if (force == PATH_AUTO && d.I > 0 && d.El > 0 && d.T <= kStreamMaxTokens) {
    Plan::Stream a, b;
    stream_shape(d, 1, d.H, d.F, &a);
    stream_shape(d, 1, d.I, d.H, &b);
    stream = (a.on && b.on) || (a.on && d.T <= kStreamMixedMaxTokens && d.El <= kStreamMixedMaxExperts);
  }
  p->decode = stream;
  p->mt = 4;
  if (p->decode) {
    const int rows = stream_rows_override();
    p->mt = rows >= 16 ? int(std::min<int64_t>(rows / 16, (d.T + 15) / 16)) : 1;
    // Tiles of 8 rows when routing gives an expert 4 rows on average (most
    // experts then fit one tile): a K range then spans twice the codes in
    // the same LDS, which halves the fp32 K-range partials both GEMMs write
    // and doubles each workgroup's contiguous run of every weight row.  An
    // expert with more than 8 rows takes several tiles and streams its
    // weights once per tile.
    if (d.I > 0 && d.El > 0 && (rows == 8 || (rows == 0 && p->S <= 4 * d.El))) {
      Plan::Stream a, b;
      stream_shape_half(d, d.H, d.F, 0, &a);
      stream_shape_half(d, d.I, d.H, 1, &b);
      p->half = a.on && b.on;
    }
  }
  p->bm = p->half ? 8 : 16 * p->mt;
  // Otherwise the LDS-tiled GEMMs when both reductions are whole 64-code
  // steps, rows are 8-code aligned and scale blocks are >= 32 codes (else
  // the register-tiled GEMMs with 64-row tiles).
  const bool aligned8 = (d.H % 8 == 0) && (d.I % 8 == 0);
  p->tiled = !p->decode && force != PATH_GEMM && d.I > 0 && aligned8 && d.H % 64 == 0 && d.I % 64 == 0 &&
             (d.bs == 0 || d.bs >= 32);
  if (p->tiled) p->bm = 128;
  // Half tiles with column-wise scales only (with block scales the tiled
  // kernel's half-tile code path was measured slower than whole tiles)
  p->half_tiles = p->tiled && d.bs == 0 && !half_tiles_off() ? 1 : 0;
  // Sum over experts of ceil(count / bm) <= ceil(S / bm) + E; when one tile
  // holds any expert's rows it is at most E (one tile per used expert).
  p->max_tiles = (p->decode && d.T <= p->bm) ? d.El : (p->S + p->bm - 1) / p->bm + d.El;
  // With I == 0 only the routing stages run (output is a zero fill).
  p->kp1 = d.I > 0 ? round_up(d.H, 128) : 0;
  p->kp2 = round_up(d.I, 128);
  // Segment scales between the tiled GEMMs: FC1's epilogue writes FC2's
  // hi/lo operand rows itself with one power-of-two scale per row tile and
  // column tile, so no split pass runs between them.  Every span FC2 folds
  // (a scale block of up to 128 codes, or two 64-code steps with
  // column-wise scales) lies in one FC1 column tile.
  if (p->tiled && (d.bs != 0 || d.I % 128 == 0) && !segments_off()) {
    p->seg_shift = d.act == QMOE_ACT_SWIGLU ? 7 : 8;  // codes of an FC1 column tile of 256 columns
    p->seg_n = (int)((d.I + (int64_t(1) << p->seg_shift) - 1) >> p->seg_shift);
  }
  // K ranges of the tiled FC2: one workgroup runs on a compute unit at a
  // time, so an FC2 with few tiles leaves units idle in its last round of
  // tiles (or in its only one).  Each range doubles the workgroups and adds
  // one partial set (S x H fp32) that the combine sums in range order.
  // Ranges double while the estimated tile count (the routed rows in
  // 128-row tiles, half a tile of padding an expert) is under 16 rounds of
  // 256 and each range keeps at least 1024 codes (shorter ones measured
  // slower: a tile's fixed costs and the combine's extra reads outweigh the
  // rounds saved).  The kernel takes ranges of any multiple of 256 codes
  // and of the scale block.
  if (p->tiled) {
    const int64_t rows = p->share ? (p->S * d.El + d.E - 1) / d.E : p->S;
    const int64_t est = ((rows + p->bm - 1) / p->bm + d.El / 2) * ((d.H + 255) / 256);
    auto ranges_ok = [&](int ks, int64_t least) {
      const int64_t kr = d.I / ks;
      return d.I % ks == 0 && kr % 256 == 0 && kr >= least && (d.bs == 0 || kr % d.bs == 0);
    };
    const int force = tiled_ksplit_override();
    int ks = 1;
    if (force > 0) {
      if (ranges_ok(force, 256)) ks = force;
    } else {
      while (ks < 4 && est * ks < 16 * 256 && ranges_ok(2 * ks, 1024)) ks *= 2;
    }
    p->ksplit2 = ks;
    p->splits2 = ks;
  }
  p->aligned = (d.H % 8 == 0) && (d.I % 8 == 0);
  p->nchunks = (p->S + p->chunk - 1) / p->chunk;
  // a share permutes over El + 1 groups (the last: slots of experts not held)
  p->small_front = !p->share && p->S <= 1024 && d.E <= 1024;
  if (p->decode && d.I > 0 && d.El > 0) {
    if (p->half) {
      stream_shape_half(d, d.H, d.F, 0, &p->s1);
      stream_shape_half(d, d.I, d.H, 1, &p->s2);
    } else {
      stream_shape(d, p->mt, d.H, d.F, &p->s1);
      stream_shape(d, p->mt, d.I, d.H, &p->s2);
    }
    if (p->s2.on) p->splits2 = p->s2.splits;
  }
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o = align256(o + bytes); return at; };
  p->off_topk_idx = take(sizeof(int32_t) * p->S);
  p->off_topk_w = take(sizeof(float) * p->S);
  const int64_t groups = p->share ? d.El + 1 : d.E;  // permutation groups
  p->off_counts = take(sizeof(int32_t) * groups);
  p->off_offsets = take(sizeof(int32_t) * (groups + 1));
  p->off_perm = take(sizeof(int32_t) * p->S);
  p->off_tiles = take(sizeof(int32_t) * 4 * p->max_tiles);
  p->off_ntiles = take(sizeof(int32_t) * 4);
  p->off_hist = take(sizeof(int32_t) * p->nchunks * groups);
  p->off_xa = take(p->s1.on ? 0 : size_t(4) * d.T * p->kp1);  // f16 hi + lo per element (streaming FC1 reads fp32 rows)
  p->off_act = take(size_t(4) * p->S * p->kp2);   // fp32 per element, or f16 hi + lo after the split pass
  p->off_exp1 = take(sizeof(int32_t) * d.T);
  p->off_exp2 = take(sizeof(int32_t) * p->S);
  p->off_seg = take(sizeof(float) * p->max_tiles * p->seg_n);
  p->off_segrows = take(sizeof(int32_t) * p->S * p->seg_n);
  p->off_segflag = take(p->seg_n > 0 ? sizeof(int32_t) : 0);
  p->off_local = take(p->share ? sizeof(int32_t) * p->S : 0);
  p->off_slot = take(d.I > 0 ? sizeof(float) * p->splits2 * p->S * d.H : 0); // FC2 rows by slot id
  p->off_part1 = take(p->s1.on && p->s1.splits > 1 ? sizeof(float) * p->s1.splits * p->S * d.F : 0);
  p->off_trows = take(p->s1.on || p->s2.on ? sizeof(int32_t) * p->max_tiles * p->bm : 0);
  p->bytes = o;
}

}  // namespace qmoe
