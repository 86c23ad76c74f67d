// C ABI of the float MoE operator (com.microsoft.MoE README; declared in
// include/qmoe.h): contract check, workspace plan and enqueue.
//
// qmoe_moe_forward enqueues, on the caller's stream:
//   router (full softmax, top-k) -> permutation (histogram, scan, stable
//   scatter) -> FC1 (and FC3) grouped GEMMs -> activation -> FC2 grouped GEMM
//   (bias, rows by slot id) -> weighted combine
// with every intermediate in the caller's workspace.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "kernels/launch.h"
#include "qmoe.h"

using namespace qmoe;

namespace {

bool aligned_to(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int64_t numel(const qmoe_tensor* t) {
  int64_t n = 1;
  for (int i = 0; i < t->rank; ++i) n *= t->dims[i];
  return n;
}

constexpr int64_t kMaxExpertsMoe = 1024;  // routing kernels hold an expert per thread / LDS entry
constexpr int64_t kChunk = 1024;          // slots per permutation block

struct MoePlan {
  int64_t T = 0, H = 0, E = 0, I = 0, F = 0, k = 0, S = 0;
  int act = QMOE_ACT_RELU, fusion = 0, normalize = 0;
  float alpha = 1.f, beta = 0.f;
  float limit = __builtin_inff();  // SwiGLU clamp (+inf: none)
  bool uses_fc3 = false;
  bool small_front = false;
  bool rows16 = false;   // at most 16 rows per used expert on average: 16-row tiles, weight streaming
  int64_t bm = 64, max_tiles = 0, nchunks = 0;
  size_t off_topk_idx = 0, off_topk_w = 0, off_counts = 0, off_offsets = 0, off_perm = 0, off_tiles = 0;
  size_t off_ntiles = 0, off_hist = 0, off_h1 = 0, off_h3 = 0, off_act = 0, off_slot = 0;
  size_t bytes = 0;
};

bool dims_are(const qmoe_tensor* t, int rank, int64_t d0, int64_t d1, int64_t d2 = 0) {
  if (t->rank != rank) return false;
  const int64_t d[3] = {d0, d1, d2};
  for (int i = 0; i < rank; ++i)
    if (t->dims[i] != d[i]) return false;
  return true;
}

qmoe_status check(const qmoe_tensor* input, const qmoe_tensor* router, const qmoe_tensor* fc1w,
                  const qmoe_tensor* fc1b, const qmoe_tensor* fc2w, const qmoe_tensor* fc2b,
                  const qmoe_tensor* fc3w, const qmoe_tensor* fc3b, const qmoe_tensor* output,
                  const qmoe_moe_attrs* a, MoePlan* p) {
  if (!input || !router || !fc1w || !fc2w || !a) return QMOE_ERR_NULL;
  // Type constraints: T = float32 for every tensor
  const qmoe_tensor* all[] = {input, router, fc1w, fc1b, fc2w, fc2b, fc3w, fc3b, output};
  for (const qmoe_tensor* t : all)
    if (t && t->dtype != QMOE_F32) return QMOE_ERR_DTYPE;
  for (const qmoe_tensor* t : all)
    if (t) {
      if (t->rank < 1 || t->rank > 3) return QMOE_ERR_SHAPE;
      for (int i = 0; i < t->rank; ++i)
        if (t->dims[i] < 0) return QMOE_ERR_SHAPE;
    }
  // input (T, H) or (B, S, H); router_probs (T, E); fc2 (E, H, I)
  if (input->rank != 2 && input->rank != 3) return QMOE_ERR_SHAPE;
  p->H = input->dims[input->rank - 1];
  p->T = 1;
  for (int i = 0; i < input->rank - 1; ++i) p->T *= input->dims[i];
  if (router->rank != 2 || router->dims[0] != p->T) return QMOE_ERR_SHAPE;
  p->E = router->dims[1];
  if (fc2w->rank != 3 || fc2w->dims[0] != p->E || fc2w->dims[1] != p->H) return QMOE_ERR_SHAPE;
  p->I = fc2w->dims[2];
  // attributes
  if (a->activation_type < QMOE_ACT_RELU || a->activation_type > QMOE_ACT_IDENTITY) return QMOE_ERR_ATTR;
  if (a->swiglu_fusion < 0 || a->swiglu_fusion > 2) return QMOE_ERR_ATTR;
  if (a->use_sparse_mixer == 1) return QMOE_ERR_UNSUPPORTED;
  if (a->use_sparse_mixer != 0) return QMOE_ERR_ATTR;
  if (a->normalize_routing_weights != 0 && a->normalize_routing_weights != 1) return QMOE_ERR_ATTR;
  if (a->k < 1 || a->k > p->E) return QMOE_ERR_ATTR;
  if (a->has_swiglu_limit != 0 && a->has_swiglu_limit != 1) return QMOE_ERR_ATTR;
  if (a->has_swiglu_limit == 1 && !(a->swiglu_limit > 0.f)) return QMOE_ERR_ATTR;
  p->limit = a->has_swiglu_limit ? a->swiglu_limit : __builtin_inff();
  p->k = a->k;
  p->act = a->activation_type;
  p->fusion = a->swiglu_fusion;
  p->normalize = a->normalize_routing_weights;
  p->alpha = a->activation_alpha;
  p->beta = a->activation_beta;
  const bool fused = p->act == QMOE_ACT_SWIGLU && p->fusion != 0;
  p->F = (fused ? 2 : 1) * p->I;
  // weights and biases
  if (!dims_are(fc1w, 3, p->E, p->F, p->H)) return QMOE_ERR_SHAPE;
  if (fc3w && !dims_are(fc3w, 3, p->E, p->I, p->H)) return QMOE_ERR_SHAPE;
  if (p->act == QMOE_ACT_SWIGLU && p->fusion == 0 && !fc3w) return QMOE_ERR_SHAPE;
  if (fc1b && !dims_are(fc1b, 2, p->E, p->F)) return QMOE_ERR_SHAPE;
  if (fc2b && !dims_are(fc2b, 2, p->E, p->H)) return QMOE_ERR_SHAPE;
  if (fc3b && (!fc3w || !dims_are(fc3b, 2, p->E, p->I))) return QMOE_ERR_SHAPE;
  if (output) {
    if (output->rank != input->rank) return QMOE_ERR_SHAPE;
    for (int i = 0; i < input->rank; ++i)
      if (output->dims[i] != input->dims[i]) return QMOE_ERR_SHAPE;
  }
  p->uses_fc3 = fc3w && (p->act == QMOE_ACT_SILU || (p->act == QMOE_ACT_SWIGLU && p->fusion == 0));
  // limits of this library
  const int64_t lim30 = int64_t(1) << 30;
  if (p->E > kMaxExpertsMoe || p->T >= lim30 || p->F >= lim30 || p->H >= lim30) return QMOE_ERR_UNSUPPORTED;
  p->S = p->T * p->k;
  if (p->S >= lim30) return QMOE_ERR_UNSUPPORTED;

  // plan
  p->small_front = p->S <= 1024 && p->E <= 1024;
  p->rows16 = p->S <= 16 * std::max<int64_t>(1, std::min(p->E, p->S));
  p->bm = p->rows16 ? gmm_rows16_tile_rows() : gmm_tile_rows();
  p->max_tiles = (p->S + p->bm - 1) / p->bm + p->E;
  p->nchunks = (p->S + kChunk - 1) / kChunk;
  if (p->T == 0 || p->H == 0) return QMOE_OK;  // empty output: nothing to enqueue
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o = align256(o + bytes); return at; };
  p->off_topk_idx = take(sizeof(int32_t) * p->S);
  p->off_topk_w = take(sizeof(float) * p->S);
  p->off_counts = take(sizeof(int32_t) * p->E);
  p->off_offsets = take(sizeof(int32_t) * (p->E + 1));
  p->off_perm = take(sizeof(int32_t) * p->S);
  p->off_tiles = take(sizeof(int32_t) * 4 * p->max_tiles);
  p->off_ntiles = take(sizeof(int32_t) * 4);
  p->off_hist = take(sizeof(int32_t) * p->nchunks * p->E);
  p->off_h1 = take(sizeof(float) * p->S * p->F);                      // FC1 rows, sorted order
  p->off_h3 = take(p->uses_fc3 ? sizeof(float) * p->S * p->I : 0);   // FC3 rows, sorted order
  p->off_act = take(sizeof(float) * p->S * p->I);                     // activation rows, sorted order
  p->off_slot = take(sizeof(float) * p->S * p->H);                    // FC2 rows by slot id
  p->bytes = o;
  return QMOE_OK;
}

#define QMOE_TRY_HIP(expr)                         \
  do {                                             \
    if ((expr) != hipSuccess) return QMOE_ERR_HIP; \
  } while (0)

const float* fptr(const qmoe_tensor* t) { return t ? static_cast<const float*>(t->data) : nullptr; }

// One float32 projection over the expert-sorted rows: weight streaming over
// 16-row tiles where the plan chose them and the shapes allow, else the
// LDS-tiled kernel.
hipError_t projection(const MoePlan& p, const F32Gemm& g, hipStream_t s) {
  const bool vec = g.K % 4 == 0 && aligned_to(g.a, 16) && aligned_to(g.w, 16);
  if (p.rows16 && vec) {
    const long est_tiles = std::max<int64_t>(1, std::min(p.E, p.S));  // experts in use, at most
    return launch_gmm_rows16(g, true, gmm_rows16_ksplit(est_tiles, g.N), (int)p.max_tiles, s);
  }
  return launch_gmm_f32(g, true, vec, (int)p.max_tiles, s);
}

qmoe_status moe_impl(const qmoe_tensor* input, const qmoe_tensor* router, const qmoe_tensor* fc1w,
                     const qmoe_tensor* fc1b, const qmoe_tensor* fc2w, const qmoe_tensor* fc2b,
                     const qmoe_tensor* fc3w, const qmoe_tensor* fc3b, const qmoe_moe_attrs* attrs,
                     const qmoe_tensor* output, void* workspace, size_t ws_bytes, void* stream,
                     const qmoe_debug* dbg) {
  if (!output) return QMOE_ERR_NULL;
  MoePlan p;
  qmoe_status st = check(input, router, fc1w, fc1b, fc2w, fc2b, fc3w, fc3b, output, attrs, &p);
  if (st != QMOE_OK) return st;
  if (p.T == 0 || p.H == 0) return QMOE_OK;
  const qmoe_tensor* all[] = {input, router, fc1w, fc1b, fc2w, fc2b, fc3w, fc3b, output};
  for (const qmoe_tensor* t : all)
    if (t && numel(t) > 0 && t->data == nullptr) return QMOE_ERR_NULL;
  for (const qmoe_tensor* t : {input, output, fc1w, fc2w, fc3w})
    if (t && !aligned_to(t->data, 16)) return QMOE_ERR_ALIGN;
  for (const qmoe_tensor* t : {router, fc1b, fc2b, fc3b})
    if (t && !aligned_to(t->data, 4)) return QMOE_ERR_ALIGN;
  if (workspace == nullptr) return QMOE_ERR_NULL;
  if (ws_bytes < p.bytes) return QMOE_ERR_WORKSPACE;
  if (!aligned_to(workspace, 256)) return QMOE_ERR_ALIGN;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  int* topk_idx = reinterpret_cast<int*>(ws + p.off_topk_idx);
  float* topk_w = reinterpret_cast<float*>(ws + p.off_topk_w);
  int* counts = reinterpret_cast<int*>(ws + p.off_counts);
  int* offsets = reinterpret_cast<int*>(ws + p.off_offsets);
  int* perm = reinterpret_cast<int*>(ws + p.off_perm);
  int* tiles = reinterpret_cast<int*>(ws + p.off_tiles);
  int* ntiles = reinterpret_cast<int*>(ws + p.off_ntiles);
  int* hist = reinterpret_cast<int*>(ws + p.off_hist);
  float* h1 = reinterpret_cast<float*>(ws + p.off_h1);
  float* h3 = reinterpret_cast<float*>(ws + p.off_h3);
  float* act = reinterpret_cast<float*>(ws + p.off_act);
  float* slot = reinterpret_cast<float*>(ws + p.off_slot);
  const int T = (int)p.T, E = (int)p.E, k = (int)p.k, S = (int)p.S;
  auto mark = [&](int i) -> hipError_t {
    if (dbg && dbg->events[i]) return hipEventRecord(reinterpret_cast<hipEvent_t>(dbg->events[i]), s);
    return hipSuccess;
  };

  QMOE_TRY_HIP(mark(0));
  const float* logits = fptr(router);
  if (p.small_front) {
    QMOE_TRY_HIP(launch_route_small(logits, T, E, k, QMOE_ROUTE_MOE, p.normalize, (int)p.bm, topk_idx, topk_w,
                                    counts, offsets, perm, tiles, ntiles, nullptr, s));
  } else {
    QMOE_TRY_HIP(launch_router(logits, T, E, k, QMOE_ROUTE_MOE, p.normalize, topk_idx, topk_w, s));
    QMOE_TRY_HIP(launch_permute(topk_idx, S, E, (int)kChunk, (int)p.nchunks, (int)p.bm, hist, counts, offsets,
                                perm, tiles, ntiles, s));
  }
  QMOE_TRY_HIP(mark(1));

  // FC1 (and FC3): operand rows are token rows gathered by slot id / k,
  // results in expert-sorted order.
  F32Gemm g{};
  g.a = fptr(input);
  g.a_perm = perm;
  g.a_div = k;
  g.perm = perm;
  g.out_by_slot = 0;
  g.tiles = tiles;
  g.ntiles = ntiles;
  g.K = (int)p.H;
  g.G = E;
  if (p.F > 0) {
    g.w = fptr(fc1w);
    g.bias = fptr(fc1b);
    g.N = (int)p.F;
    g.out = h1;
    QMOE_TRY_HIP(projection(p, g, s));
  }
  if (p.uses_fc3 && p.I > 0) {
    g.w = fptr(fc3w);
    g.bias = fptr(fc3b);
    g.N = (int)p.I;
    g.out = h3;
    QMOE_TRY_HIP(projection(p, g, s));
  }
  QMOE_TRY_HIP(mark(2));
  QMOE_TRY_HIP(launch_moe_act(p.act, h1, p.uses_fc3 ? h3 : nullptr, S, (int)p.I, (int)p.F, p.fusion, p.alpha,
                              p.beta, p.limit, act, s));
  QMOE_TRY_HIP(mark(3));
  // FC2: operand rows in sorted order, results (bias included) by slot id.
  // With I == 0 the rows are the bias alone.
  F32Gemm g2{};
  g2.a = act;
  g2.a_perm = nullptr;
  g2.a_div = 1;
  g2.w = fptr(fc2w);
  g2.bias = fptr(fc2b);
  g2.perm = perm;
  g2.out_by_slot = 1;
  g2.tiles = tiles;
  g2.ntiles = ntiles;
  g2.K = (int)p.I;
  g2.N = (int)p.H;
  g2.G = E;
  g2.out = slot;
  QMOE_TRY_HIP(projection(p, g2, s));
  QMOE_TRY_HIP(mark(4));
  QMOE_TRY_HIP(launch_combine(slot, topk_w, T, k, (int)p.H, 1, static_cast<float*>(const_cast<void*>(output->data)),
                              s));
  QMOE_TRY_HIP(mark(5));
  if (dbg) {
    if (dbg->topk_idx) QMOE_TRY_HIP(launch_copy_i32(topk_idx, dbg->topk_idx, S, s));
    if (dbg->topk_w) QMOE_TRY_HIP(launch_copy_f32(topk_w, dbg->topk_w, S, s));
    if (dbg->counts) QMOE_TRY_HIP(launch_copy_i32(counts, dbg->counts, E, s));
    if (dbg->offsets) QMOE_TRY_HIP(launch_copy_i32(offsets, dbg->offsets, E + 1, s));
    if (dbg->perm) QMOE_TRY_HIP(launch_copy_i32(perm, dbg->perm, S, s));
  }
  return QMOE_OK;
}

}  // namespace

extern "C" {

void qmoe_moe_attrs_default(qmoe_moe_attrs* a) {
  a->k = 1;
  a->activation_type = QMOE_ACT_RELU;
  a->swiglu_fusion = 0;
  a->activation_alpha = 1.f;
  a->activation_beta = 0.f;
  a->normalize_routing_weights = 0;
  a->use_sparse_mixer = 0;
  a->has_swiglu_limit = 0;
  a->swiglu_limit = 0.f;
}

qmoe_status qmoe_moe_validate(const qmoe_tensor* input, const qmoe_tensor* router_probs,
                              const qmoe_tensor* fc1_experts_weights, const qmoe_tensor* fc1_experts_bias,
                              const qmoe_tensor* fc2_experts_weights, const qmoe_tensor* fc2_experts_bias,
                              const qmoe_tensor* fc3_experts_weights, const qmoe_tensor* fc3_experts_bias,
                              const qmoe_tensor* output, const qmoe_moe_attrs* attrs) {
  MoePlan p;
  return check(input, router_probs, fc1_experts_weights, fc1_experts_bias, fc2_experts_weights, fc2_experts_bias,
               fc3_experts_weights, fc3_experts_bias, output, attrs, &p);
}

qmoe_status qmoe_moe_workspace_size(const qmoe_tensor* input, const qmoe_tensor* router_probs,
                                    const qmoe_tensor* fc1_experts_weights, const qmoe_tensor* fc1_experts_bias,
                                    const qmoe_tensor* fc2_experts_weights, const qmoe_tensor* fc2_experts_bias,
                                    const qmoe_tensor* fc3_experts_weights, const qmoe_tensor* fc3_experts_bias,
                                    const qmoe_moe_attrs* attrs, size_t* bytes) {
  if (!bytes) return QMOE_ERR_NULL;
  MoePlan p;
  const qmoe_status st = check(input, router_probs, fc1_experts_weights, fc1_experts_bias, fc2_experts_weights,
                               fc2_experts_bias, fc3_experts_weights, fc3_experts_bias, nullptr, attrs, &p);
  if (st != QMOE_OK) return st;
  *bytes = p.bytes;
  return QMOE_OK;
}

qmoe_status qmoe_moe_forward(const qmoe_tensor* input, const qmoe_tensor* router_probs,
                             const qmoe_tensor* fc1_experts_weights, const qmoe_tensor* fc1_experts_bias,
                             const qmoe_tensor* fc2_experts_weights, const qmoe_tensor* fc2_experts_bias,
                             const qmoe_tensor* fc3_experts_weights, const qmoe_tensor* fc3_experts_bias,
                             const qmoe_moe_attrs* attrs, const qmoe_tensor* output, void* workspace,
                             size_t workspace_bytes, void* stream) {
  return moe_impl(input, router_probs, fc1_experts_weights, fc1_experts_bias, fc2_experts_weights,
                  fc2_experts_bias, fc3_experts_weights, fc3_experts_bias, attrs, output, workspace,
                  workspace_bytes, stream, nullptr);
}

qmoe_status qmoe_moe_forward_debug(const qmoe_tensor* input, const qmoe_tensor* router_probs,
                                   const qmoe_tensor* fc1_experts_weights, const qmoe_tensor* fc1_experts_bias,
                                   const qmoe_tensor* fc2_experts_weights, const qmoe_tensor* fc2_experts_bias,
                                   const qmoe_tensor* fc3_experts_weights, const qmoe_tensor* fc3_experts_bias,
                                   const qmoe_moe_attrs* attrs, const qmoe_tensor* output, void* workspace,
                                   size_t workspace_bytes, void* stream, const qmoe_debug* debug) {
  return moe_impl(input, router_probs, fc1_experts_weights, fc1_experts_bias, fc2_experts_weights,
                  fc2_experts_bias, fc3_experts_weights, fc3_experts_bias, attrs, output, workspace,
                  workspace_bytes, stream, debug);
}

}  // extern "C"
