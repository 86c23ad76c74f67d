// C ABI of GroupedMatMul (ONNX operator page "GroupedMatMul - 29"; declared
// in include/qmoe.h): contract check, workspace plan and enqueue.
//
// qmoe_grouped_matmul enqueues, on the caller's stream:
//   index conversion (invalid indices -> group G) -> permutation (histogram,
//   scan, stable scatter over G + 1 groups, 64-row tiles) -> tile GEMM
// with every intermediate in the caller's workspace.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "kernels/launch.h"
#include "qmoe.h"

using namespace qmoe;

namespace {

bool aligned_to(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

constexpr int64_t kChunk = 1024;       // slots per permutation block
constexpr int64_t kMaxGroups = 1023;   // G + 1 buckets, one scan thread each

struct GmmPlan {
  int64_t M = 0, K = 0, G = 0, N = 0, S = 0, R = 0;  // R = M * S rows
  int64_t bm = 0, max_tiles = 0, nchunks = 0, nblk = 0;
  bool idx64 = false, has_bias = false;
  int32_t dtype = QMOE_F32;  // T of the Type Constraints
  bool rows16 = false;  // groups average at most 16 rows: 16-row tiles, weight-streaming kernel
  size_t off_idx = 0, off_counts = 0, off_offsets = 0, off_perm = 0, off_tiles = 0, off_ntiles = 0, off_hist = 0;
  size_t bytes = 0;
};

bool float_code(int32_t dt) { return dt == QMOE_F32 || dt == QMOE_F16 || dt == QMOE_BF16 || dt == QMOE_F64; }

qmoe_status check(const qmoe_tensor* input, const qmoe_tensor* weights, const qmoe_tensor* idx,
                  const qmoe_tensor* bias, const qmoe_tensor* output, GmmPlan* p) {
  if (!input || !weights || !idx) return QMOE_ERR_NULL;
  if (input->rank != 2 || weights->rank != 3 || idx->rank != 2) return QMOE_ERR_SHAPE;
  if (bias && bias->rank != 2) return QMOE_ERR_SHAPE;
  if (output && output->rank != 3) return QMOE_ERR_SHAPE;
  // one floating type T for input, weights, bias and output (Type Constraints)
  const int32_t T = input->dtype;
  if (!float_code(T)) return QMOE_ERR_DTYPE;
  if (weights->dtype != T || (bias && bias->dtype != T) || (output && output->dtype != T)) return QMOE_ERR_DTYPE;
  if (idx->dtype != QMOE_I32 && idx->dtype != QMOE_I64) return QMOE_ERR_DTYPE;
  const qmoe_tensor* ts[] = {input, weights, idx, bias, output};
  for (const qmoe_tensor* t : ts)
    if (t)
      for (int i = 0; i < t->rank; ++i)
        if (t->dims[i] < 0) return QMOE_ERR_SHAPE;
  p->M = input->dims[0];
  p->K = input->dims[1];
  p->G = weights->dims[0];
  p->N = weights->dims[2];
  p->S = idx->dims[1];
  if (weights->dims[1] != p->K || idx->dims[0] != p->M) return QMOE_ERR_SHAPE;
  if (bias && (bias->dims[0] != p->G || bias->dims[1] != p->N)) return QMOE_ERR_SHAPE;
  if (output && (output->dims[0] != p->M || output->dims[1] != p->S || output->dims[2] != p->N))
    return QMOE_ERR_SHAPE;
  p->dtype = T;
  const int64_t lim30 = int64_t(1) << 30;
  if (p->M > lim30 || p->S > lim30) return QMOE_ERR_UNSUPPORTED;
  p->R = p->M * p->S;
  if (p->G > kMaxGroups || p->R >= lim30 || p->K >= lim30 || p->N >= lim30) return QMOE_ERR_UNSUPPORTED;
  p->idx64 = idx->dtype == QMOE_I64;
  // Rows per group if the rows spread over min(G, R) groups: at most one
  // 16-row tile each, the weights are streamed once (16-row tiles); else
  // LDS-tiled 64-row tiles.  With misaligned pointers the tiled kernel also
  // runs the 16-row tiles.
  const int64_t spread = std::max<int64_t>(1, std::min(p->G, p->R));
  // (double streams two columns a lane: N even suffices)
  p->rows16 = p->K % 4 == 0 && p->N % (T == QMOE_F64 ? 2 : 4) == 0 && p->R <= 16 * spread;
  p->bm = p->rows16 ? gmm_rows16_tile_rows() : gmm_tile_rows();
  p->has_bias = bias != nullptr;
  p->max_tiles = (p->R + p->bm - 1) / p->bm + p->G + 1;
  p->nblk = (p->N + 127) / 128;
  if (p->max_tiles * p->nblk >= (int64_t(1) << 31)) return QMOE_ERR_UNSUPPORTED;
  p->nchunks = (p->R + kChunk - 1) / kChunk;
  if (p->R == 0 || p->N == 0) return QMOE_OK;  // empty output: nothing to enqueue
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o = align256(o + bytes); return at; };
  const int64_t buckets = p->G + 1;
  p->off_idx = take(sizeof(int32_t) * p->R);
  p->off_counts = take(sizeof(int32_t) * buckets);
  p->off_offsets = take(sizeof(int32_t) * (buckets + 1));
  p->off_perm = take(sizeof(int32_t) * p->R);
  p->off_tiles = take(sizeof(int32_t) * 4 * p->max_tiles);
  p->off_ntiles = take(sizeof(int32_t) * 4);
  p->off_hist = take(sizeof(int32_t) * p->nchunks * buckets);
  p->bytes = o;
  return QMOE_OK;
}

int64_t numel(const qmoe_tensor* t) {
  int64_t n = 1;
  for (int i = 0; i < t->rank; ++i) n *= t->dims[i];
  return n;
}

}  // namespace

extern "C" {

qmoe_status qmoe_grouped_matmul_workspace_size(const qmoe_tensor* input, const qmoe_tensor* weights,
                                               const qmoe_tensor* group_indices, const qmoe_tensor* bias,
                                               const qmoe_tensor* output, size_t* bytes) {
  if (!bytes) return QMOE_ERR_NULL;
  GmmPlan p;
  const qmoe_status st = check(input, weights, group_indices, bias, output, &p);
  if (st != QMOE_OK) return st;
  *bytes = p.bytes;
  return QMOE_OK;
}

}  // extern "C"

namespace {

qmoe_status gmm_impl(const qmoe_tensor* input, const qmoe_tensor* weights, const qmoe_tensor* group_indices,
                     const qmoe_tensor* bias, const qmoe_tensor* output, void* workspace, size_t workspace_bytes,
                     void* stream, void* const* events) {
  if (!output) return QMOE_ERR_NULL;
  GmmPlan p;
  const qmoe_status st = check(input, weights, group_indices, bias, output, &p);
  if (st != QMOE_OK) return st;
  if (p.R == 0 || p.N == 0) return QMOE_OK;
  const qmoe_tensor* all[] = {input, weights, group_indices, bias, output};
  for (const qmoe_tensor* t : all)
    if (t && numel(t) > 0 && t->data == nullptr) return QMOE_ERR_NULL;
  const uintptr_t es = p.dtype == QMOE_F64 ? 8 : p.dtype == QMOE_F32 ? 4 : 2;  // element size
  for (const qmoe_tensor* t : {input, weights, bias, output})
    if (t && !aligned_to(t->data, es)) return QMOE_ERR_ALIGN;
  if (!aligned_to(group_indices->data, p.idx64 ? 8 : 4)) return QMOE_ERR_ALIGN;
  if (workspace == nullptr) return QMOE_ERR_NULL;
  if (workspace_bytes < p.bytes) return QMOE_ERR_WORKSPACE;
  if (!aligned_to(workspace, 256)) return QMOE_ERR_ALIGN;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  int* idx = reinterpret_cast<int*>(ws + p.off_idx);
  int* counts = reinterpret_cast<int*>(ws + p.off_counts);
  int* offsets = reinterpret_cast<int*>(ws + p.off_offsets);
  int* perm = reinterpret_cast<int*>(ws + p.off_perm);
  int* tiles = reinterpret_cast<int*>(ws + p.off_tiles);
  int* ntiles = reinterpret_cast<int*>(ws + p.off_ntiles);
  int* hist = reinterpret_cast<int*>(ws + p.off_hist);
  const int R = (int)p.R, G = (int)p.G;
  auto mark = [&](int i) -> hipError_t {
    if (events && events[i]) return hipEventRecord(reinterpret_cast<hipEvent_t>(events[i]), s);
    return hipSuccess;
  };
  // float16 / bfloat16 on the register-transposed tile kernel (16-byte
  // aligned input, weights and output, K and N multiples of 8, not the
  // 16-row streaming kernel) may take 128-row tiles: fewer tiles than the
  // workspace's table was sized for
  const bool tvec = (p.K * (int64_t)es) % 16 == 0 && (p.N * (int64_t)es) % 16 == 0 &&
                    aligned_to(input->data, 16) && aligned_to(weights->data, 16);
  const uintptr_t sal = p.dtype == QMOE_F64 ? 16 : 8;  // the streaming kernels' access width
  const bool tstream16 = p.dtype != QMOE_F32 && p.rows16 && aligned_to(input->data, sal) &&
                         aligned_to(weights->data, sal) && aligned_to(output->data, sal) &&
                         (!bias || aligned_to(bias->data, sal));
  const int64_t spread = std::max<int64_t>(1, std::min<int64_t>(p.G, p.R));  // groups in use, at most
  int bm = (int)p.bm;
  int64_t max_tiles = p.max_tiles;
  if ((p.dtype == QMOE_F16 || p.dtype == QMOE_BF16) && tvec && aligned_to(output->data, 16) && !tstream16) {
    bm = gmm16_tile_rows((long)p.R, (long)spread);
    max_tiles = (p.R + bm - 1) / bm + p.G + 1;
  }
  if (mark(0) != hipSuccess) return QMOE_ERR_HIP;
  if (launch_gmm_index(group_indices->data, p.idx64, R, G, idx, s) != hipSuccess) return QMOE_ERR_HIP;
  if (launch_permute(idx, R, G + 1, (int)kChunk, (int)p.nchunks, bm, hist, counts, offsets, perm, tiles,
                     ntiles, s) != hipSuccess)
    return QMOE_ERR_HIP;
  if (mark(1) != hipSuccess) return QMOE_ERR_HIP;
  if (p.dtype != QMOE_F32) {
    TypedGemm tg{};
    tg.a = input->data;
    tg.a_perm = perm;  // slot id m * S + i -> token row m
    tg.a_div = (int)p.S;
    tg.w = weights->data;
    tg.bias = bias ? bias->data : nullptr;
    tg.perm = perm;    // output row m * S + i of [M, S, N]
    tg.tiles = tiles;
    tg.ntiles = ntiles;
    tg.K = (int)p.K;
    tg.N = (int)p.N;
    tg.G = G;
    tg.out = const_cast<void*>(output->data);
    const int ty = p.dtype == QMOE_F16 ? GMM_F16 : p.dtype == QMOE_BF16 ? GMM_BF16 : GMM_F64;
    // 16-row tiles stream the weights when every pointer allows 8-byte
    // (16-bit types) or 16-byte (double) accesses (else the tile kernel takes
    // them: its tiles hold up to 64 rows)
    hipError_t e;
    if (!tstream16) e = launch_gmm_typed(ty, tg, tvec, (int)max_tiles, s, bm);
    else if (p.dtype == QMOE_F64) e = launch_gmm64_rows16(tg, (long)spread, (int)max_tiles, s);
    else if (p.K % 8 == 0 && p.N % 8 == 0 && aligned_to(input->data, 16) && aligned_to(weights->data, 16) &&
             aligned_to(output->data, 16) && (!bias || aligned_to(bias->data, 16)))
      e = launch_gmm16_stream(ty, tg, (long)spread, (int)max_tiles, s);  // 16-byte accesses
    else e = launch_gmm16_rows16(ty, tg, gmm_rows16_ksplit(spread, tg.N), (int)max_tiles, s);
    if (e != hipSuccess) return QMOE_ERR_HIP;
    if (mark(2) != hipSuccess) return QMOE_ERR_HIP;
    return QMOE_OK;
  }
  const bool vec = p.K % 4 == 0 && p.N % 4 == 0 && aligned_to(input->data, 16) && aligned_to(weights->data, 16);
  const bool stream16 = p.rows16 && vec && aligned_to(output->data, 16) && (!bias || aligned_to(bias->data, 16));
  F32Gemm g{};
  g.a = static_cast<const float*>(input->data);
  g.a_perm = perm;  // slot id m * S + i -> token row m
  g.a_div = (int)p.S;
  g.w = static_cast<const float*>(weights->data);
  g.bias = bias ? static_cast<const float*>(bias->data) : nullptr;
  g.perm = perm;
  g.out_by_slot = 1;  // output row m * S + i of [M, S, N]
  g.tiles = tiles;
  g.ntiles = ntiles;
  g.K = (int)p.K;
  g.N = (int)p.N;
  g.G = G;
  g.out = static_cast<float*>(const_cast<void*>(output->data));
  const long est_tiles = std::max<int64_t>(1, std::min<int64_t>(p.G, p.R));  // groups in use, at most
  const hipError_t e = stream16 ? launch_gmm_rows16(g, false, gmm_rows16_ksplit(est_tiles, g.N), (int)p.max_tiles, s)
                                : launch_gmm_f32(g, false, vec, (int)p.max_tiles, s);
  if (e != hipSuccess) return QMOE_ERR_HIP;
  if (mark(2) != hipSuccess) return QMOE_ERR_HIP;
  return QMOE_OK;
}

}  // namespace

extern "C" {

qmoe_status qmoe_grouped_matmul(const qmoe_tensor* input, const qmoe_tensor* weights,
                                const qmoe_tensor* group_indices, const qmoe_tensor* bias,
                                const qmoe_tensor* output, void* workspace, size_t workspace_bytes, void* stream) {
  return gmm_impl(input, weights, group_indices, bias, output, workspace, workspace_bytes, stream, nullptr);
}

qmoe_status qmoe_grouped_matmul_debug(const qmoe_tensor* input, const qmoe_tensor* weights,
                                      const qmoe_tensor* group_indices, const qmoe_tensor* bias,
                                      const qmoe_tensor* output, void* workspace, size_t workspace_bytes,
                                      void* stream, void* const events[QMOE_GMM_EVENTS]) {
  return gmm_impl(input, weights, group_indices, bias, output, workspace, workspace_bytes, stream, events);
}

}  // extern "C"
