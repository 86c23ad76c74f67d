// C ABI entry points of the QMoE library (declared in include/qmoe.h).
//
// qmoe_forward enqueues, on the caller's stream:
//   router -> permutation (histogram, scan, stable scatter) -> FC1 operand
//   rows -> FC1 + activation -> FC2 operand rows -> FC2 -> combine
// with every intermediate in the caller's workspace.  It allocates nothing and
// never synchronises.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "kernels/launch.h"
#include "qmoe.h"
#include "qmoe_plan.h"

using namespace qmoe;

namespace {

bool aligned_to(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int64_t numel(const qmoe_tensor* t) {
  int64_t n = 1;
  for (int i = 0; i < t->rank; ++i) n *= t->dims[i];
  return n;
}

#define QMOE_TRY_HIP(expr)                      \
  do {                                          \
    if ((expr) != hipSuccess) return QMOE_ERR_HIP; \
  } while (0)

qmoe_status forward_impl(const qmoe_tensor* input, const qmoe_tensor* router, const qmoe_tensor* fc1w,
                         const qmoe_tensor* fc1s, const qmoe_tensor* fc2w, const qmoe_tensor* fc2s,
                         const qmoe_attrs* attrs, const qmoe_tensor* output, void* workspace, size_t ws_bytes,
                         void* stream, const qmoe_debug* dbg) {
  if (!output) return QMOE_ERR_NULL;
  Dims d;
  qmoe_status st = validate(input, router, fc1w, fc1s, fc2w, fc2s, output, attrs, &d);
  if (st != QMOE_OK) return st;
  Plan p;
  make_plan(d, &p);
  if (d.T == 0) return QMOE_OK;

  // Required device pointers and their alignment.
  const qmoe_tensor* all[] = {input, router, fc1w, fc1s, fc2w, fc2s, output};
  for (const qmoe_tensor* t : all)
    if (numel(t) > 0 && t->data == nullptr) return QMOE_ERR_NULL;
  if (!aligned_to(input->data, 16) || !aligned_to(output->data, 16) || !aligned_to(fc1w->data, 16) ||
      !aligned_to(fc2w->data, 16) || !aligned_to(router->data, 4) || !aligned_to(fc1s->data, 16) ||
      !aligned_to(fc2s->data, 16))
    return QMOE_ERR_ALIGN;
  if (p.bytes > 0) {
    if (workspace == nullptr) return QMOE_ERR_NULL;
    if (ws_bytes < p.bytes) return QMOE_ERR_WORKSPACE;
    if (!aligned_to(workspace, 256)) return QMOE_ERR_ALIGN;
  }

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  float* out = static_cast<float*>(const_cast<void*>(output->data));
  const int T = (int)d.T, H = (int)d.H, E = (int)d.E, I = (int)d.I, k = (int)d.k, S = (int)p.S;
  const int El = (int)d.El;
  // no FFN work: I == 0 (variant quant_zero_inter of the manifest) or a
  // share that holds no expert; every output element is zero
  const bool ffn = d.I > 0 && d.El > 0;

  if (!ffn) {
    QMOE_TRY_HIP(launch_fill_zero(out, (long)d.T * d.H, s));
    if (!dbg) return QMOE_OK;
  }
  int* topk_idx = reinterpret_cast<int*>(ws + p.off_topk_idx);
  float* topk_w = reinterpret_cast<float*>(ws + p.off_topk_w);
  int* counts = reinterpret_cast<int*>(ws + p.off_counts);
  int* offsets = reinterpret_cast<int*>(ws + p.off_offsets);
  int* perm = reinterpret_cast<int*>(ws + p.off_perm);
  int* tiles = reinterpret_cast<int*>(ws + p.off_tiles);
  int* ntiles = reinterpret_cast<int*>(ws + p.off_ntiles);
  int* hist = reinterpret_cast<int*>(ws + p.off_hist);
  uint8_t* xa = ws + p.off_xa;
  uint8_t* act = ws + p.off_act;
  float* slot = reinterpret_cast<float*>(ws + p.off_slot);
  // slot ids of the tile rows, for the weight-streaming kernels
  int* trows = p.s1.on || p.s2.on ? reinterpret_cast<int*>(ws + p.off_trows) : nullptr;
  // a share of the experts: local expert of every slot (El = not held)
  int* local = p.share ? reinterpret_cast<int*>(ws + p.off_local) : nullptr;

  auto mark = [&](int i) -> hipError_t {
    if (dbg && ffn && dbg->events[i]) return hipEventRecord(reinterpret_cast<hipEvent_t>(dbg->events[i]), s);
    return hipSuccess;
  };
  QMOE_TRY_HIP(mark(0));
  if (p.small_front) {
    QMOE_TRY_HIP(launch_route_small(static_cast<const float*>(router->data), T, E, k, d.routing, d.normalize,
                                    (int)p.bm, topk_idx, topk_w, counts, offsets, perm, tiles, ntiles, trows, s,
                                    p.half_tiles));
  } else if (p.share) {
    // routing over all E logits; the permutation groups the slots by the
    // held experts, with one more group (no tiles) for the others
    QMOE_TRY_HIP(launch_router(static_cast<const float*>(router->data), T, E, k, d.routing, d.normalize, topk_idx,
                               topk_w, s));
    QMOE_TRY_HIP(launch_local_index(topk_idx, S, (int)d.first, El, local, s));
    QMOE_TRY_HIP(launch_permute(local, S, El + 1, (int)p.chunk, (int)p.nchunks, (int)p.bm, hist, counts, offsets,
                                perm, tiles, ntiles, s, El, p.half_tiles));
    if (trows) QMOE_TRY_HIP(launch_tile_rows(perm, tiles, ntiles, (int)p.max_tiles, (int)p.bm, trows, s));
  } else {
    QMOE_TRY_HIP(launch_router(static_cast<const float*>(router->data), T, E, k, d.routing, d.normalize, topk_idx,
                               topk_w, s));
    QMOE_TRY_HIP(launch_permute(topk_idx, S, E, (int)p.chunk, (int)p.nchunks, (int)p.bm, hist, counts, offsets,
                                perm, tiles, ntiles, s, -1, p.half_tiles));
    if (trows) QMOE_TRY_HIP(launch_tile_rows(perm, tiles, ntiles, (int)p.max_tiles, (int)p.bm, trows, s));
  }
  if (ffn) {
    // Operand rows of FC1.  The streaming FC1 splits the fp32 input rows
    // itself while staging them (a single-stage launch scales each row per K
    // range on its own; a double-buffered one takes each row's exponent from
    // here); the tiled and register-tiled GEMMs read hi/lo rows prepared here.
    int* exp1 = reinterpret_cast<int*>(ws + p.off_exp1);
    int* exp2 = reinterpret_cast<int*>(ws + p.off_exp2);
    const float* x = static_cast<const float*>(input->data);
    const bool a_f32 = p.s1.on;
    // segment scales between the tiled GEMMs (the flag starts each call at
    // zero: the FC1 operand split clears it)
    float* seg = reinterpret_cast<float*>(ws + p.off_seg);
    int* segrows = reinterpret_cast<int*>(ws + p.off_segrows);
    int* segflag = p.seg_n > 0 ? reinterpret_cast<int*>(ws + p.off_segflag) : nullptr;
    if (!a_f32)
      QMOE_TRY_HIP(launch_split_rows(d.bits, x, H, H, xa, 4 * (long)p.kp1, (int)p.kp1, T, exp1, s, nullptr, segflag));
    else if (!p.s1.one)
      QMOE_TRY_HIP(launch_row_exp(x, H, T, H, exp1, s));
    QMOE_TRY_HIP(mark(1));
    GemmArgs g1{};
    g1.wq = static_cast<const uint8_t*>(fc1w->data);
    g1.ws = static_cast<const float*>(fc1s->data);
    g1.a = a_f32 ? static_cast<const uint8_t*>(input->data) : xa;
    g1.a_f32 = a_f32;
    g1.a_exp = (a_f32 && p.s1.one) ? nullptr : exp1;
    g1.a_map = perm;
    g1.a_div = k;
    g1.a_stride = a_f32 ? 4 * H : 4 * p.kp1;
    g1.tiles = tiles;
    g1.ntiles = ntiles;
    g1.split_small = p.half_tiles;
    g1.trows = trows;
    g1.N = (int)d.F;
    g1.K = H;
    g1.kb = (int)(d.H / d.pack);
    g1.nblk = (int)d.nb1;
    g1.bs = (int)d.bs;
    g1.act = act;
    g1.act_stride = 4 * p.kp2;
    g1.alpha = d.alpha;
    g1.beta = d.beta;
    g1.limit = d.limit;
    g1.S = S;
    const int epi1 = d.act == QMOE_ACT_SWIGLU ? EPI_SWIGLU : EPI_RELU;
    if (p.s1.on) {
      g1.store_by_slot = 0;
      g1.nst = p.s1.nst;
      g1.act_swiglu = d.act == QMOE_ACT_SWIGLU;
      if (p.s1.splits == 1) {
        // whole of K per workgroup: the kernel applies the activation itself
        QMOE_TRY_HIP(launch_stream(d.bits, p.mt, p.s1.one, 1, p.s1.wg_rows, p.half ? p.s1.stg : 0, g1, (int)p.max_tiles, s));
        QMOE_TRY_HIP(mark(2));
      } else {
        float* part1 = reinterpret_cast<float*>(ws + p.off_part1);
        g1.act = nullptr;
        g1.slot_out = part1;
        QMOE_TRY_HIP(launch_stream(d.bits, p.mt, p.s1.one, p.s1.splits, p.s1.wg_rows, p.half ? p.s1.stg : 0, g1, (int)p.max_tiles, s));
        QMOE_TRY_HIP(mark(2));
        QMOE_TRY_HIP(launch_act(d.bits, epi1, part1, p.s1.splits, S, (int)d.F, I, (int)p.kp2, d.alpha, d.beta, d.limit, act,
                                s));
      }
    } else if (p.tiled) {
      if (p.seg_n > 0) {
        g1.seg_scale = seg;
        g1.seg_rows = segrows;
        g1.seg_flag = segflag;
        g1.seg_n = p.seg_n;
        g1.seg_shift = p.seg_shift;
      }
      QMOE_TRY_HIP(launch_tiled(d.bits, epi1, g1, (int)p.max_tiles, s));
      QMOE_TRY_HIP(mark(2));
    } else {
      QMOE_TRY_HIP(launch_gemm(d.bits, epi1, p.mt, p.aligned, g1, (int)p.max_tiles, s));
      QMOE_TRY_HIP(mark(2));
    }
    // Operand rows of FC2: FC1 left fp32 rows (stride kp2 codes), or with
    // segment scales the hi/lo rows themselves.  The streaming FC2 splits
    // fp32 rows while staging; the other GEMMs take them as hi/lo rows,
    // converted here in place.
    float* act32 = reinterpret_cast<float*>(act);
    // (a share: only the sorted positions of held experts' slots, the first
    // offsets[El], have rows)
    if (p.seg_n > 0) {
      // only when FC1 flagged a row: back to one exponent a row (exp2)
      QMOE_TRY_HIP(launch_resplit_rows(d.bits, act, 4 * (long)p.kp2, I, S, segrows, p.seg_shift, exp2, segflag, s,
                                       p.share ? offsets + El : nullptr));
    } else if (!p.s2.on)
      QMOE_TRY_HIP(launch_split_rows(d.bits, act32, p.kp2, I, act, 4 * (long)p.kp2, (int)p.kp2, S, exp2, s,
                                     p.share ? offsets + El : nullptr));
    else if (!p.s2.one)
      QMOE_TRY_HIP(launch_row_exp(act32, p.kp2, S, I, exp2, s));
    QMOE_TRY_HIP(mark(3));
    GemmArgs g2{};
    g2.wq = static_cast<const uint8_t*>(fc2w->data);
    g2.ws = static_cast<const float*>(fc2s->data);
    g2.a = act;
    g2.a_f32 = p.s2.on;
    g2.a_exp = (p.s2.on && p.s2.one) ? nullptr : exp2;
    g2.a_map = nullptr;
    g2.a_div = 1;
    g2.a_stride = 4 * p.kp2;
    g2.tiles = tiles;
    g2.ntiles = ntiles;
    g2.split_small = p.half_tiles;
    g2.trows = trows;
    g2.N = H;
    g2.K = I;
    g2.kb = (int)(d.I / d.pack);
    g2.nblk = (int)d.nb2;
    g2.bs = (int)d.bs;
    g2.slot_out = slot;
    g2.limit = __builtin_inff();  // no activation in FC2
    g2.perm = perm;
    g2.S = S;
    g2.store_by_slot = 1;  // FC2 rows go to their slot id
    if (p.s2.on) {
      g2.nst = p.s2.nst;
      QMOE_TRY_HIP(launch_stream(d.bits, p.mt, p.s2.one, p.s2.splits, p.s2.wg_rows, p.half ? p.s2.stg : 0, g2, (int)p.max_tiles, s));
    } else if (p.tiled) {
      if (p.seg_n > 0) {
        // segment factors, or (when FC1 flagged a row) the per-row exponents
        // the re-split pass wrote
        g2.seg_scale = seg;
        g2.seg_flag = segflag;
        g2.seg_n = p.seg_n;
        g2.seg_shift = p.seg_shift;
      }
      g2.ksplit = p.ksplit2;  // K ranges: partial sets the combine sums
      QMOE_TRY_HIP(launch_tiled(d.bits, EPI_STORE, g2, (int)p.max_tiles, s));
    } else {
      QMOE_TRY_HIP(launch_gemm(d.bits, EPI_STORE, p.mt, p.aligned, g2, (int)p.max_tiles, s));
    }
    QMOE_TRY_HIP(mark(4));
    QMOE_TRY_HIP(launch_combine(slot, topk_w, T, k, H, p.splits2, out, s, local, El));
    QMOE_TRY_HIP(mark(5));
  }
  if (dbg) {
    if (dbg->topk_idx) QMOE_TRY_HIP(launch_copy_i32(topk_idx, dbg->topk_idx, S, s));
    if (dbg->topk_w) QMOE_TRY_HIP(launch_copy_f32(topk_w, dbg->topk_w, S, s));
    if (dbg->counts) QMOE_TRY_HIP(launch_copy_i32(counts, dbg->counts, El, s));
    if (dbg->offsets) QMOE_TRY_HIP(launch_copy_i32(offsets, dbg->offsets, El + 1, s));
    if (dbg->perm) QMOE_TRY_HIP(launch_copy_i32(perm, dbg->perm, S, s));
  }
  return QMOE_OK;
}

// Scratch of qmoe_forward_noalloc: one array per GPU, held until the process
// ends.  In host code its name is a host-side stand-in; the device address
// of each GPU's copy comes from hipGetSymbolAddress (kept per device).
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of the current device's scratch array (looked up once per
// device, with that device current), or nullptr if the lookup fails.
void* scratch_of_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch[dev] = ptr;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" {

int32_t qmoe_abi_version(void) { return QMOE_ABI_VERSION; }

size_t qmoe_noalloc_scratch_bytes(void) { return kScratchBytes; }

qmoe_status qmoe_forward_noalloc(const qmoe_tensor* input, const qmoe_tensor* router_probs, const qmoe_tensor* fc1w,
                                 const qmoe_tensor* fc1s, const qmoe_tensor* fc2w, const qmoe_tensor* fc2s,
                                 const qmoe_attrs* attrs, const qmoe_tensor* output, void* stream) {
  if (!output) return QMOE_ERR_NULL;
  // the same contract and plan as qmoe_forward; sizes whose workspace
  // exceeds the scratch array are refused before anything is enqueued
  Dims d;
  const qmoe_status st = validate(input, router_probs, fc1w, fc1s, fc2w, fc2s, output, attrs, &d);
  if (st != QMOE_OK) return st;
  Plan p;
  make_plan(d, &p);
  if (p.bytes > kScratchBytes) return QMOE_ERR_WORKSPACE;
  void* ws = nullptr;
  if (p.bytes > 0) {
    ws = scratch_of_current_device();
    if (!ws) return QMOE_ERR_HIP;
  }
  return forward_impl(input, router_probs, fc1w, fc1s, fc2w, fc2s, attrs, output, ws, kScratchBytes, stream,
                      nullptr);
}

void qmoe_attrs_default(qmoe_attrs* a) {
  if (!a) return;
  a->k = 1;
  a->expert_weight_bits = 4;
  a->block_size = 0;
  a->activation_type = QMOE_ACT_RELU;
  a->swiglu_fusion = 0;
  a->activation_alpha = 1.f;
  a->activation_beta = 0.f;
  a->normalize_routing_weights = 0;
  a->routing = QMOE_ROUTE_QMOE;
  a->use_sparse_mixer = 0;
  a->weights_prepacked = -1;
  a->quant_type = 0;
  a->has_swiglu_limit = 0;
  a->swiglu_limit = 0.f;
  a->first_expert = 0;
}

qmoe_status qmoe_validate(const qmoe_tensor* input, const qmoe_tensor* router_probs, const qmoe_tensor* fc1w,
                          const qmoe_tensor* fc1s, const qmoe_tensor* fc2w, const qmoe_tensor* fc2s,
                          const qmoe_tensor* output, const qmoe_attrs* attrs) {
  Dims d;
  return validate(input, router_probs, fc1w, fc1s, fc2w, fc2s, output, attrs, &d);
}

qmoe_status qmoe_workspace_size(const qmoe_tensor* input, const qmoe_tensor* router_probs, const qmoe_tensor* fc1w,
                                const qmoe_tensor* fc1s, const qmoe_tensor* fc2w, const qmoe_tensor* fc2s,
                                const qmoe_attrs* attrs, size_t* bytes) {
  if (!bytes) return QMOE_ERR_NULL;
  Dims d;
  qmoe_status st = validate(input, router_probs, fc1w, fc1s, fc2w, fc2s, nullptr, attrs, &d);
  if (st != QMOE_OK) return st;
  Plan p;
  make_plan(d, &p);
  *bytes = p.bytes;
  return QMOE_OK;
}

qmoe_status qmoe_forward(const qmoe_tensor* input, const qmoe_tensor* router_probs, const qmoe_tensor* fc1w,
                         const qmoe_tensor* fc1s, const qmoe_tensor* fc2w, const qmoe_tensor* fc2s,
                         const qmoe_attrs* attrs, const qmoe_tensor* output, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return forward_impl(input, router_probs, fc1w, fc1s, fc2w, fc2s, attrs, output, workspace, workspace_bytes,
                      stream, nullptr);
}

qmoe_status qmoe_forward_debug(const qmoe_tensor* input, const qmoe_tensor* router_probs, const qmoe_tensor* fc1w,
                               const qmoe_tensor* fc1s, const qmoe_tensor* fc2w, const qmoe_tensor* fc2s,
                               const qmoe_attrs* attrs, const qmoe_tensor* output, void* workspace,
                               size_t workspace_bytes, void* stream, const qmoe_debug* debug) {
  return forward_impl(input, router_probs, fc1w, fc1s, fc2w, fc2s, attrs, output, workspace, workspace_bytes,
                      stream, debug);
}

qmoe_status qmoe_plan_describe(const qmoe_tensor* input, const qmoe_tensor* router_probs, const qmoe_tensor* fc1w,
                               const qmoe_tensor* fc1s, const qmoe_tensor* fc2w, const qmoe_tensor* fc2s,
                               const qmoe_attrs* attrs, char* buf, size_t len) {
  if (!buf || len == 0) return QMOE_ERR_NULL;
  Dims d;
  const qmoe_status st = validate(input, router_probs, fc1w, fc1s, fc2w, fc2s, nullptr, attrs, &d);
  if (st != QMOE_OK) return st;
  Plan p;
  make_plan(d, &p);
  auto gemm = [&](const Plan::Stream& sp) { return sp.on ? "stream" : p.tiled ? "tiled" : "gemm"; };
  const bool ffn = d.T > 0 && d.I > 0 && d.El > 0;
  std::snprintf(buf, len,
                "fc1=%s fc2=%s front=%s tile_rows=%lld max_tiles=%lld share=%d "
                "s1=%d:%d:%d:%d:%d s2=%d:%d:%d:%d:%d segments=%d half_tiles=%d fc2_ranges=%d segflag=%zu "
                "workspace=%zu",
                ffn ? gemm(p.s1) : "none", ffn ? gemm(p.s2) : "none",
                p.small_front ? "one-workgroup" : "kernels", (long long)p.bm, (long long)p.max_tiles, p.share ? 1 : 0,
                p.s1.one, p.s1.stg, p.s1.nst, p.s1.splits, p.s1.wg_rows, p.s2.one, p.s2.stg, p.s2.nst,
                p.s2.splits, p.s2.wg_rows, p.seg_n, p.half_tiles, p.ksplit2, p.off_segflag, p.bytes);
  return QMOE_OK;
}

const char* qmoe_status_string(qmoe_status s) {
  switch (s) {
    case QMOE_OK: return "ok";
    case QMOE_ERR_NULL: return "null pointer";
    case QMOE_ERR_SHAPE: return "shape violates the operator contract";
    case QMOE_ERR_ATTR: return "attribute value outside the accepted set";
    case QMOE_ERR_UNSUPPORTED: return "standard value not implemented by this library";
    case QMOE_ERR_WORKSPACE: return "workspace too small";
    case QMOE_ERR_HIP: return "HIP launch failed";
    case QMOE_ERR_DTYPE: return "tensor dtype differs from the contract";
    case QMOE_ERR_ALIGN: return "pointer misaligned";
  }
  return "unknown status";
}

}  // extern "C"
