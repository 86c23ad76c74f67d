/*
 * qmoe.h -- C ABI of the QMoE routed expert FFN for AMD Instinct gfx950.
 *
 * The operator (QMoE WebGPU manifest: description, inputs, outputs,
 * attributes) takes float32 token activations x [T, H] (or [B, S, H]),
 * float32 router logits [T, E], raw uint8-packed FC1/FC2 expert weights with
 * float32 scales, and returns float32 output of x's shape:
 *
 *   sel[t]    = indices of the k largest logits of row t, largest first,
 *               equal logits ordered by ascending expert index
 *   w[t, s]   = softmax over the k selected logits           (QMoE routing)
 *             | softmax over all E logits taken at sel[t, s],
 *               renormalised iff normalize_routing_weights   (MoE routing)
 *   W[e]      = (q - mid) * scale, mid = 8 (4-bit) / 128 (8-bit);
 *               4-bit bytes hold the even code in the low nibble
 *   h         = x[t] . W1[e]^T                (FC1, rows = fusion * I)
 *   a         = relu(h)  |  g * sigmoid(alpha * g) * (u + beta),
 *               g = h[2j], u = h[2j+1]        (interleaved SwiGLU; with
 *               swiglu_limit L: g <- min(g, L), u <- clamp(u, -L, L))
 *   out[t]    = sum_s w[t, s] * (a . W2[sel[t, s]]^T)
 *
 * FC1 and FC2 are each a GroupedMatMul (ONNX GroupedMatMul-29, Summary) over
 * dequantised weights.
 *
 * Conventions shared by every entry point:
 *  - Tensors are described by qmoe_tensor: a pointer, a dtype code, a rank and
 *    up to three dims, row-major and contiguous.  For qmoe_validate and
 *    qmoe_workspace_size the pointers are not dereferenced; for qmoe_forward
 *    they are DEVICE pointers on the current HIP device.
 *  - The caller owns every buffer.  The library allocates nothing, never
 *    synchronises, and enqueues all work on the caller's stream.
 *  - A status from the contract checks (QMOE_ERR_NULL, _SHAPE, _ATTR,
 *    _UNSUPPORTED, _WORKSPACE, _DTYPE, _ALIGN) means nothing was enqueued and
 *    the output is untouched: every check runs before the first launch.
 *    QMOE_ERR_HIP reports a HIP call that failed while enqueueing (a launch,
 *    or a kernel's one-time opt-in to more than 64 KB of LDS): kernels
 *    enqueued before it stay enqueued, and the output and workspace contents
 *    are then unspecified.  On QMOE_OK every output element is written by
 *    work enqueued on stream.
 *  - Every finite input is in contract.  The matrix cores take f16 operands:
 *    each fp32 operand row (a row of x for FC1, of the activation for FC2) is
 *    multiplied by a power of two of its own, chosen so that its largest
 *    magnitude lands in [2^13, 2^14), and split into f16 hi + lo; each row's
 *    fp32 result is scaled back exactly.  An element is so carried to 2^-22
 *    of itself plus 2^-39 of its row's largest magnitude, for rows of any
 *    magnitude (GPU parity is tested on inputs scaled from 1e-7 to 1e5 and on
 *    rows twelve orders of magnitude apart).  Between the LDS-tiled GEMMs the
 *    activation rows are scaled instead by one power of two per 128-row tile
 *    and FC1 column tile (a 128- or 256-code segment of FC2's reduction):
 *    an element is then carried to 2^-22 of itself plus 2^-26 of its row's
 *    largest magnitude in the segment; a row more than 2^12 below its tile
 *    (or any row of values from 2^113 on) falls back to the per-row scaling
 *    above for the whole call.  NaN/inf in x or logits are out
 *    of contract and produce unspecified (but bounded-time) results; results
 *    beyond the float32 range are infinite.
 *  - Entry points keep no state between calls (the only process-wide
 *    record is which kernels were already granted more than 64 KB of LDS, set
 *    once and thread-safely); calls on different streams with different
 *    workspaces may overlap, and a call may be captured in a HIP graph (it
 *    enqueues kernels only: no memset or copy nodes).
 */
#ifndef QMOE_H_
#define QMOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QMOE_ABI_VERSION 3

typedef enum {
  QMOE_OK = 0,
  QMOE_ERR_NULL = 1,        /* a required pointer argument is NULL            */
  QMOE_ERR_SHAPE = 2,       /* ranks/dims violate the manifest's shape rules  */
  QMOE_ERR_ATTR = 3,        /* attribute value outside the accepted set       */
  QMOE_ERR_UNSUPPORTED = 4, /* standard value this library does not implement */
  QMOE_ERR_WORKSPACE = 5,   /* workspace smaller than qmoe_workspace_size     */
  QMOE_ERR_HIP = 6,         /* a HIP launch or device query failed            */
  QMOE_ERR_DTYPE = 7,       /* tensor dtype code differs from the contract    */
  QMOE_ERR_ALIGN = 8        /* a device pointer is not 16-byte aligned        */
} qmoe_status;

typedef enum {
  QMOE_F32 = 1,
  QMOE_U8 = 2,
  QMOE_I32 = 3,
  QMOE_I64 = 4,
  QMOE_F16 = 5,  /* GroupedMatMul only */
  QMOE_BF16 = 6, /* GroupedMatMul only */
  QMOE_F64 = 7   /* GroupedMatMul only */
} qmoe_dtype;

typedef enum {
  QMOE_ACT_RELU = 0,
  QMOE_ACT_SWIGLU = 1,
  QMOE_ACT_GELU = 2,     /* float MoE only */
  QMOE_ACT_SILU = 3,     /* float MoE only */
  QMOE_ACT_IDENTITY = 4  /* float MoE only */
} qmoe_activation;

typedef enum {
  QMOE_ROUTE_QMOE = 0, /* softmax over the k selected logits (QMoE manifest)      */
  QMOE_ROUTE_MOE = 1   /* softmax over all logits before top-k (float MoE README) */
} qmoe_routing;

typedef struct {
  const void* data;  /* device pointer for qmoe_forward; unused by validation */
  int32_t dtype;     /* qmoe_dtype */
  int32_t rank;      /* 1..3 */
  int64_t dims[3];   /* row-major extents; dims[i] for i >= rank are ignored */
} qmoe_tensor;

/* Attributes of the QMoE manifest (key "attributes"), defaults in brackets. */
typedef struct {
  int32_t k;                         /* [1]  experts per token, 1 <= k <= E      */
  int32_t expert_weight_bits;        /* [4]  4 or 8                               */
  int32_t block_size;                /* [0]  0 = column-wise scales; else a power
                                             of two >= 16 dividing H and I        */
  int32_t activation_type;           /* [RELU] qmoe_activation                    */
  int32_t swiglu_fusion;             /* [0]  0 with relu, 1 with swiglu; 2 is
                                             QMOE_ERR_UNSUPPORTED                 */
  float activation_alpha;            /* [1]  SwiGLU gate sigmoid slope            */
  float activation_beta;             /* [0]  added to the SwiGLU linear branch    */
  int32_t normalize_routing_weights; /* [0]  0 or 1; only the MoE routing mode
                                             reads it                             */
  int32_t routing;                   /* [QMOE_ROUTE_QMOE] qmoe_routing            */
  int32_t use_sparse_mixer;          /* [0]  1 is QMOE_ERR_UNSUPPORTED            */
  int32_t weights_prepacked;         /* [-1] -1 or 0; 1 is QMOE_ERR_UNSUPPORTED   */
  int32_t quant_type;                /* [0]  0 = "int"; others UNSUPPORTED        */
  int32_t has_swiglu_limit;          /* [0]  1: swiglu_limit is given              */
  float swiglu_limit;                /* [-]  SwiGLU clamp L > 0 (manifest
                                             attributeDescriptions.swiglu_limit,
                                             constants.hasSwigluLimit): the gate is
                                             bounded above by L and the linear
                                             branch to [-L, L] before the formula
                                             (a reading: no formula on the pages);
                                             read by SwiGLU only                  */
  int32_t first_expert;              /* [0]  the weights' expert 0 is global
                                             expert first_expert of the router's
                                             E: the weights (and scales) hold
                                             E_local = fc1 dims[0] consecutive
                                             experts, 0 <= first_expert and
                                             first_expert + E_local <= E
                                             (QMOE_ERR_ATTR otherwise).  Routing
                                             still ranks all E logits; slots
                                             whose expert is not held contribute
                                             nothing, so the output is this
                                             share's part of the sum over slots
                                             (one GPU's share when the experts
                                             are spread over GPUs; the pages
                                             define no such split).  E_local ==
                                             E with first_expert 0 is the whole
                                             operator; E_local == 0 gives zeros. */
} qmoe_attrs;

/* Stage boundaries at which qmoe_forward_debug records events. */
#define QMOE_STAGE_EVENTS 6

/* Optional outputs for parity checks and timing.  Any field may be NULL.
 * Device buffers: topk_idx, topk_w [T*k] (row t, slot s at t*k+s; global
 * expert indices); counts [E_local]; offsets [E_local+1]; perm [T*k] (slot id
 * t*k+s at each expert-sorted position, stable within an expert; with
 * E_local < E the slots of experts not held follow those of the held ones,
 * in slot order, from offsets[E_local] on).
 * events: caller-created hipEvent_t handles recorded on the stream at
 *   [0] before the router, [1] after the routing front end (router,
 *   permutation, FC1 operand rows), [2] after the FC1 GEMM, [3] after the
 *   FC2 operand rows (the FC1 activation pass where FC1 writes split
 *   partials, the operand split where FC2 takes hi/lo rows), [4] after the
 *   FC2 GEMM, [5] after the combine (before any debug copy).  Events are
 *   only recorded when T > 0, I > 0 and E_local > 0. */
typedef struct {
  int32_t* topk_idx;
  float* topk_w;
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm;
  void* events[QMOE_STAGE_EVENTS];
} qmoe_debug;

/* Library ABI version (QMOE_ABI_VERSION of the build). */
int32_t qmoe_abi_version(void);

/* Fill *a with the manifest defaults listed above.  a must not be NULL. */
void qmoe_attrs_default(qmoe_attrs* a);

/* Check shapes, dtypes and attributes against the manifest's derive rules
 * (quantContract: activationSupported, routingModeSupported, rawWeightLayout,
 * quantShapeOk with quantBlockSizeOk and quantScalesOk, 1 <= k <= E).  Pure
 * host code; never touches a device.  output may describe the output tensor
 * (must equal input's shape) or be NULL to skip that check. */
qmoe_status qmoe_validate(const qmoe_tensor* input, const qmoe_tensor* router_probs,
                          const qmoe_tensor* fc1_experts_weights, const qmoe_tensor* fc1_scales,
                          const qmoe_tensor* fc2_experts_weights, const qmoe_tensor* fc2_scales,
                          const qmoe_tensor* output, const qmoe_attrs* attrs);

/* Bytes of device workspace qmoe_forward needs for these shapes (validates
 * first).  *bytes receives the size; it is 0 when T == 0.  With I == 0 only
 * the (small) routing part is needed.  The size depends on the kernel plan,
 * which environment variables can change (QMOE_STREAM_SINGLE_STAGE_MAX_SPLITS:
 * most K ranges of a single-stage streaming GEMM, default 16;
 * QMOE_TILED_KSPLIT: K ranges of the LDS-tiled FC2, 1, 2 or 4, each adding
 * one set of S x H fp32 partial rows): query the size under the same
 * environment as the forward call. */
qmoe_status qmoe_workspace_size(const qmoe_tensor* input, const qmoe_tensor* router_probs,
                                const qmoe_tensor* fc1_experts_weights, const qmoe_tensor* fc1_scales,
                                const qmoe_tensor* fc2_experts_weights, const qmoe_tensor* fc2_scales,
                                const qmoe_attrs* attrs, size_t* bytes);

/* The launch plan qmoe_forward takes for these shapes and attributes, as one
 * line of text (validates first; pure host code): the kernel of each GEMM
 * (fc1=, fc2= stream | tiled | gemm | none), the routing front end, the
 * M-tile height and count, whether the weights hold a share of the experts,
 * the streaming split of each GEMM (single-stage:items per stage:stages per
 * K range:K ranges:rows per workgroup), for the LDS-tiled GEMMs the segment
 * scales per operand row (segments=), half tiles (half_tiles=) and FC2's K
 * ranges (fc2_ranges=), and the workspace bytes.  The plan
 * depends on the environment as qmoe_workspace_size says.  At most len
 * bytes are written to buf, NUL-terminated; NULL buf or len 0 is
 * QMOE_ERR_NULL. */
qmoe_status qmoe_plan_describe(const qmoe_tensor* input, const qmoe_tensor* router_probs,
                               const qmoe_tensor* fc1_experts_weights, const qmoe_tensor* fc1_scales,
                               const qmoe_tensor* fc2_experts_weights, const qmoe_tensor* fc2_scales,
                               const qmoe_attrs* attrs, char* buf, size_t len);

/* Enqueue the whole operator on stream (a hipStream_t; NULL = the null
 * stream).  Device pointers: router_probs 4-byte aligned; input, weights,
 * scales and output 16-byte aligned (QMOE_ERR_ALIGN otherwise).
 * workspace: device memory of at least qmoe_workspace_size bytes, 256-byte
 * aligned, exclusively owned by this call until the stream reaches it.  The
 * output must not alias any input. */
qmoe_status qmoe_forward(const qmoe_tensor* input, const qmoe_tensor* router_probs,
                         const qmoe_tensor* fc1_experts_weights, const qmoe_tensor* fc1_scales,
                         const qmoe_tensor* fc2_experts_weights, const qmoe_tensor* fc2_scales,
                         const qmoe_attrs* attrs, const qmoe_tensor* output,
                         void* workspace, size_t workspace_bytes, void* stream);

/* As qmoe_forward, and also copies the routing stages' results to the
 * non-NULL device buffers of *debug (debug may be NULL). */
qmoe_status qmoe_forward_debug(const qmoe_tensor* input, const qmoe_tensor* router_probs,
                               const qmoe_tensor* fc1_experts_weights, const qmoe_tensor* fc1_scales,
                               const qmoe_tensor* fc2_experts_weights, const qmoe_tensor* fc2_scales,
                               const qmoe_attrs* attrs, const qmoe_tensor* output,
                               void* workspace, size_t workspace_bytes, void* stream,
                               const qmoe_debug* debug);

/* For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): qmoe_forward without a
 * workspace argument.  Its intermediates live in a scratch array inside the
 * library, one per GPU (qmoe_noalloc_scratch_bytes() bytes, 32 MiB: enough
 * for up to about 16 decode tokens of an 8-expert hidden-4096 /
 * inter-14336 layer), held from the first call on a GPU until the process
 * ends.  Calls whose qmoe_workspace_size exceeds it return
 * QMOE_ERR_WORKSPACE before anything is enqueued; the call allocates
 * nothing (no hipMalloc, hipFree or allocating library routine).
 * The stream must belong to the current HIP device (whose array is used);
 * the first call on a device looks the array's address up (a host-side
 * query, QMOE_ERR_HIP if it fails), so make one call outside graph capture
 * first.  Every call on a GPU shares that GPU's array, which keeps the last
 * call's contents (nothing in it needs to start at zero): calls that
 * overlap on one GPU (other streams, or host threads) race and must be
 * ordered by the caller.  Otherwise as qmoe_forward. */
size_t qmoe_noalloc_scratch_bytes(void);
qmoe_status qmoe_forward_noalloc(const qmoe_tensor* input, const qmoe_tensor* router_probs,
                                 const qmoe_tensor* fc1_experts_weights, const qmoe_tensor* fc1_scales,
                                 const qmoe_tensor* fc2_experts_weights, const qmoe_tensor* fc2_scales,
                                 const qmoe_attrs* attrs, const qmoe_tensor* output, void* stream);

/* ------------------------------------------------------------------------
 * GroupedMatMul (ONNX operator page "GroupedMatMul - 29": Summary, Inputs,
 * Outputs, Type Constraints), in each floating type T of the page's list:
 *
 *   output[m, i, :] = input[m, :] @ weights[g, :, :]  (+ bias[g, :])
 *   g = group_indices[m, i]
 *
 * input [M, K], weights [G, K, N], group_indices [M, S] (int32 or int64),
 * optional bias [G, N] (NULL = no bias), output [M, S, N].  input, weights,
 * bias and output share one type T: QMOE_F32, QMOE_F16, QMOE_BF16 or
 * QMOE_F64 (any other code, or a mix, is QMOE_ERR_DTYPE); group_indices is
 * QMOE_I32 or QMOE_I64 (else QMOE_ERR_DTYPE).  Ranks or extents that
 * disagree: QMOE_ERR_SHAPE.
 * Limits (QMOE_ERR_UNSUPPORTED beyond them): G <= 1023, M * S < 2^30,
 * K < 2^30, N < 2^30, and (ceil(M * S / B) + G + 1) * ceil(N / 128)
 * < 2^31, B = 16 for float32 when M * S <= 16 min(G, M * S) and K, N are
 * multiples of 4 (weight-streaming kernel over 16-row tiles), else 64
 * (LDS-tiled kernels over 64-row, 128-column tiles); one workgroup per tile
 * and column block.
 *
 * Indices outside [0, G) are invalid input, for which the page defines no
 * result; this library writes zeros to those output rows and reads no weight
 * or bias for them (negative values do not count back from G).
 *
 * Arithmetic per type:
 *  - float32: products and sums float32; the matrix cores
 *    (v_mfma_f32_16x16x4_f32) add four K terms per instruction into a
 *    float32 accumulator, in K order from 0; the bias is added last;
 *  - float16, bfloat16: exact products of the 16-bit operands summed in a
 *    float32 accumulator (v_mfma_f32_16x16x32_f16 / _bf16, 32 K terms an
 *    instruction, in K order), the bias added in float32, the result
 *    rounded once to T (to nearest, ties to even);
 *  - double: float64 products and sums (v_mfma_f64_16x16x4_f64), bias last.
 * Conventions (ownership, streams, status, no allocation) as above.
 * ------------------------------------------------------------------------ */

/* Bytes of device workspace qmoe_grouped_matmul needs (validates first;
 * output may be NULL to skip its check).  0 when M * S * N == 0. */
qmoe_status qmoe_grouped_matmul_workspace_size(const qmoe_tensor* input, const qmoe_tensor* weights,
                                               const qmoe_tensor* group_indices, const qmoe_tensor* bias,
                                               const qmoe_tensor* output, size_t* bytes);

/* Enqueue GroupedMatMul on stream (a hipStream_t; NULL = the null stream).
 * Device pointers: float tensors aligned to their element size,
 * group_indices to its element size (QMOE_ERR_ALIGN otherwise); 16-byte
 * aligned input and weights whose rows are whole 16-byte runs (K and N
 * multiples of 16 / sizeof(T)) take the vector-load path, and the float32
 * weight-streaming kernel also needs 16-byte aligned bias and output.  workspace: at least
 * qmoe_grouped_matmul_workspace_size bytes, 256-byte aligned, owned by this
 * call until the stream reaches it.  The output must not alias an input.
 * With M * S * N == 0 nothing is enqueued. */
qmoe_status qmoe_grouped_matmul(const qmoe_tensor* input, const qmoe_tensor* weights,
                                const qmoe_tensor* group_indices, const qmoe_tensor* bias,
                                const qmoe_tensor* output, void* workspace, size_t workspace_bytes, void* stream);

/* Stage boundaries at which qmoe_grouped_matmul_debug records events. */
#define QMOE_GMM_EVENTS 3

/* As qmoe_grouped_matmul, and also records the caller-created hipEvent_t
 * handles of events (each may be NULL) on the stream: [0] before the index
 * conversion, [1] after the group permutation, [2] after the tile GEMM.
 * Nothing is recorded when M * S * N == 0. */
qmoe_status qmoe_grouped_matmul_debug(const qmoe_tensor* input, const qmoe_tensor* weights,
                                      const qmoe_tensor* group_indices, const qmoe_tensor* bias,
                                      const qmoe_tensor* output, void* workspace, size_t workspace_bytes,
                                      void* stream, void* const events[QMOE_GMM_EVENTS]);

/* ------------------------------------------------------------------------
 * Float MoE (com.microsoft.MoE README: Description, Inputs, Outputs,
 * Attributes), float32 throughout:
 *
 *   p         = softmax over all E logits of token t
 *   sel[t]    = the k largest logits, largest first, ties to the lower index
 *   w[t, s]   = p[sel[t, s]], renormalised over the k when
 *               normalize_routing_weights = 1
 *   h         = W1[e] x[t] + b1[e]        fc1 [E, F, H], bias [E, F]
 *   u3        = W3[e] x[t] + b3[e]        fc3 [E, I, H], bias [E, I]
 *   a         = relu(h) | h Phi(h) (exact GELU) | h sigmoid(h) [* u3] |
 *               g sigmoid(alpha g) (u + beta) | h
 *   y         = W2[e] a + b2[e]            fc2 [E, H, I], bias [E, H]
 *   out[t]    = sum_s w[t, s] y(sel[t, s])
 *
 * SwiGLU operands: swiglu_fusion 0: g = h, u = u3 (fc3 required);
 * 1: g = h[2j], u = h[2j+1]; 2: g = h[j], u = h[I + j].  F = 2 I for
 * swiglu with fusion 1 or 2, else F = I.  FC3 is read by swiglu with
 * fusion 0 and (optionally) by silu, where it multiplies the result; other
 * activations ignore it.  alpha and beta are read by swiglu only.
 *
 * Tensors: input [T, H] or [B, S, H]; router_probs [T, E]; output of
 * input's shape; every tensor QMOE_F32 (else QMOE_ERR_DTYPE).  Biases and
 * fc3 may be NULL; fc3_b needs fc3.  Limits (QMOE_ERR_UNSUPPORTED): E <=
 * 1024, T * k < 2^30, F, H < 2^30.  Products and sums are float32 on the
 * matrix cores (v_mfma_f32_16x16x4_f32); activations use float32 libm.
 * Conventions as above; the output must not alias an input.
 * ------------------------------------------------------------------------ */

/* Attributes of the MoE README (Attributes table), defaults in brackets. */
typedef struct {
  int32_t k;                         /* [1]  1 <= k <= E                      */
  int32_t activation_type;           /* [RELU] any qmoe_activation            */
  int32_t swiglu_fusion;             /* [0]  0, 1 or 2                        */
  float activation_alpha;            /* [1]  swiglu gate sigmoid slope         */
  float activation_beta;             /* [0]  added to the swiglu linear branch */
  int32_t normalize_routing_weights; /* [0]  0 or 1                           */
  int32_t use_sparse_mixer;          /* [0]  1 is QMOE_ERR_UNSUPPORTED        */
  int32_t has_swiglu_limit;          /* [0]  1: swiglu_limit is given          */
  float swiglu_limit;                /* [-]  SwiGLU clamp L > 0 (README
                                             Attributes), as for QMoE          */
} qmoe_moe_attrs;

/* Fill *a with the defaults listed above.  a must not be NULL. */
void qmoe_moe_attrs_default(qmoe_moe_attrs* a);

/* Contract check of the tables above (shapes, dtypes, attributes: ranks or
 * extents QMOE_ERR_SHAPE, attribute values QMOE_ERR_ATTR).  Pure host code.
 * output may be NULL to skip its check. */
qmoe_status qmoe_moe_validate(const qmoe_tensor* input, const qmoe_tensor* router_probs,
                              const qmoe_tensor* fc1_experts_weights, const qmoe_tensor* fc1_experts_bias,
                              const qmoe_tensor* fc2_experts_weights, const qmoe_tensor* fc2_experts_bias,
                              const qmoe_tensor* fc3_experts_weights, const qmoe_tensor* fc3_experts_bias,
                              const qmoe_tensor* output, const qmoe_moe_attrs* attrs);

/* Device workspace bytes of qmoe_moe_forward (validates first; 0 when
 * T * H == 0). */
qmoe_status qmoe_moe_workspace_size(const qmoe_tensor* input, const qmoe_tensor* router_probs,
                                    const qmoe_tensor* fc1_experts_weights, const qmoe_tensor* fc1_experts_bias,
                                    const qmoe_tensor* fc2_experts_weights, const qmoe_tensor* fc2_experts_bias,
                                    const qmoe_tensor* fc3_experts_weights, const qmoe_tensor* fc3_experts_bias,
                                    const qmoe_moe_attrs* attrs, size_t* bytes);

/* Enqueue the float MoE on stream.  Device pointers: input, output and the
 * weights 16-byte aligned, router_probs and biases 4-byte aligned
 * (QMOE_ERR_ALIGN otherwise).  workspace as for qmoe_forward. */
qmoe_status qmoe_moe_forward(const qmoe_tensor* input, const qmoe_tensor* router_probs,
                             const qmoe_tensor* fc1_experts_weights, const qmoe_tensor* fc1_experts_bias,
                             const qmoe_tensor* fc2_experts_weights, const qmoe_tensor* fc2_experts_bias,
                             const qmoe_tensor* fc3_experts_weights, const qmoe_tensor* fc3_experts_bias,
                             const qmoe_moe_attrs* attrs, const qmoe_tensor* output,
                             void* workspace, size_t workspace_bytes, void* stream);

/* As qmoe_moe_forward, also copying the routing results to the non-NULL
 * buffers of *debug and recording its events at [0] before the router,
 * [1] after the routing front end, [2] after FC1 (and FC3), [3] after the
 * activation, [4] after FC2, [5] after the combine (when T * H > 0). */
qmoe_status qmoe_moe_forward_debug(const qmoe_tensor* input, const qmoe_tensor* router_probs,
                                   const qmoe_tensor* fc1_experts_weights, const qmoe_tensor* fc1_experts_bias,
                                   const qmoe_tensor* fc2_experts_weights, const qmoe_tensor* fc2_experts_bias,
                                   const qmoe_tensor* fc3_experts_weights, const qmoe_tensor* fc3_experts_bias,
                                   const qmoe_moe_attrs* attrs, const qmoe_tensor* output,
                                   void* workspace, size_t workspace_bytes, void* stream,
                                   const qmoe_debug* debug);

/* Static, human-readable name of a status code. */
const char* qmoe_status_string(qmoe_status s);

#ifdef __cplusplus
}
#endif
#endif /* QMOE_H_ */
