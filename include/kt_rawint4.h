/*
 * kt_rawint4.h: C ABI of the MI355X (gfx950) RAWINT4 routed-expert LoRA layer.
 *
 * The library computes the forward and backward of the routed experts of one
 * mixture-of-experts layer whose gate/up/down projections are frozen signed
 * group-32 RAWINT4 matrices with trainable LoRA adapters.  The operation is the
 * one defined on the page "rawint4_sft_reference.py": routed_rawint4_lora
 * (forward) and run_routed_reference (its gradients with respect to the inputs,
 * the route weights and the six LoRA tensors); its calling contract follows
 * the page "test_rawint4_sft_numerical.py" (forward_sft / backward and the
 * optimizer-window rule).
 *
 * Conventions shared by every entry point:
 *   - Tensor pointers are DEVICE pointers unless stated otherwise; every tensor
 *     is dense and row-major.  bf16 values are passed as their uint16 bit
 *     patterns.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Compute entry
 *     points only enqueue work on it and return; buffers must stay alive until
 *     that work has completed.  No entry point allocates device memory.
 *   - Return codes: KT_RAWINT4_OK (0) on success; KT_RAWINT4_EINVAL for an
 *     invalid argument (nothing is enqueued); KT_RAWINT4_EWORKSPACE when the
 *     workspace is too small (nothing is enqueued); KT_RAWINT4_EHIP when the
 *     HIP runtime reports a launch error.  kt_rawint4_last_error() then returns
 *     a message (per host thread).
 *   - The library never writes weights, scales or LoRA parameters: the base is
 *     frozen by construction (there is no base-weight gradient argument).
 */
#ifndef KT_RAWINT4_H
#define KT_RAWINT4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KT_RAWINT4_OK 0
#define KT_RAWINT4_EINVAL (-1)
#define KT_RAWINT4_EWORKSPACE (-2)
#define KT_RAWINT4_EHIP (-3)

#define KT_RAWINT4_GROUP_SIZE 32
#define KT_RAWINT4_FORMAT_RAWINT4 0
#define KT_RAWINT4_FORMAT_MXFP4 1
#define KT_RAWINT4_MAX_EXPERTS 8192
#define KT_RAWINT4_MAX_RANK 128
/* bytes of the device array kt_rawint4_moe_infer_static works in (per GPU) */
#define KT_RAWINT4_STATIC_SCRATCH_BYTES (64u << 20)

/*
 * One layer.  E = num_experts, k = top_k, H = hidden, I = intermediate,
 * r = rank.  Requirements: H % 32 == 0 and I % 32 == 0 (group size 32, page
 * "rawint4_sft_reference.py", _validate_rawint4_layout), 1 <= k <= E <= 8192,
 * 1 <= r <= 128, alpha finite, swiglu_limit finite and >= 0 (0 disables the
 * clamp; page "ext_bindings.cpp" commit log, "plumb swiglu_limit").  The LoRA
 * scale is alpha / r.
 *
 * Packed weights: uint8 [E, N, K/2]; byte j of a row holds column 2j in its low
 * nibble and column 2j+1 in its high nibble; nibble c means (c - 8) times the
 * bf16 scale of its 32-column group.  Scales: bf16 bits [E, N, K/32].
 * gate and up have N = I, K = H; down has N = H, K = I.  Weight rows must be
 * 16-byte aligned (true for any base pointer aligned to 16 bytes).
 *
 * Numeric domain: the kernels multiply exact fp16 weights, which nonzero
 * scales in [2^-14, 2720] in magnitude give.  Any other finite bf16 scale is
 * handled by a power-of-two shift per expert and projection group (gate and up
 * together, down alone): the group's scales are taken times 2^-s, s the
 * smallest integer that brings the largest of them to 2720 or below, and the
 * sums are taken times 2^s again.  That is exact wherever a group's nonzero
 * scales span at most the domain's range (a factor of about 2^25).  Scales
 * that still lie outside (a group spanning more, non-finite scales) are
 * counted (see kt_rawint4_moe_diagnostics); weights decoded from them are
 * rounded to fp16 (tiny ones lose precision, non-finite ones stay so).
 *
 * weight_format = KT_RAWINT4_FORMAT_MXFP4 selects the MXFP4 base of the same
 * layer (page "ext_bindings.cpp" commit log: MXFP4_SFT_MOE, E2M1 weights with
 * a UE8M0 scale per group of 32; page "backend.py", layout
 * "mxfp4-e2m1-ue8m0-g32").  Same shapes and nibble order; nibble c is the E2M1
 * number of the OCP microscaling formats (sign bit 3, exponent bits 2..1 with
 * bias 1, mantissa bit 0: 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives)
 * times the group's scale, and the scales are the UE8M0 exponents bit-cast to
 * bf16 (e << 7, as the pages' loader converts them), i.e. powers of two.  Its
 * numeric domain: scales 0 or 2^j with -13 <= j <= 13 (UE8M0 114 .. 140), the
 * group shift above extending it to any power of two within a span of 2^26;
 * others (not a power of two, negative) are counted as above.  Everything
 * else (LoRA, clamp, gradients, window rule) is as for RAWINT4.
 *
 * LoRA tensors (fp32): gate_lora_a [E, r, H], gate_lora_b [E, I, r],
 * up_lora_a [E, r, H], up_lora_b [E, I, r], down_lora_a [E, r, I],
 * down_lora_b [E, H, r] (names and order of the page
 * "test_rawint4_sft_numerical.py", GRAD_SHAPES), each 16-byte aligned.
 */
typedef struct kt_rawint4_moe_layer {
  int32_t num_experts;
  int32_t top_k;
  int32_t hidden;
  int32_t intermediate;
  int32_t rank;
  float alpha;
  float swiglu_limit;
  const uint8_t* gate_packed;
  const uint8_t* up_packed;
  const uint8_t* down_packed;
  const uint16_t* gate_scale;
  const uint16_t* up_scale;
  const uint16_t* down_scale;
  const float* gate_lora_a;
  const float* gate_lora_b;
  const float* up_lora_a;
  const float* up_lora_b;
  const float* down_lora_a;
  const float* down_lora_b;
  int32_t weight_format; /* KT_RAWINT4_FORMAT_RAWINT4 (0, the default) or KT_RAWINT4_FORMAT_MXFP4 */
} kt_rawint4_moe_layer;

/*
 * Bytes of device workspace a forward/backward pair needs for `qlen` tokens.
 * Host-only computation; returns 0 for an invalid layer (message in
 * kt_rawint4_last_error).  The workspace is owned by the caller and must be
 * 256-byte aligned.
 */
size_t kt_rawint4_moe_workspace_bytes(const kt_rawint4_moe_layer* layer, int32_t qlen);

/*
 * Forward of the routed experts (page "rawint4_sft_reference.py",
 * routed_rawint4_lora): for every token t and slot s with e = expert_ids[t,s],
 *   g = W_g x + sc B_g A_g x,  u = W_u x + sc B_u A_u x         (x = inputs[t])
 *   h = silu(min(g, L)) * clamp(u, -L, L)    (no clamp when L = 0)
 *   y = W_d h + sc B_d A_d h
 *   output[t] = sum_s route_weights[t,s] * y
 * inputs [qlen, H] bf16, expert_ids [qlen, k] int64, route_weights [qlen, k]
 * fp32, output [qlen, H] bf16 (round to nearest even).  Expert ids outside
 * [0, E) are dropped (the slot contributes nothing) and counted.
 * The workspace keeps what the backward needs (grouping, fp32 gate/up
 * pre-activations from which the clamp masks are decided, h, LoRA-A
 * products, and the scale tensors of the experts in use converted once to
 * fp16 and transposed to [E, K/32, N]: 1/8 the size of the packed codes); a
 * later forward into the same workspace replaces it.
 * qlen == 0 is a valid no-op.
 */
int kt_rawint4_moe_fwd(const kt_rawint4_moe_layer* layer, int32_t qlen, const uint16_t* inputs,
                       const int64_t* expert_ids, const float* route_weights, uint16_t* output, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * Inference forward: the same output as kt_rawint4_moe_fwd (bit for bit, with
 * LoRA), keeping nothing for a backward (page "rawint4_sft_reference.py",
 * routed_rawint4_lora; page "test_rawint4_sft_numerical.py", the inference
 * regression, where a frozen-base inference kernel is checked against the
 * reference with zero LoRA and the base storage hash).  With all six LoRA
 * pointers NULL the layer is the frozen base alone (rank and alpha are not
 * used); otherwise every LoRA pointer must be given, as for the training
 * forward.  Arguments, alignment and errors as for kt_rawint4_moe_fwd; the
 * workspace (kt_rawint4_moe_infer_workspace_bytes, smaller: no saved
 * pre-activations, no backward buffers, no side products without LoRA) cannot
 * feed a backward.
 */
size_t kt_rawint4_moe_infer_workspace_bytes(const kt_rawint4_moe_layer* layer, int32_t qlen);
int kt_rawint4_moe_infer(const kt_rawint4_moe_layer* layer, int32_t qlen, const uint16_t* inputs,
                         const int64_t* expert_ids, const float* route_weights, uint16_t* output, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * The inference forward for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Arguments, kernels and output as kt_rawint4_moe_infer (equal to
 * it bit for bit), without a workspace: the call works in a device array of
 * KT_RAWINT4_STATIC_SCRATCH_BYTES that this library holds on each GPU it runs
 * on, from the first call there until the process ends, and allocates
 * nothing.  A call whose kt_rawint4_moe_infer_workspace_bytes exceeds that
 * size returns KT_RAWINT4_EWORKSPACE (at 384 experts, top-8, hidden 7168,
 * intermediate 2048: up to 3 tokens per call).  Every call on one GPU uses
 * the same array, which keeps the last call's contents, so calls that overlap
 * on one GPU (on other streams, from other host threads) race: order them on
 * one stream.  The call runs on the current device, records no profiling
 * events, and otherwise fails like kt_rawint4_moe_infer.
 */
int kt_rawint4_moe_infer_static(const kt_rawint4_moe_layer* layer, int32_t qlen, const uint16_t* inputs,
                                const int64_t* expert_ids, const float* route_weights, uint16_t* output,
                                void* stream);

/*
 * Backward of the same call (page "rawint4_sft_reference.py",
 * run_routed_reference: autograd with grad_output as the cotangent).  Must use
 * the workspace of the latest forward with the same layer, qlen, inputs,
 * expert_ids and route_weights: a second forward into a workspace replaces
 * what the first saved (the one pending cache of the page
 * "test_rawint4_sft_numerical.py", cache-replacement check).
 *   grad_input [qlen, H] bf16: dL/dinputs (round to nearest even);
 *   grad_route [qlen, k] fp32 or NULL: dL/droute_weights (0 for dropped slots);
 *   d_gate_a .. d_down_b: the six LoRA gradient buffers, fp32, shapes as the
 *   LoRA tensors.  Optimizer-window rule (page "test_rawint4_sft_numerical.py",
 *   the gas1/gas2/gas8 windows and the lazy clear):
 *     G = (accumulate ? G : 0) + grad_scale * dL/dLoRA
 *   for every expert row; with accumulate == 0 rows of experts absent from the
 *   call are written as 0.
 * The SwiGLU clamp gradient is boundary inclusive: the gate passes where
 * g <= L, the up projection where -L <= u <= L, decided on the fp32
 * pre-activations saved by the forward.  dX is computed transpose-free from the
 * packed [N, K] rows (page "rawint4_sft_reference.py",
 * transpose_free_rawint4_dx); no dense or transposed weight copy exists.
 * qlen == 0: only the window rule runs (zero fill when accumulate == 0).
 */
int kt_rawint4_moe_bwd(const kt_rawint4_moe_layer* layer, int32_t qlen, const uint16_t* inputs,
                       const int64_t* expert_ids, const float* route_weights, const uint16_t* grad_output,
                       uint16_t* grad_input, float* grad_route, float* d_gate_a, float* d_gate_b, float* d_up_a,
                       float* d_up_b, float* d_down_a, float* d_down_b, int32_t accumulate, float grad_scale,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward that needs no saved forward: the checkpoint-recompute form (page
 * "test_rawint4_sft_numerical.py", the cache-replacement check, where a second
 * saved forward before the backward stands for the recompute of an activation
 * checkpoint; page "ext_bindings.cpp" commit log, the checkpoint forward reuse
 * for LoRA).  It first reruns, into the workspace, the forward kernels whose
 * results the backward reads (grouping, transposed scales, LoRA side products,
 * the gate/up GEMM with its saved pre-activations, the rows of h) -- every
 * kernel but the down GEMM and the output combine -- then runs
 * kt_rawint4_moe_bwd.  All kernels are deterministic, so the results equal
 * those of kt_rawint4_moe_fwd followed by kt_rawint4_moe_bwd bit for bit.
 * The workspace (kt_rawint4_moe_workspace_bytes) may hold anything on entry:
 * a caller that keeps no activations runs the forward with kt_rawint4_moe_infer
 * and lends a training-size workspace to the backward alone.  Arguments,
 * window rule and errors as for kt_rawint4_moe_bwd.
 */
int kt_rawint4_moe_bwd_recompute(const kt_rawint4_moe_layer* layer, int32_t qlen, const uint16_t* inputs,
                                 const int64_t* expert_ids, const float* route_weights, const uint16_t* grad_output,
                                 uint16_t* grad_input, float* grad_route, float* d_gate_a, float* d_gate_b,
                                 float* d_up_a, float* d_up_b, float* d_down_a, float* d_down_b, int32_t accumulate,
                                 float grad_scale, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Test hook, the codec of page "rawint4_sft_reference.py" (unpack_rawint4):
 * packed uint8 [n, k/2] -> int8 [n, k] signed codes c - 8, low nibble first.
 * k must be even.
 */
int kt_rawint4_unpack(const uint8_t* packed, int64_t n, int64_t k, int8_t* codes, void* stream);

/*
 * Test hook, dequantize_rawint4 of the same page: packed [n, k/2] with bf16
 * scales [n, k/32] -> fp32 [n, k], (c - 8) * scale.  Runs both decoders of the
 * matrix kernels (the one of the stored orientation, whose exact fp16 values
 * are returned widened to fp32, and the one of the transposed orientation); a
 * dword where they give different values comes out as NaN.  k % 32 == 0.
 * The scales are used as given (no shift): exact for scales in the domain.
 */
int kt_rawint4_dequant(const uint8_t* packed, const uint16_t* scales, int64_t n, int64_t k, float* weights,
                       void* stream);

/*
 * Test hook, the MXFP4 twin of kt_rawint4_dequant: packed [n, k/2] E2M1 codes
 * (low nibble first) with bf16 power-of-two scales [n, k/32] -> fp32 weights
 * [n, k], through the matrix kernels' own MXFP4 decoders.  Both decoders (the
 * one of the stored orientation and the one of the transposed orientation)
 * run; a dword where they give different values comes out as NaN.
 */
int kt_rawint4_dequant_mxfp4(const uint8_t* packed, const uint16_t* scales, int64_t n, int64_t k, float* weights,
                             void* stream);

/*
 * Test hook, the token-slot grouping of the layer: offsets [E+1] int32
 * (exclusive prefix of per-expert slot counts) and sorted_slot [qlen*k] int32
 * (flat slot indices t*k+s sorted by expert, stable in slot order; entries past
 * offsets[E] are unspecified).  Ids outside [0, E) are dropped.  Needs a
 * workspace of kt_rawint4_group_workspace_bytes bytes.
 */
size_t kt_rawint4_group_workspace_bytes(int32_t qlen, int32_t top_k, int32_t num_experts);
int kt_rawint4_group(const int64_t* expert_ids, int32_t qlen, int32_t top_k, int32_t num_experts, int32_t* offsets,
                     int32_t* sorted_slot, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Synchronising read of the device-side counters of the latest forward in
 * `workspace` (written by kt_rawint4_moe_fwd or kt_rawint4_group): expert ids
 * outside [0, E) and scales outside the numeric domain that no shift of their
 * group brings in (each scale of the three projections of every expert the
 * forward routes to is checked once).
 * Host pointers out; either may be NULL.
 */
int kt_rawint4_moe_diagnostics(const void* workspace, size_t workspace_bytes, int64_t* bad_ids, int64_t* bad_scales,
                               void* stream);

/*
 * The gate and up pre-activations g = W_g x + sc B_g A_g x and
 * u = W_u x + sc B_u A_u x of every slot, as the latest forward in `workspace`
 * saved them for the backward (page "rawint4_sft_reference.py",
 * routed_rawint4_lora / rawint4_swiglu: the values the clamp masks are decided
 * on).  `layer` and `qlen` are those of that forward.  gate and up are device
 * fp32 arrays [qlen * top_k][I] in slot order (slot = token * top_k + j); a
 * dropped slot's row is zero.  Enqueued on `stream`; nothing is allocated.
 * Use: checking the masks against another computation of the layer, where a
 * value on a clamp bound to within rounding may fall either side.
 */
int kt_rawint4_moe_saved_preactivations(const kt_rawint4_moe_layer* layer, int32_t qlen, const void* workspace,
                                        size_t workspace_bytes, float* gate, float* up, void* stream);

/*
 * Per-phase timing of the layer's launches, for measurement.  While enabled,
 * every forward/backward records a hipEvent pair around each phase (grouping,
 * activation conversion, LoRA side products, each grouped GEMM, combine,
 * route-weight gradient, LoRA gradient reductions, the forward's one
 * conversion of the scales to fp16, and the passes that give h and dG|dU one
 * exponent per row) on the caller's stream.
 * kt_rawint4_profile_read waits for the recorded events, writes the summed
 * milliseconds and the number of recorded launches of each phase into
 * ms[capacity] / launches[capacity] (host arrays), clears the records and
 * returns the number of phases (or a negative error code; capacity must cover
 * every phase, 18 at present).  Phase names: kt_rawint4_profile_phase_name.
 */
int kt_rawint4_profile_enable(int32_t on);
int kt_rawint4_profile_read(float* ms, int32_t* launches, int32_t capacity);
const char* kt_rawint4_profile_phase_name(int32_t phase);

/* Message of the last failing call on this host thread ("" if none). */
const char* kt_rawint4_last_error(void);

/* "compressed-tensors-rawint4-g32-v1" (page "backend.py", RAWINT4_WEIGHT_LAYOUT). */
const char* kt_rawint4_weight_layout(void);

#ifdef __cplusplus
}
#endif

#endif /* KT_RAWINT4_H */
