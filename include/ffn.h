/*
 * ffn.h -- C ABI of libffn.so: the fused two-layer feed-forward network on one
 * AMD Instinct MI355X (gfx950), and its grouped Mixture-of-Experts form.
 *
 * Operation (the kernel-fusion / tensor-parallelism post, brunomaga.github.io,
 * section "Megatron-LM tensor parallelism", equations for H and Y):
 *
 *     H = act1(X W1 + b1)          X: M x N, W1: N x O, b1: O
 *     Y = act2(H W2 + b2)          W2: O x P, b2: P, Y: M x P
 *
 * computed for one GPU's tensor-parallel shard: O is the shard's share of the
 * hidden width.  H never goes to global memory on the bf16 path with M > 16:
 * it is produced tile by tile into LDS and consumed there by the second
 * product (same page, section "Step 1: fusing the two linear layers").  For a
 * shard's partial output in a tensor-parallel layer pass b2 = NULL and
 * act2 = NONE on every shard but one (the bias is added once, after the sum).
 *
 * Conventions for every entry point:
 *  - Memory.  All array arguments are DEVICE pointers on the current HIP
 *    device, row-major and contiguous, and must be 16-byte aligned; the
 *    workspace must be 256-byte aligned.  The caller allocates and owns every
 *    buffer, the workspace included; the library never allocates, frees or
 *    keeps a pointer after the call returns.
 *  - Workspace.  Query the size with the matching *_workspace_size call.
 *    The workspace holds only per-call intermediates (split partials, the
 *    decode shape's H, the routing tables, the decode stream's flags, which
 *    carry a number that is new for every call); it needs no initialisation
 *    and keeps nothing between calls.  Calls that share a workspace must be
 *    ordered (same stream).
 *  - Asynchrony.  Calls only enqueue work on `stream` (a hipStream_t; NULL is
 *    the default stream) and return without synchronising.
 *  - Errors.  Every argument check runs on the host before anything is
 *    enqueued.  A failed check returns a negative FFN_E* code, sets the text
 *    returned by ffn_last_error() (per host thread) and leaves every output
 *    untouched.  A failed launch returns FFN_ELAUNCH.
 *  - Shapes.  M >= 1 (M == 0 is a no-op); N, O, P >= 8 and multiples of 8;
 *    N and O below 2^24, P below 2^23 and each weight matrix below 2^30
 *    elements (the kernels use 32-bit byte offsets), else FFN_EUNSUPPORTED.
 *    Any M works
 *    (partial row tiles are handled).
 *  - Numerics.  bf16 storage, fp32 accumulation; H is rounded to bf16 once,
 *    Y once (round to nearest even).  No floating-point atomics: repeated
 *    calls with the same inputs give bitwise-identical outputs.
 *  - Aliasing.  Outputs must not overlap any input or the workspace.
 */
#ifndef FFN_MI355X_H
#define FFN_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { FFN_F32 = 0, FFN_BF16 = 1 } ffn_dtype_t;

/* act1 / act2.  GELU_TANH is 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))). */
typedef enum { FFN_ACT_NONE = 0, FFN_ACT_RELU = 1, FFN_ACT_GELU_TANH = 2 } ffn_act_t;

/* Kernel family.  AUTO picks DECODE for bf16 with M <= 16 where it applies
 * (N = P = 4096, O a multiple of 256 up to 2048, a device of 256 CUs), SKINNY
 * for other bf16 shapes with M <= 16, FUSED for other bf16 shapes and F32 for
 * fp32 data; the others force a family (tests).  The SwiGLU entry points
 * resolve AUTO by the same rule (their DECODE form streams Wg, Wu and Wd).
 * DECODE (the dense form of the tensor-parallelism post, brunomaga.github.io,
 * "Megatron-LM tensor parallelism", at decode batch sizes): one kernel
 * streams W1 and W2 together, cuts the hidden dimension into one slice per
 * XCD and passes each slice of H between the workgroups of that XCD through
 * its L2; a second kernel sums the 8 slice partials of Y.  Its 256
 * workgroups (one per CU) wait on each other, so the first kernel needs the
 * whole device at once: other kernels that hold CUs meanwhile (another
 * stream, another process) delay it, and two such calls that run at the
 * same time can hold each other's CUs.  Every wait is bounded (about a
 * second): if one expires, or the hardware deals workgroups to XCDs
 * otherwise than round-robin, every element of Y is NaN rather than wrong.
 * Order concurrent decode calls on one stream, or force FFN_VARIANT_SKINNY. */
typedef enum {
    FFN_VARIANT_AUTO = 0,
    FFN_VARIANT_FUSED = 1,   /* bf16, H in LDS, split-O partials + ordered reduce */
    FFN_VARIANT_SKINNY = 2,  /* bf16, M <= 16: two weight-streaming layers        */
    FFN_VARIANT_F32 = 3,     /* fp32 data, fp32 arithmetic                       */
    FFN_VARIANT_DECODE = 4   /* bf16, M <= 16: one streaming kernel + reduction  */
} ffn_variant_t;

enum {
    FFN_OK = 0,
    FFN_EINVAL = -1,       /* null pointer, size out of range, unknown enum      */
    FFN_EWORKSPACE = -2,   /* workspace smaller than *_workspace_size()          */
    FFN_EUNSUPPORTED = -3, /* shape or combination the kernels do not implement  */
    FFN_EALIGN = -4,       /* pointer not 16-byte (workspace: 256-byte) aligned  */
    FFN_ELAUNCH = -5       /* the HIP runtime refused a launch                   */
};

/* Workspace bytes ffn_forward needs for this shape (0 if the shape is invalid). */
size_t ffn_workspace_size(int64_t M, int64_t N, int64_t O, int64_t P, int dtype);
size_t ffn_workspace_size_ex(int64_t M, int64_t N, int64_t O, int64_t P, int dtype, int variant);

/* Y = act2(act1(X W1 + b1) W2 + b2).
 *   X  : M x N  (dtype)          W1 : N x O (dtype)     b1 : O (dtype) or NULL
 *   W2 : O x P  (dtype)          b2 : P (dtype) or NULL Y  : M x P (dtype), written
 *   dtype: ffn_dtype_t; act1, act2: ffn_act_t.
 * Returns FFN_OK or a negative FFN_E* code (see the conventions above). */
int ffn_forward(const void* X, const void* W1, const void* b1, const void* W2, const void* b2,
                void* Y, int64_t M, int64_t N, int64_t O, int64_t P, int dtype, int act1,
                int act2, void* workspace, size_t workspace_bytes, void* stream);

/* The kernel family (FFN_VARIANT_FUSED, _SKINNY, _F32 or _DECODE) that
 * ffn_forward_ex runs for this shape, dtype and variant on the current
 * device; AUTO resolves as described at ffn_variant_t.  Returns a negative
 * FFN_E* code for an invalid shape, dtype or variant; it does not check that
 * a forced family supports the shape. */
int ffn_forward_family(int64_t M, int64_t N, int64_t O, int64_t P, int dtype, int variant);

/* As ffn_forward, with the kernel family forced (FFN_VARIANT_*). */
int ffn_forward_ex(const void* X, const void* W1, const void* b1, const void* W2,
                   const void* b2, void* Y, int64_t M, int64_t N, int64_t O, int64_t P,
                   int dtype, int act1, int act2, int variant, void* workspace,
                   size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------- no allocation
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): as
 * ffn_forward_ex, with the workspace taken from a static device array of
 * FFN_NOALLOC_SCRATCH_BYTES inside the library instead of an argument.  The
 * call allocates and frees nothing.  Each device holds its own copy of the
 * array from the library's first call on it until the process ends.
 *  - A shape whose ffn_workspace_size_ex() exceeds FFN_NOALLOC_SCRATCH_BYTES
 *    is refused with FFN_EWORKSPACE before any HIP call, outputs untouched.
 *    16 MiB holds every decode-shaped call (M <= 16) up to 16 x 8192 x 3584 x
 *    8192 (14.1 MiB) and fused calls with up to 16 MiB of split partials
 *    (S*M*P*3 bytes: up to 341 rows at 4096 x 1792 x 4096).
 *  - Every call on one device shares that device's array, which keeps the
 *    last call's contents (nothing in it needs clearing between calls).
 *    Calls that overlap on one device -- on different streams, from different
 *    host threads, or from processes sharing the device context -- race on
 *    it; order them (one stream) or use ffn_forward_ex with a workspace each.
 *  - Otherwise as ffn_forward_ex: the same kernels, so the same output bits. */
#define FFN_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int ffn_forward_noalloc(const void* X, const void* W1, const void* b1, const void* W2,
                        const void* b2, void* Y, int64_t M, int64_t N, int64_t O, int64_t P,
                        int dtype, int act1, int act2, int variant, void* stream);

/* As ffn_forward_ex, and records caller-created HIP events (hipEvent_t cast
 * to void*) on `stream` around the path's kernels, for per-kernel timing:
 * events[0] before the first kernel, events[1] between the first (the fused
 * FFN, the fp32 FFN, skinny layer 1 or the decode streaming kernel) and the
 * second (the split reduction, skinny layer 2 or the decode slice
 * reduction), events[2] after the second.  n_events >= 3. */
int ffn_forward_traced(const void* X, const void* W1, const void* b1, const void* W2,
                       const void* b2, void* Y, int64_t M, int64_t N, int64_t O, int64_t P,
                       int dtype, int act1, int act2, int variant, void* workspace,
                       size_t workspace_bytes, void* stream, void** events, int n_events);

/* ---------------------------------------------------------------- backward
 * Gradients of the dense FFN for act2 = NONE (the kernel-fusion post,
 * brunomaga.github.io, names a fused backward pass as its next step: the
 * forward keeps no H, so the backward recomputes it).  With a = X W1 + b1,
 * h = act1(a), Y = h W2 + b2 and the output gradient dY (M x P):
 *
 *   dX = (dY W2^T * act1'(a)) W1^T           M x N, bf16
 *   dW1 = X^T (dY W2^T * act1'(a))           N x O, fp32
 *   db1 = column sums of dY W2^T * act1'(a)  O, fp32 (may be NULL)
 *   dW2 = h^T dY                             O x P, fp32
 *   db2 = column sums of dY                  P, fp32 (may be NULL)
 *
 * act1'(x): ReLU' = 1 for x > 0 else 0; GELU-tanh' the derivative of the
 * tanh form; NONE: 1.  bf16 inputs (X, W1, b1 or NULL, W2, dY) only; the
 * intermediates h, act1'(a) and dY W2^T * act1'(a) are rounded to bf16 once
 * (they live in the workspace); sums accumulate in fp32 in a fixed order (no
 * atomics: repeated calls are bitwise identical).  M*N, M*O and M*P must be
 * below 2^30.  With M == 0 the weight and bias gradients are zero-filled. */
size_t ffn_backward_workspace_size(int64_t M, int64_t N, int64_t O, int64_t P, int dtype);

int ffn_backward(const void* X, const void* W1, const void* b1, const void* W2, const void* dY,
                 void* dX, float* dW1, float* db1, float* dW2, float* db2, int64_t M, int64_t N,
                 int64_t O, int64_t P, int dtype, int act1, void* workspace,
                 size_t workspace_bytes, void* stream);

/* As ffn_backward, recording events[0..6] on `stream` around its six steps
 * (h and act1'(a); da; dX; dW1; dW2; the bias sums).  n_events >= 7. */
int ffn_backward_traced(const void* X, const void* W1, const void* b1, const void* W2,
                        const void* dY, void* dX, float* dW1, float* db1, float* dW2, float* db2,
                        int64_t M, int64_t N, int64_t O, int64_t P, int dtype, int act1,
                        void* workspace, size_t workspace_bytes, void* stream, void** events,
                        int n_events);

/* ---------------------------------------------------------------- SwiGLU
 * The gated FFN the benchmarked models use (the kernel-fusion post,
 * brunomaga.github.io, section "Benchmarks": a third weight matrix whose
 * product with the input gates the activation; no biases):
 *
 *     H = silu(X Wg) * (X Wu)      X: M x N, Wg, Wu: N x O   (* elementwise)
 *     Y = H Wd                     Wd: O x P, Y: M x P
 *
 * with silu(x) = x / (1 + exp(-x)) (the page names the unit; this definition
 * is the published SiLU / Swish-1 one).  Same conventions as ffn_forward: for
 * a tensor-parallel shard pass the shard's columns of Wg and Wu and rows of Wd
 * and sum the shards' Y.  H is rounded to bf16 once (bf16 data) and never goes
 * to global memory on the FUSED family.  Variants as for ffn_forward: AUTO
 * picks SKINNY for bf16 with M <= 16 (the gated first layer writes H, 16 x O
 * bf16, to the workspace), FUSED for other bf16 shapes, F32 for fp32 data. */
size_t ffn_swiglu_workspace_size(int64_t M, int64_t N, int64_t O, int64_t P, int dtype,
                                 int variant);

/* Y = (silu(X Wg) * (X Wu)) Wd.  All of X, Wg, Wu, Wd, Y in `dtype`; none may be
 * NULL (X and Y may be NULL when M == 0).  Returns FFN_OK or FFN_E*. */
int ffn_swiglu_forward(const void* X, const void* Wg, const void* Wu, const void* Wd, void* Y,
                       int64_t M, int64_t N, int64_t O, int64_t P, int dtype, int variant,
                       void* workspace, size_t workspace_bytes, void* stream);

/* As ffn_swiglu_forward, with events recorded as for ffn_forward_traced:
 * events[0] before, events[1] between the first kernel (the fused FFN, the
 * fp32 FFN or the gated first layer) and the rest, events[2] after. */
int ffn_swiglu_forward_traced(const void* X, const void* Wg, const void* Wu, const void* Wd,
                              void* Y, int64_t M, int64_t N, int64_t O, int64_t P, int dtype,
                              int variant, void* workspace, size_t workspace_bytes, void* stream,
                              void** events, int n_events);

/* ---------------------------------------------------------------- MoE
 * Grouped form over the per-expert token lists of a top-k Mixture-of-Experts
 * layer (the MoE tile-signalling review, zhongzhuzhou.org, sections 2.1-2.2:
 * route, expert computation, gate-weighted sum).  bf16 only; 1 <= E <= 256,
 * 1 <= k <= min(E, 8).
 *
 * Routing (from the fp32 gate logits, M x E): per token the k largest logits
 * (ties: smaller expert index first; slot 0 = largest), gate weights =
 * softmax over those k logits (fp32).  Entry t*k+s is token t's s-th choice;
 * each expert's list holds its entries in ascending token order, lists
 * concatenated by expert index. */
size_t moe_workspace_size(int64_t M, int64_t E, int k, int64_t N, int64_t O, int64_t P,
                          int dtype);

/* Routing alone.  Outputs (device, caller-owned; each may be NULL):
 *   topk_ids M x k int32, topk_w M x k float, expert_offsets E+1 int32
 *   (exclusive prefix of the per-expert counts; [E] = M*k),
 *   sorted_entries M*k int32 (the concatenated per-expert lists).
 * workspace: at least moe_workspace_size(M, E, k, 8, 8, 8, FFN_BF16) bytes. */
int moe_route(const float* logits, int64_t M, int64_t E, int k, int32_t* topk_ids,
              float* topk_w, int32_t* expert_offsets, int32_t* sorted_entries,
              void* workspace, size_t workspace_bytes, void* stream);

/* Y[t] = sum_s w[t,s] * act2( act1(X[t] W1_e + b1_e) W2_e + b2_e ), e = topk_ids[t,s].
 *   X: M x N bf16; logits: M x E fp32; W1: E x N x O; b1: E x O or NULL;
 *   W2: E x O x P; b2: E x P or NULL; Y: M x P bf16.
 *   The routing outputs are optional copies, as in moe_route. */
int moe_ffn_forward(const void* X, const float* logits, int64_t M, int64_t E, int k,
                    const void* W1, const void* b1, const void* W2, const void* b2, void* Y,
                    int64_t N, int64_t O, int64_t P, int dtype, int act1, int act2,
                    int32_t* topk_ids, float* topk_w, int32_t* expert_offsets,
                    int32_t* sorted_entries, void* workspace, size_t workspace_bytes,
                    void* stream);

/* As moe_ffn_forward without the routing copies, recording events[0..3]
 * around the routing, grouped-FFN and combine kernels.  n_events >= 4. */
int moe_ffn_forward_traced(const void* X, const float* logits, int64_t M, int64_t E, int k,
                           const void* W1, const void* b1, const void* W2, const void* b2,
                           void* Y, int64_t N, int64_t O, int64_t P, int dtype, int act1,
                           int act2, void* workspace, size_t workspace_bytes, void* stream,
                           void** events, int n_events);

/* ---------------------------------------------------------------- MoE with the router
 * The same layer with the gate network on the GPU (the review, section 2.2,
 * step 1: the gate runs on the tokens and yields the assignments and gate
 * weights), read as one linear layer:
 *
 *     logits = X Wr + br           Wr: N x E bf16, br: E fp32 or NULL
 *
 * accumulated in fp32 (bf16 products, one fixed summation order), then routed
 * exactly as moe_route does.  The router form needs E % 8 == 0; Wr must be
 * 16-byte aligned.  logits_out (M x E fp32, may be NULL) receives the logits
 * the routing used.  Workspace: as for moe_workspace_size. */

/* Router + routing alone (the outputs as in moe_route, plus logits_out). */
int moe_router(const void* X, const void* Wr, const float* br, int64_t M, int64_t N, int64_t E,
               int k, float* logits_out, int32_t* topk_ids, float* topk_w,
               int32_t* expert_offsets, int32_t* sorted_entries, void* workspace,
               size_t workspace_bytes, void* stream);

/* As moe_ffn_forward with the logits computed from X, Wr and br. */
int moe_ffn_forward_router(const void* X, const void* Wr, const float* br, int64_t M, int64_t E,
                           int k, const void* W1, const void* b1, const void* W2, const void* b2,
                           void* Y, int64_t N, int64_t O, int64_t P, int dtype, int act1,
                           int act2, float* logits_out, int32_t* topk_ids, float* topk_w,
                           int32_t* expert_offsets, int32_t* sorted_entries, void* workspace,
                           size_t workspace_bytes, void* stream);

/* Text describing the last non-zero return on this host thread ("" if none). */
const char* ffn_last_error(void);

/* Library version (major * 10000 + minor * 100 + patch). */
int ffn_version(void);

/* ---- Measurement support (not part of the FFN path) --------------------
 * Two kernels that give a benchmark this GPU's own ceilings beside the
 * published peaks: a loop of independent bf16 MFMAs on register operands, and
 * a streaming 16-byte read of a device buffer.  Both only enqueue on `stream`;
 * time them with events.  `sink` is a device buffer of at least
 * ffn_ceiling_sink_bytes() bytes that the kernels may write (in practice they
 * never do; it keeps their work from being optimised away). */
size_t ffn_ceiling_sink_bytes(void);
/* Enqueues the MFMA loop (`iters` steps per wave) and returns in
 * *flops_per_launch the floating-point operations one launch performs. */
int ffn_ceiling_mfma(void* sink, size_t sink_bytes, int iters, double* flops_per_launch,
                     void* stream);
/* Enqueues one read of `bytes` bytes (a positive multiple of 16) at `src`
 * (16-byte aligned). */
int ffn_ceiling_read(const void* src, size_t bytes, void* sink, size_t sink_bytes, void* stream);

/* Host-only self-check of the LDS layouts the fused kernel relies on, using the
 * kernel's own layout functions: the H-tile fragment reads, the weight-stage
 * blocks (direct-load slots, coalesced lane quads, transposing-read addresses
 * and their bank spread) and the X fragments.  Returns 0 when all hold, else
 * the number of the first failed check.  Makes no HIP call. */
int ffn_selftest_layout(void);

/* Self-test of the decode stream's failure path (FFN_VARIANT_DECODE): as
 * ffn_forward_ex with that variant and bf16 data, but the workgroups' flags
 * never hold the call's number and every wait gives up after 64 polls, so
 * the call must write NaN to every element of Y (what a wait that expires in
 * a real call does).  Every kernel ends normally.  For tests only. */
int ffn_selftest_decode_expiry(const void* X, const void* W1, const void* b1, const void* W2,
                               const void* b2, void* Y, int64_t M, int64_t N, int64_t O,
                               int64_t P, int act1, int act2, void* workspace,
                               size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FFN_MI355X_H */
