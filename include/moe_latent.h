/*
 * moe_latent.h -- C ABI of one latent mixture-of-experts decode layer on MI355X (gfx950).
 *
 * The layer (TensorFold pull request 1038, «What's in it», the latent MoE bullet) runs, per
 * row of the input, in this order:
 *   bf16 router gate gemv -> sigmoid, group-limited top-k with a correction bias ->
 *   fc1_latent_proj (hidden -> latent) -> routed experts (4-bit affine up, relu^2, 4-bit
 *   down) in the latent -> weighted combine over the picks -> fc2_latent_proj (latent ->
 *   hidden) -> + shared expert -> + residual.
 * A non-latent variant (latent = 0: experts act on the hidden vector, no fc1/fc2) with fp16
 * activations and an fp32 router covers the fp16 family router of TensorFold pull request
 * 1295 («What this changes», family kernels: fp32 router, sigmoid top-8, per-expert norm
 * and sum).
 *
 * Every pointer handed to this library is a device pointer (hipMalloc'd or from a torch
 * tensor on the current GPU) unless stated otherwise. All calls are host calls; forward
 * work is enqueued on the handle's HIP stream and does not synchronise.
 *
 * Errors: every int-returning call returns MOE_OK (0) or one of the moe_status codes;
 * moe_latent_last_error() then returns a message (per calling thread) that names the
 * refused parameter or tensor.
 */
#ifndef MOE_LATENT_H
#define MOE_LATENT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types of moe_tensor.dtype and of the activation / router switches */
enum moe_dtype { MOE_DT_BF16 = 1, MOE_DT_F16 = 2, MOE_DT_F32 = 3, MOE_DT_U32 = 4, MOE_DT_I32 = 5 };

/* expert activation (the only one the layer uses: relu^2 of the up projection) */
enum moe_activation { MOE_ACT_RELU2 = 1 };

enum moe_status {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1,      /* NULL handle / pointer, unknown enum value */
    MOE_ERR_TOPK_GT_EXPERTS = 2,  /* top_k larger than the layer's own expert count */
    MOE_ERR_GROUPS = 3,           /* n_experts % n_group, topk_group > n_group, too few candidates */
    MOE_ERR_SHAPE = 4,            /* a size the kernels do not take (see moe_latent_config) */
    MOE_ERR_MISSING_TENSOR = 5,   /* a tensor the configuration needs has data == NULL */
    MOE_ERR_DTYPE = 6,            /* e.g. a quantized or non-bf16 latent projection */
    MOE_ERR_LAYOUT = 7,           /* wrong rank, shape, or strides (transposed / non-contiguous) */
    MOE_ERR_EXPERTS_OVER_HIDDEN = 8, /* latent layer whose experts are stored over hidden */
    MOE_ERR_DEVICE = 9,           /* no device, or the current device is not gfx950 */
    MOE_ERR_ROWS = 10,            /* rows < 1 or rows > max_rows */
    MOE_ERR_ALIAS = 11,           /* out partially overlaps hidden_in */
    MOE_ERR_HIP = 12,             /* a HIP runtime call failed (message holds its error) */
    MOE_ERR_OOM = 13,             /* device allocation failed */
    MOE_ERR_DEVICE_CHECK = 14     /* a kernel's own consistency check failed (see the message) */
};

/* A borrowed view of one weight tensor: data is a device pointer, shape/stride in elements,
 * row-major expected (stride of the last dim 1, each outer stride the product of the inner
 * extents). Unused trailing entries are ignored. */
typedef struct {
    const void *data;
    int32_t dtype;   /* moe_dtype */
    int32_t ndim;    /* 1..4 */
    int64_t shape[4];
    int64_t stride[4];
} moe_tensor;

/* Layer configuration. Sizes the kernels take: hidden % 512 == 0; latent == 0 or
 * latent % 128 == 0; expert_inter % 64 == 0; shared_inter == 0 or % 128 == 0; expert input
 * and inter widths <= 6144; n_experts <= 1024; n_group <= 256; top_k <= 16;
 * 1 <= max_rows <= 4096 (a decode pass takes at most 256 rows, a prefill up to max_rows). latent == 0 selects the non-latent layer; shared_inter == 0 drops
 * the shared expert. A shared expert needs a latent layer (MOE_ERR_SHAPE otherwise): its
 * output is added in the fc2 epilogue.
 * Routed expert format: quant_bits-bit affine codes in groups of group_size inputs (the
 * affine family whose decode speed the mlx-bun program measures, §7.4 experiment axes:
 * 2..8 bits, groups of 32, 64 or 128). quant_bits 4 with group_size 64 is the layer's own
 * format (the fused 4-bit expert path, fp16 activations allowed); any other pair of
 * quant_bits in {2, 3, 4, 5, 6, 8} and group_size in {32, 64, 128} runs the width-generic
 * expert kernels, which need bf16 activations and expert input and inter widths that are
 * multiples of 128 (MOE_ERR_SHAPE / MOE_ERR_DTYPE otherwise). quant_bits 0 reads as 4. */
typedef struct {
    int32_t hidden;         /* H */
    int32_t latent;         /* L, or 0 (non-latent) */
    int32_t n_experts;      /* E */
    int32_t n_group;        /* G: contiguous groups of E / G experts */
    int32_t topk_group;     /* groups kept per row */
    int32_t top_k;          /* k experts picked per row */
    int32_t expert_inter;   /* I: routed expert intermediate width */
    int32_t shared_inter;   /* SI: shared expert width, or 0 */
    int32_t group_size;     /* quantization group along the input dim (64) */
    int32_t act_dtype;      /* MOE_DT_BF16 or MOE_DT_F16 (F16 only with latent == 0, no shared) */
    int32_t router_dtype;   /* MOE_DT_BF16 (bf16 gate, bf16 logits) or MOE_DT_F32 */
    int32_t activation;     /* MOE_ACT_RELU2 */
    int32_t has_bias;       /* 1: fp32 correction bias added for selection only */
    int32_t norm_topk;      /* 1: weights = scores / (sum over picks), then * routed_scaling */
    int32_t max_rows;       /* largest rows a forward may pass; sizes the workspace */
    float routed_scaling;   /* rho */
    int32_t quant_bits;     /* routed expert code width: 2, 3, 4, 5, 6 or 8 (0: 4) */
} moe_latent_config;

/* The layer's weights (borrowed: the caller keeps every buffer alive until destroy; every
 * data pointer 16-byte aligned, MOE_ERR_LAYOUT otherwise).
 *   gate_w      [E][H]     bf16 (router_dtype BF16) or fp32 (F32)
 *   corr_bias   [E]        fp32 (only read when has_bias)
 *   fc1_w       [L][H]     bf16 (latent layers only)
 *   fc2_w       [H][L]     bf16 (latent layers only)
 *   up_q        [E][I][D b/32]  u32 (b = quant_bits): each output row's codes as one
 *                             little-endian bit string, the code of input k in bits
 *                             [k b, k b + b) (4 bits: 8 codes per word, code of input k in word
 *                             k/8 at bits 4*(k%8), lowest nibble = lowest k); D = L, or H if
 *                             non-latent
 *   up_scales   [E][I][D/gs]  bf16 scale per group of gs = group_size inputs
 *   up_biases   [E][I][D/gs]  bf16 bias per group: weight = code * scale + bias
 *   down_q      [E][D][I b/32]  u32, same packing
 *   down_scales [E][D][I/gs]  bf16
 *   down_biases [E][D][I/gs]  bf16
 *   shared_up   [SI][H]   bf16 (shared_inter > 0 only)
 *   shared_down [H][SI]   bf16 (shared_inter > 0 only) */
typedef struct {
    moe_tensor gate_w, corr_bias, fc1_w, fc2_w;
    moe_tensor up_q, up_scales, up_biases, down_q, down_scales, down_biases;
    moe_tensor shared_up, shared_down;
} moe_latent_weights;

typedef struct moe_latent moe_latent_t;

/* Create a layer handle (TensorFold pull request 1038, «What's in it»: refusals before
 * load, per-layer loader; the review thread: release of device resources on every
 * refusal). Checks, in order, the configuration (top_k against this layer's own expert
 * count, groups, sizes), then every tensor descriptor (presence, dtype, shape, row-major
 * strides; a latent projection that is missing, quantized, transposed or not bf16 is
 * refused by name, and so are experts stored over hidden in a latent layer), then that the
 * current device is gfx950 -- all before any weight byte is read. Then it allocates the
 * workspace for max_rows rows on the current device. hip_stream: the hipStream_t forwards
 * are enqueued on (NULL = the null stream). On failure *out is NULL and nothing stays
 * allocated. */
int moe_latent_create(const moe_latent_config *cfg, const moe_latent_weights *w,
                      void *hip_stream, moe_latent_t **out);

/* One forward of `rows` independent rows (TensorFold pull request 1038, «What's in it»,
 * layer order; «Per operator and row invariance»: each row of a multi-row pass equals its
 * own one-row pass). hidden_in: [rows][H] activations (act_dtype); out: [rows][H] (same
 * dtype); both 16-byte aligned (MOE_ERR_LAYOUT otherwise). out == hidden_in (in place) is
 * allowed; any other overlap is refused. Enqueued as
 * a short chain of launches (no host synchronisation, no allocation, no memset: it can be
 * captured in a HIP graph) that starts and ends on the handle's stream: in a pass of more than
 * one row (by default) the shared expert runs on the handle's own side stream, forked off the
 * handle's stream by an event at the start and joined back by an event before the fc2 launch,
 * so a graph captured on the handle's stream holds both branches; returns launch errors only -- device-side
 * faults surface at the caller's next synchronisation / moe_latent_status(). The handle is
 * not reentrant: forwards on one handle must not overlap in time on different streams. */
int moe_latent_forward(moe_latent_t *h, int32_t rows, const void *hidden_in, void *out);

/* The fused prefill: one pass of `rows` rows (1 .. max_rows, up to 4096) through the same
 * layer, for prompts (TensorFold pull request 1038, «Not yet / next»: a fused prefill for the
 * latent MoE, where prompts otherwise run through the decode kernels 16 rows at a time).
 * The projections and the routed experts run as MFMA GEMMs over all rows at once: the picks
 * are grouped by expert (a counting sort on the device) and each expert's weights are read
 * once per tile of 64 of its picks. Same arithmetic as moe_latent_forward -- the same gate
 * order, so the same logits and routing bit for bit; the same route, combine and rounding
 * points -- with other fp32 summation orders in the projections and experts, so outputs
 * agree with a decode pass within the parity bar, not bit for bit. Each row of a prefill
 * equals that row passed alone through moe_latent_prefill, bit for bit. Takes bf16
 * activations, 4-bit codes in groups of 64, expert_inter a multiple of 128 and
 * n_experts * hidden below 2^31 (MOE_ERR_DTYPE / MOE_ERR_SHAPE otherwise). Buffers and
 * errors as moe_latent_forward (in
 * place allowed); enqueued on the handle's stream as a chain of launches, no allocation;
 * moe_latent_get_routing and moe_latent_read_stage then report this pass. moe_latent_forward
 * itself takes at most 256 rows (MOE_ERR_ROWS above). */
int moe_latent_prefill(moe_latent_t *h, int32_t rows, const void *hidden_in, void *out);

/* Release the workspace and the handle (NULL-safe; a handle already destroyed or never
 * created is ignored). Synchronises the handle's stream first, so no enqueued forward still
 * uses what it frees. Every device resource create took is released here, as the loader on
 * TensorFold pull request 1038 releases what it built (review thread: device resources of a
 * failed or finished load are freed, checked by counting live allocations; see
 * moe_latent_live_allocations). */
void moe_latent_destroy(moe_latent_t *h);

/* Launch groups of a forward, in enqueue order.
 * Variant 2 (two streams; the default for passes of more than one row): 0 gate + fc1 (one-row pass: its first workgroup
 * routes the row once the gate workgroups have handed it their logits; that wait is bounded,
 * and a timeout sets bit 8 of the device error flag, reported by moe_latent_status); with a
 * shared expert, on the side stream: 1 shared up, 2 and 3 the two halves of shared down;
 * then on the handle's stream: route (multi-row passes only: one workgroup per row, the last
 * builds the expert schedule); routed expert up; routed expert down (multi-row: the last
 * workgroup of each output block combines it; a non-latent layer also adds the residual
 * there); combine + fc2 + shared + residual (latent layers; it waits for the side stream;
 * one-row pass: each fc2 workgroup combines the slice of the expert outputs it reads).
 * Variant 1 (one stream; the default for a one-row pass): one-row pass: 0 gate + fc1 + shared up (+ the route as above);
 * 1 routed expert up + shared down (first half); 2 routed expert down + shared down (second
 * half); 3 combine + fc2 + shared + residual. Multi-row pass: 0 as above without the route;
 * 1 route + shared down (first half); 2 routed expert up + shared down (second half); 3 routed
 * expert down + combine; 4 fc2 + shared + residual. A non-latent layer has no fc1 / fc2 /
 * shared launches: its combine adds the residual. */

/* Enqueue only launch group `group` of a forward of `rows` rows, for timing one
 * kernel on its own. Its inputs are what the earlier groups of the same forward wrote, so
 * call it after a full moe_latent_forward with the same rows, hidden_in and out; it then
 * rewrites the same values. A group with no work for this pass enqueues nothing. */
int moe_latent_launch_group(moe_latent_t *h, int32_t rows, const void *hidden_in, void *out,
                            int32_t group);

/* Number of workgroups launch group `group` runs for a pass of `rows` rows (0: nothing to
 * launch, or no such group), or -1 for an invalid handle or rows. */
int moe_latent_group_items(moe_latent_t *h, int32_t rows, int32_t group);

/* The same count, and the group's stages (enum values of the work-item table, in layer
 * order: 0 gate, 1 fc1, 2 shared up, 3 route, 4 shared down first half, 5 routed expert up,
 * 6 shared down second half, 7 routed expert down, 8 fc2) and stream (0: the handle's
 * stream, 1: its side stream) into the non-NULL pointers; for labelling per-launch
 * measurements. */
int moe_latent_group_stages(moe_latent_t *h, int32_t rows, int32_t group, int32_t *first_stage,
                            int32_t *last_stage, int32_t *side);

/* The name of the kernel launch group `group` runs for a pass of `rows` rows, as a profiler
 * lists it without namespace and arguments (e.g. "moe_front_kernel", "moe_stage_kernel<3, 5,
 * false, 0>"), written NUL-terminated into name (at most cap bytes, cut to fit); for matching
 * per-launch measurements with profiler records. Returns its length, 0 (empty name) when
 * there is no such group, or -1 for an invalid handle, rows, name or cap. */
int moe_latent_group_kernel(moe_latent_t *h, int32_t rows, int32_t group, char *name, int32_t cap);

/* A forward like moe_latent_forward, whose launch i (launch group i) also records the start
 * and the end of its own kernel into events[2 i] and events[2 i + 1] (hipEvent_t handles the
 * caller created with timing enabled; the timestamps come from the kernel's dispatch itself,
 * on the stream the launch runs on, no extra packets), so that hipEventElapsedTime gives each
 * launch's duration inside the forward. For per-launch timing; it cannot be captured in a
 * graph. n_events must be at least twice the
 * number of launch groups of the pass (MOE_ERR_INVALID_ARG otherwise); a launch with no work
 * leaves its two events untouched. */
int moe_latent_forward_timed(moe_latent_t *h, int32_t rows, const void *hidden_in, void *out,
                             void *const *events, int32_t n_events);

/* Change the stream later forwards are enqueued on (e.g. a graph-capture stream). */
int moe_latent_set_stream(moe_latent_t *h, void *hip_stream);

/* Execution variant (see the launch groups above): 2: the routed chain on the handle's stream
 * and the shared expert on the handle's side stream, in parallel; 1: one chain of launches on
 * the handle's stream, the shared expert's workgroups filling its launches; 3 (the default):
 * variant 1 for a one-row pass and variant 2 for more rows (the side stream's fork and join
 * cost more than they save in a one-row pass); 4: variant 1, but the first launch of a one-row
 * pass as work items of the stage kernel (gate, route, fc1 and shared up items) instead of the
 * front kernel (fc1 and shared up in slices spread evenly over the compute units, the gate
 * rows and the route beside them). All give the same bits. 0 (one fused launch per forward, a dependency-ordered work queue)
 * is reserved and refused with MOE_ERR_INVALID_ARG: its first GPU run did not complete, and
 * it is not built. Synchronises the handle's stream first. */
int moe_latent_set_variant(moe_latent_t *h, int32_t variant);

/* Copy the last forward's routing to device buffers, enqueued on the handle's stream:
 * idx_dev [rows][top_k] int32 expert ids in pick order, w_dev [rows][top_k] fp32 weights
 * (either may be NULL to skip it); rows is the last forward's row count. The routing is
 * what TensorFold pull request 1038 checks bit for bit per row («Per operator and row
 * invariance»: group_expert_select at k = 9; per-row equality of a multi-row pass with its
 * one-row passes), so the tests read it back here. MOE_ERR_INVALID_ARG before any forward;
 * MOE_ERR_HIP if a copy cannot be enqueued. */
int moe_latent_get_routing(moe_latent_t *h, int32_t *idx_dev, float *w_dev);

/* Intermediate values of the last forward, for stage-by-stage checks. */
enum moe_stage {
    MOE_STAGE_LOGITS = 1,      /* [rows][E] bf16 (router BF16) or fp32 (router F32) */
    MOE_STAGE_LATENT = 2,      /* [rows][D] act: fc1 output (or hidden_in when non-latent) */
    MOE_STAGE_EXPERT_ACT = 3,  /* [rows][top_k][I] act: relu^2 of each pick's up projection */
    MOE_STAGE_EXPERT_OUT = 4,  /* [rows][top_k][D] act: each pick's down projection */
    MOE_STAGE_COMBINE = 5,     /* [rows][D] act */
    MOE_STAGE_SHARED_ACT = 6,  /* [rows][SI] act: relu^2 of the shared up projection */
    MOE_STAGE_SHARED_OUT = 7   /* [rows][H] act: shared expert output */
};

/* Copy `bytes` bytes of stage `stage` of the last forward to dst_dev (enqueued on the
 * handle's stream). bytes must not exceed the stage's size for the last forward's rows. */
int moe_latent_read_stage(moe_latent_t *h, int32_t stage, void *dst_dev, size_t bytes);

/* Synchronise the handle's stream, then report device-side errors of past forwards
 * (MOE_ERR_DEVICE_CHECK) or MOE_ERR_HIP; clears the device error flag. */
int moe_latent_status(moe_latent_t *h);

/* Message of the last failed call on this thread ("" if none; a successful create clears
 * it). The message names the refused parameter or tensor and the reason, as the refusals of
 * TensorFold pull request 1038 do («What's in it»: a layer whose top-k exceeds its expert
 * count, a missing, quantized or transposed latent projection, experts stored over hidden,
 * an unsupported chip -- each refused by name before any weight is read). The pointer stays
 * valid until this thread's next call into the library; the library owns it. */
const char *moe_latent_last_error(void);

/* Number of device allocations, streams and events the library currently holds (all
 * handles); a handle holds its workspace, its side stream and two events. */
int32_t moe_latent_live_allocations(void);

/* A plain read-only stream over device memory, the reference beside the published HBM peak
 * that the measured bandwidth of the layer is judged against (mlx-bun 0.3.0
 * decode-speed program, the bandwidth-wall model and its measurement discipline: what a
 * pure read of the same bytes achieves on the same machine). Enqueues on hip_stream (NULL:
 * the null stream) one launch that reads `bytes` bytes at src (device, 16-byte aligned,
 * bytes a multiple of 16, at most 2^40) with 16-byte nontemporal loads, one workgroup per
 * compute unit, and
 * folds the data into *sink_dev (one device uint32, XOR-accumulated, so the reads are not
 * elided). No allocation. MOE_ERR_INVALID_ARG for a NULL pointer, a misaligned src or a bad
 * size. */
int moe_latent_stream_read(const void *src, size_t bytes, uint32_t *sink_dev, void *hip_stream);

/* The bf16 lm_head gemv beside the layer (TensorFold pull request 1038, «Per operator and
 * row invariance», its lm_head rows: K = 4096 inputs, N = 131072 outputs, at 1 and 16 rows):
 * out[r][n] = sum_k w[n][k] * x[r][k], products exact in fp32 and summed in fp32, then stored
 * as fp32 (out_dtype MOE_DT_F32) or rounded to bf16 (MOE_DT_BF16, round to nearest even).
 *   w    [N][K] bf16, row-major (borrowed; N a multiple of 16, K a multiple of 128)
 *   x    [rows][K] bf16, 1 <= rows <= 256
 *   out  [rows][N] fp32 or bf16 (caller's; may not overlap x or w)
 * All device pointers, 16-byte aligned. Each row's result does not depend on the other rows
 * of the call (bit for bit). One launch on hip_stream (NULL: the null stream); no allocation,
 * no synchronisation; it can be captured in a HIP graph. Errors: MOE_ERR_LAYOUT (rank, strides,
 * alignment), MOE_ERR_DTYPE, MOE_ERR_SHAPE (N or K), MOE_ERR_ROWS, MOE_ERR_ALIAS,
 * MOE_ERR_DEVICE (not gfx950), MOE_ERR_HIP (launch). */
int moe_lm_head_gemv(const moe_tensor *w, int32_t rows, const void *x, void *out, int32_t out_dtype,
                     void *hip_stream);

/* Size of the static workspace of moe_latent_forward_static, per GPU (16 MiB: a Bolt-like
 * layer of hidden 4096, latent 1024, 9 picks of 2048-wide experts and a 4096-wide shared
 * expert fits up to about 100 rows). */
#define MOE_LATENT_STATIC_SCRATCH_BYTES (16u << 20)

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): one forward like moe_latent_forward, without a
 * handle and without any allocation. cfg and w are validated as moe_latent_create validates
 * them (same refusals and codes; nothing is kept after the call), hidden_in / out / rows as
 * moe_latent_forward checks them (rows <= cfg->max_rows). The workspace for `rows` rows lives
 * in a library-owned array of MOE_LATENT_STATIC_SCRATCH_BYTES per GPU, held until the process
 * ends; a forward whose workspace does not fit is refused with MOE_ERR_SHAPE. Enqueued on
 * hip_stream (NULL: the null stream) as the single-stream launch chain of moe_latent_forward,
 * preceded by two fill kernels that zero the array's counters and error flag (no memset, no
 * host synchronisation): it can be captured in a HIP graph. Every call on a GPU shares that
 * GPU's array, which keeps the last call's contents, so calls that overlap in time on one GPU
 * (on different streams, or replays of graphs on different streams) race and give wrong
 * results; calls in stream order do not. The output equals moe_latent_forward's bit for bit.
 * Device-side check flags are cleared by the next call and are not reported. */
int moe_latent_forward_static(const moe_latent_config *cfg, const moe_latent_weights *w, int32_t rows,
                              const void *hidden_in, void *out, void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_LATENT_H */
