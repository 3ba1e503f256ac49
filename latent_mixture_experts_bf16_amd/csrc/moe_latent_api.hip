// moe_latent_api.hip -- host side of the C ABI declared in include/moe_latent.h.
//
// Refusal conventions follow TensorFold pull request 1038 («What's in it»: refusals before
// load -- a layer whose top-k exceeds its own expert count; a latent projection that is
// missing, quantized, transposed or not bf16; experts stored over hidden; an unsupported
// chip -- each by name, before any weight is read; review thread: the device resources a
// failed load created are released). Here: configuration, then tensor descriptors, then the
// device, then allocation; every failure frees what was allocated and returns a named code.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "moe_latent.h"
#include "layer_plan.h"

namespace moe {
template <int FIRST, int LAST, bool WIDE, int QB>
__global__ void moe_stage_kernel(LayerParams p, int lo, int hi, int mid, int pre);
__global__ void moe_clear_kernel(uint32_t *ctr, int n);
__global__ void moe_stream_read_kernel(const uint4 *src, size_t n, uint32_t *sink);
__global__ void moe_lm_head_kernel(LayerParams p, const uint16_t *W, const uint16_t *X, int K, int lo);
__global__ void moe_front_kernel(LayerParams p, int nwg);
// the prefill (prefill_kernels.hip)
template <bool F32W> __global__ void pf_gate_kernel(LayerParams p);
template <int ME> __global__ void pf_route_kernel(LayerParams p);
__global__ void pf_sched_kernel(LayerParams p);
template <int EPI, int KS>
__global__ void pf_gemm_kernel(LayerParams p, const uint16_t *X, const uint16_t *W, int N, int K);
template <bool UP> __global__ void pf_expert_kernel(LayerParams p);
template <int EPI, int TN>
__global__ void pf_gemm_big_kernel(LayerParams p, const uint16_t *X, const uint16_t *W, int N, int K);
__global__ void pf_combine_kernel(LayerParams p);
}  // namespace moe

using namespace moe;

struct moe_latent {
    moe_latent_config cfg;
    LayerParams base;       // sizes, weights and workspace pointers; per-forward fields set later
    hipStream_t stream;     // the caller's stream: forwards start and end on it
    hipStream_t side;       // the handle's own stream (default priority) for the shared expert
    hipEvent_t ev_fork;     // recorded on `stream` when a forward starts; `side` waits for it
    hipEvent_t ev_join;     // recorded on `side` after its work; `stream` waits for it
    int variant;            // 1: one stream; 2: two streams; 3 (default): by row count
    int device;
    int last_rows;
    void *ws;               // one workspace allocation
    size_t ws_bytes;
    int n_ctr;             // completion counters in the workspace
    int cus;               // compute units of the device
    uint32_t magic;
};

static const uint32_t kMagic = 0x4D4F454Cu;
static thread_local std::string g_err;
static std::atomic<int> g_live_allocs{0};
static std::atomic<int> g_alloc_calls{0};

static int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

// Device allocation with leak accounting. MOE_LATENT_FAIL_ALLOC_AT=n makes the n-th
// allocation after the variable was set (or last changed) fail, to test the release paths.
static std::mutex g_fail_mu;
static std::string g_fail_seen;
static bool inject_failure() {
    const char *f = getenv("MOE_LATENT_FAIL_ALLOC_AT");
    std::lock_guard<std::mutex> lk(g_fail_mu);
    const std::string v = f ? f : "";
    if (v != g_fail_seen) { g_fail_seen = v; g_alloc_calls = 0; }
    const int n = ++g_alloc_calls;
    return !v.empty() && atoi(v.c_str()) == n;
}

static hipError_t dev_alloc(void **p, size_t bytes) {
    if (inject_failure()) { *p = nullptr; return hipErrorOutOfMemory; }
    hipError_t e = hipMalloc(p, bytes);
    if (e == hipSuccess) ++g_live_allocs;
    return e;
}

static void dev_free(void *p) {
    if (p && hipFree(p) == hipSuccess) --g_live_allocs;
}

// The handle's side stream and events, counted and failure-injected like allocations.
static hipError_t side_stream_create(hipStream_t *s) {
    if (inject_failure()) { *s = nullptr; return hipErrorOutOfMemory; }
    hipError_t e = hipStreamCreateWithFlags(s, hipStreamNonBlocking);   // default priority
    if (e == hipSuccess) ++g_live_allocs;
    return e;
}
static void side_stream_destroy(hipStream_t s) {
    if (s && hipStreamDestroy(s) == hipSuccess) --g_live_allocs;
}
static hipError_t event_create(hipEvent_t *ev) {
    if (inject_failure()) { *ev = nullptr; return hipErrorOutOfMemory; }
    hipError_t e = hipEventCreateWithFlags(ev, hipEventDisableTiming);
    if (e == hipSuccess) ++g_live_allocs;
    return e;
}
static void event_destroy(hipEvent_t ev) {
    if (ev && hipEventDestroy(ev) == hipSuccess) --g_live_allocs;
}

// ------------------------------------------------------------------ validation

static const char *dt_name(int dt) {
    switch (dt) {
    case MOE_DT_BF16: return "bf16";
    case MOE_DT_F16: return "f16";
    case MOE_DT_F32: return "f32";
    case MOE_DT_U32: return "u32";
    case MOE_DT_I32: return "i32";
    default: return "unknown";
    }
}

// Output rows of one expert item: the largest power of two <= 64 that divides N, whose
// codes, scales and biases fit the item's LDS, and whose codes and scales fill whole 16-byte
// units. bits: code width; gs: inputs per scale.
static int expert_block(int N, int Kin, int bits = 4, int gs = 64) {
    for (int nb = EXPERT_MAX_BLOCK; nb > 1; nb >>= 1) {
        const size_t code_bytes = (size_t)nb * Kin * bits / 8, groups = (size_t)nb * (Kin / gs);
        if (N % nb == 0 && code_bytes <= EXPERT_LDS_CODES && groups * 2 <= EXPERT_LDS_SCALES &&
            code_bytes % 256 == 0 && groups % 8 == 0)
            return nb;
    }
    return 1;
}

static int quant_bits_of(const moe_latent_config &c) { return c.quant_bits ? c.quant_bits : 4; }
static bool generic_format(const moe_latent_config &c) { return quant_bits_of(c) != 4 || c.group_size != 64; }

static int check_config(const moe_latent_config &c) {
    if (c.hidden <= 0 || c.n_experts <= 0 || c.n_group <= 0 || c.topk_group <= 0 || c.top_k <= 0 ||
        c.expert_inter <= 0 || c.latent < 0 || c.shared_inter < 0)
        return fail(MOE_ERR_INVALID_ARG, "config: sizes must be positive (latent, shared_inter >= 0)");
    if (c.top_k > c.n_experts)
        return fail(MOE_ERR_TOPK_GT_EXPERTS, "config: top_k %d exceeds this layer's n_experts %d",
                    c.top_k, c.n_experts);
    if (c.n_experts > MAX_EXPERTS)
        return fail(MOE_ERR_SHAPE, "config: n_experts %d > %d", c.n_experts, (int)MAX_EXPERTS);
    if (c.top_k > MAX_TOPK) return fail(MOE_ERR_SHAPE, "config: top_k %d > %d", c.top_k, (int)MAX_TOPK);
    if (c.n_group > 256 || c.n_experts % c.n_group)
        return fail(MOE_ERR_GROUPS, "config: n_experts %d not divisible into n_group %d groups (<= 256)",
                    c.n_experts, c.n_group);
    const int per = c.n_experts / c.n_group;
    if (c.topk_group > c.n_group)
        return fail(MOE_ERR_GROUPS, "config: topk_group %d > n_group %d", c.topk_group, c.n_group);
    if (c.n_group > 1 && per < 2)
        return fail(MOE_ERR_GROUPS, "config: groups of %d expert; a group score needs two", per);
    if (c.topk_group * per < c.top_k)
        return fail(MOE_ERR_GROUPS, "config: %d kept groups of %d experts cannot hold top_k %d",
                    c.topk_group, per, c.top_k);
    const int qb = quant_bits_of(c);
    if (qb != 2 && qb != 3 && qb != 4 && qb != 5 && qb != 6 && qb != 8)
        return fail(MOE_ERR_SHAPE, "config: quant_bits %d (2, 3, 4, 5, 6 or 8)", c.quant_bits);
    if (c.group_size != 32 && c.group_size != 64 && c.group_size != 128)
        return fail(MOE_ERR_SHAPE, "config: group_size %d (32, 64 or 128)", c.group_size);
    if (c.hidden % 512) return fail(MOE_ERR_SHAPE, "config: hidden %d not a multiple of 512", c.hidden);
    if (c.latent % 128) return fail(MOE_ERR_SHAPE, "config: latent %d not a multiple of 128", c.latent);
    if (c.shared_inter % 128)
        return fail(MOE_ERR_SHAPE, "config: shared_inter %d not a multiple of 128", c.shared_inter);
    const int D = c.latent ? c.latent : c.hidden;
    if (c.expert_inter % 64 || c.expert_inter > 6144 || D > 6144)
        return fail(MOE_ERR_SHAPE, "config: expert dims (in %d, inter %d) must be multiples of 64, <= 6144",
                    D, c.expert_inter);
    if (generic_format(c)) {
        if (D % 128 || c.expert_inter % 128)
            return fail(MOE_ERR_SHAPE, "config: %d-bit codes in groups of %d need expert dims (in %d, inter %d) "
                        "that are multiples of 128", qb, c.group_size, D, c.expert_inter);
        if (c.act_dtype != MOE_DT_BF16)
            return fail(MOE_ERR_DTYPE, "config: %d-bit codes in groups of %d need bf16 activations", qb,
                        c.group_size);
    }
    {
        const int nb_up = expert_block(c.expert_inter, D, qb, c.group_size);
        const int nb_dn = expert_block(D, c.expert_inter, qb, c.group_size);
        if (((size_t)nb_up * D * qb / 8) % 256 || ((size_t)nb_dn * c.expert_inter * qb / 8) % 256 ||
            (nb_up * (D / c.group_size)) % 8 || (nb_dn * (c.expert_inter / c.group_size)) % 8)
            return fail(MOE_ERR_SHAPE, "config: no expert block fits the item LDS for in %d, inter %d", D,
                        c.expert_inter);
    }
    if (c.act_dtype != MOE_DT_BF16 && c.act_dtype != MOE_DT_F16)
        return fail(MOE_ERR_DTYPE, "config: act_dtype %s (bf16 or f16)", dt_name(c.act_dtype));
    if (c.act_dtype == MOE_DT_F16 && (c.latent || c.shared_inter))
        return fail(MOE_ERR_DTYPE, "config: f16 activations only for the non-latent layer without a shared expert");
    if (!c.latent && c.shared_inter)
        return fail(MOE_ERR_SHAPE, "config: a shared expert needs a latent layer (its output is added in the fc2 "
                    "epilogue)");
    if (c.router_dtype != MOE_DT_BF16 && c.router_dtype != MOE_DT_F32)
        return fail(MOE_ERR_DTYPE, "config: router_dtype %s (bf16 or f32)", dt_name(c.router_dtype));
    if (c.activation != MOE_ACT_RELU2) return fail(MOE_ERR_INVALID_ARG, "config: activation %d", c.activation);
    if (c.max_rows < 1 || c.max_rows > MAX_PREFILL_ROWS)
        return fail(MOE_ERR_ROWS, "config: max_rows %d outside 1..%d", c.max_rows, (int)MAX_PREFILL_ROWS);
    return MOE_OK;
}

// shape expected row-major with the given extents
static int check_tensor(const char *name, const moe_tensor &t, int dtype, int ndim, const int64_t *shape) {
    if (!t.data) return fail(MOE_ERR_MISSING_TENSOR, "%s: missing (data == NULL)", name);
    if (t.dtype != dtype) {
        if (dtype == MOE_DT_BF16 && t.dtype == MOE_DT_U32)
            return fail(MOE_ERR_DTYPE, "%s: quantized (u32 codes); a bf16 tensor is required", name);
        return fail(MOE_ERR_DTYPE, "%s: dtype %s, expected %s", name, dt_name(t.dtype), dt_name(dtype));
    }
    if (t.ndim != ndim) return fail(MOE_ERR_LAYOUT, "%s: rank %d, expected %d", name, t.ndim, ndim);
    bool transposed = ndim == 2 && t.shape[0] == shape[1] && t.shape[1] == shape[0] && shape[0] != shape[1];
    for (int i = 0; i < ndim; ++i)
        if (t.shape[i] != shape[i]) {
            if (transposed) return fail(MOE_ERR_LAYOUT, "%s: transposed ([%lld][%lld], expected [%lld][%lld])", name,
                                        (long long)t.shape[0], (long long)t.shape[1], (long long)shape[0],
                                        (long long)shape[1]);
            return fail(MOE_ERR_LAYOUT, "%s: dim %d is %lld, expected %lld", name, i, (long long)t.shape[i],
                        (long long)shape[i]);
        }
    int64_t st = 1;
    for (int i = ndim - 1; i >= 0; --i) {
        if (t.stride[i] != st) {
            if (ndim == 2 && t.stride[0] == 1 && t.stride[1] == shape[0])
                return fail(MOE_ERR_LAYOUT, "%s: transposed (column-major strides)", name);
            return fail(MOE_ERR_LAYOUT, "%s: not contiguous row-major (stride[%d] = %lld, expected %lld)", name, i,
                        (long long)t.stride[i], (long long)st);
        }
        st *= shape[i];
    }
    if ((uintptr_t)t.data & 15)   // the kernels read every tensor with 16-byte loads
        return fail(MOE_ERR_LAYOUT, "%s: data pointer not 16-byte aligned", name);
    return MOE_OK;
}

static int check_weights(const moe_latent_config &c, const moe_latent_weights &w) {
    const int64_t H = c.hidden, L = c.latent, E = c.n_experts, I = c.expert_inter, SI = c.shared_inter;
    const int64_t D = L ? L : H;
    int rc;
    {
        const int64_t s[2] = {E, H};
        if ((rc = check_tensor("gate_w", w.gate_w, c.router_dtype, 2, s))) return rc;
    }
    if (c.has_bias) {
        const int64_t s[1] = {E};
        if ((rc = check_tensor("corr_bias", w.corr_bias, MOE_DT_F32, 1, s))) return rc;
    }
    if (L) {
        const int64_t s1[2] = {L, H}, s2[2] = {H, L};
        if ((rc = check_tensor("fc1_latent_proj", w.fc1_w, MOE_DT_BF16, 2, s1))) return rc;
        if ((rc = check_tensor("fc2_latent_proj", w.fc2_w, MOE_DT_BF16, 2, s2))) return rc;
        // experts must live in the latent: refuse expert tensors laid out over hidden
        if (w.up_q.data && w.up_q.ndim == 3 && w.up_q.shape[2] == H * quant_bits_of(c) / 32 && H != L)
            return fail(MOE_ERR_EXPERTS_OVER_HIDDEN, "up_q: experts stored over hidden (%lld inputs), latent is %lld",
                        (long long)H, (long long)L);
        if (w.down_q.data && w.down_q.ndim == 3 && w.down_q.shape[1] == H && H != L)
            return fail(MOE_ERR_EXPERTS_OVER_HIDDEN, "down_q: experts stored over hidden (%lld outputs), latent is %lld",
                        (long long)H, (long long)L);
    }
    const int64_t qb = quant_bits_of(c), gs = c.group_size;
    {
        const int64_t q[3] = {E, I, D * qb / 32}, g[3] = {E, I, D / gs};
        if ((rc = check_tensor("up_q", w.up_q, MOE_DT_U32, 3, q))) return rc;
        if ((rc = check_tensor("up_scales", w.up_scales, MOE_DT_BF16, 3, g))) return rc;
        if ((rc = check_tensor("up_biases", w.up_biases, MOE_DT_BF16, 3, g))) return rc;
    }
    {
        const int64_t q[3] = {E, D, I * qb / 32}, g[3] = {E, D, I / gs};
        if ((rc = check_tensor("down_q", w.down_q, MOE_DT_U32, 3, q))) return rc;
        if ((rc = check_tensor("down_scales", w.down_scales, MOE_DT_BF16, 3, g))) return rc;
        if ((rc = check_tensor("down_biases", w.down_biases, MOE_DT_BF16, 3, g))) return rc;
    }
    if (SI) {
        const int64_t s1[2] = {SI, H}, s2[2] = {H, SI};
        if ((rc = check_tensor("shared_up", w.shared_up, MOE_DT_BF16, 2, s1))) return rc;
        if ((rc = check_tensor("shared_down", w.shared_down, MOE_DT_BF16, 2, s2))) return rc;
    }
    return MOE_OK;
}

static int check_device(int *dev_out, int *cus) {
    int n = 0;
    hipError_t e = hipGetDeviceCount(&n);
    if (e != hipSuccess || n < 1) return fail(MOE_ERR_DEVICE, "no HIP device (%s)", hipGetErrorString(e));
    int dev = 0;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return fail(MOE_ERR_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
    hipDeviceProp_t prop;
    if ((e = hipGetDeviceProperties(&prop, dev)) != hipSuccess)
        return fail(MOE_ERR_DEVICE, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        return fail(MOE_ERR_DEVICE, "device %d is %s; this library is built for gfx950 (MI355X)", dev,
                    prop.gcnArchName);
    *dev_out = dev;
    *cus = prop.multiProcessorCount;
    return MOE_OK;
}

// ------------------------------------------------------------------ workspace

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Items per 16-output tile of a dense projection over K inputs: each item takes K / splits
// inputs (a multiple of 128); the last of a tile's items to finish adds their partial sums.
// Tiles of 4096 inputs and more are cut in parts of 2048 (64 KB of weights, all in flight
// at once), so that a launch's items fit the machine in one round and spread evenly.
static int dense_splits_host(int K) { return K >= 4096 && K % 2048 == 0 ? K / 2048 : 1; }

// Lays out the workspace of `R` rows over `base` (nullptr: sizes only) and fills the
// workspace fields of p (split counts, counter offsets, region pointers). Returns its size in
// bytes; *n_ctr gets the number of completion counters.
static size_t layout_workspace(const moe_latent_config &c, LayerParams &p, size_t R, char *base, int *n_ctr) {
    const size_t E = c.n_experts, K = c.top_k, I = c.expert_inter, H = c.hidden;
    const size_t D = c.latent ? c.latent : c.hidden, SI = c.shared_inter, L = c.latent;
    p.ks_fc1 = dense_splits_host((int)H);
    p.ks_shup = dense_splits_host((int)H);
    // the shared down projection: whole tiles of up to 4096 inputs (128 KB), parts of 4096
    // beyond; the same for every row count, so that its sums keep one order
    p.ks_shdn = SI > 4096 && SI % 4096 == 0 ? (int)(SI / 4096) : 1;
    p.ks_fc2 = dense_splits_host(L ? (int)L : 1);
    // dense tile counters after the fixed ones
    p.ctr_fc1 = CTR_DENSE;
    p.ctr_shup = p.ctr_fc1 + (int)(L / DENSE_TILE);
    p.ctr_shdn = p.ctr_shup + (int)(SI / DENSE_TILE);
    p.ctr_fc2 = p.ctr_shdn + (SI ? (int)(H / DENSE_TILE) : 0);
    // the logit handoff words [rows][E] of decode passes (8-byte aligned, zero between forwards)
    p.ctr_hand = (p.ctr_fc2 + (L ? (int)(H / DENSE_TILE) : 0) + 1) & ~1;
    *n_ctr = p.ctr_hand + 2 * (int)E * (int)(R < (size_t)MAX_ROWS ? R : (size_t)MAX_ROWS);
    p.wait_ticks = 10000000u;   // 100 ms: far beyond any forward
    // split-K partials of decode passes: [tile][split][row][16] floats = N * splits * rows
    // floats (a decode pass takes at most MAX_ROWS rows; a prefill none of these); fc1 and
    // shared up hold at least [tile][split][wave slice][16], the front kernel's slices
    const size_t Rd = R < (size_t)MAX_ROWS ? R : (size_t)MAX_ROWS;
    const size_t Rf = Rd > (size_t)(WG_THREADS / 64) ? Rd : (size_t)(WG_THREADS / 64);
    const size_t part_fc1 = L * p.ks_fc1 * Rf * 4;
    const size_t part_shup = SI * p.ks_shup * Rf * 4;
    const size_t part_shdn = SI ? H * p.ks_shdn * Rd * 4 : 0;
    const size_t part_fc2 = L ? H * p.ks_fc2 * Rd * 4 : 0;
    const size_t max_tiles = (R * K + 63) / 64 + (E < R * K ? E : R * K);   // prefill row tiles
    enum { NREG = 22 };
    const size_t sizes[NREG] = {R * E * 4, R * K * 4, R * K * 4, (size_t)SCH_COUNT * 4, R * (L ? L : 1) * 2,
                                R * (SI ? SI : 1) * 2, R * K * I * 2, R * K * D * 2, R * D * 2,
                                R * H * 2, 256, (size_t)*n_ctr * 4, part_fc1, part_shup, part_shdn,
                                part_fc2, E * 4, R * K * 4, (E + 1) * 4, (E + 1) * 4, R * K * 4,
                                max_tiles * 4};
    size_t off[NREG], total = 0;
    for (int i = 0; i < NREG; ++i) { off[i] = total; total += align256(sizes[i]); }
    if (base) {
        p.logits = base + off[0];
        p.idx = (int32_t *)(base + off[1]);
        p.wts = (float *)(base + off[2]);
        p.sched = (int32_t *)(base + off[3]);
        p.u = (uint16_t *)(base + off[4]);
        p.shact = (uint16_t *)(base + off[5]);
        p.eact = (uint16_t *)(base + off[6]);
        p.eout = (uint16_t *)(base + off[7]);
        p.comb = (uint16_t *)(base + off[8]);
        p.shout = (uint16_t *)(base + off[9]);
        p.err = (uint32_t *)(base + off[10]);
        p.ctr = (uint32_t *)(base + off[11]);
        p.part_fc1 = (float *)(base + off[12]);
        p.part_shup = (float *)(base + off[13]);
        p.part_shdn = (float *)(base + off[14]);
        p.part_fc2 = (float *)(base + off[15]);
        p.pf_count = (int32_t *)(base + off[16]);
        p.pf_slot = (int32_t *)(base + off[17]);
        p.pf_off = (int32_t *)(base + off[18]);
        p.pf_tile = (int32_t *)(base + off[19]);
        p.pf_pairs = (int32_t *)(base + off[20]);
        p.pf_tmap = (int32_t *)(base + off[21]);
    }
    return total;
}

static int setup_workspace(moe_latent *h) {
    h->ws_bytes = layout_workspace(h->cfg, h->base, (size_t)h->cfg.max_rows, nullptr, &h->n_ctr);
    hipError_t e = dev_alloc(&h->ws, h->ws_bytes);
    if (e != hipSuccess) return fail(MOE_ERR_OOM, "workspace of %zu bytes: %s", h->ws_bytes, hipGetErrorString(e));
    layout_workspace(h->cfg, h->base, (size_t)h->cfg.max_rows, (char *)h->ws, &h->n_ctr);
    return MOE_OK;
}

// zero the error flag and the completion counters (at create, and after a device error)
static hipError_t clear_flag(moe_latent *h) {
    hipLaunchKernelGGL(moe_clear_kernel, dim3(1), dim3(64), 0, h->stream, h->base.err, 64);
    hipLaunchKernelGGL(moe_clear_kernel, dim3((h->n_ctr + 255) / 256), dim3(256), 0, h->stream, h->base.ctr,
                       h->n_ctr);
    return hipGetLastError();
}

// ------------------------------------------------------------------ API

extern "C" const char *moe_latent_last_error(void) { return g_err.c_str(); }

extern "C" int32_t moe_latent_live_allocations(void) { return g_live_allocs.load(); }

// Release everything a handle holds (each part may be missing after a failed create).
static void release(moe_latent *h) {
    if (h->side) (void)hipStreamSynchronize(h->side);
    event_destroy(h->ev_fork);
    event_destroy(h->ev_join);
    side_stream_destroy(h->side);
    dev_free(h->ws);
    h->magic = 0;
    delete h;
}

extern "C" void moe_latent_destroy(moe_latent_t *h) {
    if (!h || h->magic != kMagic) return;
    (void)hipStreamSynchronize(h->stream);
    release(h);
}

// Sizes, switches and weight pointers of a validated configuration.
static void fill_params(const moe_latent_config &c, const moe_latent_weights &w, LayerParams &p) {
    p.H = c.hidden;
    p.L = c.latent;
    p.D = c.latent ? c.latent : c.hidden;
    p.E = c.n_experts;
    p.G = c.n_group;
    p.TG = c.topk_group;
    p.K = c.top_k;
    p.I = c.expert_inter;
    p.SI = c.shared_inter;
    p.act_f16 = c.act_dtype == MOE_DT_F16;
    p.router_f32 = c.router_dtype == MOE_DT_F32;
    p.has_bias = c.has_bias != 0;
    p.norm_topk = c.norm_topk != 0;
    p.rho = c.routed_scaling;
    p.qbits = quant_bits_of(c);
    p.gs_log2 = __builtin_ctz((unsigned)c.group_size);
    p.generic = generic_format(c) ? 1 : 0;
    p.gate_w16 = p.router_f32 ? nullptr : (const uint16_t *)w.gate_w.data;
    p.gate_w32 = p.router_f32 ? (const float *)w.gate_w.data : nullptr;
    p.bias = c.has_bias ? (const float *)w.corr_bias.data : nullptr;
    p.fc1 = (const uint16_t *)w.fc1_w.data;
    p.fc2 = (const uint16_t *)w.fc2_w.data;
    p.up_q = (const uint32_t *)w.up_q.data;
    p.up_s = (const uint16_t *)w.up_scales.data;
    p.up_b = (const uint16_t *)w.up_biases.data;
    p.dn_q = (const uint32_t *)w.down_q.data;
    p.dn_s = (const uint16_t *)w.down_scales.data;
    p.dn_b = (const uint16_t *)w.down_biases.data;
    p.su = (const uint16_t *)w.shared_up.data;
    p.sd = (const uint16_t *)w.shared_down.data;
}

extern "C" int moe_latent_create(const moe_latent_config *cfg, const moe_latent_weights *w, void *hip_stream,
                                 moe_latent_t **out) {
    g_err.clear();
    if (!out) return fail(MOE_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    if (!cfg || !w) return fail(MOE_ERR_INVALID_ARG, "cfg or weights is NULL");
    int rc;
    if ((rc = check_config(*cfg))) return rc;
    if ((rc = check_weights(*cfg, *w))) return rc;
    int dev = 0, cus = 0;
    if ((rc = check_device(&dev, &cus))) return rc;

    moe_latent *h = new moe_latent();
    memset(&h->base, 0, sizeof h->base);
    h->cfg = *cfg;
    h->stream = (hipStream_t)hip_stream;
    h->side = nullptr;
    h->ev_fork = h->ev_join = nullptr;
    h->variant = 3;
    h->ws = nullptr;
    h->device = dev;
    h->magic = kMagic;
    h->last_rows = 0;
    h->cus = cus;
    h->base.cus = cus;
    fill_params(*cfg, *w, h->base);

    if ((rc = setup_workspace(h))) {
        release(h);
        return rc;
    }
    hipError_t e;
    if ((e = side_stream_create(&h->side)) != hipSuccess || (e = event_create(&h->ev_fork)) != hipSuccess ||
        (e = event_create(&h->ev_join)) != hipSuccess) {
        release(h);
        return fail(e == hipErrorOutOfMemory ? MOE_ERR_OOM : MOE_ERR_HIP, "side stream or events: %s",
                    hipGetErrorString(e));
    }
    if ((e = clear_flag(h)) != hipSuccess || (e = hipStreamSynchronize(h->stream)) != hipSuccess) {
        release(h);
        return fail(MOE_ERR_HIP, "initialising the workspace: %s", hipGetErrorString(e));
    }
    *out = h;
    return MOE_OK;
}

static bool valid(moe_latent_t *h) { return h && h->magic == kMagic; }

extern "C" int moe_latent_set_stream(moe_latent_t *h, void *hip_stream) {
    if (!valid(h)) return fail(MOE_ERR_INVALID_ARG, "invalid handle");
    h->stream = (hipStream_t)hip_stream;
    return MOE_OK;
}

// One launch of a forward: the items of stages [first, last], run by the kernel instance
// `kernel` (its template range covers them), dispatched in table order, except that with
// split >= 0 the first `pre` items of stage `split` on are dispatched first (see
// moe_stage_kernel). side: 0 on the caller's stream, 1 on the handle's side stream; join: the
// launch first waits for the side stream's work of this forward.
enum Kernel { K_GATE_SHUP, K_ROUTE_UP, K_UP_DOWN, K_FC2, K_SHUP, K_SHDN_A, K_SHDN_B, K_FRONT };
struct Launch {
    int first, last, kernel, split, pre, side, join, fork;
};
constexpr int MAX_LAUNCHES = 10;

// The launches of one forward, in enqueue order (see layer_kernels.hip). Returns their number.
//   variant 2 (two streams): the shared expert depends on nothing but the layer input, so it
//     runs on the side stream (shared up, then the two halves of shared down) while the
//     caller's stream runs the routed chain; fc2, which adds the shared output, waits for it.
//   variant 1 (one stream): the shared expert's items fill the chain's launches.
static int plan_launches(const LayerParams &p, int cus, int variant, Launch *out) {
    int n = 0;
    // variant 3 (the default): one stream for a one-row pass, two streams above. Measured on
    // the Bolt-like layer: a one-row forward takes 52 us on two streams against 38 us on one
    // (the side stream's fork and join cost more than the overlap saves in so short a pass);
    // the 64-row stack 361 us per layer against 394, the 16-row pass 149 against 151.
    if (variant == 3) variant = p.single_row ? 1 : 2;
    // variant 4: variant 1 with the first launch of a one-row pass as stage-kernel items
    const bool front = p.single_row && p.front_wgs > 0 && variant != 4;
    if (variant == 4) variant = 1;
    auto add = [&](int f, int l, int k, int split = -1, int pre = 0, int side = 0, int join = 0, int fork = 0) {
        out[n++] = Launch{f, l, k, split, pre, side, join, fork};
    };
    if (variant == 2) {
        // the side stream forks after the gate launch, but the routed chain's expert up launch
        // is enqueued (and so captured) before the side launches, so that it is dispatched
        // first when both become ready
        add(ST_GATE, ST_FC1, K_GATE_SHUP, -1, 0, 0, 0, p.SI ? 1 : 0);   // the route items end the gate stage
        if (!p.hand) add(ST_ROUTE, ST_ROUTE, K_ROUTE_UP);
        add(ST_UP, ST_UP, K_ROUTE_UP);
        if (p.SI) {
            add(ST_SHUP, ST_SHUP, K_SHUP, -1, 0, 1);
            add(ST_SHDN_A, ST_SHDN_A, K_SHDN_A, -1, 0, 1);
            add(ST_SHDN_B, ST_SHDN_B, K_SHDN_B, -1, 0, 1);
        }
        add(ST_DOWN, ST_DOWN, K_UP_DOWN);
        if (p.L) add(ST_FC2, ST_FC2, K_FC2, -1, 0, 0, p.SI ? 1 : 0);
        return n;
    }
    if (p.single_row) {
        // Expert launches: the workgroups go to the compute units round-robin in dispatch
        // order, so (cus - shared down items) expert items go first, then the 128 KB shared
        // down items, each on a compute unit of its own, then the other expert items.
        auto pre = [&](int shdn, int ex) {
            const int sd = p.item_base[shdn + 1] - p.item_base[shdn], e = p.item_base[ex + 1] - p.item_base[ex];
            const int a = cus - sd;
            return a <= 0 ? 0 : (a < e ? a : e);
        };
        add(ST_GATE, ST_SHUP, front ? K_FRONT : K_GATE_SHUP);
        add(ST_ROUTE, ST_UP, K_ROUTE_UP, ST_UP, pre(ST_SHDN_A, ST_UP));
        add(ST_SHDN_B, ST_DOWN, K_UP_DOWN, ST_DOWN, pre(ST_SHDN_B, ST_DOWN));
    } else if (p.hand) {
        // the route items (and the schedule) end the gate launch: the launches of a one-row pass
        add(ST_GATE, ST_SHUP, K_GATE_SHUP);
        add(ST_ROUTE, ST_UP, K_ROUTE_UP);
        add(ST_SHDN_B, ST_DOWN, K_UP_DOWN);
    } else {
        add(ST_GATE, ST_SHUP, K_GATE_SHUP);
        add(ST_ROUTE, ST_SHDN_A, K_ROUTE_UP);
        add(ST_UP, ST_SHDN_B, K_UP_DOWN);
        add(ST_DOWN, ST_DOWN, K_UP_DOWN);
    }
    add(ST_FC2, ST_FC2, K_FC2);
    return n;
}

// ev0, ev1: when set, the kernel's start and end are recorded into them by its own dispatch
template <int KF, int KL, bool WIDE, int QB = 0>
static void launch_kernel(const LayerParams &p, const Launch &l, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
    const int lo = p.item_base[l.first], hi = p.item_base[l.last + 1];
    const int mid = l.split >= 0 ? p.item_base[l.split] : lo, pre = l.split >= 0 ? l.pre : 0;
    if (hi <= lo) return;
    if (ev0 || ev1)
        hipExtLaunchKernelGGL((moe_stage_kernel<KF, KL, WIDE, QB>), dim3(hi - lo), dim3(WG_THREADS), 0, st, ev0, ev1,
                              0, p, lo, hi, mid, pre);
    else
        hipLaunchKernelGGL((moe_stage_kernel<KF, KL, WIDE, QB>), dim3(hi - lo), dim3(WG_THREADS), 0, st, p, lo, hi,
                           mid, pre);
}

// A launch holding routed expert items: the instance for the input width and expert format.
template <int KF, int KL>
static void launch_expert(const LayerParams &p, const Launch &l, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
    const bool wide = p.D > 2048 || p.I > 2048;
    const int qb = p.generic ? p.qbits : 0;
#define MOE_CASE(QB)                                                  \
    case QB:                                                          \
        if (wide) launch_kernel<KF, KL, true, QB>(p, l, st, ev0, ev1); \
        else launch_kernel<KF, KL, false, QB>(p, l, st, ev0, ev1);     \
        break;
    switch (qb) {
        MOE_CASE(0)
        MOE_CASE(2)
        MOE_CASE(3)
        MOE_CASE(4)
        MOE_CASE(5)
        MOE_CASE(6)
        MOE_CASE(8)
        default: break;   // widths are checked at create
    }
#undef MOE_CASE
}

// The first launch of a one-row pass as the front kernel: an empty workgroup, the row blocks,
// then the route workgroup.
static void launch_front(const LayerParams &p, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
    const int n = p.front_wgs;
    if (ev0 || ev1)
        hipExtLaunchKernelGGL(moe_front_kernel, dim3(n + 2), dim3(FRONT_THREADS), 0, st, ev0, ev1, 0, p, n);
    else
        hipLaunchKernelGGL(moe_front_kernel, dim3(n + 2), dim3(FRONT_THREADS), 0, st, p, n);
}

// Workgroups of a launch.
static int launch_items(const LayerParams &p, const Launch &l) {
    if (l.kernel == K_FRONT) return p.front_wgs + 2;
    return p.item_base[l.last + 1] - p.item_base[l.first];
}

static void launch_one(const LayerParams &p, const Launch &l, hipStream_t st, hipEvent_t ev0 = nullptr,
                       hipEvent_t ev1 = nullptr) {
    switch (l.kernel) {
        case K_FRONT: launch_front(p, st, ev0, ev1); break;
        case K_GATE_SHUP: launch_kernel<ST_GATE, ST_SHUP, false>(p, l, st, ev0, ev1); break;
        case K_ROUTE_UP: launch_expert<ST_ROUTE, ST_UP>(p, l, st, ev0, ev1); break;
        case K_UP_DOWN: launch_expert<ST_UP, ST_DOWN>(p, l, st, ev0, ev1); break;
        case K_SHUP: launch_kernel<ST_SHUP, ST_SHUP, false>(p, l, st, ev0, ev1); break;
        case K_SHDN_A: launch_kernel<ST_SHDN_A, ST_SHDN_A, false>(p, l, st, ev0, ev1); break;
        case K_SHDN_B: launch_kernel<ST_SHDN_B, ST_SHDN_B, false>(p, l, st, ev0, ev1); break;
        default: launch_kernel<ST_FC2, ST_FC2, false>(p, l, st, ev0, ev1); break;
    }
}

// Enqueue a whole forward (g == -1) on the handle's streams, or launch g alone on the caller's
// stream. A whole forward forks the side stream off the caller's stream before its first
// launch and joins it back before the launch marked `join` (or at the end), so that the
// forward starts and ends on the caller's stream (and a graph captured there holds both
// branches). evs: per launch i, events to record its kernel's start and end into (or null).
static void enqueue(const moe_latent *h, const LayerParams &p, int g, void *const *evs = nullptr) {
    Launch ls[MAX_LAUNCHES];
    const int n = plan_launches(p, h->cus, h->variant, ls);
    bool forked = false, fork_recorded = false, joined = false;
    for (int i = 0; i < n; ++i) {
        if (g != -1 && g != i) continue;
        const Launch &l = ls[i];
        hipStream_t st = h->stream;
        if (g == -1 && l.side) {
            if (!forked) {
                if (!fork_recorded) (void)hipEventRecord(h->ev_fork, h->stream);
                (void)hipStreamWaitEvent(h->side, h->ev_fork, 0);
                forked = true;
            }
            st = h->side;
        }
        if (g == -1 && l.join && forked && !joined) {
            (void)hipEventRecord(h->ev_join, h->side);
            (void)hipStreamWaitEvent(h->stream, h->ev_join, 0);
            joined = true;
        }
        launch_one(p, l, st, evs ? (hipEvent_t)evs[2 * i] : nullptr, evs ? (hipEvent_t)evs[2 * i + 1] : nullptr);
        if (g == -1 && l.fork) {   // the side stream starts after this launch
            (void)hipEventRecord(h->ev_fork, h->stream);
            fork_recorded = true;
        }
    }
    if (forked && !joined) {
        (void)hipEventRecord(h->ev_join, h->side);
        (void)hipStreamWaitEvent(h->stream, h->ev_join, 0);
    }
}

extern "C" int moe_latent_set_variant(moe_latent_t *h, int32_t variant) {
    if (!valid(h)) return fail(MOE_ERR_INVALID_ARG, "invalid handle");
    if (variant == 0)
        return fail(MOE_ERR_INVALID_ARG, "variant 0 (one fused launch per forward) is disabled: its first "
                    "GPU run did not complete (see the description of moe_latent_set_variant)");
    if (variant < 1 || variant > 4)
        return fail(MOE_ERR_INVALID_ARG, "variant %d (1: one stream, 2: two streams, 3: by row count, 4: one "
                    "stream, a one-row pass without the front kernel)", variant);
    (void)hipStreamSynchronize(h->stream);
    h->variant = variant;
    return MOE_OK;
}

static void plan_items(LayerParams &p, int rows) {
    int n[NSTAGE];
    p.rows = rows;
    p.single_row = rows == 1;
    // the route items join the gate launch, handed the logits in place (measured on the
    // Bolt-like layer against a route launch of its own: 64-row stack 338 against 354 us per
    // layer, 16-row pass 145 against 147)
    p.hand = 1;
    p.inline_comb = rows == 1 && p.L && p.L / p.ks_fc2 <= DENSE_XLDS;
    p.umax = p.E < rows * p.K ? p.E : rows * p.K;
    p.up_nb = expert_block(p.I, p.D, p.qbits, 1 << p.gs_log2);
    p.dn_nb = expert_block(p.D, p.I, p.qbits, 1 << p.gs_log2);
    p.up_blocks = p.I / p.up_nb;
    p.dn_blocks = p.D / p.dn_nb;
    // a one-row latent pass of bf16 activations: fc1 and shared up in the front kernel's row
    // blocks (one per compute unit but one, at most FRONT_ROWS_MAX rows each; K slices of at
    // most FRONT_KW_MAX inputs, at most FRONT_U_MAX of them)
    p.front_wgs = 0;
    if (rows == 1 && p.L && !p.act_f16 && p.ks_fc1 == p.ks_shup) {
        const int kpart = p.H / p.ks_fc1, ns = dense_nsplit(kpart, WG_THREADS / 64);
        const int R = p.L + p.SI;
        if (kpart / ns <= FRONT_KW_MAX && p.ks_fc1 * ns <= FRONT_U_MAX) {
            const int nb = p.cus > 1 ? p.cus - 1 : 1;
            p.front_wgs = nb > (R + FRONT_ROWS_MAX - 1) / FRONT_ROWS_MAX ? nb : (R + FRONT_ROWS_MAX - 1) / FRONT_ROWS_MAX;
        }
    }
    // dense projections: (tile of 16 outputs, K split) per item; the shared down projection's
    // tiles are cut in two halves for two launches
    const int shdn = p.SI ? p.H / DENSE_TILE : 0, ks_sd = p.ks_shdn;
    // gate: groups of 4 experts; a multi-row pass of gate rows up to 4096 (bf16) or 5120 (fp32)
    // wide splits its rows in chunks that fit the item's 32 KB of LDS
    p.gate_rc = rows > 1 && p.H <= (p.router_f32 ? 5120 : 4096) ? 16384 / p.H : rows;
    if (p.gate_rc > 16) p.gate_rc = 16;
    n[ST_GATE] = (p.E + WG_THREADS / 64 - 1) / (WG_THREADS / 64) * ((rows + p.gate_rc - 1) / p.gate_rc) +
                 (p.hand ? rows : 0);
    n[ST_FC1] = p.L ? p.L / DENSE_TILE * p.ks_fc1 : 0;
    n[ST_SHUP] = p.SI / DENSE_TILE * p.ks_shup;
    n[ST_ROUTE] = p.hand ? 0 : rows;
    n[ST_SHDN_A] = shdn / 2 * ks_sd;
    n[ST_UP] = p.umax * p.up_blocks;
    n[ST_SHDN_B] = (shdn - shdn / 2) * ks_sd;
    n[ST_DOWN] = p.umax * p.dn_blocks;
    n[ST_FC2] = p.L ? p.H / DENSE_TILE * p.ks_fc2 : 0;
    p.item_base[0] = 0;
    for (int s = 0; s < NSTAGE; ++s) p.item_base[s + 1] = p.item_base[s] + n[s];
}

// The checks of a forward's arguments (shared by the forward and its launch groups).
static int check_io(moe_latent_t *h, int32_t rows, const void *hidden_in, void *out) {
    if (!valid(h)) return fail(MOE_ERR_INVALID_ARG, "invalid handle");
    if (!hidden_in || !out) return fail(MOE_ERR_INVALID_ARG, "hidden_in or out is NULL");
    if (((uintptr_t)hidden_in | (uintptr_t)out) & 15)
        return fail(MOE_ERR_LAYOUT, "hidden_in and out must be 16-byte aligned");
    if (rows < 1 || rows > h->cfg.max_rows)
        return fail(MOE_ERR_ROWS, "rows %d outside 1..max_rows %d", rows, h->cfg.max_rows);
    if (rows > MAX_ROWS)
        return fail(MOE_ERR_ROWS, "rows %d: a decode pass takes at most %d rows (moe_latent_prefill takes up "
                    "to max_rows)", rows, (int)MAX_ROWS);
    const size_t bytes = (size_t)rows * h->cfg.hidden * 2;
    const char *a = (const char *)hidden_in, *b = (const char *)out;
    if (a != b && a < b + bytes && b < a + bytes)
        return fail(MOE_ERR_ALIAS, "out partially overlaps hidden_in");
    return MOE_OK;
}

extern "C" int moe_latent_forward(moe_latent_t *h, int32_t rows, const void *hidden_in, void *out) {
    if (int rc = check_io(h, rows, hidden_in, out)) return rc;
    LayerParams p = h->base;
    p.x = (const uint16_t *)hidden_in;
    p.out = (uint16_t *)out;
    plan_items(p, rows);
    enqueue(h, p, -1);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "launch: %s", hipGetErrorString(e));
    h->last_rows = rows;
    return MOE_OK;
}

// The layers the prefill takes: bf16 activations, 4-bit codes in groups of 64, and every
// projection's outputs a multiple of 128 (its tiles), inputs a multiple of 64.
static int check_prefill_layer(const moe_latent_config &c) {
    if (c.act_dtype != MOE_DT_BF16) return fail(MOE_ERR_DTYPE, "prefill: bf16 activations only");
    if (generic_format(c))
        return fail(MOE_ERR_SHAPE, "prefill: 4-bit codes in groups of 64 only (%d-bit, groups of %d)",
                    quant_bits_of(c), c.group_size);
    if (c.expert_inter % 128)
        return fail(MOE_ERR_SHAPE, "prefill: expert_inter %d not a multiple of 128", c.expert_inter);
    if ((long long)c.n_experts * c.hidden >= (1LL << 31))   // the gate's 32-bit row offsets
        return fail(MOE_ERR_SHAPE, "prefill: n_experts %d x hidden %d gate elements exceed 2^31 - 1",
                    c.n_experts, c.hidden);
    return MOE_OK;
}

static int grid8(long n) { return (int)(8 * ((n + 7) / 8)); }

// A launch of 128 x 128 GEMM tiles: 128 inputs a step when it has at most one tile per compute
// unit (their 128 KB of LDS then cost no occupancy) and K allows, else 64 (same bits).
template <int EPI>
static void small_gemm(const LayerParams &p, int cus, long tiles, hipStream_t st, const uint16_t *X,
                       const uint16_t *W, int N, int K) {
    if (tiles <= cus && K % 128 == 0)
        hipLaunchKernelGGL((pf_gemm_kernel<EPI, 128>), dim3(grid8(tiles)), dim3(256), 0, st, p, X, W, N, K);
    else
        hipLaunchKernelGGL((pf_gemm_kernel<EPI, 64>), dim3(grid8(tiles)), dim3(256), 0, st, p, X, W, N, K);
}

extern "C" int moe_latent_prefill(moe_latent_t *h, int32_t rows, const void *hidden_in, void *out) {
    if (!valid(h)) return fail(MOE_ERR_INVALID_ARG, "invalid handle");
    if (!hidden_in || !out) return fail(MOE_ERR_INVALID_ARG, "hidden_in or out is NULL");
    if (((uintptr_t)hidden_in | (uintptr_t)out) & 15)
        return fail(MOE_ERR_LAYOUT, "hidden_in and out must be 16-byte aligned");
    if (rows < 1 || rows > h->cfg.max_rows)
        return fail(MOE_ERR_ROWS, "rows %d outside 1..max_rows %d", rows, h->cfg.max_rows);
    {
        const size_t bytes = (size_t)rows * h->cfg.hidden * 2;
        const char *a = (const char *)hidden_in, *b = (const char *)out;
        if (a != b && a < b + bytes && b < a + bytes) return fail(MOE_ERR_ALIAS, "out partially overlaps hidden_in");
    }
    if (int rc = check_prefill_layer(h->cfg)) return rc;
    LayerParams p = h->base;
    p.x = (const uint16_t *)hidden_in;
    p.out = (uint16_t *)out;
    p.rows = rows;
    p.single_row = 0;
    p.hand = 0;   // the prefill's route kernel reads the logits from memory
    p.inline_comb = 0;
    const hipStream_t st = h->stream;
    const int E = p.E, K = p.K, NP = rows * K;
    hipLaunchKernelGGL(moe_clear_kernel, dim3((E + 255) / 256), dim3(256), 0, st, (uint32_t *)p.pf_count, E);
    {
        // waves of 8 rows x 8 experts, 4 a workgroup
        const long wb = (long)((rows + 7) / 8) * ((E + 7) / 8);
        if (p.router_f32) hipLaunchKernelGGL(pf_gate_kernel<true>, dim3((unsigned)((wb + 3) / 4)), dim3(256), 0, st, p);
        else hipLaunchKernelGGL(pf_gate_kernel<false>, dim3((unsigned)((wb + 3) / 4)), dim3(256), 0, st, p);
    }
    if (E <= 256) hipLaunchKernelGGL(pf_route_kernel<256>, dim3(rows), dim3(WG_THREADS), 0, st, p);
    else hipLaunchKernelGGL(pf_route_kernel<MAX_EXPERTS>, dim3(rows), dim3(WG_THREADS), 0, st, p);
    hipLaunchKernelGGL(pf_sched_kernel, dim3((NP + 1023) / 1024), dim3(WG_THREADS), 0, st, p);
    const int mt = (rows + 127) / 128;
    // 256 x 256 tiles for a projection of N outputs once they alone fill about the machine
    const auto big = [&](int N) { return N % 256 == 0 && (long)((rows + 255) / 256) * (N / 256) * 4 >= 3L * h->cus; };
    const auto big_tiles = [&](int N) { return grid8((long)((rows + 255) / 256) * (N / 256)); };
    // fc1 with the shared up projection in the same launch (a shared expert needs a latent
    // layer): as one matrix in big tiles of 320 outputs when those fill about the machine,
    // else the shared up projection in big tiles and fc1 alone, else 128 x 128 tiles
    const int NC = p.L + p.SI;
    const long cat_tiles = (long)((rows + 255) / 256) * (NC / 320);
    if (p.L && p.SI && NC % 320 == 0 && cat_tiles * 4 >= 3L * h->cus) {
        hipLaunchKernelGGL((pf_gemm_big_kernel<0, 320>), dim3(grid8(cat_tiles)), dim3(512), 0, st, p, p.x, p.fc1, NC,
                           p.H);
    } else if (p.L) {
        if (p.SI && big(p.SI)) {
            hipLaunchKernelGGL((pf_gemm_big_kernel<1, 256>), dim3(big_tiles(p.SI)), dim3(512), 0, st, p, p.x, p.su,
                               p.SI, p.H);
            LayerParams q = p;
            q.SI = 0;   // the fc1 launch's tiles only
            small_gemm<0>(q, h->cus, (long)mt * (p.L / 128), st, p.x, p.fc1, p.L, p.H);
        } else {
            small_gemm<0>(p, h->cus, (long)mt * ((p.L + p.SI) / 128), st, p.x, p.fc1, p.L, p.H);
        }
    }
    // expert tiles: at most one partial tile of 64 picks per expert beyond the full ones
    const long max_tiles = (NP + 63) / 64 + (E < NP ? E : NP);
    // three expert workgroups (50 KB of LDS each) to a compute unit once the launch spans
    // several rounds of them; otherwise 24 KB of unused dynamic LDS holds it to two (with few
    // rounds the last one's idle slots cost more than the third workgroup gains)
    const long up_wgs = max_tiles * ((p.I + 255) / 256), dn_wgs = max_tiles * ((p.D + 255) / 256);
    const auto pad = [&](long wgs) { return wgs >= 12L * h->cus ? 0u : 24u * 1024u; };
    hipLaunchKernelGGL(pf_expert_kernel<true>, dim3(grid8(up_wgs)), dim3(256), pad(up_wgs), st, p);
    hipLaunchKernelGGL(pf_expert_kernel<false>, dim3(grid8(dn_wgs)), dim3(256), pad(dn_wgs), st, p);
    if (p.SI && big(p.H))
        hipLaunchKernelGGL((pf_gemm_big_kernel<2, 256>), dim3(big_tiles(p.H)), dim3(512), 0, st, p, p.shact, p.sd, p.H,
                           p.SI);
    else if (p.SI)
        small_gemm<2>(p, h->cus, (long)mt * (p.H / 128), st, p.shact, p.sd, p.H, p.SI);
    hipLaunchKernelGGL(pf_combine_kernel, dim3((unsigned)(((long)rows * (p.D / 4) + 255) / 256)), dim3(256), 0, st, p);
    if (p.L && big(p.H))
        hipLaunchKernelGGL((pf_gemm_big_kernel<3, 256>), dim3(big_tiles(p.H)), dim3(512), 0, st, p, p.comb, p.fc2, p.H,
                           p.L);
    else if (p.L)
        small_gemm<3>(p, h->cus, (long)mt * (p.H / 128), st, p.comb, p.fc2, p.H, p.L);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "prefill launch: %s", hipGetErrorString(e));
    h->last_rows = rows;
    return MOE_OK;
}

extern "C" int moe_latent_launch_group(moe_latent_t *h, int32_t rows, const void *hidden_in, void *out,
                                       int32_t group) {
    if (int rc = check_io(h, rows, hidden_in, out)) return rc;
    LayerParams p = h->base;
    p.x = (const uint16_t *)hidden_in;
    p.out = (uint16_t *)out;
    plan_items(p, rows);
    Launch ls[MAX_LAUNCHES];
    const int n = plan_launches(p, h->cus, h->variant, ls);
    if (group < 0 || group >= n) return fail(MOE_ERR_INVALID_ARG, "group %d outside 0..%d", group, n - 1);
    enqueue(h, p, group);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "launch: %s", hipGetErrorString(e));
    return MOE_OK;
}

extern "C" int moe_latent_forward_timed(moe_latent_t *h, int32_t rows, const void *hidden_in, void *out,
                                        void *const *events, int32_t n_events) {
    if (int rc = check_io(h, rows, hidden_in, out)) return rc;
    LayerParams p = h->base;
    p.x = (const uint16_t *)hidden_in;
    p.out = (uint16_t *)out;
    plan_items(p, rows);
    Launch ls[MAX_LAUNCHES];
    const int n = plan_launches(p, h->cus, h->variant, ls);
    if (!events || n_events < 2 * n)
        return fail(MOE_ERR_INVALID_ARG, "events: %d given, 2 per launch group (%d groups) needed", n_events, n);
    for (int i = 0; i < 2 * n; ++i)
        if (!events[i]) return fail(MOE_ERR_INVALID_ARG, "events[%d] is NULL", i);
    enqueue(h, p, -1, events);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "launch: %s", hipGetErrorString(e));
    h->last_rows = rows;
    return MOE_OK;
}

extern "C" int moe_latent_stream_read(const void *src, size_t bytes, uint32_t *sink_dev, void *hip_stream) {
    if (!src || !sink_dev) return fail(MOE_ERR_INVALID_ARG, "stream_read: src or sink is NULL");
    if (((uintptr_t)src & 15) || (bytes & 15) || bytes == 0 || bytes > ((size_t)1 << 40))
        return fail(MOE_ERR_INVALID_ARG, "stream_read: src must be 16-byte aligned and bytes a nonzero multiple of 16 "
                    "up to 2^40 (%zu)", bytes);
    // one workgroup of 256 threads per compute unit, each thread with 8 loads in flight
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < 1)
        cus = 256;
    hipLaunchKernelGGL(moe_stream_read_kernel, dim3(cus), dim3(256), 0, (hipStream_t)hip_stream,
                       (const uint4 *)src, bytes / 16, sink_dev);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "stream_read launch: %s", hipGetErrorString(e));
    return MOE_OK;
}

extern "C" int moe_latent_group_items(moe_latent_t *h, int32_t rows, int32_t group) {
    if (!valid(h) || rows < 1 || rows > h->cfg.max_rows || rows > MAX_ROWS) return -1;
    LayerParams p = h->base;
    plan_items(p, rows);
    Launch ls[MAX_LAUNCHES];
    const int n = plan_launches(p, h->cus, h->variant, ls);
    if (group < 0 || group >= n) return 0;
    return launch_items(p, ls[group]);
}

extern "C" int moe_latent_group_stages(moe_latent_t *h, int32_t rows, int32_t group, int32_t *first_stage,
                                       int32_t *last_stage, int32_t *side) {
    if (!valid(h) || rows < 1 || rows > h->cfg.max_rows || rows > MAX_ROWS) return -1;
    LayerParams p = h->base;
    plan_items(p, rows);
    Launch ls[MAX_LAUNCHES];
    const int n = plan_launches(p, h->cus, h->variant, ls);
    if (group < 0 || group >= n) return 0;
    if (first_stage) *first_stage = ls[group].first;
    if (last_stage) *last_stage = ls[group].last;
    if (side) *side = ls[group].side;
    return launch_items(p, ls[group]);
}

// The kernel a launch runs, as a profiler names it (without namespace and arguments).
static void kernel_name(const LayerParams &p, const Launch &l, char *buf, size_t cap) {
    const char *wide = p.D > 2048 || p.I > 2048 ? "true" : "false";
    const int qb = p.generic ? p.qbits : 0;
    switch (l.kernel) {
        case K_FRONT: snprintf(buf, cap, "moe_front_kernel"); break;
        case K_GATE_SHUP: snprintf(buf, cap, "moe_stage_kernel<%d, %d, false, 0>", ST_GATE, ST_SHUP); break;
        case K_ROUTE_UP: snprintf(buf, cap, "moe_stage_kernel<%d, %d, %s, %d>", ST_ROUTE, ST_UP, wide, qb); break;
        case K_UP_DOWN: snprintf(buf, cap, "moe_stage_kernel<%d, %d, %s, %d>", ST_UP, ST_DOWN, wide, qb); break;
        case K_SHUP: snprintf(buf, cap, "moe_stage_kernel<%d, %d, false, 0>", ST_SHUP, ST_SHUP); break;
        case K_SHDN_A: snprintf(buf, cap, "moe_stage_kernel<%d, %d, false, 0>", ST_SHDN_A, ST_SHDN_A); break;
        case K_SHDN_B: snprintf(buf, cap, "moe_stage_kernel<%d, %d, false, 0>", ST_SHDN_B, ST_SHDN_B); break;
        default: snprintf(buf, cap, "moe_stage_kernel<%d, %d, false, 0>", ST_FC2, ST_FC2); break;
    }
}

extern "C" int moe_latent_group_kernel(moe_latent_t *h, int32_t rows, int32_t group, char *name, int32_t cap) {
    if (!valid(h) || rows < 1 || rows > h->cfg.max_rows || rows > MAX_ROWS || !name || cap < 1) return -1;
    LayerParams p = h->base;
    plan_items(p, rows);
    Launch ls[MAX_LAUNCHES];
    const int n = plan_launches(p, h->cus, h->variant, ls);
    name[0] = 0;
    if (group < 0 || group >= n) return 0;
    char buf[96];
    kernel_name(p, ls[group], buf, sizeof buf);
    snprintf(name, (size_t)cap, "%s", buf);
    return (int)strlen(name);
}

extern "C" int moe_latent_get_routing(moe_latent_t *h, int32_t *idx_dev, float *w_dev) {
    if (!valid(h)) return fail(MOE_ERR_INVALID_ARG, "invalid handle");
    if (!h->last_rows) return fail(MOE_ERR_INVALID_ARG, "no forward yet");
    const size_t n = (size_t)h->last_rows * h->cfg.top_k;
    hipError_t e = hipSuccess;
    if (idx_dev) e = hipMemcpyAsync(idx_dev, h->base.idx, n * 4, hipMemcpyDeviceToDevice, h->stream);
    if (e == hipSuccess && w_dev) e = hipMemcpyAsync(w_dev, h->base.wts, n * 4, hipMemcpyDeviceToDevice, h->stream);
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "routing copy: %s", hipGetErrorString(e));
    return MOE_OK;
}

extern "C" int moe_latent_read_stage(moe_latent_t *h, int32_t stage, void *dst_dev, size_t bytes) {
    if (!valid(h)) return fail(MOE_ERR_INVALID_ARG, "invalid handle");
    if (!dst_dev) return fail(MOE_ERR_INVALID_ARG, "dst is NULL");
    if (!h->last_rows) return fail(MOE_ERR_INVALID_ARG, "no forward yet");
    const LayerParams &p = h->base;
    const size_t R = h->last_rows;
    const void *src = nullptr;
    size_t avail = 0;
    switch (stage) {
    case MOE_STAGE_LOGITS: src = p.logits; avail = R * p.E * (p.router_f32 ? 4 : 2); break;
    case MOE_STAGE_LATENT:
        if (!p.L) return fail(MOE_ERR_INVALID_ARG, "non-latent layer: the latent is hidden_in");
        src = p.u; avail = R * p.L * 2; break;
    case MOE_STAGE_EXPERT_ACT: src = p.eact; avail = R * p.K * p.I * 2; break;
    case MOE_STAGE_EXPERT_OUT: src = p.eout; avail = R * p.K * p.D * 2; break;
    case MOE_STAGE_COMBINE: src = p.comb; avail = R * p.D * 2; break;
    case MOE_STAGE_SHARED_ACT:
        if (!p.SI) return fail(MOE_ERR_INVALID_ARG, "no shared expert");
        src = p.shact; avail = R * p.SI * 2; break;
    case MOE_STAGE_SHARED_OUT:
        if (!p.SI) return fail(MOE_ERR_INVALID_ARG, "no shared expert");
        src = p.shout; avail = R * p.H * 2; break;
    default: return fail(MOE_ERR_INVALID_ARG, "unknown stage %d", stage);
    }
    if (bytes > avail) return fail(MOE_ERR_INVALID_ARG, "stage %d holds %zu bytes, %zu asked", stage, avail, bytes);
    hipError_t e = hipMemcpyAsync(dst_dev, src, bytes, hipMemcpyDeviceToDevice, h->stream);
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "stage copy: %s", hipGetErrorString(e));
    return MOE_OK;
}

extern "C" int moe_latent_status(moe_latent_t *h) {
    if (!valid(h)) return fail(MOE_ERR_INVALID_ARG, "invalid handle");
    hipError_t e = hipStreamSynchronize(h->stream);
    if (e == hipSuccess) e = hipStreamSynchronize(h->side);
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "stream: %s", hipGetErrorString(e));
    uint32_t flag = 0;
    e = hipMemcpy(&flag, h->base.err, 4, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "reading the error flag: %s", hipGetErrorString(e));
    if (flag) {
        (void)clear_flag(h);
        (void)hipStreamSynchronize(h->stream);
        return fail(MOE_ERR_DEVICE_CHECK, "device-side error flag %u (2: a route found no candidate, "
                    "4: an invalid schedule)", flag);
    }
    return MOE_OK;
}

// ------------------------------------------------------------------ forward without allocation

// The workspace of moe_latent_forward_static: one array per GPU, held until the process ends.
// Host code never uses its name as an address (that is a host-side stand-in): the device
// address of each GPU's copy is taken once, with that GPU current, and kept in g_scratch.
static __device__ __align__(256) unsigned char scratch[MOE_LATENT_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices];   // device address of scratch on each GPU (nullptr: not taken yet)
int g_scratch_cus[kMaxDevices];
}  // namespace

// The current device's scratch address and compute-unit count (taken on its first use).
static int scratch_of_current_device(void **ptr, int *cus) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_DEVICE, "device %d beyond the %d this library tracks", dev, kMaxDevices);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess || !p)
            return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        int n = 0;
        if ((e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess || n < 1)
            return fail(MOE_ERR_HIP, "compute unit count: %s", hipGetErrorString(e));
        g_scratch[dev] = p;
        g_scratch_cus[dev] = n;
    }
    *ptr = g_scratch[dev];
    *cus = g_scratch_cus[dev];
    return MOE_OK;
}

extern "C" int moe_latent_forward_static(const moe_latent_config *cfg, const moe_latent_weights *w, int32_t rows,
                                         const void *hidden_in, void *out, void *hip_stream) {
    g_err.clear();
    if (!cfg || !w) return fail(MOE_ERR_INVALID_ARG, "cfg or weights is NULL");
    int rc;
    if ((rc = check_config(*cfg))) return rc;
    if ((rc = check_weights(*cfg, *w))) return rc;
    int dev = 0, cus = 0;
    if ((rc = check_device(&dev, &cus))) return rc;
    if (!hidden_in || !out) return fail(MOE_ERR_INVALID_ARG, "hidden_in or out is NULL");
    if (((uintptr_t)hidden_in | (uintptr_t)out) & 15)
        return fail(MOE_ERR_LAYOUT, "hidden_in and out must be 16-byte aligned");
    if (rows < 1 || rows > cfg->max_rows || rows > MAX_ROWS)
        return fail(MOE_ERR_ROWS, "rows %d outside 1..%d (max_rows, at most %d)", rows, cfg->max_rows, (int)MAX_ROWS);
    const size_t bytes = (size_t)rows * cfg->hidden * 2;
    const char *a = (const char *)hidden_in, *b = (const char *)out;
    if (a != b && a < b + bytes && b < a + bytes) return fail(MOE_ERR_ALIAS, "out partially overlaps hidden_in");

    LayerParams p;
    memset(&p, 0, sizeof p);
    fill_params(*cfg, *w, p);
    int n_ctr = 0;
    const size_t need = layout_workspace(*cfg, p, (size_t)rows, nullptr, &n_ctr);
    if (need > MOE_LATENT_STATIC_SCRATCH_BYTES)
        return fail(MOE_ERR_SHAPE, "the workspace of %d rows of this layer needs %zu bytes; the static scratch "
                    "holds %zu (use moe_latent_create / moe_latent_forward, or fewer rows)",
                    rows, need, (size_t)MOE_LATENT_STATIC_SCRATCH_BYTES);
    void *base = nullptr;
    if ((rc = scratch_of_current_device(&base, &cus))) return rc;
    layout_workspace(*cfg, p, (size_t)rows, (char *)base, &n_ctr);
    p.cus = cus;
    p.x = (const uint16_t *)hidden_in;
    p.out = (uint16_t *)out;
    plan_items(p, rows);
    hipStream_t st = (hipStream_t)hip_stream;
    // the counters and the error flag start at zero (the previous call, maybe of another
    // layer, left its own contents): fill kernels, no memset
    hipLaunchKernelGGL(moe_clear_kernel, dim3(1), dim3(64), 0, st, p.err, 64);
    hipLaunchKernelGGL(moe_clear_kernel, dim3((n_ctr + 255) / 256), dim3(256), 0, st, p.ctr, n_ctr);
    Launch ls[MAX_LAUNCHES];
    const int n = plan_launches(p, cus, 1, ls);   // one stream: this call owns no side stream
    for (int i = 0; i < n; ++i) launch_one(p, ls[i], st);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "launch: %s", hipGetErrorString(e));
    return MOE_OK;
}

// ------------------------------------------------------------------ lm_head gemv

extern "C" int moe_lm_head_gemv(const moe_tensor *w, int32_t rows, const void *x, void *out, int32_t out_dtype,
                                void *hip_stream) {
    g_err.clear();
    if (!w) return fail(MOE_ERR_INVALID_ARG, "lm_head: weight descriptor is NULL");
    if (w->ndim != 2) return fail(MOE_ERR_LAYOUT, "lm_head: rank %d, expected 2 ([N][K])", w->ndim);
    const int64_t N = w->shape[0], K = w->shape[1];
    {
        const int64_t shape[2] = {N, K};
        int rc = check_tensor("lm_head", *w, MOE_DT_BF16, 2, shape);
        if (rc) return rc;
    }
    if (N < 16 || N % 16 || N / 16 > (int64_t)1 << 30)
        return fail(MOE_ERR_SHAPE, "lm_head: N %lld must be a positive multiple of 16 (tiles of 16 outputs)",
                    (long long)N);
    if (K < 128 || K % 128 || K > (int64_t)1 << 20)
        return fail(MOE_ERR_SHAPE, "lm_head: K %lld must be a multiple of 128, at most 2^20", (long long)K);
    if (rows < 1 || rows > MAX_ROWS) return fail(MOE_ERR_ROWS, "lm_head: rows %d outside 1..%d", rows, (int)MAX_ROWS);
    if (out_dtype != MOE_DT_BF16 && out_dtype != MOE_DT_F32)
        return fail(MOE_ERR_DTYPE, "lm_head: out dtype %s (bf16 or f32)", dt_name(out_dtype));
    if (!x || !out) return fail(MOE_ERR_INVALID_ARG, "lm_head: x or out is NULL");
    if (((uintptr_t)x | (uintptr_t)out) & 15) return fail(MOE_ERR_LAYOUT, "lm_head: x and out must be 16-byte aligned");
    const size_t xb = (size_t)rows * K * 2, ob = (size_t)rows * N * (out_dtype == MOE_DT_F32 ? 4 : 2);
    const char *xa = (const char *)x, *oa = (const char *)out, *wa = (const char *)w->data;
    const size_t wb = (size_t)N * K * 2;
    if ((xa < oa + ob && oa < xa + xb) || (wa < oa + ob && oa < wa + wb))
        return fail(MOE_ERR_ALIAS, "lm_head: out overlaps x or the weights");
    int dev = 0, cus = 0, rc;
    if ((rc = check_device(&dev, &cus))) return rc;
    LayerParams p;
    memset(&p, 0, sizeof p);
    p.rows = rows;
    p.lm_out = out;
    p.lm_n = (int)N;
    p.lm_f32 = out_dtype == MOE_DT_F32;
    hipLaunchKernelGGL(moe_lm_head_kernel, dim3((unsigned)(N / 16)), dim3(WG_THREADS), 0, (hipStream_t)hip_stream, p,
                       (const uint16_t *)w->data, (const uint16_t *)x, (int)K, 0);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "lm_head launch: %s", hipGetErrorString(e));
    return MOE_OK;
}
