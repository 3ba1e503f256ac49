// layer_kernels.hip -- the decode kernels of one latent mixture-of-experts layer (gfx950):
// the stage kernel that runs any contiguous range of a forward's work items (layer_items.h
// describes the items and their arithmetic), the lm_head gemv, and small helpers.
#include "layer_items.h"

namespace moe {

// ------------------------------------------------------------------ driver

constexpr int NW = WG_THREADS / 64;    // waves of a workgroup

// Kernels: each covers the stages [FIRST, LAST] (the host launches any contiguous range of
// items inside them); WIDE selects the expert variant for inputs wider than 2048.
struct NoLds {};

// widest expert input row of a kernel variant
#define XMAX_OF(wide) ((wide) ? 6144 : 2048)

template <int FIRST, int LAST, bool WIDE>
struct StageLds {
    static constexpr bool has(int s) { return FIRST <= s && s <= LAST; }
    static constexpr bool dense = has(ST_FC1) || has(ST_SHUP) || has(ST_SHDN_A) || has(ST_SHDN_B) || has(ST_FC2);
    union U {
        typename std::conditional<dense, DenseLds<NW>, NoLds>::type dense;
        typename std::conditional<has(ST_GATE) || has(ST_ROUTE), RouteLds<WG_THREADS>, NoLds>::type route;
        typename std::conditional<has(ST_GATE), GateLds, NoLds>::type gate;
        typename std::conditional<has(ST_GATE) || has(ST_ROUTE), SchedLds, NoLds>::type sched;
        typename std::conditional<has(ST_UP) || has(ST_DOWN), ExpertLds<XMAX_OF(WIDE)>, NoLds>::type ex;
    };
};

// QB: 0 for the fused 4-bit expert items (codes in groups of 64), else the code width of the
// width-generic expert items.
template <int S, bool WIDE, int QB, class LdsT>
__device__ __forceinline__ void run_stage(const LayerParams &p, int local, LdsT &lds, int *s_flag) {
    if constexpr (S == ST_GATE) {
        // with the hand-off, the last `rows` items route the rows with the logits the gate
        // items (all dispatched before them) hand them; the last of them builds the schedule
        const int ngate = p.item_base[ST_GATE + 1] - p.item_base[ST_GATE] - (p.hand ? p.rows : 0);
        if (local >= ngate) {
            route_item<WG_THREADS>(p, local - ngate, lds.route);
            if (!p.single_row && last_arriver(p.ctr + CTR_ROUTE, (uint32_t)p.rows, s_flag)) {
                __syncthreads();
                sched_item(p, lds.sched);
            }
        } else {
            gate_item<NW>(p, local, lds.gate);
        }
    } else if constexpr (S == ST_FC1) {
        const int ks = p.ks_fc1;
        dense_item<EPI_FC1, NW>(p, p.fc1, p.x, p.H, local / ks, local % ks, ks, p.part_fc1, p.ctr + p.ctr_fc1,
                                lds.dense, s_flag);
    } else if constexpr (S == ST_SHUP) {
        const int ks = p.ks_shup;
        dense_item<EPI_SHUP, NW>(p, p.su, p.x, p.H, local / ks, local % ks, ks, p.part_shup, p.ctr + p.ctr_shup,
                                 lds.dense, s_flag);
    } else if constexpr (S == ST_ROUTE) {
        route_item<WG_THREADS>(p, local, lds.route);
        if (last_arriver(p.ctr + CTR_ROUTE, (uint32_t)p.rows, s_flag)) {
            __syncthreads();
            sched_item(p, lds.sched);
        }
    } else if constexpr (S == ST_SHDN_A || S == ST_SHDN_B) {
        const int ks = p.ks_shdn;
        const int it = local + (S == ST_SHDN_B ? p.item_base[ST_SHDN_A + 1] - p.item_base[ST_SHDN_A] : 0);
        dense_item<EPI_SHDN, NW>(p, p.sd, p.shact, p.SI, it / ks, it % ks, ks, p.part_shdn, p.ctr + p.ctr_shdn,
                                 lds.dense, s_flag);
    } else if constexpr (S == ST_UP) {
        const int slot = local / p.up_blocks, blk = local % p.up_blocks;
        if constexpr (QB != 0) qexpert_item<QB, true, XMAX_OF(WIDE)>(p, slot, blk, lds.ex);
        else if (p.act_f16) expert_item<true, XMAX_OF(WIDE), true>(p, slot, blk, lds.ex);
        else expert_item<true, XMAX_OF(WIDE), false>(p, slot, blk, lds.ex);
    } else if constexpr (S == ST_DOWN) {
        const int slot = local / p.dn_blocks, blk = local % p.dn_blocks;
        int U;
        if constexpr (QB != 0) U = qexpert_item<QB, false, XMAX_OF(WIDE)>(p, slot, blk, lds.ex);
        else U = p.act_f16 ? expert_item<false, XMAX_OF(WIDE), true>(p, slot, blk, lds.ex)
                           : expert_item<false, XMAX_OF(WIDE), false>(p, slot, blk, lds.ex);
        if (slot < U && !p.inline_comb && last_arriver(p.ctr + CTR_BLOCK + blk, (uint32_t)U, s_flag))
            combine_block(p, blk * p.dn_nb, p.dn_nb);
    } else if constexpr (S == ST_FC2) {
        const int ks = p.ks_fc2;
        dense_item<EPI_FC2, NW>(p, p.fc2, p.comb, p.L, local / ks, local % ks, ks, p.part_fc2, p.ctr + p.ctr_fc2,
                                lds.dense, s_flag);
    }
}

template <int FIRST, int LAST, bool WIDE, int QB, int S, class LdsT>
__device__ __forceinline__ void dispatch(const LayerParams &p, int it, LdsT &lds, int *s_flag) {
    if constexpr (S <= LAST) {
        if (it < p.item_base[S + 1]) {
            run_stage<S, WIDE, QB>(p, it - p.item_base[S], lds, s_flag);
            return;
        }
        dispatch<FIRST, LAST, WIDE, QB, S + 1>(p, it, lds, s_flag);
    }
}

// Waves per SIMD the register allocation aims for: 3 (three items per compute unit: what
// the expert stages' LDS allows, and enough for every item of the first launch at once), and
// 2 for fc2 (one item per compute unit).
constexpr int waves_target(int first, int last, bool wide) {
    (void)last;
    (void)wide;
    return first == ST_FC2 ? 2 : 3;
}

// Runs items [lo, hi) of the table, which must lie in the stages [FIRST, LAST]. The hardware
// dispatches workgroups in index order: workgroups 0 .. pre - 1 take items mid .. mid + pre
// - 1, the next ones items lo .. mid - 1, the rest items mid + pre .. hi - 1 (pre = 0: table
// order). QB: the routed expert items' code width (0: the fused 4-bit items).
template <int FIRST, int LAST, bool WIDE, int QB>
__global__ void __launch_bounds__(WG_THREADS) __attribute__((amdgpu_waves_per_eu(waves_target(FIRST, LAST, WIDE), 8)))
moe_stage_kernel(LayerParams p, int lo, int hi, int mid, int pre) {
    __shared__ typename StageLds<FIRST, LAST, WIDE>::U lds;
    __shared__ int s_flag;
    const int b = (int)blockIdx.x;
    const int it = b < pre ? mid + b : b < pre + (mid - lo) ? lo + b - pre : lo + b;
    if (it >= hi) return;
    dispatch<FIRST, LAST, WIDE, QB, FIRST>(p, it, lds, &s_flag);
}

template __global__ void moe_stage_kernel<ST_GATE, ST_SHUP, false, 0>(LayerParams, int, int, int, int);
template __global__ void moe_stage_kernel<ST_FC2, ST_FC2, false, 0>(LayerParams, int, int, int, int);
// the shared expert on its own stream
template __global__ void moe_stage_kernel<ST_SHUP, ST_SHUP, false, 0>(LayerParams, int, int, int, int);
template __global__ void moe_stage_kernel<ST_SHDN_A, ST_SHDN_A, false, 0>(LayerParams, int, int, int, int);
template __global__ void moe_stage_kernel<ST_SHDN_B, ST_SHDN_B, false, 0>(LayerParams, int, int, int, int);
// the launches holding routed expert items, for each expert format
#define MOE_EXPERT_KERNELS(QB)                                                                        \
    template __global__ void moe_stage_kernel<ST_ROUTE, ST_UP, false, QB>(LayerParams, int, int, int, int); \
    template __global__ void moe_stage_kernel<ST_ROUTE, ST_UP, true, QB>(LayerParams, int, int, int, int);  \
    template __global__ void moe_stage_kernel<ST_UP, ST_DOWN, false, QB>(LayerParams, int, int, int, int);  \
    template __global__ void moe_stage_kernel<ST_UP, ST_DOWN, true, QB>(LayerParams, int, int, int, int);
MOE_EXPERT_KERNELS(0)
MOE_EXPERT_KERNELS(2)
MOE_EXPERT_KERNELS(3)
MOE_EXPERT_KERNELS(4)
MOE_EXPERT_KERNELS(5)
MOE_EXPERT_KERNELS(6)
MOE_EXPERT_KERNELS(8)
#undef MOE_EXPERT_KERNELS

// The first launch of a one-row pass. Workgroup 0 does nothing: the route workgroup,
// dispatched last, goes to the compute unit it leaves, where no weights stream (a compute
// unit holds one workgroup of this kernel's size at 4 waves per SIMD, so that unit is the
// only one with room). Workgroups 1 .. n take the row blocks of fc1 and the shared up
// projection (rows [(b-1) R / n, b R / n) of the R rows), their last wave the gate rows b - 1,
// b - 1 + n, ...; workgroup n + 1 routes the row with the logits the gate waves hand it (its
// wait is bounded, see route_item; every workgroup it waits for was dispatched before it).
__global__ void __launch_bounds__(FRONT_THREADS) __attribute__((amdgpu_waves_per_eu(4, 8)))
moe_front_kernel(LayerParams p, int n) {
    __shared__ FrontLds lds;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, b = (int)blockIdx.x;
    if (b > n) {
        route_item<FRONT_THREADS>(p, 0, lds.route);
        return;
    }
    if (b == 0) return;
    const int w = b - 1, R = p.L + p.SI;
    const int r0 = (int)((long)w * R / n), r1 = (int)((long)(w + 1) * R / n);
    if (wave == FRONT_SW) {
        for (int e = w; e < p.E; e += n) gate_expert(p, e, 0, 1, lane);
    } else {
        front_rows<MOE_FRONT_DEP>(p, r0, r1, wave, lane, lds);
    }
    __syncthreads();
    front_join(p, r0, r1, lds);
}

// Read-only stream: n 16-byte units, 8 nontemporal loads in flight per thread per round,
// grid-stride (one workgroup per compute unit: the fastest shape measured on this machine);
// the data is folded into one XOR per workgroup so that the loads are kept.
__global__ void __launch_bounds__(256) moe_stream_read_kernel(const uint4 *__restrict__ src, size_t n, uint32_t *sink) {
    __shared__ uint32_t red[256];
    const size_t stride = (size_t)gridDim.x * 256;
    uint32_t acc = 0;
    size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    for (; i + 7 * stride < n; i += 8 * stride) {
        uint4 v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = ld_weight16(src + i + q * stride);
#pragma unroll
        for (int q = 0; q < 8; ++q) acc ^= v[q].x ^ v[q].y ^ v[q].z ^ v[q].w;
    }
    for (; i < n; i += stride) {
        const uint4 v = src[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    red[threadIdx.x] = acc;
    __syncthreads();
    if (threadIdx.x < 64) {
        uint32_t r = red[threadIdx.x] ^ red[threadIdx.x + 64] ^ red[threadIdx.x + 128] ^ red[threadIdx.x + 192];
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) r ^= __shfl_xor(r, d, 64);
        if (threadIdx.x == 0) atomicXor(sink, r);
    }
}

// The bf16 lm_head gemv (TensorFold pull request 1038, «Per operator and row invariance»,
// the lm_head rows: K = 4096 inputs, N = 131072 outputs, at 1 and 16 rows): out = W . x for
// every row, fp32 sums, with the layer's dense tiles -- 16 outputs over all K per workgroup,
// each input row its own MFMA column, so a row's result does not depend on the other rows.
// One workgroup per tile; tiles [lo, hi) of this launch.
__global__ void __launch_bounds__(WG_THREADS) __attribute__((amdgpu_waves_per_eu(3, 8)))
moe_lm_head_kernel(LayerParams p, const uint16_t *__restrict__ W, const uint16_t *__restrict__ X, int K, int lo) {
    __shared__ DenseLds<WG_THREADS / 64> lds;
    __shared__ int s_flag;
    dense_item<EPI_LMH, WG_THREADS / 64>(p, W, X, K, lo + (int)blockIdx.x, 0, 1, nullptr, nullptr, lds, &s_flag);
}

// zero a small device buffer (the error flag) without a memset node in captured graphs
__global__ void moe_clear_kernel(uint32_t *ctr, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) ctr[i] = 0u;
}

}  // namespace moe
