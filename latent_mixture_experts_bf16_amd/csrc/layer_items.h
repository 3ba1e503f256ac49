// layer_items.h -- the work items of one latent mixture-of-experts layer (gfx950 device code
// shared by the decode kernels, layer_kernels.hip, and the prefill kernels, prefill_kernels.hip).
//
// A forward is a table of work items (tiles of each stage, see layer_plan.h) run as a short
// chain of launches on one stream; stages that do not depend on each other share a launch,
// and steps that need every item of a stage (schedule after the route, the adding of a
// split tile's parts, combine after the experts of a block) are run by the last item to
// finish. The one exception: in a one-row pass the route item (the last gate item of the first
// launch) waits, bounded, for the logits the gate items dispatched before it hand it.
//   one row:   [gate, route, fc1, shared up] -> [expert up, shared down A] ->
//              [expert down, shared down B] -> [combine + fc2 + shared + residual]
//   more rows: [gate, fc1, shared up] -> [route; schedule, shared down A] ->
//              [expert up, shared down B] -> [expert down; combine] -> [fc2 + ...]
//   (passes of more rows run the shared expert on a second stream by default: see
//   moe_latent_api.hip, plan_launches)
// One workgroup of 4 waves runs one item; a launch's items are sized (about 32-64 KB of
// weights each) so that all of them are resident at once (three per compute unit: the
// expert launches' LDS holds a 32 KB block of codes, and the dense tiles' registers hold four
// steps of weights and their way into MFMA fragments).
//
// Arithmetic of each stage (TensorFold pull request 1038, «What's in it»: gate gemv ->
// route top-k -> fc1_latent_proj -> routed experts -> combine -> fc2_latent_proj -> +
// shared -> + residual), with fp32 accumulation and rounding to the activation dtype after
// every step:
//   gate     z = rnd(sum x*w) in a fixed order: lane t of a wave accumulates k = 512j+8t+i
//            (j outer, i inner) from +0 with fused multiply-adds, then the 64 partials are
//            joined by an xor butterfly 32, 16, 8, 4, 2, 1 -- so logits are reproducible
//            bit for bit and routing with them.
//   route    sigmoid evaluated in binary64 and rounded once to fp32; bias added for
//            selection only; group score = sum of the two best biased scores of a group;
//            top groups, then top-k experts by (score desc, id asc), NaN lowest; weights
//            = (s / sum of s in pick order) * rho.
//   dense    (fc1, shared up/down, fc2): bf16 MFMA 16x16x32 tiles, K split over the 4
//            waves of a workgroup and joined in a fixed order (projections of 4096 inputs
//            and more are also split over items, the last of which adds their partial
//            sums in split order). A row's result never depends
//            on the other rows of the pass (each output row of a tile is its own column of
//            the MFMA), so a multi-row pass equals its one-row passes bit for bit.
//   experts  4-bit affine weights w = q*scale + bias (groups of 64 along k); per 32 inputs
//            the kernel forms sum(q*x) and sum(x) and adds scale*sum(q*x) + bias*sum(x):
//            the same value as sum(w*x) up to fp32 summation order. Each picked expert's
//            weights are read once for all the rows that picked it.
//   combine  8 lanes: lane t sums w_j*y_j over picks j = t, t+8, ... (pick 8 onto pick 0),
//            joined as ((T0+T4)+(T2+T6)) + ((T1+T5)+(T3+T7)).
//   final    out = rnd(x + rnd(rnd(fc2) + shared)).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layer_plan.h"
#include <type_traits>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ number formats

__device__ __forceinline__ float bf2f(uint32_t h) { return __uint_as_float(h << 16); }

__device__ __forceinline__ uint16_t f2bf(float f) {
    uint32_t b = __float_as_uint(f);
    if ((b & 0x7F800000u) == 0x7F800000u && (b & 0x007FFFFFu)) return (uint16_t)((b >> 16) | 0x40u);
    return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ float h2f(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

__device__ __forceinline__ uint16_t f2h(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// both conversions, then a select: no branch per element
__device__ __forceinline__ float act2f(int f16, uint32_t h) {
    const float a = h2f(h), b = bf2f(h);
    return f16 ? a : b;
}
__device__ __forceinline__ uint16_t f2act(int f16, float v) { return f16 ? f2h(v) : f2bf(v); }
__device__ __forceinline__ float rnd(int f16, float v) { return act2f(f16, f2act(f16, v)); }

__device__ __forceinline__ float relu_sq(int f16, float h) {
    float r = h > 0.0f ? h : 0.0f;
    return rnd(f16, r * r);
}

// 8 packed 16-bit activations -> fp32
__device__ __forceinline__ void unpack8(int f16, uint4 v, float *o) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        o[2 * i] = act2f(f16, w[i] & 0xFFFFu);
        o[2 * i + 1] = act2f(f16, w[i] >> 16);
    }
}

// the 8 codes of one word, in k order (lowest nibble first), as fp32: the even and the odd
// nibbles are first masked into bytes, each then converted by a byte-to-float conversion
// (the empty asm keeps the compiler from re-extracting single nibbles instead)
__device__ __forceinline__ void nibbles8(uint32_t w, float *q) {
    uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
    asm("" : "+v"(lo), "+v"(hi));
    q[0] = (float)(lo & 0xFFu);
    q[1] = (float)(hi & 0xFFu);
    q[2] = (float)((lo >> 8) & 0xFFu);
    q[3] = (float)((hi >> 8) & 0xFFu);
    q[4] = (float)((lo >> 16) & 0xFFu);
    q[5] = (float)((hi >> 16) & 0xFFu);
    q[6] = (float)(lo >> 24);
    q[7] = (float)(hi >> 24);
}

// A 16-byte weight load marked nontemporal, for weights that a wave reads in whole 1 KB runs
// (every weight byte is read once per forward; such streaming loads measured 10-15 % faster
// than plain ones on this machine, but much slower where several instructions share a line).
typedef unsigned int w32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_weight16(const void *p) {
    const w32x4 v = __builtin_nontemporal_load((const __attribute__((address_space(1))) w32x4 *)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}
// the cache policy of direct global->LDS weight copies (whole 1 KB runs): nontemporal
constexpr int AUX_NT = 2;

// ------------------------------------------------------------------ cross-workgroup data

// Data a "last arriver" reads from other workgroups of the same launch is written through to
// memory and read around the caches (agent-scope relaxed atomic stores and loads); the
// counter is only bumped once those stores have completed. No L2 write-back or invalidate.
__device__ __forceinline__ void st_shared16(uint16_t *p, uint16_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint16_t ld_shared16(const uint16_t *p) {
    return __hip_atomic_load(const_cast<uint16_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_shared32(int32_t *p, int32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t ld_shared32(const int32_t *p) {
    return __hip_atomic_load(const_cast<int32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_sharedf(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_sharedf(const float *p) {
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// wait until this thread's vector memory operations (the stores above) have completed
__device__ __forceinline__ void wait_vmem() {
    __builtin_amdgcn_s_waitcnt(0 | (0x7 << 4) | (0xF << 8));   // vmcnt(0) only
}

// Count this item done on *c once its write-through stores have completed. Returns true, in
// every thread of the item, for the item that brings the count to `target`: that item then
// reads the other items' data with read-around loads, and resets the counter for the next
// forward. Nothing waits: the other items just finish.
__device__ __forceinline__ bool last_arriver(uint32_t *c, uint32_t target, int *s_flag) {
    wait_vmem();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t old = __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int last = old + 1 == target;
        if (last) __hip_atomic_store(c, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *s_flag = last;
    }
    __syncthreads();
    const bool last = *s_flag != 0;
    if (last) {
        wait_vmem();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    }
    return last;
}

// ------------------------------------------------------------------ gate

// The handoff word of logit (r, e) (see LayerParams::ctr_hand).
__device__ __forceinline__ uint64_t *hand_word(const LayerParams &p, int r, int e) {
    return (uint64_t *)(p.ctr + p.ctr_hand) + (size_t)r * p.E + e;
}

// Store logit (r, e) (raw bits: bf16, or fp32 for the fp32 router). When the route items run
// in the gate launch (p.hand), the logit is handed to them in one 64-bit store (value and
// presence bit together, so a route item never sees one without the other) and a plain copy
// is kept for the stage readback; otherwise it is written through for the route items of the
// next launch.
__device__ __forceinline__ void put_logit(const LayerParams &p, int r, int e, uint32_t bits) {
    if (p.hand) {
        __hip_atomic_store(hand_word(p, r, e), (1ull << 32) | bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (p.router_f32) ((uint32_t *)p.logits)[(size_t)r * p.E + e] = bits;
        else ((uint16_t *)p.logits)[(size_t)r * p.E + e] = (uint16_t)bits;
    } else if (p.router_f32) {
        st_shared32((int32_t *)p.logits + (size_t)r * p.E + e, (int32_t)bits);
    } else {
        st_shared16((uint16_t *)p.logits + (size_t)r * p.E + e, (uint16_t)bits);
    }
}

// Input rows of a multi-row gate item, staged in LDS (16-bit values).
constexpr int GATE_LDS_ELEMS = 16384;
struct GateLds {
    uint4 x[GATE_LDS_ELEMS / 8];
};

// Expert e's logits for the rows [r0, r1): one wave, the order above, the gate row held in
// registers (bf16 rows of up to 4096 inputs) and each input row read from global memory.
__device__ __forceinline__ void gate_expert(const LayerParams &p, int e, int r0, int r1, int lane) {
    const int nj = p.H / 512;
    if (!p.router_f32 && nj <= 8) {
        const uint16_t *wr = p.gate_w16 + (size_t)e * p.H + 8 * lane;
        uint4 wv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (j < nj) wv[j] = ld_weight16(wr + 512 * j);
        for (int r = r0; r < r1; ++r) {
            const uint16_t *xr = p.x + (size_t)r * p.H + 8 * lane;
            uint4 xv[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (j < nj) xv[j] = *(const uint4 *)(xr + 512 * j);
            float acc = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (j < nj) {
                    float xf[8], wf[8];
                    unpack8(p.act_f16, xv[j], xf);
                    unpack8(0, wv[j], wf);
#pragma unroll
                    for (int i = 0; i < 8; ++i) acc = __builtin_fmaf(xf[i], wf[i], acc);
                }
            }
#pragma unroll
            for (int d = 32; d >= 1; d >>= 1) acc = acc + __shfl_xor(acc, d, 64);
            if (lane == 0) put_logit(p, r, e, f2bf(acc));
        }
        return;
    }
    for (int r = r0; r < r1; ++r) {
        const uint16_t *xr = p.x + (size_t)r * p.H;
        float acc = 0.0f;
        for (int j0 = 0; j0 < nj; j0 += 4) {
            uint4 xv[4], wv[4][2];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (j0 + q < nj) {
                    const int k0 = 512 * (j0 + q) + 8 * lane;
                    xv[q] = *(const uint4 *)(xr + k0);
                    if (p.router_f32) {
                        wv[q][0] = ld_weight16(p.gate_w32 + (size_t)e * p.H + k0);
                        wv[q][1] = ld_weight16(p.gate_w32 + (size_t)e * p.H + k0 + 4);
                    } else {
                        wv[q][0] = ld_weight16(p.gate_w16 + (size_t)e * p.H + k0);
                    }
                }
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (j0 + q < nj) {
                    float xf[8], wf[8];
                    unpack8(p.act_f16, xv[q], xf);
                    if (p.router_f32) {
                        const uint32_t w8[8] = {wv[q][0].x, wv[q][0].y, wv[q][0].z, wv[q][0].w,
                                                wv[q][1].x, wv[q][1].y, wv[q][1].z, wv[q][1].w};
#pragma unroll
                        for (int i = 0; i < 8; ++i) wf[i] = __uint_as_float(w8[i]);
                    } else {
                        unpack8(0, wv[q][0], wf);
                    }
#pragma unroll
                    for (int i = 0; i < 8; ++i) acc = __builtin_fmaf(xf[i], wf[i], acc);
                }
            }
        }
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) acc = acc + __shfl_xor(acc, d, 64);
        if (lane == 0) put_logit(p, r, e, p.router_f32 ? __float_as_uint(acc) : (uint32_t)f2bf(acc));
    }
}

// Item: NW experts (one per wave) for the rows [r0, r1) of chunk item / groups (all rows when
// gate_rc >= rows). Fixed summation order described above. Gate rows of up to 4096 bf16 or
// 5120 fp32 inputs stay in registers across the rows; a one-row pass loads its input row into
// registers with them, a multi-row item first copies its chunk of input rows into LDS (all
// rows' loads in flight at once) and reads each row from there.
constexpr int GATE_NJ_F32 = 10;   // 512-input chunks of an fp32 gate row held in registers
template <int NW>
__device__ __forceinline__ void gate_item(const LayerParams &p, int item, GateLds &L) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int groups = (p.E + NW - 1) / NW;
    const int e = (item % groups) * NW + wave;
    const int r0 = (item / groups) * p.gate_rc;
    const int r1 = r0 + p.gate_rc < p.rows ? r0 + p.gate_rc : p.rows;
    const int nj = p.H / 512;
    if (p.router_f32 && nj <= GATE_NJ_F32 && p.rows > 1) {
        // the fp32 router: the same, with each chunk of the gate row in two registers
        const int units = (r1 - r0) * (p.H >> 3);
        const uint4 *src = (const uint4 *)(p.x + (size_t)r0 * p.H);
        for (int u0 = wave * 64; u0 < units; u0 += NW * 64) {
            if (u0 + lane < units)
                __builtin_amdgcn_global_load_lds((const void *)(src + u0 + lane),
                                                 (__attribute__((address_space(3))) void *)(L.x + u0), 16, 0, 0);
        }
        uint4 wv[GATE_NJ_F32][2];
        if (e < p.E) {
            const float *wr = p.gate_w32 + (size_t)e * p.H + 8 * lane;
#pragma unroll
            for (int j = 0; j < GATE_NJ_F32; ++j)
                if (j < nj) {
                    wv[j][0] = ld_weight16(wr + 512 * j);
                    wv[j][1] = ld_weight16(wr + 512 * j + 4);
                }
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (e >= p.E) return;
        for (int r = r0; r < r1; ++r) {
            const uint4 *xr = L.x + (size_t)(r - r0) * (p.H >> 3) + lane;
            float acc = 0.0f;
#pragma unroll
            for (int j = 0; j < GATE_NJ_F32; ++j) {
                if (j < nj) {
                    float xf[8];
                    unpack8(p.act_f16, xr[64 * j], xf);
                    const uint32_t w8[8] = {wv[j][0].x, wv[j][0].y, wv[j][0].z, wv[j][0].w,
                                            wv[j][1].x, wv[j][1].y, wv[j][1].z, wv[j][1].w};
#pragma unroll
                    for (int i = 0; i < 8; ++i) acc = __builtin_fmaf(xf[i], __uint_as_float(w8[i]), acc);
                }
            }
#pragma unroll
            for (int d = 32; d >= 1; d >>= 1) acc = acc + __shfl_xor(acc, d, 64);
            if (lane == 0) put_logit(p, r, e, __float_as_uint(acc));
        }
        return;
    }
    if (!p.router_f32 && nj <= 8 && p.rows > 1) {
        // the chunk's rows: direct global -> LDS copies, 1 KB per wave instruction
        const int units = (r1 - r0) * (p.H >> 3);
        const uint4 *src = (const uint4 *)(p.x + (size_t)r0 * p.H);
        for (int u0 = wave * 64; u0 < units; u0 += NW * 64) {
            if (u0 + lane < units)
                __builtin_amdgcn_global_load_lds((const void *)(src + u0 + lane),
                                                 (__attribute__((address_space(3))) void *)(L.x + u0), 16, 0, 0);
        }
        uint4 wv[8];
        if (e < p.E) {
            const uint16_t *wr = p.gate_w16 + (size_t)e * p.H + 8 * lane;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (j < nj) wv[j] = ld_weight16(wr + 512 * j);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (e >= p.E) return;
        for (int r = r0; r < r1; ++r) {
            const uint4 *xr = L.x + (size_t)(r - r0) * (p.H >> 3) + lane;
            float acc = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (j < nj) {
                    float xf[8], wf[8];
                    unpack8(p.act_f16, xr[64 * j], xf);
                    unpack8(0, wv[j], wf);
#pragma unroll
                    for (int i = 0; i < 8; ++i) acc = __builtin_fmaf(xf[i], wf[i], acc);
                }
            }
#pragma unroll
            for (int d = 32; d >= 1; d >>= 1) acc = acc + __shfl_xor(acc, d, 64);
            if (lane == 0) put_logit(p, r, e, f2bf(acc));
        }
        return;
    }
    if (e >= p.E) return;
    gate_expert(p, e, r0, r1, lane);
}

// ------------------------------------------------------------------ route

// 64-bit rank key: larger key ranks first. High word orders the float (NaN lowest, -0 ==
// +0), low word orders ids ascending.
__device__ __forceinline__ uint64_t rank_key(float v, int id) {
    uint32_t b = __float_as_uint(v);
    uint32_t o;
    if (v != v) o = 0u;
    else if (v == 0.0f) o = 0x80000000u;
    else o = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    return ((uint64_t)o << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)id);
}


// Number of keys in v[0..n) larger than k (v in LDS, 16-byte aligned). Batches of 16
// independent broadcast reads keep the LDS pipeline full.
__device__ __forceinline__ int count_greater(const uint64_t *v, int n, uint64_t k) {
    int c = 0, f = 0;
    for (; f + 16 <= n; f += 16) {
        uint64_t t[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) t[q] = v[f + q];
#pragma unroll
        for (int q = 0; q < 16; ++q) c += t[q] > k;
    }
    for (; f < n; ++f) c += v[f] > k;
    return c;
}

// The same for any alignment of v.
__device__ __forceinline__ int count_greater_any(const uint64_t *v, int n, uint64_t k) {
    int c = 0, f = 0;
    for (; f + 16 <= n; f += 16) {
        uint64_t t[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) t[q] = v[f + q];
#pragma unroll
        for (int q = 0; q < 16; ++q) c += t[q] > k;
    }
    for (; f + 4 <= n; f += 4) {
        uint64_t t[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) t[q] = v[f + q];
#pragma unroll
        for (int q = 0; q < 4; ++q) c += t[q] > k;
    }
    for (; f < n; ++f) c += v[f] > k;
    return c;
}

// ME: the most experts the item serves (the candidates never outnumber the experts: at most
// top_k per kept group, or top_k per block of 64 when blocked, with top_k <= 16)
template <int NT, int ME = MAX_EXPERTS>
struct RouteLds {
    float s[ME];
    float b[ME];
    alignas(16) uint64_t key[ME];    // rank keys of the biased scores
    alignas(16) uint64_t ckey[ME];   // the candidates' keys
    alignas(16) uint64_t gkey[256];  // rank keys of the group scores
    int rank[ME];                    // candidate ranks, summed over counting threads
    int inr[ME];                     // each expert's rank inside its group
    int top[256][2];              // the two best members of each group
    int keep[256];                // 1: the group is kept
    int picks[MAX_TOPK];
};

// Item: one row (TensorFold pull request 1038, «Per operator and row invariance»:
// group_expert_select at k = 9; pull request 1295, «What this changes»: sigmoid top-8 with
// per-expert norm and sum). Every selection is by rank: an element's rank is the number of
// elements whose 64-bit key is larger, counted by the element's own thread from LDS (group
// keys, up to 64 groups: by the group's lane of every wave, from the other lanes) -- keys
// are unique, so ranks are a permutation and no thread waits on another's choice.
template <int NT, int ME = MAX_EXPERTS>
__device__ __forceinline__ void route_item(const LayerParams &p, int r, RouteLds<NT, ME> &L) {
    const int tid = threadIdx.x;
    const int E = p.E, G = p.G, per = p.E / p.G;
    for (int e = tid; e < E; e += NT) {
        // both loads are issued before either value is used
        const float bias = p.has_bias ? p.bias[e] : 0.0f;
        uint32_t raw;
        if (p.hand) {
            // the gate items of this launch hand the logits over: poll the word (read around
            // the caches) until it is present, for at most wait_ticks (then error bit 8), and
            // clear it for the next forward
            uint64_t *hw = hand_word(p, r, e);
            uint64_t v = __hip_atomic_load(hw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (!(v >> 32)) {
                const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
                do {
                    __builtin_amdgcn_s_sleep(1);
                    v = __hip_atomic_load(hw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    if (!(v >> 32) && __builtin_amdgcn_s_memrealtime() - t0 > (uint64_t)p.wait_ticks) {
                        atomicOr(p.err, 8u);
                        break;
                    }
                } while (!(v >> 32));
            }
            __hip_atomic_store(hw, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            raw = (uint32_t)v;
        } else {
            raw = p.router_f32 ? (uint32_t)ld_shared32((const int32_t *)p.logits + (size_t)r * E + e)
                               : (uint32_t)ld_shared16((const uint16_t *)p.logits + (size_t)r * E + e);
        }
        const float z = p.router_f32 ? __uint_as_float(raw) : __uint_as_float(raw << 16);
        const float s = (float)(1.0 / (1.0 + exp(-(double)z)));
        const float b = p.has_bias ? s + bias : s;
        L.s[e] = s;
        L.b[e] = b;
        L.key[e] = rank_key(b, e);
    }
    if (tid < MAX_TOPK) L.picks[tid] = -1;
    for (int c = tid; c < E; c += NT) L.rank[c] = 0;
    __syncthreads();
    // every expert's rank inside its group. Without group selection: among all experts, which
    // picks the top_k directly, or for more than 64 experts inside blocks of 64, whose top_k
    // are the candidates (a pick is among the top_k of its block)
    const bool grouped = p.TG < G, blocked = !grouped && E > 64;
    const int gsz = grouped ? per : blocked ? 64 : E;
    const int nblk = (E + 63) >> 6;
    if (blocked)   // a block of fewer than top_k experts leaves candidate slots that rank last
        for (int c = tid; c < nblk * p.K; c += NT) L.ckey[c] = 0;
    for (int e = tid; e < E; e += NT) {
        const int g = e / gsz, n = E - g * gsz < gsz ? E - g * gsz : gsz;
        const int rank = count_greater_any(L.key + g * gsz, n, L.key[e]);
        L.inr[e] = rank;
        if (grouped && rank < 2) L.top[g][rank] = e;
        if (!grouped && !blocked && rank < p.K) L.picks[rank] = e;
    }
    __syncthreads();
    if (grouped || blocked) {
        // candidates: a pick is among the top_k of its own group, so only those members of the
        // kept groups enter; candidate slot = (kept groups before g) * KK + rank in the group
        const int KK = blocked ? p.K : p.K < per ? p.K : per;
        if (blocked) {
            for (int e = tid; e < E; e += NT)
                if (L.inr[e] < KK) L.ckey[(e >> 6) * KK + L.inr[e]] = L.key[e];
        } else if (G <= 64) {
            // up to 64 groups: every wave scores the groups itself, lane g taking group g, and
            // ranks them with lane reads, so the kept groups are a mask in every wave and no
            // barrier is needed before the candidates
            const int lane = tid & 63;
            uint64_t gk = 0;
            if (lane < G) {
                const float gam = per > 1 ? L.b[L.top[lane][0]] + L.b[L.top[lane][1]] : L.b[L.top[lane][0]];
                gk = rank_key(gam, lane);
            }
            int c = 0;
            for (int h = 0; h < G; ++h) {
                const uint64_t o = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(gk >> 32), h) << 32) |
                                   (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)gk, h);
                c += o > gk;
            }
            const uint64_t keepm = __ballot(lane < G && c < p.TG);
            for (int e = tid; e < E; e += NT) {
                const int g = e / per, rank = L.inr[e];
                if (((keepm >> g) & 1ull) && rank < KK)
                    L.ckey[__popcll(keepm & ((1ull << g) - 1ull)) * KK + rank] = L.key[e];
            }
        } else {
            for (int g = tid; g < G; g += NT) {
                const float gam = per > 1 ? L.b[L.top[g][0]] + L.b[L.top[g][1]] : L.b[L.top[g][0]];
                L.gkey[g] = rank_key(gam, g);
            }
            __syncthreads();
            // kept groups: rank < TG
            for (int g = tid; g < G; g += NT) L.keep[g] = count_greater(L.gkey, G, L.gkey[g]) < p.TG;
            __syncthreads();
            for (int e = tid; e < E; e += NT) {
                const int g = e / per, rank = L.inr[e];
                if (L.keep[g] && rank < KK) {
                    int before = 0;
                    for (int h = 0; h < g; ++h) before += L.keep[h];
                    L.ckey[before * KK + rank] = L.key[e];
                }
            }
        }
        __syncthreads();
        // the top_k of the candidates: rank among them, counted by T threads per candidate
        // (each over a contiguous part of the list) and summed in LDS
        const int nc = blocked ? nblk * KK : p.TG * KK;
        int T = 1;
        while (T < 16 && 2 * T * nc <= NT) T *= 2;
        for (int i = tid; i < nc * T; i += NT) {
            const int c = i / T, part = i % T;
            const int lo = part * nc / T, hi = (part + 1) * nc / T;
            const int cnt = count_greater_any(L.ckey + lo, hi - lo, L.ckey[c]);
            atomicAdd(&L.rank[c], cnt);
        }
        __syncthreads();
        for (int c = tid; c < nc; c += NT) {
            const int rank = L.rank[c];
            if (rank < p.K) L.picks[rank] = (int)(0xFFFFFFFFu - (uint32_t)L.ckey[c]);
        }
        __syncthreads();
    }
    // thread j < K finishes pick j: every such thread reads all picks (a missing one, which
    // the host checks exclude, counts as expert 0), sums the picked scores in pick order and
    // writes its index and weight; a one-row pass also gets its schedule here, slot u holding
    // the u-th smallest picked expert
    if (tid < p.K) {
        const int j = tid;
        int pk[MAX_TOPK];
        bool missing = false;
#pragma unroll
        for (int i = 0; i < MAX_TOPK; ++i) {
            pk[i] = i < p.K ? L.picks[i] : 0;
            if (pk[i] < 0 || pk[i] >= E) { pk[i] = 0; missing = true; }
        }
        if (missing && j == 0) atomicOr(p.err, 2u);
        float sv[MAX_TOPK];
#pragma unroll
        for (int i = 0; i < MAX_TOPK; ++i) sv[i] = i < p.K ? L.s[pk[i]] : 0.0f;
        float S = sv[0];
#pragma unroll
        for (int i = 1; i < MAX_TOPK; ++i)
            if (i < p.K) S = S + sv[i];
        float sj = sv[0];
        int ej = pk[0], u = 0;
#pragma unroll
        for (int i = 0; i < MAX_TOPK; ++i) if (i == j) { sj = sv[i]; ej = pk[i]; }
#pragma unroll
        for (int i = 0; i < MAX_TOPK; ++i)
            if (i < p.K) u += pk[i] < ej || (pk[i] == ej && i < j);
        const float v = p.norm_topk ? sj / S : sj;
        st_shared32(p.idx + (size_t)r * p.K + j, ej);
        p.wts[(size_t)r * p.K + j] = v * p.rho;
        if (p.single_row) {
            *(int4 *)(p.sched + SCH_REC + SCH_RECW * u) = make_int4(ej, u, 1, j);
            *(int4 *)(p.sched + SCH_REC + SCH_RECW * u + 4) = make_int4(-1, 0, 0, 0);
            p.sched[SCH_PAIRS + u] = j;
            if (j == 0) p.sched[SCH_U] = p.K;
        }
    }
}

// ------------------------------------------------------------------ schedule

struct SchedLds {
    int slot[MAX_EXPERTS];   // slot of each picked expert
    int cnt[MAX_EXPERTS];
    int off[MAX_EXPERTS + 1];
    int cur[MAX_EXPERTS];
    int scan[WG_THREADS];
    int pairs[MAX_ROWS * MAX_TOPK];
};

// Item: the whole pass. Slots are the distinct picked experts in increasing id; each slot
// lists its (row * top_k + pick) pairs in increasing row. The picks are read once (one round
// trip) and everything is built in LDS; the schedule is written after the last barrier, since
// a barrier waits for the stores before it.
__device__ __forceinline__ void sched_item(const LayerParams &p, SchedLds &L) {
    const int tid = threadIdx.x, E = p.E, NP = p.rows * p.K;
    constexpr int PPT = MAX_ROWS * MAX_TOPK / WG_THREADS;   // picks per thread at most
    int pick[PPT];
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
        const int i = tid + k * WG_THREADS;
        pick[k] = i < NP ? ld_shared32(p.idx + i) : 0;
    }
    for (int e = tid; e < E; e += WG_THREADS) { L.cnt[e] = 0; L.cur[e] = 0; }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < PPT; ++k)
        if (tid + k * WG_THREADS < NP) atomicAdd(&L.cnt[pick[k]], 1);
    __syncthreads();
    // exclusive scans of cnt (pair offsets) and of (cnt > 0) (slot ids), 4 experts per thread
    const int per_t = (E + WG_THREADS - 1) / WG_THREADS;
    int local_pairs = 0, local_slots = 0;
    for (int m = 0; m < per_t; ++m) {
        const int e = tid * per_t + m;
        if (e < E) { local_pairs += L.cnt[e]; local_slots += L.cnt[e] > 0; }
    }
    L.scan[tid] = (local_slots << 16) | local_pairs;   // both < 2^16
    __syncthreads();
    for (int d = 1; d < WG_THREADS; d <<= 1) {
        const int v = tid >= d ? L.scan[tid - d] : 0;
        __syncthreads();
        L.scan[tid] += v;
        __syncthreads();
    }
    int run = tid ? L.scan[tid - 1] : 0;
    int run_pairs = run & 0xFFFF, run_slots = run >> 16;
    for (int m = 0; m < per_t; ++m) {
        const int e = tid * per_t + m;
        if (e < E) {
            L.off[e] = run_pairs;
            L.slot[e] = run_slots;
            run_slots += L.cnt[e] > 0;
            run_pairs += L.cnt[e];
        }
    }
    const int U = L.scan[WG_THREADS - 1] >> 16, umax = E < NP ? E : NP;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
        const int i = tid + k * WG_THREADS;
        if (i < NP) L.pairs[L.off[pick[k]] + atomicAdd(&L.cur[pick[k]], 1)] = i;
    }
    __syncthreads();
    // order each expert's list by row (insertion sort: lists are short)
    for (int e = tid; e < E; e += WG_THREADS) {
        const int o = L.off[e], n = L.cnt[e];
        for (int a = 1; a < n; ++a) {
            const int v = L.pairs[o + a];
            int b = a - 1;
            while (b >= 0 && L.pairs[o + b] > v) { L.pairs[o + b + 1] = L.pairs[o + b]; --b; }
            L.pairs[o + b + 1] = v;
        }
    }
    __syncthreads();
    // the schedule: U, each slot's record (slots past U, up to the slots the item grid
    // enumerates, marked empty), the pair lists
    if (tid == 0) p.sched[SCH_U] = U;
    for (int e = tid; e < E; e += WG_THREADS) {
        const int o = L.off[e], n = L.cnt[e];
        if (n > 0) {
            *(int4 *)(p.sched + SCH_REC + SCH_RECW * L.slot[e]) = make_int4(e, o, n, L.pairs[o]);
            *(int4 *)(p.sched + SCH_REC + SCH_RECW * L.slot[e] + 4) = make_int4(n > 1 ? L.pairs[o + 1] : -1, 0, 0, 0);
        }
    }
    for (int u = U + tid; u < umax; u += WG_THREADS) *(int4 *)(p.sched + SCH_REC + SCH_RECW * u) = make_int4(-1, 0, 0, 0);
    for (int i = tid; i < NP; i += WG_THREADS) p.sched[SCH_PAIRS + i] = L.pairs[i];
}

// ------------------------------------------------------------------ combine

// The combine of row r at latent output d, before rounding (lane order described at the top).
// COH: the expert outputs were written by the same launch (read around the non-coherent
// caches); otherwise by an earlier one (plain loads).
template <bool COH>
__device__ __forceinline__ float combine_value(const LayerParams &p, int r, int d) {
    // all MAX_TOPK loads are issued unconditionally (picks past K re-read pick K - 1) so that
    // none waits for another; the picks past K are then left out of the sum
    float w[MAX_TOPK];
    uint16_t v[MAX_TOPK];
#pragma unroll
    for (int j = 0; j < MAX_TOPK; ++j) {
        const size_t pr = (size_t)r * p.K + (j < p.K ? j : p.K - 1);
        w[j] = p.wts[pr];
        v[j] = COH ? ld_shared16(p.eout + pr * p.D + d) : p.eout[pr * p.D + d];
    }
    float T[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) T[t] = 0.0f;
#pragma unroll
    for (int j = 0; j < MAX_TOPK; ++j) {
        const float t = T[j & 7] + w[j] * act2f(p.act_f16, v[j]);
        T[j & 7] = j < p.K ? t : T[j & 7];
    }
    return ((T[0] + T[4]) + (T[2] + T[6])) + ((T[1] + T[5]) + (T[3] + T[7]));
}

__device__ __forceinline__ uint32_t pack2(uint16_t lo, uint16_t hi) { return (uint32_t)lo | ((uint32_t)hi << 16); }

// The same combine at latent outputs d..d+3 (d a multiple of 4) of row r, the expert outputs
// written by an earlier launch: one 8-byte load per pick, each output summed exactly as
// combine_value does.
__device__ __forceinline__ void combine4(const LayerParams &p, int r, int d, float *out) {
    float w[MAX_TOPK];
    uint2 v[MAX_TOPK];
    // picks past K load nothing (the branches are uniform; the loads still go out together)
#pragma unroll
    for (int j = 0; j < MAX_TOPK; ++j) {
        w[j] = 0.0f;
        v[j] = make_uint2(0u, 0u);
        if (j < p.K) {
            const size_t pr = (size_t)r * p.K + j;
            w[j] = p.wts[pr];
            v[j] = *(const uint2 *)(p.eout + pr * p.D + d);
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float T[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) T[t] = 0.0f;
#pragma unroll
        for (int j = 0; j < MAX_TOPK; ++j) {
            const uint32_t word = i < 2 ? v[j].x : v[j].y;
            const uint32_t h = i & 1 ? word >> 16 : word & 0xFFFFu;
            const float t = T[j & 7] + w[j] * act2f(p.act_f16, h);
            T[j & 7] = j < p.K ? t : T[j & 7];
        }
        out[i] = ((T[0] + T[4]) + (T[2] + T[6])) + ((T[1] + T[5]) + (T[3] + T[7]));
    }
}

// ------------------------------------------------------------------ dense bf16 tiles (MFMA)

enum Epi { EPI_FC1 = 0, EPI_SHUP = 1, EPI_SHDN = 2, EPI_FC2 = 3, EPI_LMH = 4 };

// Weight steps of 128 inputs a wave of a dense tile keeps in flight (1, 2 or 4; build-time
// knobs). Fewer steps keep the memory queues shorter, and with them the round trips of every
// other item of the launch -- the gate's loads and the route's logit hand-off in the first
// launch. Measured on the one-row Bolt-like forward (38.96 us with 4 everywhere): fc1 and
// shared up at 1 and shared down at 2, 37.17 us; the lm_head at 2, 160 us at one row against
// 171 (at 16 rows 211 against 224).
#ifndef MOE_DEP_L0
#define MOE_DEP_L0 1
#endif
#ifndef MOE_DEP_SHDN
#define MOE_DEP_SHDN 2
#endif
#ifndef MOE_DEP_LMH
#define MOE_DEP_LMH 2
#endif
constexpr int dense_depth(int epi) {
    return epi == EPI_FC1 || epi == EPI_SHUP ? MOE_DEP_L0 : epi == EPI_SHDN ? MOE_DEP_SHDN : epi == EPI_LMH ? MOE_DEP_LMH : 4;
}

template <int NW>
struct DenseLds {
    // per wave: one step's weights (16 rows x 128 inputs, rows 272 bytes apart) on their way
    // from row runs to MFMA fragments; after the wave's last step, its partial sums
    // [row tile][lane]
    union WaveBuf {
        uint4 wt[16 * 17];
        f32x4 part[2][64];
    } w[NW];
    // the item's slice of the input rows, [row][kpart], when it fits (the combine itself in
    // fc2 of a one-row pass)
    uint16_t xs[DENSE_XLDS];
};

// 16-byte loads through a pointer of a known address space (p must point into LDS, resp.
// global memory), so that a wait for one kind of access never counts the other.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 lds_ld16(const void *p) {
    const u32x4 v = *(const __attribute__((address_space(3))) u32x4 *)p;
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void lds_st16(void *p, uint4 v) {
    *(__attribute__((address_space(3))) u32x4 *)p = (u32x4){v.x, v.y, v.z, v.w};
}
__device__ __forceinline__ uint4 glb_ld16(const void *p) {
    const u32x4 v = *(const __attribute__((address_space(1))) u32x4 *)p;
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Inputs of the fc2 epilogue (shared expert output and residual) of 4 outputs.
struct EpiIn {
    float sh[4], xv[4];
};

__device__ __forceinline__ EpiIn epi_load(const LayerParams &p, int row, int n) {
    // two 8-byte loads (n is a multiple of 4); the shared output buffer exists even when the
    // layer has no shared expert
    const uint2 sh = *(const uint2 *)(p.shout + (size_t)row * p.H + n);
    const uint2 xv = *(const uint2 *)(p.x + (size_t)row * p.H + n);
    const uint32_t shw[2] = {sh.x, sh.y}, xw[2] = {xv.x, xv.y};
    EpiIn v;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float s16 = __uint_as_float((i & 1 ? shw[i >> 1] >> 16 : shw[i >> 1] & 0xFFFFu) << 16);
        v.sh[i] = p.SI ? s16 : 0.0f;
        v.xv[i] = __uint_as_float((i & 1 ? xw[i >> 1] >> 16 : xw[i >> 1] & 0xFFFFu) << 16);
    }
    return v;
}

__device__ __forceinline__ void fc2_out(const LayerParams &p, int row, int n, float a, float sh, float xv) {
    const float m = rnd(0, a);
    p.out[(size_t)row * p.H + n] = f2bf(xv + rnd(0, m + sh));
}

__device__ __forceinline__ void dense_epilogue(const LayerParams &p, int epi, int row, int n, float a) {
    if (epi == EPI_FC1) {
        p.u[(size_t)row * p.L + n] = f2bf(a);
    } else if (epi == EPI_SHUP) {
        p.shact[(size_t)row * p.SI + n] = f2bf(relu_sq(0, rnd(0, a)));
    } else if (epi == EPI_SHDN) {
        p.shout[(size_t)row * p.H + n] = f2bf(a);
    } else if (epi == EPI_LMH) {
        if (p.lm_f32) ((float *)p.lm_out)[(size_t)row * p.lm_n + n] = a;
        else ((uint16_t *)p.lm_out)[(size_t)row * p.lm_n + n] = f2bf(a);
    } else {
        // both loads unconditional (the shared output buffer always exists), so they overlap
        const float sh = bf2f(p.shout[(size_t)row * p.H + n]);
        const float xv = bf2f(p.x[(size_t)row * p.H + n]);
        fc2_out(p, row, n, a, p.SI ? sh : 0.0f, xv);
    }
}

// Item: part `split` (of `ks`) of K for outputs n0..n0+15 of W [N][K] (bf16, row-major)
// against X [rows][K] (bf16), all rows. Inside the item K is split again over up to NW waves
// in contiguous slices (each a multiple of 128). A step of 128 inputs is 4 MFMAs of 32: lane
// L holds 8 consecutive k of weight row L % 16 and of one input row (k = 32 j + 8 (L / 16) for
// MFMA j). The weights are loaded in 256-byte row runs (load instruction i of a step: rows
// 4i..4i+3, 16 lanes per row, streamed nontemporal) and rearranged into those fragments
// through the wave's LDS buffer. A wave issues the loads of up to 4 steps of its weight
// slice, then multiplies. The waves'
// partial sums are joined in wave order; with ks > 1 the item's partial goes to the
// workspace and the last of the ks items to finish adds them in split order and applies the
// epilogue. For the fc2 of a one-row pass (p.inline_comb) the item first computes its slice
// of the combine into LDS, while its first weights are in flight.
template <int EPI, int NW>
__device__ __forceinline__ void dense_item(const LayerParams &p, const uint16_t *__restrict__ W,
                                           const uint16_t *__restrict__ X, int K, int tile, int split, int ks,
                                           float *part, uint32_t *ctr, DenseLds<NW> &L, int *s_flag) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nr = lane & 15, grp = lane >> 4;
    const int n0 = tile * DENSE_TILE;
    const int kpart = K / ks, kbase = split * kpart;
    const int nsplit = dense_nsplit(kpart, NW);
    const int kw = kpart / nsplit, nit = kw / 128;
    const int nrt = (p.rows + 15) >> 4;
    float *mypart = part + ((size_t)(tile * ks + split) * p.rows) * DENSE_TILE;
    constexpr int RT = 2;   // row tiles (16 rows each) per pass over the weights
    const bool inl = EPI == EPI_FC2 && p.inline_comb;
    // the input slice staged in LDS when it fits (always for a one-row fc2 pass that combines)
    const bool xl = inl || p.rows * kpart <= DENSE_XLDS;
    // weight loads: lane (16 r + c) reads inputs 8c..8c+7 of the step from row 4i + r in
    // instruction i (whole 256-byte runs of a row: measured about 10 % faster than 64 bytes
    // of each of 16 rows, the LDS round trip included)
    const int rr = lane >> 4, kk = lane & 15;
    const uint16_t *wrow = W + (size_t)(n0 + rr) * K + kbase + wave * kw + 8 * kk;
    const size_t xoff = (size_t)kbase + wave * kw + 8 * grp;
    uint4 *wt = L.w[wave].wt;

    uint4 a[4][4];
    // steps in flight per wave: fewer keep the memory queues, and with them every other item's
    // round trips, shorter
    constexpr int dep = dense_depth(EPI);
    auto load_w = [&](int i0) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (q < dep && i0 + q < nit) {
                const uint16_t *wp = wrow + 128 * (i0 + q);
#pragma unroll
                for (int i = 0; i < 4; ++i) a[q][i] = ld_weight16(wp + (size_t)(4 * i) * K);
            }
        }
    };
    // the fc2 epilogue's inputs, when one pass finishes every row here
    const bool epi_pre = EPI == EPI_FC2 && ks == 1 && nrt <= RT;
    EpiIn pre = {};
    if (epi_pre && wave < nrt) {
        const int row = wave * 16 + nr;
        if (row < p.rows) pre = epi_load(p, row, n0 + 4 * grp);
    }
    // the passes over the weights, compiled once per input source (LDS or global memory); the
    // first weights are loaded inside, so that no weight register is live across the choice
    auto passes = [&](auto xl_c) {
    if (wave < nsplit) load_w(0);
    if constexpr (decltype(xl_c)::value) {
        if (inl) {
            for (int i = 4 * threadIdx.x; i < kpart; i += 4 * NW * 64) {
                float c4[4];
                combine4(p, 0, kbase + i, c4);
                const uint2 c = {pack2(f2bf(c4[0]), f2bf(c4[1])), pack2(f2bf(c4[2]), f2bf(c4[3]))};
                *(uint2 *)(L.xs + i) = c;
                if (tile == 0) *(uint2 *)(p.comb + kbase + i) = c;
            }
        } else {
            const int cpr = kpart >> 3;   // 16-byte chunks per row
#pragma unroll 4
            for (int c = threadIdx.x; c < p.rows * cpr; c += NW * 64) {
                const int r = c / cpr, o = (c - r * cpr) << 3;
                *(uint4 *)(L.xs + r * kpart + o) = glb_ld16(X + (size_t)r * K + kbase + o);
            }
        }
        __syncthreads();
    }
    for (int rt0 = 0; rt0 < nrt; rt0 += RT) {
        f32x4 acc[RT];
#pragma unroll
        for (int t = 0; t < RT; ++t) acc[t] = (f32x4){0.f, 0.f, 0.f, 0.f};
        if (wave < nsplit) {
            for (int i0 = 0; i0 < nit; i0 += dep) {
                if (rt0 > 0 || i0 > 0) load_w(i0);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (q < dep && i0 + q < nit) {
                        const int kb = 128 * (i0 + q);
                        // the step's weights through the wave's buffer: written as loaded,
                        // read as fragments (MFMA j: row nr, inputs 32 j + 8 grp ..); LDS
                        // accesses of a wave are carried out in order
#pragma unroll
                        for (int i = 0; i < 4; ++i) lds_st16(&wt[(4 * i + rr) * 17 + kk], a[q][i]);
                        uint4 f[4];
#pragma unroll
                        for (int j = 0; j < 4; ++j) f[j] = lds_ld16(&wt[nr * 17 + 4 * j + grp]);
#pragma unroll
                        for (int t = 0; t < RT; ++t) {
                            const int row = (rt0 + t) * 16 + nr;
                            if (rt0 + t < nrt) {
                                uint4 b0 = {0, 0, 0, 0}, b1 = b0, b2 = b0, b3 = b0;
                                if (row < p.rows) {
                                    if constexpr (decltype(xl_c)::value) {
                                        const uint16_t *xp = L.xs + row * kpart + wave * kw + 8 * grp + kb;
                                        b0 = lds_ld16(xp); b1 = lds_ld16(xp + 32);
                                        b2 = lds_ld16(xp + 64); b3 = lds_ld16(xp + 96);
                                    } else {
                                        const uint16_t *xp = X + (size_t)row * K + xoff + kb;
                                        b0 = glb_ld16(xp); b1 = glb_ld16(xp + 32);
                                        b2 = glb_ld16(xp + 64); b3 = glb_ld16(xp + 96);
                                    }
                                }
                                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                    __builtin_bit_cast(bf16x8, f[0]), __builtin_bit_cast(bf16x8, b0), acc[t], 0, 0, 0);
                                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                    __builtin_bit_cast(bf16x8, f[1]), __builtin_bit_cast(bf16x8, b1), acc[t], 0, 0, 0);
                                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                    __builtin_bit_cast(bf16x8, f[2]), __builtin_bit_cast(bf16x8, b2), acc[t], 0, 0, 0);
                                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                    __builtin_bit_cast(bf16x8, f[3]), __builtin_bit_cast(bf16x8, b3), acc[t], 0, 0, 0);
                            }
                        }
                    }
                    // one step's inputs live at a time (keeps the scheduler from hoisting
                    // the input reads of every step ahead of the first multiply)
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
#pragma unroll
        for (int t = 0; t < RT; ++t) L.w[wave].part[t][lane] = acc[t];
        __syncthreads();
        // wave t finishes row tile rt0 + t: partials joined in wave order
        if (wave < RT && rt0 + wave < nrt) {
            const int t = wave;
            f32x4 v = L.w[0].part[t][lane];
            for (int q = 1; q < nsplit; ++q) v = v + L.w[q].part[t][lane];
            const int row = (rt0 + t) * 16 + nr;
            if (row < p.rows) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (ks > 1) st_sharedf(mypart + (size_t)row * DENSE_TILE + 4 * grp + i, v[i]);
                    else if (epi_pre) fc2_out(p, row, n0 + 4 * grp + i, v[i], pre.sh[i], pre.xv[i]);
                    else dense_epilogue(p, EPI, row, n0 + 4 * grp + i, v[i]);
                }
            }
        }
        __syncthreads();
    }
    };
    if (xl) passes(std::true_type{});
    else passes(std::false_type{});
    if (ks > 1 && last_arriver(ctr + tile, (uint32_t)ks, s_flag)) {
        for (int i = threadIdx.x; i < p.rows * DENSE_TILE; i += NW * 64) {
            const int row = i / DENSE_TILE, nn = i % DENSE_TILE;
            const float *pp = part + ((size_t)tile * ks * p.rows + row) * DENSE_TILE + nn;
            float v = ld_sharedf(pp);
            for (int q = 1; q < ks; ++q) v = v + ld_sharedf(pp + (size_t)q * p.rows * DENSE_TILE);
            dense_epilogue(p, EPI, row, n0 + nn, v);
        }
    }
}

// ------------------------------------------------------------------ first launch of a one-row pass

// Weight steps of 128 inputs a slice wave keeps in flight (a build-time knob).
#ifndef MOE_FRONT_DEP
#define MOE_FRONT_DEP 1
#endif

// The fc1 and shared up projections of a one-row pass, as blocks of whole output rows (of the
// rows of W1 followed by those of the shared up projection) spread evenly over the compute
// units, each block in one workgroup over all of K: no sums cross workgroups. Wave s of a
// block takes K slice s: the K range that wave s % nsplit of K part s / nsplit takes in a
// dense item, with the same MFMA chain from zero over the same inputs in the same order (an
// MFMA computes each output row alike, whatever rows share its tile); the block then adds
// each row's slices as the dense items do (the waves' sums in wave order within a part, then
// the parts in order). So every output equals the dense items', and so those of every
// multi-row pass, bit for bit.
struct FrontLds {
    union {
        struct {
            uint4 wt[FRONT_SW][16 * 17];                // per slice wave: one step's weights (as in DenseLds)
            uint4 xs[FRONT_SW][64];                     // per slice wave: the inputs of its slice
            float part[FRONT_U_MAX][32];                // [slice][row of the block's two row tiles]
        } s;
        RouteLds<FRONT_THREADS> route;
    };
};

// Row r of the concatenated projections: its weight row and its epilogue.
__device__ __forceinline__ const uint16_t *front_row(const LayerParams &p, int r) {
    return r < p.L ? p.fc1 + (size_t)r * p.H : p.su + (size_t)(r - p.L) * p.H;
}

// Slice wave `wave`: its K slices (wave, wave + FRONT_SW, ...) for the rows [r0, r1). A step
// is 128 inputs of every row of the block (instruction i loads rows 4 i .. 4 i + 3, 16 lanes
// per row, 256-byte runs; rows past r1 are not loaded), DEP steps in flight; the rows are
// multiplied as MFMA row tiles of 16 (the last one partial: its missing rows are not kept),
// one accumulator each, and each tile's sums go to part[slice][row].
template <int DEP>
__device__ __forceinline__ void front_rows(const LayerParams &p, int r0, int r1, int wave, int lane, FrontLds &L) {
    const int nr = lane & 15, grp = lane >> 4, rr = lane >> 4, kk = lane & 15;
    const int K = p.H, ks = p.ks_fc1, kpart = K / ks, nsplit = dense_nsplit(kpart, WG_THREADS / 64);
    const int kw = kpart / nsplit, nit = kw >> 7, U = ks * nsplit, nrow = r1 - r0;
    constexpr int NI = (FRONT_ROWS_MAX + 3) / 4;   // load instructions of a step at most
    uint4 *wt = L.s.wt[wave], *xs = L.s.xs[wave];
    for (int s = wave; s < U; s += FRONT_SW) {
        const int kb = (s / nsplit) * kpart + (s % nsplit) * kw;
        // the slice's inputs first: loads complete in order, so the first weights wait on
        // nothing else
        uint4 xv = make_uint4(0, 0, 0, 0);
        if (8 * lane < kw) xv = glb_ld16(p.x + kb + 8 * lane);
        // loads of step g's row tile tt (instructions 4 tt .. 4 tt + 3)
        auto load = [&](int g, int tt, uint4 *dst) {
#pragma unroll
            for (int i = 4 * tt; i < 4 * tt + 4; ++i) {
                if (i < NI) {
                    dst[i] = make_uint4(0, 0, 0, 0);
                    if (4 * i + rr < nrow) dst[i] = ld_weight16(front_row(p, r0 + 4 * i + rr) + kb + 128 * g + 8 * kk);
                }
            }
        };
        uint4 a[DEP][NI];
#pragma unroll
        for (int q = 0; q < DEP; ++q)
            if (q < nit) {
                load(q, 0, a[q]);
                load(q, 1, a[q]);
            }
        lds_st16(&xs[lane], xv);
        f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        for (int g0 = 0; g0 < nit; g0 += DEP) {
#pragma unroll
            for (int q = 0; q < DEP; ++q) {
                const int g = g0 + q;
                if (g < nit) {
                    // the step's input fragments, for both row tiles
                    uint4 b[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) b[j] = lds_ld16(xs + 16 * g + 4 * j + grp);
#pragma unroll
                    for (int tt = 0; tt < 2; ++tt) {
                        if (16 * tt < nrow) {
                            // the tile's rows through the wave's buffer into fragments (LDS
                            // accesses of a wave are carried out in order); the same rows of
                            // the step DEP ahead into the registers at once
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                if (4 * tt + i < NI && 16 * tt + 4 * i < nrow)
                                    lds_st16(&wt[(4 * i + rr) * 17 + kk], a[q][4 * tt + i]);
                            if (g + DEP < nit) load(g + DEP, tt, a[q]);
                            uint4 f[4];
#pragma unroll
                            for (int j = 0; j < 4; ++j) f[j] = lds_ld16(&wt[nr * 17 + 4 * j + grp]);
                            // every column of the MFMA gets the input row; column 0 is kept
#pragma unroll
                            for (int j = 0; j < 4; ++j)
                                acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                    __builtin_bit_cast(bf16x8, f[j]), __builtin_bit_cast(bf16x8, b[j]), acc[tt], 0, 0, 0);
                        }
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if (nr == 0) {
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int i = 0; i < 4; ++i) L.s.part[s][16 * tt + 4 * grp + i] = acc[tt][i];
        }
    }
}

// After the block's barrier: row r0 + t's slices added up in the dense items' order, then its
// epilogue (fc1: rounding; shared up: relu^2).
__device__ __forceinline__ void front_join(const LayerParams &p, int r0, int r1, const FrontLds &L) {
    const int t = threadIdx.x;
    if (t >= r1 - r0) return;
    const int ks = p.ks_fc1, nsplit = dense_nsplit(p.H / ks, WG_THREADS / 64);
    float v = 0.0f;
    for (int q = 0; q < ks; ++q) {
        float w = L.s.part[q * nsplit][t];
        for (int s = 1; s < nsplit; ++s) w = w + L.s.part[q * nsplit + s][t];
        v = q ? v + w : w;
    }
    const int r = r0 + t;
    dense_epilogue(p, r < p.L ? EPI_FC1 : EPI_SHUP, 0, r < p.L ? r : r - p.L, v);
}

// ------------------------------------------------------------------ routed experts (4-bit)

// LDS of one expert item: a block of NB output rows' codes, scales and biases (NB chosen on
// the host so that they fit), and the input rows (16-bit values) of the pairs in work: two
// rows of up to 2048 inputs, or one wider row in the wide variant. XMAX: the widest input row
// (2048, or 6144 in the wide variant).
template <int XMAX>
struct ExpertLds {
    static constexpr int XROWS = XMAX <= 2048 ? 2 : 1;
    uint4 q[EXPERT_LDS_CODES / 16];
    uint16_t s[EXPERT_LDS_SCALES / 2];
    uint16_t b[EXPERT_LDS_SCALES / 2];
    uint4 x[XROWS * XMAX / 8];
};

// Copy `units` 16-byte units from global src to LDS dst with direct global->LDS loads
// (each wave moves 1 KB per instruction, lane i the i-th 16 bytes); AUX: their cache policy.
template <int AUX = 0>
__device__ __forceinline__ void stage_lds(const uint4 *src, uint4 *dst, int units) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    for (int u0 = wave * 64; u0 < units; u0 += WG_THREADS) {
        if (u0 + lane < units)
            __builtin_amdgcn_global_load_lds((const void *)(src + u0 + lane),
                                             (__attribute__((address_space(3))) void *)(dst + u0), 16, 0, AUX);
    }
}

// v of the lane t ^ m(b), where m(b) = 2^(b+1) - 1 for bit b <= 3 (within quads and rows of
// 16 lanes: data-parallel-primitive moves) and m(b) = 2^b for b = 4, 5 (a swizzle, a
// permute). m(b) has bit b as its highest bit, so the masks of distinct bits are linearly
// independent and pair up every lane group of size 2^k exactly.
__device__ __forceinline__ float lane_mirror(float v, int b) {
    const int i = __float_as_int(v);
    int r;
    switch (b) {
        case 0: r = __builtin_amdgcn_update_dpp(i, i, 0xB1, 0xF, 0xF, false); break;    // quad_perm 1,0,3,2
        case 1: r = __builtin_amdgcn_update_dpp(i, i, 0x1B, 0xF, 0xF, false); break;    // quad_perm 3,2,1,0
        case 2: r = __builtin_amdgcn_update_dpp(i, i, 0x141, 0xF, 0xF, false); break;   // row_half_mirror
        case 3: r = __builtin_amdgcn_update_dpp(i, i, 0x140, 0xF, 0xF, false); break;   // row_mirror
        case 4: r = __builtin_amdgcn_ds_swizzle(i, 0x401F); break;                       // xor 16
        default: r = __builtin_amdgcn_ds_bpermute((int)((threadIdx.x ^ 32) << 2), i); break;   // xor 32
    }
    return __int_as_float(r);
}

__device__ __forceinline__ int mirror_mask(int b) { return b >= 4 ? 1 << b : (2 << b) - 1; }

// Sum each of the R values of v over the P lanes of a lane group (P, R powers of two,
// R <= P <= 64; t = lane index in the group, groups aligned to P lanes). Halving steps
// first, over the top bits of t: the lane whose bit is set keeps the upper half of its
// values and adds its partner's (lane t ^ m(bit)), the other the lower half; then plain
// exchanges over the remaining bits. Afterwards v[0] of lane t holds the full sum of value
// row(t) = the top log2(R) bits of t read high to low. Fixed order.
template <int R>
__device__ __forceinline__ int reduce_rows(float *v, int P, int t) {
    int n = R, bit = 31 - __builtin_clz(P) - 1, row = 0;
#pragma unroll
    for (int step = 0; (1 << step) < R; ++step) {
        n >>= 1;
        const bool upper = (t >> bit) & 1;
        row = 2 * row + (upper ? 1 : 0);
#pragma unroll
        for (int i = 0; i < R / 2; ++i) {
            if (i < n) {
                const float send = upper ? v[i] : v[i + n];
                const float keep = upper ? v[i + n] : v[i];
                v[i] = keep + lane_mirror(send, bit);
            }
        }
        --bit;
    }
    for (; bit >= 0; --bit) v[0] = v[0] + lane_mirror(v[0], bit);
    return row;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// a.lo * b.lo + a.hi * b.hi + c in fp32, a and b packed bf16 (F16: fp16) pairs
template <bool F16>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    if constexpr (F16)
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c, false);
    else
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

// Codes i and i + 4 of the word w (inputs 8j+i and 8j+i+4 of its 8) as a packed pair of
// 16-bit values, with one mask-and-insert: nibble bits placed under the exponent of 128 (bf16:
// 0x4300 | q is 128 + q exactly) or of 1024 (fp16: 0x6400 | q is 1024 + q, less 1024 exactly
// gives q).
template <bool F16>
__device__ __forceinline__ uint32_t code_pair(uint32_t w, int i) {
    const uint32_t m = ((w >> (4 * i)) & 0x000F000Fu) | (F16 ? 0x64006400u : 0x43004300u);
    if constexpr (F16) {
        const f16x2 h = __builtin_bit_cast(f16x2, m) - (f16x2){(_Float16)1024.0f, (_Float16)1024.0f};
        return __builtin_bit_cast(uint32_t, h);
    } else {
        return m;
    }
}

// All four pairs of a word, code_pair(w, 0..3): for bf16 the even and the odd nibbles are
// first masked into bytes (nibble 2i and 2i + 1 in byte i of m0 and m1), then each pair is one
// byte permute that puts two code bytes under 0x43 high bytes (0x43 0q is 128 + q): 7
// instructions for 4 pairs instead of 11.
template <bool F16>
__device__ __forceinline__ void code_pairs(uint32_t w, uint32_t *cp) {
    if constexpr (F16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) cp[i] = code_pair<true>(w, i);
    } else {
        const uint32_t m0 = w & 0x0F0F0F0Fu, m1 = (w >> 4) & 0x0F0F0F0Fu, hi = 0x43434343u;
        // result bytes: [code byte, 0x43, code byte, 0x43]; selectors 0-3 pick from m, 4-7 from hi
        cp[0] = __builtin_amdgcn_perm(hi, m0, 0x05020400u);   // nibbles 0 and 4
        cp[1] = __builtin_amdgcn_perm(hi, m1, 0x05020400u);   // nibbles 1 and 5
        cp[2] = __builtin_amdgcn_perm(hi, m0, 0x05030401u);   // nibbles 2 and 6
        cp[3] = __builtin_amdgcn_perm(hi, m1, 0x05030401u);   // nibbles 3 and 7
    }
}

// Chunk c (32 inputs) of an input row in LDS as packed 16-bit pairs (x[8j+i], x[8j+i+4]),
// i < 4 (the order code_pair decodes the codes in); returns the chunk's sum.
template <bool F16>
__device__ __forceinline__ float x_chunk(const uint4 *x, int c, uint32_t *xq) {
    uint32_t xw[16];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
        const uint4 v4 = lds_ld16(&x[4 * c + q4]);
        xw[4 * q4] = v4.x; xw[4 * q4 + 1] = v4.y; xw[4 * q4 + 2] = v4.z; xw[4 * q4 + 3] = v4.w;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        xq[4 * j] = __builtin_amdgcn_perm(xw[4 * j + 2], xw[4 * j], 0x05040100u);
        xq[4 * j + 1] = __builtin_amdgcn_perm(xw[4 * j + 2], xw[4 * j], 0x07060302u);
        xq[4 * j + 2] = __builtin_amdgcn_perm(xw[4 * j + 3], xw[4 * j + 1], 0x05040100u);
        xq[4 * j + 3] = __builtin_amdgcn_perm(xw[4 * j + 3], xw[4 * j + 1], 0x07060302u);
    }
    float sx = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) sx = dot2<F16>(F16 ? 0x3C003C00u : 0x3F803F80u, xw[k], sx);
    return sx;
}

// Item: outputs [blk*NB, +NB) of the up (UP) or down projection of slot `slot`, for every
// pair (row, pick) of that slot. The block's 4-bit codes, scales and biases and the first
// pairs' input rows are staged in LDS (all in flight at once; every weight byte is read from
// HBM once, whatever the number of rows). Each output row's inputs are cut in chunks of 32
// (16 bytes of codes). A group of P lanes covers the chunks of its output rows, lane t taking
// chunks t, t + P, ... (at most 4): it keeps their inputs in registers as packed pairs and
// adds, per row and chunk, scale * sum(q * x) + bias * sum(x), the products summed by
// 2-element dot products in fp32; reduce_rows then joins the P lanes of each row.
// Where two pairs remain (and two input rows fit in LDS), they go through the block together:
// each code word is decoded once for both, and every (row, pair) sum takes the same operations
// in the same order as it does alone.
template <bool UP, int XMAX, bool F16>
__device__ __forceinline__ int expert_item(const LayerParams &p, int slot, int blk, ExpertLds<XMAX> &L) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    // the number of slots and the slot's record (expert, pairs, first two pairs): independent loads
    const int U = p.sched[SCH_U];
    const int4 rec = *(const int4 *)(p.sched + SCH_REC + SCH_RECW * slot);
    const int4 rec2 = *(const int4 *)(p.sched + SCH_REC + SCH_RECW * slot + 4);
    const int e = rec.x, off = rec.y, R = rec.z;
    int pr = rec.w, pr2 = rec2.x;
    const int NP = p.rows * p.K;
    if (e == -1) return U;   // no expert in this slot for this pass
    if (e < 0 || e >= p.E || off < 0 || R < 1 || off + R > NP || pr < 0 || pr >= NP ||
        (R >= 2 && (pr2 < 0 || pr2 >= NP))) {   // never for a valid schedule
        if (threadIdx.x == 0) atomicOr(p.err, 4u);
        return 0;
    }
    const int Kin = UP ? p.D : p.I, N = UP ? p.I : p.D;
    const int NB = UP ? p.up_nb : p.dn_nb;
    const int n0 = blk * NB;
    const int C = Kin >> 5, G64 = Kin >> 6;
    const size_t qrow = (size_t)(Kin >> 3);
    const uint32_t *Q = (UP ? p.up_q : p.dn_q) + ((size_t)e * N + n0) * qrow;
    const uint16_t *S = (UP ? p.up_s : p.dn_s) + ((size_t)e * N + n0) * G64;
    const uint16_t *B = (UP ? p.up_b : p.dn_b) + ((size_t)e * N + n0) * G64;
    const uint16_t *xin = UP ? (p.L ? p.u : p.x) : p.eact;
    auto xrow = [&](int q) { return xin + (UP ? (size_t)(q / p.K) * Kin : (size_t)q * Kin); };
    // P lanes per row, each keeping up to XCH chunks (32 inputs each) of the input row, so that
    // a row is joined over few lanes (within a row of 16 lanes: data-parallel moves only)
    constexpr int XCH = 4;
    int P = 2;
    while (P * XCH < C && P < 64) P <<= 1;
    const int nch = (C + P - 1) / P;          // chunks per lane, <= XCH (inputs <= 6144)
    const int gpw = 64 / P, t = lane % P, grp = lane / P;
    const int NG = (WG_THREADS / 64) * gpw;   // lane groups of the item
    int RG = NB / NG;                          // rows per lane group (1 or 2: NB * C <= 2048)
    if (RG < 1) RG = 1;
    const int g = wave * gpw + grp;
    // The codes go to LDS in the order the lanes read them when the lanes tile the block
    // exactly: unit ((m * RG + row in group) * NG + group) * P + t holds chunk t + P m of that
    // row, so each read instruction of a wave takes 1 KB of consecutive LDS (no bank
    // conflicts); otherwise row-major (row * C + chunk).
    const bool tiled = nch * P == C && RG * NG == NB;
    const int xu = Kin >> 3;   // 16-byte units of one input row
    auto pair_at = [&](int j) {
        const int q = p.sched[SCH_PAIRS + off + j];
        return q < 0 || q >= NP ? NP - 1 : q;   // never for a valid schedule
    };
    auto put = [&](int q, int n, float acc) {
        if (UP) p.eact[(size_t)q * p.I + n] = f2act(F16, relu_sq(F16, rnd(F16, acc)));
        else if (p.inline_comb) p.eout[(size_t)q * p.D + n] = f2act(F16, acc);   // read next launch
        else st_shared16(p.eout + (size_t)q * p.D + n, f2act(F16, acc));   // combined in this one
    };
    constexpr bool PAIR2 = ExpertLds<XMAX>::XROWS == 2;
    // scales, biases and the first pairs' input rows first, the codes last
    stage_lds<AUX_NT>((const uint4 *)S, (uint4 *)L.s, NB * G64 / 8);
    stage_lds<AUX_NT>((const uint4 *)B, (uint4 *)L.b, NB * G64 / 8);
    stage_lds((const uint4 *)xrow(pr), L.x, xu);
    if (PAIR2 && R >= 2) stage_lds((const uint4 *)xrow(pr2), L.x + xu, xu);
    if (tiled) {
        const uint4 *src = (const uint4 *)Q;
        const int lp = __builtin_ctz(P), lg = __builtin_ctz(NG), lr = __builtin_ctz(RG);   // powers of two
        for (int u0 = wave * 64; u0 < NB * C; u0 += WG_THREADS) {
            const int u = u0 + lane;
            const int ut = u & (P - 1), ug = (u >> lp) & (NG - 1), ur = (u >> (lp + lg)) & (RG - 1);
            const int um = u >> (lp + lg + lr);
            if (u < NB * C)
                __builtin_amdgcn_global_load_lds((const void *)(src + (ug * RG + ur) * C + ut + P * um),
                                                 (__attribute__((address_space(3))) void *)(L.q + u0), 16, 0, AUX_NT);
        }
    } else {
        stage_lds<AUX_NT>((const uint4 *)Q, L.q, NB * C);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int r = 0; r < R;) {
        const bool two = PAIR2 && R - r >= 2;
        if (r > 0) {
            pr = pair_at(r);
            if (two) pr2 = pair_at(r + 1);
            __syncthreads();   // every lane is done with the previous input rows
            stage_lds((const uint4 *)xrow(pr), L.x, xu);
            if (two) stage_lds((const uint4 *)xrow(pr2), L.x + xu, xu);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
        if (two) {
            for (int rb = 0; rb < RG; rb += 2) {
                float va[2] = {0.0f, 0.0f}, vb[2] = {0.0f, 0.0f};
#pragma unroll
                for (int m = 0; m < XCH; ++m) {
                    const int c = t + P * m;
                    if (m < nch && c < C) {
                        uint32_t qa[16], qb[16];
                        const float sa = x_chunk<F16>(L.x, c, qa), sb = x_chunk<F16>(L.x + xu, c, qb);
                        uint4 qv[2];
                        float sc[2], bi[2];
#pragma unroll
                        for (int ii = 0; ii < 2; ++ii) {
                            int nl = g * RG + rb + ii;
                            nl = nl < NB ? nl : NB - 1;
                            qv[ii] = lds_ld16(&L.q[tiled ? ((m * RG + rb + ii) * NG + g) * P + t : nl * C + c]);
                            sc[ii] = bf2f(L.s[nl * G64 + (c >> 1)]);
                            bi[ii] = bf2f(L.b[nl * G64 + (c >> 1)]);
                        }
#pragma unroll
                        for (int ii = 0; ii < 2; ++ii) {
                            float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
                            for (int j = 0; j < 4; ++j) {
                                const uint32_t w = j == 0 ? qv[ii].x : j == 1 ? qv[ii].y : j == 2 ? qv[ii].z : qv[ii].w;
                                uint32_t cp[4];
                                code_pairs<F16>(w, cp);
#pragma unroll
                                for (int i = 0; i < 4; ++i) {
                                    a0 = dot2<F16>(cp[i], qa[4 * j + i], a0);
                                    a1 = dot2<F16>(cp[i], qb[4 * j + i], a1);
                                }
                            }
                            const float bb = F16 ? bi[ii] : __builtin_fmaf(-128.0f, sc[ii], bi[ii]);
                            va[ii] = __builtin_fmaf(sc[ii], a0, va[ii]);
                            va[ii] = __builtin_fmaf(bb, sa, va[ii]);
                            vb[ii] = __builtin_fmaf(sc[ii], a1, vb[ii]);
                            vb[ii] = __builtin_fmaf(bb, sb, vb[ii]);
                        }
                    }
                }
                const int rr = reduce_rows<2>(va, P, t);
                reduce_rows<2>(vb, P, t);
                const int nl = g * RG + rb + rr;
                if ((t & (P / 2 - 1)) == 0 && nl < NB && rb + rr < RG) {
                    put(pr, n0 + nl, va[0]);
                    put(pr2, n0 + nl, vb[0]);
                }
            }
            r += 2;
            continue;
        }
        // the lane's chunks of the input row: packed 16-bit pairs (x[8j+i], x[8j+i+4]), i < 4,
        // matching the code pairs decoded below, and each chunk's sum
        uint32_t xq[XCH][16];
        float xs[XCH];
#pragma unroll
        for (int m = 0; m < XCH; ++m) {
            const int c = t + P * m;
            xs[m] = 0.0f;
#pragma unroll
            for (int k = 0; k < 16; ++k) xq[m][k] = 0u;
            if (m < nch && c < C) xs[m] = x_chunk<F16>(L.x, c, xq[m]);
        }
        for (int rb = 0; rb < RG; rb += 2) {
            // 2 rows at a time, without branches (rows past NB read row NB - 1, dropped below)
            float v[2] = {0.0f, 0.0f};
#pragma unroll
            for (int m = 0; m < XCH; ++m) {
                const int c = t + P * m;
                if (m < nch && c < C) {
                    uint4 qv[2];
                    float sc[2], bi[2];
#pragma unroll
                    for (int ii = 0; ii < 2; ++ii) {
                        int nl = g * RG + rb + ii;
                        nl = nl < NB ? nl : NB - 1;
                        qv[ii] = lds_ld16(&L.q[tiled ? ((m * RG + rb + ii) * NG + g) * P + t : nl * C + c]);
                        sc[ii] = bf2f(L.s[nl * G64 + (c >> 1)]);
                        bi[ii] = bf2f(L.b[nl * G64 + (c >> 1)]);
                    }
#pragma unroll
                    for (int ii = 0; ii < 2; ++ii) {
                        float a = 0.0f;
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const uint32_t w = j == 0 ? qv[ii].x : j == 1 ? qv[ii].y : j == 2 ? qv[ii].z : qv[ii].w;
                            uint32_t cp[4];
                            code_pairs<F16>(w, cp);
#pragma unroll
                            for (int i = 0; i < 4; ++i) a = dot2<F16>(cp[i], xq[m][4 * j + i], a);
                        }
                        // bf16 pairs carry 128 + q: scale * sum(q x) = scale * a - 128 scale * sum(x)
                        v[ii] = __builtin_fmaf(sc[ii], a, v[ii]);
                        v[ii] = __builtin_fmaf(F16 ? bi[ii] : __builtin_fmaf(-128.0f, sc[ii], bi[ii]), xs[m], v[ii]);
                    }
                }
            }
            const int rr = reduce_rows<2>(v, P, t);
            // lane t holds row rb + rr; the lowest lane of those holding it stores it
            const int nl = g * RG + rb + rr;
            if ((t & (P / 2 - 1)) == 0 && nl < NB && rb + rr < RG) put(pr, n0 + nl, v[0]);
        }
        ++r;
    }
    return U;
}

// ------------------------------------------------------------------ routed experts, other widths

// Code k (0..31) of a 32-input chunk whose BITS * 32 bits sit in the words w[0..BITS) as one
// little-endian bit string (k and BITS known at compile time, so w stays in registers).
template <int BITS>
__device__ __forceinline__ uint32_t chunk_code(const uint32_t *w, int k) {
    const int o = k * BITS, wi = o >> 5, sh = o & 31;
    const uint32_t mask = (1u << BITS) - 1u;
    if (sh + BITS <= 32) return (w[wi] >> sh) & mask;
    return __builtin_amdgcn_alignbit(w[wi + 1], w[wi], (uint32_t)sh) & mask;
}

// Codes k and k + 4 of a chunk as a packed pair of bf16 values: 128 + q for widths up to 7
// bits (q under the exponent of 128, exact), q itself for 8 bits (an integer below 256 is a
// bf16 value: its fp32 image has 16 trailing zero bits).
template <int BITS>
__device__ __forceinline__ uint32_t chunk_pair(const uint32_t *w, int k) {
    const uint32_t a = chunk_code<BITS>(w, k), b = chunk_code<BITS>(w, k + 4);
    if constexpr (BITS <= 7) {
        return a | (b << 16) | 0x43004300u;
    } else {
        return __builtin_amdgcn_perm(__float_as_uint((float)b), __float_as_uint((float)a), 0x07060302u);
    }
}

// Item: outputs [blk*NB, +NB) of the up (UP) or down projection of slot `slot`, for every
// pair of that slot, with BITS-bit affine codes in groups of p.gs along the input (the
// affine family of the mlx-bun decode-speed program, §7.4 experiment axes: 2..8-bit, groups
// of 32/64/128). As expert_item, but the block's codes sit in LDS row by row (a 32-input
// chunk is BITS words), one pair per pass, bf16 activations; per chunk the lane adds
// scale * sum(q' x) + (bias - OFF scale) * sum(x) with q' = q + OFF (OFF = 128 for widths up
// to 7 bits, 0 for 8).
template <int BITS, bool UP, int XMAX>
__device__ __forceinline__ int qexpert_item(const LayerParams &p, int slot, int blk, ExpertLds<XMAX> &L) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int U = p.sched[SCH_U];
    const int4 rec = *(const int4 *)(p.sched + SCH_REC + SCH_RECW * slot);
    const int e = rec.x, off = rec.y, R = rec.z;
    int pr = rec.w;
    const int NP = p.rows * p.K;
    if (e == -1) return U;
    if (e < 0 || e >= p.E || off < 0 || R < 1 || off + R > NP || pr < 0 || pr >= NP) {   // never for a valid schedule
        if (threadIdx.x == 0) atomicOr(p.err, 4u);
        return 0;
    }
    const int Kin = UP ? p.D : p.I, N = UP ? p.I : p.D;
    const int NB = UP ? p.up_nb : p.dn_nb;
    const int n0 = blk * NB;
    const int C = Kin >> 5, G = Kin >> p.gs_log2, RW = (Kin >> 5) * BITS;   // words per row
    const uint32_t *Q = (UP ? p.up_q : p.dn_q) + ((size_t)e * N + n0) * RW;
    const uint16_t *S = (UP ? p.up_s : p.dn_s) + ((size_t)e * N + n0) * G;
    const uint16_t *B = (UP ? p.up_b : p.dn_b) + ((size_t)e * N + n0) * G;
    const uint16_t *xin = UP ? (p.L ? p.u : p.x) : p.eact;
    auto xrow = [&](int q) { return xin + (UP ? (size_t)(q / p.K) * Kin : (size_t)q * Kin); };
    constexpr int XCH = 4;
    constexpr float OFF = BITS <= 7 ? 128.0f : 0.0f;
    int P = 2;
    while (P * XCH < C && P < 64) P <<= 1;
    const int nch = (C + P - 1) / P;
    const int gpw = 64 / P, t = lane % P, grp = lane / P;
    const int NG = (WG_THREADS / 64) * gpw;
    int RG = NB / NG;
    if (RG < 1) RG = 1;
    const int g = wave * gpw + grp;
    const int xu = Kin >> 3;
    auto put = [&](int q, int n, float acc) {
        if (UP) p.eact[(size_t)q * p.I + n] = f2bf(relu_sq(0, rnd(0, acc)));
        else if (p.inline_comb) p.eout[(size_t)q * p.D + n] = f2bf(acc);
        else st_shared16(p.eout + (size_t)q * p.D + n, f2bf(acc));
    };
    stage_lds<AUX_NT>((const uint4 *)S, (uint4 *)L.s, NB * G / 8);
    stage_lds<AUX_NT>((const uint4 *)B, (uint4 *)L.b, NB * G / 8);
    stage_lds((const uint4 *)xrow(pr), L.x, xu);
    stage_lds<AUX_NT>((const uint4 *)Q, L.q, NB * RW / 4);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const uint32_t *LQ = (const uint32_t *)L.q;
    for (int r = 0; r < R; ++r) {
        if (r > 0) {
            const int q = p.sched[SCH_PAIRS + off + r];
            pr = q < 0 || q >= NP ? NP - 1 : q;
            __syncthreads();
            stage_lds((const uint4 *)xrow(pr), L.x, xu);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
        uint32_t xq[XCH][16];
        float xs[XCH];
#pragma unroll
        for (int m = 0; m < XCH; ++m) {
            const int c = t + P * m;
            xs[m] = 0.0f;
#pragma unroll
            for (int k = 0; k < 16; ++k) xq[m][k] = 0u;
            if (m < nch && c < C) xs[m] = x_chunk<false>(L.x, c, xq[m]);
        }
        for (int rb = 0; rb < RG; rb += 2) {
            float v[2] = {0.0f, 0.0f};
#pragma unroll
            for (int m = 0; m < XCH; ++m) {
                const int c = t + P * m;
                if (m < nch && c < C) {
#pragma unroll
                    for (int ii = 0; ii < 2; ++ii) {
                        int nl = g * RG + rb + ii;
                        nl = nl < NB ? nl : NB - 1;
                        uint32_t w[BITS];
                        const uint32_t *src = LQ + nl * RW + c * BITS;   // 16-byte aligned for 4 and 8 bits,
                        if constexpr (BITS % 4 == 0) {                   // 8-byte for 2 and 6
#pragma unroll
                            for (int i = 0; i < BITS; i += 4) {
                                const uint4 v4 = lds_ld16(src + i);
                                w[i] = v4.x; w[i + 1] = v4.y; w[i + 2] = v4.z; w[i + 3] = v4.w;
                            }
                        } else if constexpr (BITS % 2 == 0) {
#pragma unroll
                            for (int i = 0; i < BITS; i += 2) {
                                const uint2 v2 = *(const uint2 *)(src + i);
                                w[i] = v2.x; w[i + 1] = v2.y;
                            }
                        } else {
#pragma unroll
                            for (int i = 0; i < BITS; ++i) w[i] = src[i];
                        }
                        const int gi = nl * G + ((c << 5) >> p.gs_log2);
                        const float sc = bf2f(L.s[gi]), bi = bf2f(L.b[gi]);
                        float a = 0.0f;
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
#pragma unroll
                            for (int i = 0; i < 4; ++i) a = dot2<false>(chunk_pair<BITS>(w, 8 * j + i), xq[m][4 * j + i], a);
                        }
                        v[ii] = __builtin_fmaf(sc, a, v[ii]);
                        v[ii] = __builtin_fmaf(__builtin_fmaf(-OFF, sc, bi), xs[m], v[ii]);
                    }
                }
            }
            const int rr = reduce_rows<2>(v, P, t);
            const int nl = g * RG + rb + rr;
            if ((t & (P / 2 - 1)) == 0 && nl < NB && rb + rr < RG) put(pr, n0 + nl, v[0]);
        }
    }
    return U;
}

// ------------------------------------------------------------------ combine

// Combine of latent outputs [n0, n0 + nb) for every row of the pass (the last down item of
// that block to finish runs it); a non-latent layer also adds the residual here (fc2 is the
// identity and there is no shared expert).
__device__ __forceinline__ void combine_block(const LayerParams &p, int n0, int nb) {
    for (int i = threadIdx.x; i < p.rows * nb; i += WG_THREADS) {
        const int r = i / nb, d = n0 + i % nb;
        const uint16_t c = f2act(p.act_f16, combine_value<true>(p, r, d));
        p.comb[(size_t)r * p.D + d] = c;
        if (!p.L) {
            const float m = act2f(p.act_f16, c), sh = 0.0f;
            const float xv = act2f(p.act_f16, p.x[(size_t)r * p.H + d]);
            p.out[(size_t)r * p.H + d] = f2act(p.act_f16, xv + rnd(p.act_f16, m + sh));
        }
    }
}

}  // namespace moe
