// layer_kernels.hip -- HIP kernels of one latent mixture-of-experts decode layer (gfx950).
//
// A forward is a table of work items (tiles of each stage, see layer_plan.h) run as a short
// chain of launches on one stream. Stages that do not depend on each other share a launch:
//   [gate, fc1, shared up] -> [route, shared down] -> [schedule] -> [expert up] ->
//   [expert down] -> [combine] -> [fc2 + shared + residual]
// (for a one-row pass the route writes the schedule and each fc2 item forms the combine
// itself, so that pass is five launches). One workgroup of 4 waves runs one item.
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
//            waves of a workgroup and joined in a fixed order. A row's result never depends
//            on the other rows of the pass (each output row of a tile is its own column of
//            the MFMA), so a multi-row pass equals its one-row passes bit for bit.
//   experts  4-bit affine weights w = q*scale + bias (groups of 64 along k); per 32 inputs
//            the kernel forms sum(q*x) and sum(x) and adds scale*sum(q*x) + bias*sum(x):
//            the same value as sum(w*x) up to fp32 summation order. Each picked expert's
//            weights are read once for all the rows that picked it.
//   combine  8 lanes: lane t sums w_j*y_j over picks j = t, t+8, ... (pick 8 onto pick 0),
//            joined as ((T0+T4)+(T2+T6)) + ((T1+T5)+(T3+T7)).
//   final    out = rnd(x + rnd(rnd(fc2) + shared)).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layer_plan.h"

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

__device__ __forceinline__ float act2f(int f16, uint32_t h) { return f16 ? h2f(h) : bf2f(h); }
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

// the 8 codes of one word, in k order (lowest nibble first), as fp32
__device__ __forceinline__ void nibbles8(uint32_t w, float *q) {
    const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
    q[0] = (float)(lo & 0xFFu);
    q[1] = (float)(hi & 0xFFu);
    q[2] = (float)((lo >> 8) & 0xFFu);
    q[3] = (float)((hi >> 8) & 0xFFu);
    q[4] = (float)((lo >> 16) & 0xFFu);
    q[5] = (float)((hi >> 16) & 0xFFu);
    q[6] = (float)(lo >> 24);
    q[7] = (float)(hi >> 24);
}

// ------------------------------------------------------------------ gate

// Item: NW experts (one per wave), all rows. Fixed summation order described above. The
// loads of a row are issued before its arithmetic; bf16 gate rows of up to 4096 inputs stay
// in registers across the rows of the pass.
template <int NW>
__device__ __forceinline__ void gate_item(const LayerParams &p, int item) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int e = item * NW + wave;
    if (e >= p.E) return;
    const int nj = p.H / 512;
    if (!p.router_f32 && nj <= 8) {
        const uint16_t *wr = p.gate_w16 + (size_t)e * p.H + 8 * lane;
        uint4 wv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (j < nj) wv[j] = *(const uint4 *)(wr + 512 * j);
        for (int r = 0; r < p.rows; ++r) {
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
            if (lane == 0) ((uint16_t *)p.logits)[(size_t)r * p.E + e] = f2bf(acc);
        }
        return;
    }
    for (int r = 0; r < p.rows; ++r) {
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
                        wv[q][0] = *(const uint4 *)(p.gate_w32 + (size_t)e * p.H + k0);
                        wv[q][1] = *(const uint4 *)(p.gate_w32 + (size_t)e * p.H + k0 + 4);
                    } else {
                        wv[q][0] = *(const uint4 *)(p.gate_w16 + (size_t)e * p.H + k0);
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
        if (lane == 0) {
            if (p.router_f32) ((float *)p.logits)[(size_t)r * p.E + e] = acc;
            else ((uint16_t *)p.logits)[(size_t)r * p.E + e] = f2bf(acc);
        }
    }
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

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
        const uint32_t lo = __shfl_xor((uint32_t)v, d, 64);
        const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), d, 64);
        const uint64_t o = ((uint64_t)hi << 32) | lo;
        v = o > v ? o : v;
    }
    return v;
}

template <int NT>
struct RouteLds {
    float s[MAX_EXPERTS];
    float b[MAX_EXPERTS];
    float gam[256];
    int keep[256];
    uint64_t best[NT / 64];
    int picks[MAX_TOPK];
};

// Item: one row (TensorFold pull request 1038, «Per operator and row invariance»:
// group_expert_select at k = 9; pull request 1295, «What this changes»: sigmoid top-8 with
// per-expert norm and sum).
template <int NT>
__device__ __forceinline__ void route_item(const LayerParams &p, int r, RouteLds<NT> &L) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int E = p.E, G = p.G, per = p.E / p.G;
    for (int e = tid; e < E; e += NT) {
        const float z = p.router_f32 ? ((const float *)p.logits)[(size_t)r * E + e]
                                     : bf2f(((const uint16_t *)p.logits)[(size_t)r * E + e]);
        const float s = (float)(1.0 / (1.0 + exp(-(double)z)));
        L.s[e] = s;
        L.b[e] = p.has_bias ? s + p.bias[e] : s;
    }
    __syncthreads();
    // group scores: one thread per group, two best members by rank
    for (int g = tid; g < G; g += NT) {
        uint64_t k1 = 0, k2 = 0;
        int i1 = -1, i2 = -1;
        for (int e = g * per; e < (g + 1) * per; ++e) {
            const uint64_t k = rank_key(L.b[e], e);
            if (i1 < 0 || k > k1) { k2 = k1; i2 = i1; k1 = k; i1 = e; }
            else if (i2 < 0 || k > k2) { k2 = k; i2 = e; }
        }
        L.gam[g] = (i2 >= 0) ? L.b[i1] + L.b[i2] : L.b[i1];
    }
    __syncthreads();
    // kept groups: rank among groups < topk_group
    for (int g = tid; g < G; g += NT) {
        const uint64_t kg = rank_key(L.gam[g], g);
        int rank = 0;
        for (int h = 0; h < G; ++h) rank += rank_key(L.gam[h], h) > kg;
        L.keep[g] = rank < p.TG;
    }
    __syncthreads();
    // top-k among candidates: k rounds of a workgroup-wide max of 64-bit keys
    uint64_t mine[MAX_EXPERTS / NT];
#pragma unroll
    for (int m = 0; m < MAX_EXPERTS / NT; ++m) {
        const int e = tid + m * NT;
        mine[m] = (e < E && L.keep[e / per]) ? rank_key(L.b[e], e) : 0ull;
    }
    for (int j = 0; j < p.K; ++j) {
        uint64_t v = 0;
#pragma unroll
        for (int m = 0; m < MAX_EXPERTS / NT; ++m) v = mine[m] > v ? mine[m] : v;
        v = wave_max_u64(v);
        if (lane == 0) L.best[wave] = v;
        __syncthreads();
        uint64_t w = L.best[0];
#pragma unroll
        for (int q = 1; q < NT / 64; ++q) w = L.best[q] > w ? L.best[q] : w;
        int e = (int)(0xFFFFFFFFu - (uint32_t)w);
#pragma unroll
        for (int m = 0; m < MAX_EXPERTS / NT; ++m)
            if (mine[m] == w) mine[m] = 0ull;
        if (w == 0ull || e < 0 || e >= E) {   // no candidate left: excluded by the host checks
            e = 0;
            if (tid == 0) atomicOr(p.err, 2u);
        }
        if (tid == 0) L.picks[j] = e;
        __syncthreads();
    }
    if (tid == 0) {
        float S = L.s[L.picks[0]];
        for (int j = 1; j < p.K; ++j) S = S + L.s[L.picks[j]];
        for (int j = 0; j < p.K; ++j) {
            const float sj = L.s[L.picks[j]];
            const float v = p.norm_topk ? sj / S : sj;
            p.idx[(size_t)r * p.K + j] = L.picks[j];
            p.wts[(size_t)r * p.K + j] = v * p.rho;
        }
        if (p.single_row) {
            // schedule of a one-row pass: one slot per pick, slots in increasing expert id
            int order[MAX_TOPK];
            for (int j = 0; j < p.K; ++j) {
                int a = j;
                while (a > 0 && L.picks[order[a - 1]] > L.picks[j]) { order[a] = order[a - 1]; --a; }
                order[a] = j;
            }
            for (int u = 0; u < p.K; ++u) {
                p.sched[SCH_EXPERT + u] = L.picks[order[u]];
                p.sched[SCH_OFF + u] = u;
                p.sched[SCH_PAIRS + u] = order[u];
            }
            p.sched[SCH_OFF + p.K] = p.K;
            p.sched[SCH_U] = p.K;
        }
    }
}

// ------------------------------------------------------------------ schedule

struct SchedLds {
    int cnt[MAX_EXPERTS];
    int off[MAX_EXPERTS + 1];
    int cur[MAX_EXPERTS];
    int scan[WG_THREADS];
    int pairs[MAX_ROWS * MAX_TOPK];
};

// Item: the whole pass. Slots are the distinct picked experts in increasing id; each slot
// lists its (row * top_k + pick) pairs in increasing row.
__device__ __forceinline__ void sched_item(const LayerParams &p, SchedLds &L) {
    const int tid = threadIdx.x, E = p.E, NP = p.rows * p.K;
    for (int e = tid; e < E; e += WG_THREADS) { L.cnt[e] = 0; L.cur[e] = 0; }
    __syncthreads();
    for (int i = tid; i < NP; i += WG_THREADS) atomicAdd(&L.cnt[p.idx[i]], 1);
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
            if (L.cnt[e] > 0) {
                p.sched[SCH_EXPERT + run_slots] = e;
                p.sched[SCH_OFF + run_slots] = run_pairs;
                ++run_slots;
            }
            run_pairs += L.cnt[e];
        }
    }
    if (tid == WG_THREADS - 1) {
        p.sched[SCH_U] = run_slots;
        p.sched[SCH_OFF + run_slots] = run_pairs;
    }
    __syncthreads();
    for (int i = tid; i < NP; i += WG_THREADS) {
        const int e = p.idx[i];
        L.pairs[L.off[e] + atomicAdd(&L.cur[e], 1)] = i;
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
    for (int i = tid; i < NP; i += WG_THREADS) p.sched[SCH_PAIRS + i] = L.pairs[i];
}

// ------------------------------------------------------------------ dense bf16 tiles (MFMA)

enum Epi { EPI_FC1 = 0, EPI_SHUP = 1, EPI_SHDN = 2, EPI_FC2 = 3 };

template <int NW>
struct DenseLds {
    f32x4 part[NW][2][64];   // [wave][row tile][lane]
};

// Item: outputs n0..n0+15 of W [N][K] (bf16, row-major) against X [rows][K] (bf16), all rows.
// K is split over up to NW waves in contiguous slices (each a multiple of 128); per 128
// inputs each lane holds 32 consecutive k of one weight row (64 B) and of one input row,
// fed to 4 MFMAs of 32. A wave first issues the loads of up to 4 such steps of its weight
// slice, then multiplies. The slices' partial sums are joined in wave order.
template <int EPI, int NW>
__device__ __forceinline__ void dense_item(const LayerParams &p, const uint16_t *__restrict__ W,
                                           const uint16_t *__restrict__ X, int K, int n0, DenseLds<NW> &L) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nr = lane & 15, grp = lane >> 4;
    int nsplit = NW;
    while (nsplit > 1 && K % (128 * nsplit)) nsplit >>= 1;
    const int kw = K / nsplit, nit = kw / 128;
    const int nrt = (p.rows + 15) >> 4;
    constexpr int RT = 2;   // row tiles (16 rows each) per pass over the weights
    for (int rt0 = 0; rt0 < nrt; rt0 += RT) {
        f32x4 acc[RT];
#pragma unroll
        for (int t = 0; t < RT; ++t) acc[t] = (f32x4){0.f, 0.f, 0.f, 0.f};
        if (wave < nsplit) {
            const uint16_t *wrow = W + (size_t)(n0 + nr) * K + wave * kw + 32 * grp;
            const size_t xoff = (size_t)wave * kw + 32 * grp;
            for (int i0 = 0; i0 < nit; i0 += 4) {
                uint4 a[4][4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (i0 + q < nit) {
                        const uint4 *wp = (const uint4 *)(wrow + 128 * (i0 + q));
                        a[q][0] = wp[0]; a[q][1] = wp[1]; a[q][2] = wp[2]; a[q][3] = wp[3];
                    }
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (i0 + q < nit) {
                        const int kb = 128 * (i0 + q);
#pragma unroll
                        for (int t = 0; t < RT; ++t) {
                            const int row = (rt0 + t) * 16 + nr;
                            if (rt0 + t < nrt) {
                                uint4 b0 = {0, 0, 0, 0}, b1 = b0, b2 = b0, b3 = b0;
                                if (row < p.rows) {
                                    const uint4 *xp = (const uint4 *)(X + (size_t)row * K + xoff + kb);
                                    b0 = xp[0]; b1 = xp[1]; b2 = xp[2]; b3 = xp[3];
                                }
                                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                    __builtin_bit_cast(bf16x8, a[q][0]), __builtin_bit_cast(bf16x8, b0), acc[t], 0, 0, 0);
                                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                    __builtin_bit_cast(bf16x8, a[q][1]), __builtin_bit_cast(bf16x8, b1), acc[t], 0, 0, 0);
                                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                    __builtin_bit_cast(bf16x8, a[q][2]), __builtin_bit_cast(bf16x8, b2), acc[t], 0, 0, 0);
                                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                    __builtin_bit_cast(bf16x8, a[q][3]), __builtin_bit_cast(bf16x8, b3), acc[t], 0, 0, 0);
                            }
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int t = 0; t < RT; ++t) L.part[wave][t][lane] = acc[t];
        __syncthreads();
        // wave t finishes row tile rt0 + t: partials joined in wave order
        if (wave < RT && rt0 + wave < nrt) {
            const int t = wave;
            f32x4 v = L.part[0][t][lane];
            for (int q = 1; q < nsplit; ++q) v = v + L.part[q][t][lane];
            const int row = (rt0 + t) * 16 + nr;
            if (row < p.rows) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int n = n0 + 4 * grp + i;
                    const float a = v[i];
                    if (EPI == EPI_FC1) {
                        p.u[(size_t)row * p.L + n] = f2bf(a);
                    } else if (EPI == EPI_SHUP) {
                        p.shact[(size_t)row * p.SI + n] = f2bf(relu_sq(0, rnd(0, a)));
                    } else if (EPI == EPI_SHDN) {
                        p.shout[(size_t)row * p.H + n] = f2bf(a);
                    } else {
                        const float m = rnd(0, a);
                        const float sh = p.SI ? bf2f(p.shout[(size_t)row * p.H + n]) : 0.0f;
                        const float xv = bf2f(p.x[(size_t)row * p.H + n]);
                        p.out[(size_t)row * p.H + n] = f2bf(xv + rnd(0, m + sh));
                    }
                }
            }
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------------ routed experts (4-bit)

// LDS of one expert item: a block of NB output rows' codes, scales and biases (NB chosen on
// the host so that they fit).
struct ExpertLds {
    uint4 q[EXPERT_LDS_CODES / 16];
    uint16_t s[EXPERT_LDS_SCALES / 2];
    uint16_t b[EXPERT_LDS_SCALES / 2];
};

// Copy `units` 16-byte units from global src to LDS dst with direct global->LDS loads
// (each wave moves 1 KB per instruction, lane i the i-th 16 bytes).
__device__ __forceinline__ void stage_lds(const uint4 *src, uint4 *dst, int units) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    for (int u0 = wave * 64; u0 < units; u0 += WG_THREADS) {
        if (u0 + lane < units)
            __builtin_amdgcn_global_load_lds((const void *)(src + u0 + lane),
                                             (__attribute__((address_space(3))) void *)(dst + u0), 16, 0, 0);
    }
}

// Item: outputs [blk*NB, +NB) of the up (UP) or down projection of slot `slot`, for every
// pair (row, pick) of that slot. The block's 4-bit codes, scales and biases are first staged
// in LDS (all the item's weight bytes in flight at once; each is read from HBM once, whatever
// the number of rows). Each output row's inputs are split in chunks of 32 (16 bytes of
// codes); a row is handled by Cp lanes (Cp = chunks rounded up to a power of two, at most
// 64; NCH chunks per lane when there are more than 64).
template <int NCH, bool UP>
__device__ __forceinline__ void expert_item(const LayerParams &p, int slot, int blk, ExpertLds &L) {
    const int U = p.sched[SCH_U];
    if (slot >= U) return;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int e = p.sched[SCH_EXPERT + slot];
    const int off = p.sched[SCH_OFF + slot];
    const int R = p.sched[SCH_OFF + slot + 1] - off;
    const int NP = p.rows * p.K;
    if (e < 0 || e >= p.E || off < 0 || R < 0 || off + R > NP) {   // never for a valid schedule
        if (threadIdx.x == 0) atomicOr(p.err, 4u);
        return;
    }
    const int Kin = UP ? p.D : p.I, N = UP ? p.I : p.D;
    const int NB = UP ? p.up_nb : p.dn_nb;
    const int n0 = blk * NB;
    const int C = Kin >> 5, G64 = Kin >> 6;
    const size_t qrow = (size_t)(Kin >> 3);
    const uint32_t *Q = (UP ? p.up_q : p.dn_q) + ((size_t)e * N + n0) * qrow;
    const uint16_t *S = (UP ? p.up_s : p.dn_s) + ((size_t)e * N + n0) * G64;
    const uint16_t *B = (UP ? p.up_b : p.dn_b) + ((size_t)e * N + n0) * G64;
    stage_lds((const uint4 *)Q, L.q, NB * C);
    stage_lds((const uint4 *)S, (uint4 *)L.s, NB * G64 / 8);
    stage_lds((const uint4 *)B, (uint4 *)L.b, NB * G64 / 8);

    int Cp = 1;
    while (Cp < C && Cp < 64) Cp <<= 1;
    const int rpp = 64 / Cp;
    const int lrow = lane / Cp, c0 = lane % Cp;
    const uint16_t *xin = UP ? (p.L ? p.u : p.x) : p.eact;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    for (int r = 0; r < R; ++r) {
        int pr = p.sched[SCH_PAIRS + off + r];
        if (pr >= NP) pr = NP - 1;
        const uint16_t *xrow = xin + (UP ? (size_t)(pr / p.K) * Kin : (size_t)pr * Kin);
        // this lane's input chunks: summed, and with one chunk per lane also kept in
        // registers (fp32); with more they are re-read from cache for every output row
        float xf[NCH == 1 ? 32 : 1];
        float xs[NCH];
#pragma unroll
        for (int m = 0; m < NCH; ++m) {
            const int c = c0 + 64 * m;
            float t[32];
#pragma unroll
            for (int i = 0; i < 32; ++i) t[i] = 0.0f;
            if (c < C) {
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) unpack8(p.act_f16, ((const uint4 *)(xrow + 32 * c))[q4], &t[8 * q4]);
            }
            float sum = 0.0f;
#pragma unroll
            for (int i = 0; i < 32; ++i) sum = sum + t[i];
            xs[m] = sum;
            if constexpr (NCH == 1) {
#pragma unroll
                for (int i = 0; i < 32; ++i) xf[i] = t[i];
            }
        }
        for (int nb = wave * rpp; nb < NB; nb += 4 * rpp) {
            const int nl = nb + lrow;                 // row within the block
            float acc = 0.0f;
#pragma unroll
            for (int m = 0; m < NCH; ++m) {
                const int c = c0 + 64 * m;
                if (nl < NB && c < C) {
                    const uint4 qv = L.q[nl * C + c];
                    const float sc = bf2f(L.s[nl * G64 + (c >> 1)]);
                    const float bi = bf2f(L.b[nl * G64 + (c >> 1)]);
                    const uint32_t qw[4] = {qv.x, qv.y, qv.z, qv.w};
                    float part = 0.0f;
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        float qf[8], xv[8];
                        nibbles8(qw[q4], qf);
                        if constexpr (NCH == 1) {
#pragma unroll
                            for (int i = 0; i < 8; ++i) xv[i] = xf[8 * q4 + i];
                        } else {
                            unpack8(p.act_f16, ((const uint4 *)(xrow + 32 * c))[q4], xv);
                        }
#pragma unroll
                        for (int i = 0; i < 8; ++i) part = __builtin_fmaf(qf[i], xv[i], part);
                    }
                    acc = __builtin_fmaf(sc, part, acc);
                    acc = __builtin_fmaf(bi, xs[m], acc);
                }
            }
            for (int d = Cp >> 1; d >= 1; d >>= 1) acc = acc + __shfl_xor(acc, d, 64);
            if (c0 == 0 && nl < NB) {
                const int n = n0 + nl;
                if (UP) p.eact[(size_t)pr * p.I + n] = f2act(p.act_f16, relu_sq(p.act_f16, rnd(p.act_f16, acc)));
                else p.eout[(size_t)pr * p.D + n] = f2act(p.act_f16, acc);
            }
        }
    }
}

// ------------------------------------------------------------------ combine

// The combine of row r at latent output d, before rounding (lane order described at the top).
__device__ __forceinline__ float combine_value(const LayerParams &p, int r, int d) {
    float T[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) T[t] = 0.0f;
#pragma unroll
    for (int j = 0; j < MAX_TOPK; ++j) {
        if (j < p.K) {
            const size_t pr = (size_t)r * p.K + j;
            const float pj = p.wts[pr] * act2f(p.act_f16, p.eout[pr * p.D + d]);
            T[j & 7] = T[j & 7] + pj;
        }
    }
    return ((T[0] + T[4]) + (T[2] + T[6])) + ((T[1] + T[5]) + (T[3] + T[7]));
}

// Item: (row, 256 outputs).
__device__ __forceinline__ void combine_item(const LayerParams &p, int item) {
    const int r = item / p.comb_blocks, blk = item % p.comb_blocks;
    const int d = blk * COMBINE_BLOCK + threadIdx.x;
    if (d >= p.D) return;
    const uint16_t c = f2act(p.act_f16, combine_value(p, r, d));
    p.comb[(size_t)r * p.D + d] = c;
    if (!p.L) {
        // non-latent: fc2 is the identity and there is no shared expert
        const float m = act2f(p.act_f16, c), sh = 0.0f;
        const float xv = act2f(p.act_f16, p.x[(size_t)r * p.H + d]);
        p.out[(size_t)r * p.H + d] = f2act(p.act_f16, xv + rnd(p.act_f16, m + sh));
    }
}

// ------------------------------------------------------------------ driver

constexpr int MAX_LATENT = 6144;
constexpr int DW = DENSE_THREADS / 64;    // waves of a dense workgroup

struct Fc2Lds {
    DenseLds<DW> dense;
    uint16_t c[MAX_LATENT];   // the row's combine, when formed inline
};

// Launch groups: stages [first, last] of one launch (no item of a group depends on another
// item of the same group), its workgroup size and its LDS.
template <int G> struct Group;
template <> struct Group<0> {
    static constexpr int first = ST_GATE, last = ST_SHUP, threads = DENSE_THREADS;
    union Lds { DenseLds<DW> dense; };
};
template <> struct Group<1> {
    static constexpr int first = ST_ROUTE, last = ST_SHDN, threads = DENSE_THREADS;
    union Lds { RouteLds<DENSE_THREADS> route; DenseLds<DW> dense; };
};
template <> struct Group<2> {
    static constexpr int first = ST_SCHED, last = ST_SCHED, threads = WG_THREADS;
    union Lds { SchedLds sched; };
};
template <> struct Group<3> {
    static constexpr int first = ST_UP, last = ST_UP, threads = WG_THREADS;
    union Lds { ExpertLds ex; };
};
template <> struct Group<4> {
    static constexpr int first = ST_DOWN, last = ST_DOWN, threads = WG_THREADS;
    union Lds { ExpertLds ex; };
};
template <> struct Group<5> {
    static constexpr int first = ST_COMBINE, last = ST_COMBINE, threads = WG_THREADS;
    union Lds { int unused; };
};
template <> struct Group<7> {   // expert up for inputs wider than 2048 (several chunks per lane)
    static constexpr int first = ST_UP, last = ST_UP, threads = WG_THREADS;
    union Lds { ExpertLds ex; };
};
template <> struct Group<8> {   // expert down for intermediates wider than 2048
    static constexpr int first = ST_DOWN, last = ST_DOWN, threads = WG_THREADS;
    union Lds { ExpertLds ex; };
};
template <> struct Group<6> {
    static constexpr int first = ST_FC2, last = ST_FC2, threads = DENSE_THREADS;
    union Lds { DenseLds<DW> dense; Fc2Lds fc2; };
};

template <int G, int S, class LdsT>
__device__ __forceinline__ void run_stage(const LayerParams &p, int local, LdsT &lds) {
    constexpr bool wide = G >= 7;
    if constexpr (S == ST_GATE) {
        gate_item<DW>(p, local);
    } else if constexpr (S == ST_FC1) {
        dense_item<EPI_FC1, DW>(p, p.fc1, p.x, p.H, local * DENSE_TILE, lds.dense);
    } else if constexpr (S == ST_SHUP) {
        dense_item<EPI_SHUP, DW>(p, p.su, p.x, p.H, local * DENSE_TILE, lds.dense);
    } else if constexpr (S == ST_ROUTE) {
        route_item<DENSE_THREADS>(p, local, lds.route);
    } else if constexpr (S == ST_SHDN) {
        dense_item<EPI_SHDN, DW>(p, p.sd, p.shact, p.SI, local * DENSE_TILE, lds.dense);
    } else if constexpr (S == ST_SCHED) {
        sched_item(p, lds.sched);
    } else if constexpr (S == ST_UP) {
        const int slot = local / p.up_blocks, blk = local % p.up_blocks;
        if constexpr (wide) expert_item<3, true>(p, slot, blk, lds.ex);
        else expert_item<1, true>(p, slot, blk, lds.ex);
    } else if constexpr (S == ST_DOWN) {
        const int slot = local / p.dn_blocks, blk = local % p.dn_blocks;
        if constexpr (wide) expert_item<3, false>(p, slot, blk, lds.ex);
        else expert_item<1, false>(p, slot, blk, lds.ex);
    } else if constexpr (S == ST_COMBINE) {
        combine_item(p, local);
    } else if constexpr (S == ST_FC2) {
        if (p.single_row) {
            // one-row pass: form the whole combine in LDS first (the same arithmetic as the
            // combine stage); the first item also stores it for inspection
            for (int d = threadIdx.x; d < p.L; d += DENSE_THREADS) {
                const uint16_t c = f2bf(combine_value(p, 0, d));
                lds.fc2.c[d] = c;
                if (local == 0) p.comb[d] = c;
            }
            __syncthreads();
            dense_item<EPI_FC2, DW>(p, p.fc2, lds.fc2.c, p.L, local * DENSE_TILE, lds.fc2.dense);
        } else {
            dense_item<EPI_FC2, DW>(p, p.fc2, p.comb, p.L, local * DENSE_TILE, lds.dense);
        }
    }
}

template <int G, int S, class LdsT>
__device__ __forceinline__ void dispatch(const LayerParams &p, int it, LdsT &lds) {
    if constexpr (S <= Group<G>::last) {
        if (it < p.item_base[S + 1]) {
            run_stage<G, S>(p, it - p.item_base[S], lds);
            return;
        }
        dispatch<G, S + 1>(p, it, lds);
    }
}

template <int G>
__global__ void __launch_bounds__(Group<G>::threads) __attribute__((amdgpu_waves_per_eu(4, 8)))
moe_group_kernel(LayerParams p) {
    __shared__ typename Group<G>::Lds lds;
    const int it = p.item_base[Group<G>::first] + (int)blockIdx.x;
    if (it >= p.item_base[Group<G>::last + 1]) return;
    dispatch<G, Group<G>::first>(p, it, lds);
}

template __global__ void moe_group_kernel<0>(LayerParams);
template __global__ void moe_group_kernel<1>(LayerParams);
template __global__ void moe_group_kernel<2>(LayerParams);
template __global__ void moe_group_kernel<3>(LayerParams);
template __global__ void moe_group_kernel<4>(LayerParams);
template __global__ void moe_group_kernel<5>(LayerParams);
template __global__ void moe_group_kernel<6>(LayerParams);
template __global__ void moe_group_kernel<7>(LayerParams);
template __global__ void moe_group_kernel<8>(LayerParams);

// zero a small device buffer (the error flag) without a memset node in captured graphs
__global__ void moe_clear_kernel(uint32_t *ctr, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) ctr[i] = 0u;
}

}  // namespace moe
