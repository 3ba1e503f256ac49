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

// Item: 4 experts (one per wave), all rows. Fixed summation order described above.
__device__ __forceinline__ void gate_item(const LayerParams &p, int item) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int e = item * 4 + wave;
    if (e >= p.E) return;
    const int nj = p.H / 512;
    for (int r = 0; r < p.rows; ++r) {
        const uint16_t *xr = p.x + (size_t)r * p.H;
        float acc = 0.0f;
        for (int j = 0; j < nj; ++j) {
            const int k0 = 512 * j + 8 * lane;
            float xf[8], wf[8];
            unpack8(p.act_f16, *(const uint4 *)(xr + k0), xf);
            if (p.router_f32) {
                const float4 *wp = (const float4 *)(p.gate_w32 + (size_t)e * p.H + k0);
                const float4 a = wp[0], b = wp[1];
                wf[0] = a.x; wf[1] = a.y; wf[2] = a.z; wf[3] = a.w;
                wf[4] = b.x; wf[5] = b.y; wf[6] = b.z; wf[7] = b.w;
            } else {
                unpack8(0, *(const uint4 *)(p.gate_w16 + (size_t)e * p.H + k0), wf);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) acc = __builtin_fmaf(xf[i], wf[i], acc);
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

struct RouteLds {
    float s[MAX_EXPERTS];
    float b[MAX_EXPERTS];
    float gam[256];
    int keep[256];
    uint64_t best[4];
    int picks[MAX_TOPK];
};

// Item: one row (TensorFold pull request 1038, «Per operator and row invariance»:
// group_expert_select at k = 9; pull request 1295, «What this changes»: sigmoid top-8 with
// per-expert norm and sum).
__device__ __forceinline__ void route_item(const LayerParams &p, int r, RouteLds &L) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int E = p.E, G = p.G, per = p.E / p.G;
    for (int e = tid; e < E; e += WG_THREADS) {
        const float z = p.router_f32 ? ((const float *)p.logits)[(size_t)r * E + e]
                                     : bf2f(((const uint16_t *)p.logits)[(size_t)r * E + e]);
        const float s = (float)(1.0 / (1.0 + exp(-(double)z)));
        L.s[e] = s;
        L.b[e] = p.has_bias ? s + p.bias[e] : s;
    }
    __syncthreads();
    // group scores: one thread per group, two best members by rank
    for (int g = tid; g < G; g += WG_THREADS) {
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
    for (int g = tid; g < G; g += WG_THREADS) {
        const uint64_t kg = rank_key(L.gam[g], g);
        int rank = 0;
        for (int h = 0; h < G; ++h) rank += rank_key(L.gam[h], h) > kg;
        L.keep[g] = rank < p.TG;
    }
    __syncthreads();
    // top-k among candidates: k rounds of a workgroup-wide max of 64-bit keys
    uint64_t mine[MAX_EXPERTS / WG_THREADS];
#pragma unroll
    for (int m = 0; m < MAX_EXPERTS / WG_THREADS; ++m) {
        const int e = tid + m * WG_THREADS;
        mine[m] = (e < E && L.keep[e / per]) ? rank_key(L.b[e], e) : 0ull;
    }
    for (int j = 0; j < p.K; ++j) {
        uint64_t v = 0;
#pragma unroll
        for (int m = 0; m < MAX_EXPERTS / WG_THREADS; ++m) v = mine[m] > v ? mine[m] : v;
        v = wave_max_u64(v);
        if (lane == 0) L.best[wave] = v;
        __syncthreads();
        uint64_t w = L.best[0];
#pragma unroll
        for (int q = 1; q < 4; ++q) w = L.best[q] > w ? L.best[q] : w;
        int e = (int)(0xFFFFFFFFu - (uint32_t)w);
#pragma unroll
        for (int m = 0; m < MAX_EXPERTS / WG_THREADS; ++m)
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

struct DenseLds {
    f32x4 part[4][4][64];   // [wave][row tile][lane]
};

// Item: outputs n0..n0+15 of W [N][K] (bf16, row-major) against X [rows][K] (bf16), all rows.
// Wave w sums a contiguous quarter (or half / all) of K; per 128 inputs each lane holds 32
// consecutive k of one weight row (64 B) and of one input row, fed to 4 MFMAs of 32.
template <int EPI>
__device__ __forceinline__ void dense_item(const LayerParams &p, const uint16_t *__restrict__ W,
                           const uint16_t *__restrict__ X, int K, int n0, DenseLds &L) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nr = lane & 15, grp = lane >> 4;
    const int nsplit = (K % 512 == 0) ? 4 : ((K % 256 == 0) ? 2 : 1);
    const int kw = K / nsplit;
    const int nrt = (p.rows + 15) >> 4;
    for (int rt0 = 0; rt0 < nrt; rt0 += 4) {
        f32x4 acc[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t] = (f32x4){0.f, 0.f, 0.f, 0.f};
        if (wave < nsplit) {
            const uint16_t *wrow = W + (size_t)(n0 + nr) * K + wave * kw + 32 * grp;
            for (int kb = 0; kb < kw; kb += 128) {
                const uint4 *wp = (const uint4 *)(wrow + kb);
                const uint4 a0 = wp[0], a1 = wp[1], a2 = wp[2], a3 = wp[3];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int row = (rt0 + t) * 16 + nr;
                    if (rt0 + t < nrt) {
                        uint4 b0 = {0, 0, 0, 0}, b1 = b0, b2 = b0, b3 = b0;
                        if (row < p.rows) {
                            const uint4 *xp = (const uint4 *)(X + (size_t)row * K + wave * kw + 32 * grp + kb);
                            b0 = xp[0]; b1 = xp[1]; b2 = xp[2]; b3 = xp[3];
                        }
                        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8, a0), __builtin_bit_cast(bf16x8, b0), acc[t], 0, 0, 0);
                        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8, a1), __builtin_bit_cast(bf16x8, b1), acc[t], 0, 0, 0);
                        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8, a2), __builtin_bit_cast(bf16x8, b2), acc[t], 0, 0, 0);
                        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8, a3), __builtin_bit_cast(bf16x8, b3), acc[t], 0, 0, 0);
                    }
                }
            }
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) L.part[wave][t][lane] = acc[t];
        __syncthreads();
        // wave t4 finishes row tile rt0 + t4: partials joined in wave order
        {
            const int t = wave;
            if (rt0 + t < nrt) {
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
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------------ routed experts (4-bit)

// Item: outputs [blk*NB, +NB) of the up (UP) or down projection of slot `slot`, for every
// pair (row, pick) of that slot. Each output row's K inputs are split in chunks of 32 (one
// 16-byte load of codes); a row is handled by Cp lanes (Cp = chunks rounded up to a power of
// two, at most 64; NCH chunks per lane when there are more than 64).
template <int NCH, int RB, bool UP>
__device__ __forceinline__ void expert_item(const LayerParams &p, int slot, int blk) {
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
    const int NB = UP ? UP_BLOCK : DOWN_BLOCK;
    const int n0 = blk * NB, n1 = min(N, n0 + NB);
    const int C = Kin >> 5;
    int Cp = 1;
    while (Cp < C && Cp < 64) Cp <<= 1;
    const int rpp = 64 / Cp;
    const int lrow = lane / Cp, c0 = lane % Cp;
    const size_t qrow = (size_t)(Kin >> 3), grow = (size_t)(Kin >> 6);
    const uint32_t *Q = (UP ? p.up_q : p.dn_q) + (size_t)e * N * qrow;
    const uint16_t *S = (UP ? p.up_s : p.dn_s) + (size_t)e * N * grow;
    const uint16_t *B = (UP ? p.up_b : p.dn_b) + (size_t)e * N * grow;
    const uint16_t *xin = UP ? (p.L ? p.u : p.x) : p.eact;

    for (int rb0 = 0; rb0 < R; rb0 += RB) {
        // per pair: the row of the input, and each of this lane's chunks summed; with one
        // chunk per lane the chunk itself is also kept in registers (fp32), with more it is
        // re-read from cache for every output row
        const uint16_t *xrow[RB];
        float xf[RB][NCH == 1 ? 32 : 1];
        float xs[RB][NCH];
        int pr[RB];
#pragma unroll
        for (int rr = 0; rr < RB; ++rr) {
            pr[rr] = (rb0 + rr < R) ? p.sched[SCH_PAIRS + off + rb0 + rr] : -1;
            if (pr[rr] >= NP) pr[rr] = -1;
            xrow[rr] = xin + (pr[rr] < 0 ? 0 : (UP ? (size_t)(pr[rr] / p.K) * Kin : (size_t)pr[rr] * Kin));
#pragma unroll
            for (int m = 0; m < NCH; ++m) {
                const int c = c0 + 64 * m;
                float t[32];
#pragma unroll
                for (int i = 0; i < 32; ++i) t[i] = 0.0f;
                if (pr[rr] >= 0 && c < C) {
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4)
                        unpack8(p.act_f16, ((const uint4 *)(xrow[rr] + 32 * c))[q4], &t[8 * q4]);
                }
                float sum = 0.0f;
#pragma unroll
                for (int i = 0; i < 32; ++i) sum = sum + t[i];
                xs[rr][m] = sum;
                if constexpr (NCH == 1) {
#pragma unroll
                    for (int i = 0; i < 32; ++i) xf[rr][i] = t[i];
                }
            }
        }
        for (int nb = n0 + wave * rpp; nb < n1; nb += 4 * rpp) {
            const int n = nb + lrow;
            float acc[RB];
#pragma unroll
            for (int rr = 0; rr < RB; ++rr) acc[rr] = 0.0f;
            if (n < n1) {
#pragma unroll
                for (int m = 0; m < NCH; ++m) {
                    const int c = c0 + 64 * m;
                    if (c < C) {
                        const uint4 qv = *(const uint4 *)(Q + (size_t)n * qrow + 4 * c);
                        const float sc = bf2f(S[(size_t)n * grow + (c >> 1)]);
                        const float bi = bf2f(B[(size_t)n * grow + (c >> 1)]);
                        const uint32_t qw[4] = {qv.x, qv.y, qv.z, qv.w};
                        float part[RB];
#pragma unroll
                        for (int rr = 0; rr < RB; ++rr) part[rr] = 0.0f;
#pragma unroll
                        for (int q4 = 0; q4 < 4; ++q4) {
                            float qf[8];
                            nibbles8(qw[q4], qf);
#pragma unroll
                            for (int rr = 0; rr < RB; ++rr) {
                                float xv[8];
                                if constexpr (NCH == 1) {
#pragma unroll
                                    for (int i = 0; i < 8; ++i) xv[i] = xf[rr][8 * q4 + i];
                                } else if (pr[rr] >= 0) {
                                    unpack8(p.act_f16, ((const uint4 *)(xrow[rr] + 32 * c))[q4], xv);
                                } else {
#pragma unroll
                                    for (int i = 0; i < 8; ++i) xv[i] = 0.0f;
                                }
#pragma unroll
                                for (int i = 0; i < 8; ++i) part[rr] = __builtin_fmaf(qf[i], xv[i], part[rr]);
                            }
                        }
#pragma unroll
                        for (int rr = 0; rr < RB; ++rr) {
                            acc[rr] = __builtin_fmaf(sc, part[rr], acc[rr]);
                            acc[rr] = __builtin_fmaf(bi, xs[rr][m], acc[rr]);
                        }
                    }
                }
            }
#pragma unroll
            for (int rr = 0; rr < RB; ++rr) {
                float v = acc[rr];
                for (int d = Cp >> 1; d >= 1; d >>= 1) v = v + __shfl_xor(v, d, 64);
                if (c0 == 0 && n < n1 && pr[rr] >= 0) {
                    if (UP) p.eact[(size_t)pr[rr] * p.I + n] = f2act(p.act_f16, relu_sq(p.act_f16, rnd(p.act_f16, v)));
                    else p.eout[(size_t)pr[rr] * p.D + n] = f2act(p.act_f16, v);
                }
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

struct Fc2Lds {
    DenseLds dense;
    uint16_t c[MAX_LATENT];   // the row's combine, when formed inline
};

union ItemLds {
    RouteLds route;
    SchedLds sched;
    DenseLds dense;
    Fc2Lds fc2;
};

// Launch groups: stages [first, last] of one launch (no item of a group waits on another).
template <int G> struct Group;
template <> struct Group<0> { static constexpr int first = ST_GATE, last = ST_SHUP; };
template <> struct Group<1> { static constexpr int first = ST_ROUTE, last = ST_SHDN; };
template <> struct Group<2> { static constexpr int first = ST_SCHED, last = ST_SCHED; };
template <> struct Group<3> { static constexpr int first = ST_UP, last = ST_UP; };
template <> struct Group<4> { static constexpr int first = ST_DOWN, last = ST_DOWN; };
template <> struct Group<5> { static constexpr int first = ST_COMBINE, last = ST_COMBINE; };
template <> struct Group<6> { static constexpr int first = ST_FC2, last = ST_FC2; };

template <int S>
__device__ __forceinline__ void run_stage(const LayerParams &p, int local, ItemLds &lds) {
    if constexpr (S == ST_GATE) {
        gate_item(p, local);
    } else if constexpr (S == ST_FC1) {
        dense_item<EPI_FC1>(p, p.fc1, p.x, p.H, local * DENSE_TILE, lds.dense);
    } else if constexpr (S == ST_SHUP) {
        dense_item<EPI_SHUP>(p, p.su, p.x, p.H, local * DENSE_TILE, lds.dense);
    } else if constexpr (S == ST_ROUTE) {
        route_item(p, local, lds.route);
    } else if constexpr (S == ST_SHDN) {
        dense_item<EPI_SHDN>(p, p.sd, p.shact, p.SI, local * DENSE_TILE, lds.dense);
    } else if constexpr (S == ST_SCHED) {
        sched_item(p, lds.sched);
    } else if constexpr (S == ST_UP) {
        const int slot = local / p.up_blocks, blk = local % p.up_blocks;
        if (p.D > 2048) expert_item<3, 1, true>(p, slot, blk);
        else expert_item<1, 2, true>(p, slot, blk);
    } else if constexpr (S == ST_DOWN) {
        const int slot = local / p.dn_blocks, blk = local % p.dn_blocks;
        if (p.I > 2048) expert_item<3, 1, false>(p, slot, blk);
        else expert_item<1, 2, false>(p, slot, blk);
    } else if constexpr (S == ST_COMBINE) {
        combine_item(p, local);
    } else if constexpr (S == ST_FC2) {
        if (p.single_row) {
            // one-row pass: form the whole combine in LDS first (the same arithmetic as the
            // combine stage); the first item also stores it for inspection
            for (int d = threadIdx.x; d < p.L; d += WG_THREADS) {
                const uint16_t c = f2bf(combine_value(p, 0, d));
                lds.fc2.c[d] = c;
                if (local == 0) p.comb[d] = c;
            }
            __syncthreads();
            dense_item<EPI_FC2>(p, p.fc2, lds.fc2.c, p.L, local * DENSE_TILE, lds.fc2.dense);
        } else {
            dense_item<EPI_FC2>(p, p.fc2, p.comb, p.L, local * DENSE_TILE, lds.dense);
        }
    }
}

template <int G, int S>
__device__ __forceinline__ void dispatch(const LayerParams &p, int it, ItemLds &lds) {
    if constexpr (S <= Group<G>::last) {
        if (it < p.item_base[S + 1]) {
            run_stage<S>(p, it - p.item_base[S], lds);
            return;
        }
        dispatch<G, S + 1>(p, it, lds);
    }
}

template <int G>
__global__ void __launch_bounds__(WG_THREADS) moe_group_kernel(LayerParams p) {
    __shared__ ItemLds lds;
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

// zero a small device buffer (the error flag) without a memset node in captured graphs
__global__ void moe_clear_kernel(uint32_t *ctr, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) ctr[i] = 0u;
}

}  // namespace moe
