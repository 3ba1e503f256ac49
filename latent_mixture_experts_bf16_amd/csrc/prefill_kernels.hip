// prefill_kernels.hip -- the fused prefill of one latent mixture-of-experts layer (gfx950):
// many rows (hundreds to thousands) through the layer in a handful of launches, with the
// projections and the routed experts as MFMA GEMMs over all rows at once, instead of the
// decode kernels' tiles of 16 rows (TensorFold pull request 1038, «Not yet / next»: a fused
// prefill for the latent MoE, where prompts otherwise run through the decode kernels 16 rows
// at a time).
//
// The layer's arithmetic is that of the decode path (layer_items.h): the same gate order (so
// the logits and the routing are the same bits), the same route and combine items, and the
// same rounding points; only the fp32 summation order of the projections and of the experts
// differs. Launches, in order:
//   gate     logits of every row, the decode gate's lane order (8 rows x 8 experts a wave)
//   route    one row per workgroup (the decode route item); each pick takes a place in its
//            expert's list with an atomic counter
//   sched    prefix sums of the per-expert counts (list starts, row-tile starts) and the
//            pick ids scattered into the per-expert lists
//   gemm     fc1 (u = rnd(W1 x)) and shared up (rnd(relu^2(rnd(Su x)))) in one launch: 128 x 128
//            tiles, or one matrix of L + SI rows in 256 x 320 tiles when those fill the machine
//   expert   routed up / down: tiles of 64 picks of one expert x 256 outputs, 4-bit codes
//            decoded in registers, MFMA per group of 64 inputs, then the scale per group (the
//            bias terms by an fp32 MFMA every four groups)
//   gemm     shared down (rnd(Sd a)): 128 x 128 or 256 x 256 tiles
//   combine  every row (the decode combine: lane order and rounding)
//   gemm     fc2 with the final adds: out = rnd(x + rnd(rnd(W2 c) + sh)): as shared down
// Every output's sum runs over its inputs in one fixed order whatever the number of rows and
// the tile shape, so each row of a pass equals that row passed alone, bit for bit.
#include "layer_items.h"

namespace moe {

// ------------------------------------------------------------------ gate

// Logits of rows [8 rb, +8) x experts [8 eb, +8) per wave, each the decode gate's fixed
// order: lane t accumulates, from +0 with fused
// multiply-adds, the terms k = 512 j + 8 t + i (j outer, i inner), and the 64 lane partials
// are joined as the xor butterfly 32 .. 1 joins them in lane 0: ((P0 + P32) + (P16 + P48)) ...
// Here each lane writes its partials to LDS and lane o then sums those of output o in that
// tree: 63 additions and 64 LDS reads instead of 6 cross-lane steps per output, which cut the
// kernel by a third. Rows and experts past the end
// are clamped (computed again, not stored). F32W: fp32 gate weights (fp32 logits); else bf16
// weights, logits rounded to bf16.
constexpr int PF_GATE_RED = 64 * 65;   // one wave's partials: [output][lane], rows 65 apart
template <bool F32W>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 8))) pf_gate_kernel(LayerParams p) {
    constexpr int ET = 8;
    __shared__ float red[4][PF_GATE_RED];
    const int wave = threadIdx.x >> 6, t = threadIdx.x & 63;
    const int nEB = (p.E + ET - 1) / ET, nRB = (p.rows + 7) >> 3;
    const int wb = blockIdx.x * 4 + wave;
    if (wb >= nEB * nRB) return;
    const int eb = wb % nEB, rb = wb / nEB;
    const int H = p.H;
    const uint16_t *xr[8];
    int er[ET];   // gate rows, then their offsets (E H < 2^31)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int r = rb * 8 + i;
        xr[i] = p.x + (size_t)(r < p.rows ? r : p.rows - 1) * H;
    }
#pragma unroll
    for (int i = 0; i < ET; ++i) {
        const int e = eb * ET + i;
        er[i] = (e < p.E ? e : p.E - 1) * H;
    }
    float acc[8][ET];
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int e = 0; e < ET; ++e) acc[r][e] = 0.0f;
    for (int j = 0; j < H / 512; ++j) {
        const int k = 512 * j + 8 * t;
        if constexpr (F32W) {
            uint4 xv[8];
#pragma unroll
            for (int r = 0; r < 8; ++r) xv[r] = *(const uint4 *)(xr[r] + k);
            float4 w0[8], w1[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float *wp = p.gate_w32 + er[e] + k;
                w0[e] = *(const float4 *)wp;
                w1[e] = *(const float4 *)(wp + 4);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float xf[8];
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    const uint32_t wd = i < 2 ? xv[r].x : i < 4 ? xv[r].y : i < 6 ? xv[r].z : xv[r].w;
                    xf[r] = bf2f(i & 1 ? wd >> 16 : wd & 0xFFFFu);
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float4 &q = i < 4 ? w0[e] : w1[e];
                    const float wf = (i & 3) == 0 ? q.x : (i & 3) == 1 ? q.y : (i & 3) == 2 ? q.z : q.w;
#pragma unroll
                    for (int r = 0; r < 8; ++r) acc[r][e] = __builtin_fmaf(xf[r], wf, acc[r][e]);
                }
            }
        } else {
            // the lane's 8 inputs in two halves of 4 (i = 4 h .. 4 h + 3, in order)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                uint2 xv[8], wv[ET];
#pragma unroll
                for (int r = 0; r < 8; ++r) xv[r] = *(const uint2 *)(xr[r] + k + 4 * h);
#pragma unroll
                for (int e = 0; e < ET; ++e) wv[e] = *(const uint2 *)(p.gate_w16 + er[e] + k + 4 * h);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float xf[8], wf[ET];
#pragma unroll
                    for (int r = 0; r < 8; ++r) {
                        const uint32_t wd = i < 2 ? xv[r].x : xv[r].y;
                        xf[r] = bf2f(i & 1 ? wd >> 16 : wd & 0xFFFFu);
                    }
#pragma unroll
                    for (int e = 0; e < ET; ++e) {
                        const uint32_t wd = i < 2 ? wv[e].x : wv[e].y;
                        wf[e] = bf2f(i & 1 ? wd >> 16 : wd & 0xFFFFu);
                    }
#pragma unroll
                    for (int r = 0; r < 8; ++r)
#pragma unroll
                        for (int e = 0; e < ET; ++e) acc[r][e] = __builtin_fmaf(xf[r], wf[e], acc[r][e]);
                }
            }
        }
    }
    // the 64 outputs (expert e of row r is output 8 r + e): lane t writes its partials, lane o
    // sums output o over the lanes
    float *R = red[wave];
#pragma unroll
    for (int c = 0; c < ET / 8; ++c) {
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
            for (int e = 0; e < 8; ++e) R[(8 * r + e) * 65 + t] = acc[r][8 * c + e];
        __builtin_amdgcn_wave_barrier();
        float v[32];
#pragma unroll
        for (int u = 0; u < 32; ++u) v[u] = R[t * 65 + u] + R[t * 65 + u + 32];
#pragma unroll
        for (int d = 16; d >= 1; d >>= 1)
#pragma unroll
            for (int u = 0; u < d; ++u) v[u] = v[u] + v[u + d];
        const int row = rb * 8 + (t >> 3), ex = eb * ET + 8 * c + (t & 7);
        if (row < p.rows && ex < p.E) {
            if constexpr (F32W) ((float *)p.logits)[(size_t)row * p.E + ex] = v[0];
            else ((uint16_t *)p.logits)[(size_t)row * p.E + ex] = f2bf(v[0]);
        }
        __builtin_amdgcn_wave_barrier();   // every lane has read before the next writes
    }
}

// ------------------------------------------------------------------ route and lists

// One row per workgroup: the decode route item, then each pick counts itself in its expert's
// list (its place there is the count before it; the order of the places inside a list does
// not change any result, since every row of a tile is its own MFMA column).
template <int ME>
__global__ void __launch_bounds__(WG_THREADS) pf_route_kernel(LayerParams p) {
    __shared__ RouteLds<WG_THREADS, ME> lds;   // E <= ME (a small table lets more rows run at once)
    const int r = blockIdx.x;
    route_item<WG_THREADS, ME>(p, r, lds);
    __syncthreads();
    if (threadIdx.x < p.K) {
        const int i = r * p.K + (int)threadIdx.x;
        int e = ld_shared32(p.idx + i);
        e = e < 0 || e >= p.E ? 0 : e;   // never: the route writes valid ids
        p.pf_slot[i] = atomicAdd(p.pf_count + e, 1);
    }
}

// Exclusive prefix sums of the per-expert counts (list starts) and of their row tiles of
// PF_BM picks (tile starts), computed by every workgroup (workgroup 0 stores them), then each
// workgroup scatters its 1024 picks into the lists.
constexpr int PF_BM = 64;    // picks per expert tile
constexpr int PF_BN = 128;   // outputs per expert tile and per dense tile
constexpr int PF_DM = 128;   // rows per dense tile

__global__ void __launch_bounds__(WG_THREADS) pf_sched_kernel(LayerParams p) {
    __shared__ int off[MAX_EXPERTS + 1], toff[MAX_EXPERTS + 1];
    __shared__ int sa[WG_THREADS], sb[WG_THREADS];
    const int tid = threadIdx.x, E = p.E;
    // thread t: experts [4t, 4t + 4)
    int c[4], tl[4], s0 = 0, s1 = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = 4 * tid + i;
        c[i] = e < E ? p.pf_count[e] : 0;
        tl[i] = (c[i] + PF_BM - 1) / PF_BM;
        s0 += c[i];
        s1 += tl[i];
    }
    sa[tid] = s0;
    sb[tid] = s1;
    __syncthreads();
    for (int d = 1; d < WG_THREADS; d <<= 1) {   // inclusive scan (Hillis-Steele)
        const int a = tid >= d ? sa[tid - d] : 0, b = tid >= d ? sb[tid - d] : 0;
        __syncthreads();
        sa[tid] += a;
        sb[tid] += b;
        __syncthreads();
    }
    int o0 = sa[tid] - s0, o1 = sb[tid] - s1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = 4 * tid + i;
        if (e < E) { off[e] = o0; toff[e] = o1; }
        o0 += c[i];
        o1 += tl[i];
    }
    if (tid == WG_THREADS - 1) { off[E] = sa[tid]; toff[E] = sb[tid]; }
    __syncthreads();
    if (blockIdx.x == 0) {
        for (int e = tid; e <= E; e += WG_THREADS) {
            p.pf_off[e] = off[e];
            p.pf_tile[e] = toff[e];
        }
        // each row tile's expert and its place among that expert's tiles
        for (int e = tid; e < E; e += WG_THREADS)
            for (int mt = 0; mt < toff[e + 1] - toff[e]; ++mt) p.pf_tmap[toff[e] + mt] = (e << 8) | mt;
    }
    const int NP = p.rows * p.K;
    for (int i = blockIdx.x * 1024 + tid; i < NP && i < (blockIdx.x + 1) * 1024; i += WG_THREADS) {
        int e = p.idx[i];
        e = e < 0 || e >= E ? 0 : e;
        p.pf_pairs[off[e] + p.pf_slot[i]] = i;
    }
}

// ------------------------------------------------------------------ MFMA tiles

// 16-byte units of a tile row of 64 bf16 (128 bytes) are stored at unit (c ^ (row & 7)), so
// that the 16 rows a fragment read touches fall in distinct banks.
__device__ __forceinline__ int swz(int row, int c) { return row * 8 + (c ^ (row & 7)); }

// vmcnt(n) with the other counters left alone
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 15) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

__device__ __forceinline__ void lds_dma16(const void *src, void *lds_dst) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)lds_dst, 16, 0, 0);
}

// A workgroup's place in the logical order of `total` tiles: consecutive workgroups go to
// the 8 XCDs in turn, so logical tile i is run by XCD i / per (per = ceil(total / 8)) and
// neighbouring tiles share an XCD's L2. Returns -1 past the end.
__device__ __forceinline__ int xcd_tile(int total) {
    const int b = (int)blockIdx.x, per = (total + 7) >> 3;
    const int i = b >> 3, x = b & 7;
    if (i >= per) return -1;
    const int l = x * per + i;
    return l < total ? l : -1;
}

enum PfEpi { PF_FC1 = 0, PF_SHUP = 1, PF_SHDN = 2, PF_FC2 = 3 };

template <int KS>
struct PfGemmLds {
    uint4 a[2][PF_DM * KS / 8];    // [buffer][row][KS / 8 units of 16 bytes]: KS inputs of each row
    uint4 b[2][PF_BN * KS / 8];
};

// unit c of a row of U units: the 16 rows of a fragment read fall in distinct banks
template <int U>
__device__ __forceinline__ int swz_u(int row, int c) { return row * U + (c ^ (row & (U - 1))); }

// Outputs n .. n + 3 of row m from their fp32 sums v, through the launch's epilogue (epi is
// EPI, or PF_SHUP for the shared up tiles of an fc1 launch): fc1 (rounded), shared up (relu^2
// of the rounded sum, rounded), shared down (rounded), fc2 (out = rnd(x + rnd(rnd(sum) + sh))).
template <int EPI>
__device__ __forceinline__ void pf_store4(const LayerParams &p, int epi, int m, int n, f32x4 v) {
    uint16_t o[4];
    if constexpr (EPI == PF_FC2) {
        const uint2 sh = *(const uint2 *)(p.shout + (size_t)m * p.H + n);
        const uint2 xv = *(const uint2 *)(p.x + (size_t)m * p.H + n);
        const uint32_t shw[2] = {sh.x, sh.y}, xw[2] = {xv.x, xv.y};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float s16 = bf2f(q & 1 ? shw[q >> 1] >> 16 : shw[q >> 1] & 0xFFFFu);
            const float x16 = bf2f(q & 1 ? xw[q >> 1] >> 16 : xw[q >> 1] & 0xFFFFu);
            const float mm = rnd(0, v[q]);
            o[q] = f2bf(x16 + rnd(0, mm + (p.SI ? s16 : 0.0f)));
        }
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = epi == PF_SHUP ? f2bf(relu_sq(0, rnd(0, v[q]))) : f2bf(v[q]);
    }
    const uint2 ov = {pack2(o[0], o[1]), pack2(o[2], o[3])};
    uint16_t *dst = epi == PF_FC1 ? p.u + (size_t)m * p.L + n
                  : epi == PF_SHUP ? p.shact + (size_t)m * p.SI + n
                  : EPI == PF_SHDN ? p.shout + (size_t)m * p.H + n
                                   : p.out + (size_t)m * p.H + n;
    *(uint2 *)dst = ov;
}

// C[m][n] = sum_k X[m][k] W[n][k] for m < rows (X = [rows][K] bf16, W = [N][K] bf16), tiles
// of 128 rows x 128 outputs, KS inputs a step (double-buffered direct copies to LDS; 128 for
// launches of at most one tile per compute unit, whose 128 KB then cost no occupancy, and
// half the barriers per input). Wave w
// holds rows 64 (w & 1) .. +63 and outputs 64 (w >> 1) .. +63 as 4 x 4 MFMA 16x16x32 tiles
// with the weights as the first operand, so lane l ends with outputs 4 (l >> 4) .. +3 of row
// l & 15 of each tile; each output's sum runs over k in one fixed order (the epilogue is
// pf_store4's). An fc1 launch also runs the shared up tiles when p.SI is set.
template <int EPI, int KS>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(KS == 128 ? 1 : 2, 8))) pf_gemm_kernel(LayerParams p, const uint16_t *__restrict__ X,
                                                         const uint16_t *W, int N, int K) {
    constexpr int UPR = KS / 8, NI = UPR / 2;   // units of a row a step; copies a thread and operand
    __shared__ PfGemmLds<KS> L;
    const int nbm = (p.rows + PF_DM - 1) / PF_DM, t1 = (N / PF_BN) * nbm;
    // fc1 launches carry the shared up projection too (the same input): its tiles follow
    const int total = EPI == PF_FC1 && p.SI ? t1 + (p.SI / PF_BN) * nbm : t1;
    int tile = xcd_tile(total);
    if (tile < 0) return;
    int epi = EPI;
    if (EPI == PF_FC1 && tile >= t1) {
        tile -= t1;
        W = p.su;
        N = p.SI;
        epi = PF_SHUP;
    }
    const int nbn = N / PF_BN;
    const int m0 = (tile / nbn) * PF_DM, n0 = (tile % nbn) * PF_BN;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wm = wave & 1, wn = wave >> 1;
    // the copies: instruction i of wave w moves units 64 (4 i + w) .. +63 of each tile of
    // 128 UPR units, lane l the unit u = 64 (4 i + w) + l: row u / UPR, stored swizzled
    const uint16_t *xs[NI], *ws[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int u = 64 * (4 * i + wave) + lane, row = u / UPR, cs = u % UPR;
        const int c = swz_u<UPR>(row, cs) - row * UPR;   // the swizzle is its own inverse
        const int m = m0 + row < p.rows ? m0 + row : p.rows - 1;
        xs[i] = X + (size_t)m * K + 8 * c;
        ws[i] = W + (size_t)(n0 + row) * K + 8 * c;
    }
    auto issue = [&](int ks, int buf) {
        const int k0 = KS * ks;
#pragma unroll
        for (int i = 0; i < NI; ++i) lds_dma16(xs[i] + k0, &L.a[buf][64 * (4 * i + wave)]);
#pragma unroll
        for (int i = 0; i < NI; ++i) lds_dma16(ws[i] + k0, &L.b[buf][64 * (4 * i + wave)]);
    };
    f32x4 acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = (f32x4){0.f, 0.f, 0.f, 0.f};
    const int nk = K / KS;
    issue(0, 0);
    for (int ks = 0; ks < nk; ++ks) {
        const int buf = ks & 1;
        wait_vm<0>();
        __syncthreads();   // step ks is in LDS; every wave is done with step ks - 1
        if (ks + 1 < nk) issue(ks + 1, buf ^ 1);
#pragma unroll
        for (int s = 0; s < KS / 32; ++s) {
            uint4 xf[4], wf[4];
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
                xf[mi] = lds_ld16(&L.a[buf][swz_u<UPR>(wm * 64 + mi * 16 + (lane & 15), 4 * s + (lane >> 4))]);
#pragma unroll
            for (int ni = 0; ni < 4; ++ni)
                wf[ni] = lds_ld16(&L.b[buf][swz_u<UPR>(wn * 64 + ni * 16 + (lane & 15), 4 * s + (lane >> 4))]);
#pragma unroll
            for (int ni = 0; ni < 4; ++ni)
#pragma unroll
                for (int mi = 0; mi < 4; ++mi)
                    acc[ni][mi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, wf[ni]), __builtin_bit_cast(bf16x8, xf[mi]), acc[ni][mi], 0, 0, 0);
        }
    }
    // epilogue: lane l has outputs n .. n + 3 of row m of each tile
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
        const int m = m0 + wm * 64 + mi * 16 + (lane & 15);
        if (m >= p.rows) continue;
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) pf_store4<EPI>(p, epi, m, n0 + wn * 64 + ni * 16 + 4 * (lane >> 4), acc[ni][mi]);
    }
}

template __global__ void pf_gemm_kernel<PF_FC1, 64>(LayerParams, const uint16_t *, const uint16_t *, int, int);
template __global__ void pf_gemm_kernel<PF_SHDN, 64>(LayerParams, const uint16_t *, const uint16_t *, int, int);
template __global__ void pf_gemm_kernel<PF_FC2, 64>(LayerParams, const uint16_t *, const uint16_t *, int, int);
template __global__ void pf_gemm_kernel<PF_FC1, 128>(LayerParams, const uint16_t *, const uint16_t *, int, int);
template __global__ void pf_gemm_kernel<PF_SHDN, 128>(LayerParams, const uint16_t *, const uint16_t *, int, int);
template __global__ void pf_gemm_kernel<PF_FC2, 128>(LayerParams, const uint16_t *, const uint16_t *, int, int);

// The same products in tiles of 256 rows x TN outputs (8 waves; wave w holds rows 128 (w & 1)
// .. +127 and outputs TN / 4 (w >> 1) .. + TN / 4 - 1 as MFMA 16x16x32 tiles), for passes with
// enough rows to fill the machine with them: per product they copy about half the bytes of
// the 128 x 128 tiles. Every output's sum is formed as in pf_gemm_kernel (the same MFMA,
// operand order and input chunks, in the same order), so both give the same bits. N is a
// multiple of TN. An fc1 launch with p.SI set carries fc1 and the shared up projection as one
// matrix of L + SI rows (fc1's rows first), in tiles of 320 outputs: 256 tiles at 4096 rows
// of the Bolt-like layer, one per compute unit.
constexpr int PF_GM = 256;

template <int TN>
struct PfBigLds {
    uint4 a[2][PF_GM * 8];   // [buffer][row][8 units of 16 bytes]: 64 inputs of each row
    uint4 b[2][TN * 8];
};

template <int EPI, int TN>
__global__ void __launch_bounds__(512) pf_gemm_big_kernel(LayerParams p, const uint16_t *__restrict__ X,
                                                          const uint16_t *__restrict__ W, int N, int K) {
    constexpr int NW = TN / 4, NIT = NW / 16, WI = TN / 64;   // outputs, MFMA tiles, copies a wave
    constexpr bool CAT = EPI == PF_FC1;   // fc1 rows, then the shared up rows
    __shared__ PfBigLds<TN> L;
    const int nbn = N / TN, total = ((p.rows + PF_GM - 1) / PF_GM) * nbn;
    const int tile = xcd_tile(total);
    if (tile < 0) return;
    const int m0 = (tile / nbn) * PF_GM, n0 = (tile % nbn) * TN;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wm = wave & 1, wn = wave >> 1;
    // the copies: instruction i of wave w moves units 64 (8 i + w) .. +63 of each tile, lane l
    // the unit u = 64 (8 i + w) + l: row u >> 3, stored swizzled
    const uint16_t *xs[4], *ws[WI];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int u = 64 * (8 * i + wave) + lane, row = u >> 3, c = (u & 7) ^ (row & 7);
        const int m = m0 + row < p.rows ? m0 + row : p.rows - 1;
        xs[i] = X + (size_t)m * K + 8 * c;
    }
#pragma unroll
    for (int i = 0; i < WI; ++i) {
        const int u = 64 * (8 * i + wave) + lane, row = u >> 3, c = (u & 7) ^ (row & 7);
        const int n = n0 + row;
        ws[i] = (CAT && n >= p.L ? p.su + (size_t)(n - p.L) * K : W + (size_t)n * K) + 8 * c;
    }
    auto issue = [&](int ks, int buf) {
        const int k0 = 64 * ks;
#pragma unroll
        for (int i = 0; i < 4; ++i) lds_dma16(xs[i] + k0, &L.a[buf][64 * (8 * i + wave)]);
#pragma unroll
        for (int i = 0; i < WI; ++i) lds_dma16(ws[i] + k0, &L.b[buf][64 * (8 * i + wave)]);
    };
    f32x4 acc[NIT][8];
#pragma unroll
    for (int a = 0; a < NIT; ++a)
#pragma unroll
        for (int b = 0; b < 8; ++b) acc[a][b] = (f32x4){0.f, 0.f, 0.f, 0.f};
    const int nk = K / 64;
    issue(0, 0);
    for (int ks = 0; ks < nk; ++ks) {
        const int buf = ks & 1;
        wait_vm<0>();
        __syncthreads();   // step ks is in LDS; every wave is done with step ks - 1
        if (ks + 1 < nk) issue(ks + 1, buf ^ 1);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            uint4 xf[8], wf[NIT];
#pragma unroll
            for (int mi = 0; mi < 8; ++mi)
                xf[mi] = lds_ld16(&L.a[buf][swz(wm * 128 + mi * 16 + (lane & 15), 4 * s + (lane >> 4))]);
#pragma unroll
            for (int ni = 0; ni < NIT; ++ni)
                wf[ni] = lds_ld16(&L.b[buf][swz(wn * NW + ni * 16 + (lane & 15), 4 * s + (lane >> 4))]);
#pragma unroll
            for (int ni = 0; ni < NIT; ++ni)
#pragma unroll
                for (int mi = 0; mi < 8; ++mi)
                    acc[ni][mi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, wf[ni]), __builtin_bit_cast(bf16x8, xf[mi]), acc[ni][mi], 0, 0, 0);
        }
    }
#pragma unroll
    for (int mi = 0; mi < 8; ++mi) {
        const int m = m0 + wm * 128 + mi * 16 + (lane & 15);
        if (m >= p.rows) continue;
#pragma unroll
        for (int ni = 0; ni < NIT; ++ni) {
            const int n = n0 + wn * NW + ni * 16 + 4 * (lane >> 4);   // L is a multiple of 4
            if (CAT && n >= p.L) pf_store4<EPI>(p, PF_SHUP, m, n - p.L, acc[ni][mi]);
            else pf_store4<EPI>(p, EPI, m, n, acc[ni][mi]);
        }
    }
}

template __global__ void pf_gemm_big_kernel<PF_FC1, 320>(LayerParams, const uint16_t *, const uint16_t *, int, int);
template __global__ void pf_gemm_big_kernel<PF_SHUP, 256>(LayerParams, const uint16_t *, const uint16_t *, int, int);
template __global__ void pf_gemm_big_kernel<PF_SHDN, 256>(LayerParams, const uint16_t *, const uint16_t *, int, int);
template __global__ void pf_gemm_big_kernel<PF_FC2, 256>(LayerParams, const uint16_t *, const uint16_t *, int, int);

// ------------------------------------------------------------------ routed experts

constexpr int PF_EBN = 256;   // outputs per expert tile (64 per wave)

// Two input steps (groups of 64 inputs) in LDS: one copy in flight while the other is used.
struct PfExpertLds {
    uint4 a[2][PF_BM * 8];         // [buffer][pick][8 units]: 64 inputs of each pick's row, as copied
    uint32_t q[2][PF_EBN * 8];     // [buffer][output][8 words]: 64 codes of each output row
    uint4 ap[PF_BM * 8];           // the step's inputs as pairs (x[i], x[i + 4]) of each 8 (unit c of
                                   // pick r at swz(r, c))
    float sc[PF_EBN];              // the step's scale of each output
    float xs4[4][PF_BM];           // group sums of each pick, for groups g with g % 4 = slot
    float cb4[4][PF_EBN];          // bias - 128 scale of each output, for the same groups
    uint32_t scp[2][PF_EBN], bcp[2][PF_EBN];   // scales and biases of two groups of each output
};

// Tile: picks [m0, m0 + 64) of expert e's list x outputs [n0, n0 + 256) of its up (UP) or
// down projection, one group of 64 inputs (of the 4-bit codes) a step. Per group g and
// output n the tile forms, per pick, a = sum over the group of (128 + q) x (MFMA: the codes
// decoded into bf16 128 + q exactly, the inputs reordered to the codes' pairing) and sx =
// sum of x; sum(w x) with w = q scale + bias is the sum over groups of scale * a (added
// group by group) and of (bias - 128 scale) * sx (added four groups at a time as one fp32
// MFMA 16x16x4 of those factors). A step: its copies wait, then the workgroup reorders the
// inputs and sums each pick's group once (in a fixed order), then wave w multiplies outputs
// 64 w .. +63 for all 64 picks (4 x 4 MFMA 16x16 tiles). MFMA step s of a group takes input
// chunk 2 (l >> 4) + s in lane l's group of 16 -- any order of k serves when both operands
// use the same. Up: eact = rnd(relu^2(rnd(sum))); down: eout = rnd(sum). Three workgroups
// fit a compute unit; the host holds a launch to two with unused dynamic LDS when it has too
// few tiles for a third to pay.
template <bool UP>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 8))) pf_expert_kernel(LayerParams p) {
    __shared__ PfExpertLds L;
    const int Kin = UP ? p.D : p.I, N = UP ? p.I : p.D;
    const int nbn = (N + PF_EBN - 1) / PF_EBN, G = Kin >> 6;
    const int total_tiles = p.pf_tile[p.E];
    const int lt = xcd_tile(total_tiles * nbn);
    if (lt < 0) return;
    const int t = lt / nbn, n0 = (lt % nbn) * PF_EBN;
    const int tcode = p.pf_tmap[t];
    const int e = tcode >> 8;
    const int list0 = p.pf_off[e], cnt = p.pf_off[e + 1] - list0;
    const int m0 = (tcode & 255) * PF_BM;
    // 16-pick MFMA tiles that hold picks: a tile short of 64 picks (the last of its expert)
    // skips the products, copies and reordering of the empty ones
    const int mlim = cnt - m0 >= PF_BM ? 4 : (cnt - m0 + 15) >> 4;
    const int tid = threadIdx.x, wn = tid >> 6, lane = tid & 63, lg = lane >> 4, lr = lane & 15;
    auto pick = [&](int m) { return p.pf_pairs[list0 + (m0 + m < cnt ? m0 + m : cnt - 1)]; };
    auto out_row = [&](int nl) { return n0 + nl < N ? n0 + nl : N - 1; };
    const size_t eN = (size_t)e * N;
    const uint16_t *S = UP ? p.up_s : p.dn_s, *Bs = UP ? p.up_b : p.dn_b;
    const uint16_t *sp = S + (eN + out_row(tid)) * G, *bp = Bs + (eN + out_row(tid)) * G;
    // the scales and biases of groups 2 j and 2 j + 1 of every output, copied into pair buffer
    // j & 1 (G is even): lane l of wave w copies those of output 64 w + l
    auto issue_sc = [&](int j) {
        __builtin_amdgcn_global_load_lds((const void *)(sp + 2 * j),
                                         (__attribute__((address_space(3))) void *)&L.scp[j & 1][64 * wn], 4, 0, 0);
        __builtin_amdgcn_global_load_lds((const void *)(bp + 2 * j),
                                         (__attribute__((address_space(3))) void *)&L.bcp[j & 1][64 * wn], 4, 0, 0);
    };
    issue_sc(0);
    // copies per step: the picks' inputs (64 x 128 bytes: two 1 KB instructions a wave, unit
    // u = 128 w + 64 i + l is chunk u & 7 of pick row u >> 3) and the codes (256 x 32 bytes: two
    // a wave, unit u is half u & 1 of output row u >> 1)
    const uint16_t *xsrc[2];
    const uint32_t *qsrc[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int u = 128 * wn + 64 * i + lane;
        const int pr = pick(u >> 3);
        xsrc[i] = (UP ? (p.L ? p.u : p.x) + (size_t)(pr / p.K) * Kin : p.eact + (size_t)pr * Kin) + 8 * (u & 7);
        qsrc[i] = (UP ? p.up_q : p.dn_q) + (eN + out_row(u >> 1)) * (Kin >> 3) + 4 * (u & 1);
    }
    auto issue = [&](int g, int buf) {
        if (wn < mlim)   // wave w copies the inputs of picks 16 w .. +15
#pragma unroll
            for (int i = 0; i < 2; ++i) lds_dma16(xsrc[i] + 64 * g, &L.a[buf][128 * wn + 64 * i]);
#pragma unroll
        for (int i = 0; i < 2; ++i) lds_dma16(qsrc[i] + 8 * g, &((uint4 *)L.q[buf])[128 * wn + 64 * i]);
    };
    const bool active = n0 + 64 * wn < N;   // the wave has outputs in this tile
    f32x4 acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = (f32x4){0.f, 0.f, 0.f, 0.f};
    issue(0, 0);
    for (int g = 0; g < G; ++g) {
        const int buf = g & 1;
        wait_vm<0>();
        __syncthreads();   // step g and its scales are in LDS; every wave is done with step g - 1
        if (g + 1 < G) issue(g + 1, buf ^ 1);
        if ((g & 1) && g + 1 < G) issue_sc((g + 1) >> 1);
        {
            // thread t: 16 inputs (units 2 (t & 3), +1) of pick t >> 2 (wave w: picks 16 w .. +15)
            const int r = tid >> 2, part = tid & 3, slot = g & 3;
            if (wn < mlim) {
            const uint4 v0 = lds_ld16(&L.a[buf][r * 8 + 2 * part]), v1 = lds_ld16(&L.a[buf][r * 8 + 2 * part + 1]);
            float sx = 0.0f;
            sx = dot2<false>(0x3F803F80u, v0.x, sx);
            sx = dot2<false>(0x3F803F80u, v0.y, sx);
            sx = dot2<false>(0x3F803F80u, v0.z, sx);
            sx = dot2<false>(0x3F803F80u, v0.w, sx);
            sx = dot2<false>(0x3F803F80u, v1.x, sx);
            sx = dot2<false>(0x3F803F80u, v1.y, sx);
            sx = dot2<false>(0x3F803F80u, v1.z, sx);
            sx = dot2<false>(0x3F803F80u, v1.w, sx);
            sx = sx + __shfl_xor(sx, 1, 64);
            sx = sx + __shfl_xor(sx, 2, 64);
            const uint4 p0 = {__builtin_amdgcn_perm(v0.z, v0.x, 0x05040100u), __builtin_amdgcn_perm(v0.z, v0.x, 0x07060302u),
                              __builtin_amdgcn_perm(v0.w, v0.y, 0x05040100u), __builtin_amdgcn_perm(v0.w, v0.y, 0x07060302u)};
            const uint4 p1 = {__builtin_amdgcn_perm(v1.z, v1.x, 0x05040100u), __builtin_amdgcn_perm(v1.z, v1.x, 0x07060302u),
                              __builtin_amdgcn_perm(v1.w, v1.y, 0x05040100u), __builtin_amdgcn_perm(v1.w, v1.y, 0x07060302u)};
            lds_st16(&L.ap[swz(r, 2 * part)], p0);
            lds_st16(&L.ap[swz(r, 2 * part + 1)], p1);
            if (part == 0) L.xs4[slot][r] = sx;
            }
            // thread t: output t's scale and bias for this group
            const uint32_t sw = L.scp[(g >> 1) & 1][tid], bw = L.bcp[(g >> 1) & 1][tid];
            const float sct = bf2f(g & 1 ? sw >> 16 : sw & 0xFFFFu);
            L.sc[tid] = sct;
            L.cb4[slot][tid] = __builtin_fmaf(-128.0f, sct, bf2f(g & 1 ? bw >> 16 : bw & 0xFFFFu));
            // the last group: the slots after it add nothing
            if (g == G - 1)
                for (int z = slot + 1; z < 4; ++z) {
                    L.cb4[z][tid] = 0.0f;
                    if (tid < PF_BM) L.xs4[z][tid] = 0.0f;
                }
        }
        __syncthreads();
        // the products of the first MT pick tiles (MT = 4, or 2 when the tile holds at most 32
        // picks): the same operations in the same order either way
        auto products = [&](auto mt) {
            constexpr int MT = decltype(mt)::value;
            uint4 xf[MT][2];
#pragma unroll
            for (int mi = 0; mi < MT; ++mi) {
                xf[mi][0] = lds_ld16(&L.ap[swz(16 * mi + lr, 2 * lg)]);
                xf[mi][1] = lds_ld16(&L.ap[swz(16 * mi + lr, 2 * lg + 1)]);
            }
#pragma unroll
            for (int ni = 0; ni < 4; ++ni) {
                const int nl = 64 * wn + 16 * ni;
                const uint2 w = *(const uint2 *)&L.q[buf][(nl + lr) * 8 + 2 * lg];
                uint32_t c0[4], c1[4];
                code_pairs<false>(w.x, c0);
                code_pairs<false>(w.y, c1);
                const uint4 wf0 = make_uint4(c0[0], c0[1], c0[2], c0[3]);
                const uint4 wf1 = make_uint4(c1[0], c1[1], c1[2], c1[3]);
                // the pick tiles' products first (independent), then their scaling
                f32x4 a[MT];
#pragma unroll
                for (int mi = 0; mi < MT; ++mi) {
                    a[mi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wf0),
                                                                    __builtin_bit_cast(bf16x8, xf[mi][0]),
                                                                    (f32x4){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                    a[mi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wf1),
                                                                    __builtin_bit_cast(bf16x8, xf[mi][1]), a[mi], 0, 0, 0);
                }
                // the scale of the 4 outputs this lane ends with
                const f32x4 sc = *(const f32x4 *)&L.sc[nl + 4 * lg];
#pragma unroll
                for (int mi = 0; mi < MT; ++mi)
#pragma unroll
                    for (int q = 0; q < 4; ++q) acc[ni][mi][q] = __builtin_fmaf(sc[q], a[mi][q], acc[ni][mi][q]);
            }
            if ((g & 3) == 3 || g == G - 1) {
                // the bias terms of the last four groups: lane l supplies (bias - 128 scale) of
                // output l & 15 of the tile and the group sum of pick l & 15, group slot l >> 4
#pragma unroll
                for (int ni = 0; ni < 4; ++ni) {
                    const float cbl = L.cb4[lg][64 * wn + 16 * ni + lr];
#pragma unroll
                    for (int mi = 0; mi < MT; ++mi)
                        acc[ni][mi] = __builtin_amdgcn_mfma_f32_16x16x4f32(cbl, L.xs4[lg][16 * mi + lr], acc[ni][mi], 0, 0, 0);
                }
            }
        };
        if (active) {
            if (mlim > 2) products(std::integral_constant<int, 4>{});
            else products(std::integral_constant<int, 2>{});
        }
    }
    if (!active) return;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
        const int m = 16 * mi + lr;
        if (m0 + m >= cnt) continue;
        const int pr = pick(m);
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
            const int n = n0 + 64 * wn + 16 * ni + 4 * lg;
            const f32x4 v = acc[ni][mi];
            uint16_t o[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) o[q] = UP ? f2bf(relu_sq(0, rnd(0, v[q]))) : f2bf(v[q]);
            const uint2 ov = {pack2(o[0], o[1]), pack2(o[2], o[3])};
            *(uint2 *)((UP ? p.eact + (size_t)pr * p.I : p.eout + (size_t)pr * p.D) + n) = ov;
        }
    }
}

template __global__ void pf_expert_kernel<true>(LayerParams);
template __global__ void pf_expert_kernel<false>(LayerParams);

// ------------------------------------------------------------------ combine

// comb = rnd(combine) of every row (the decode combine's lane order), 4 outputs a thread; a
// non-latent layer writes out = rnd(x + rnd(comb)) instead (no fc2, no shared expert).
__global__ void __launch_bounds__(256) pf_combine_kernel(LayerParams p) {
    const int per_row = p.D / 4;
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= p.rows * per_row) return;
    const int r = i / per_row, d = 4 * (i % per_row);
    float c4[4];
    combine4(p, r, d, c4);
    uint16_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint16_t c = f2bf(c4[q]);
        if (p.L) {
            o[q] = c;
        } else {
            const float xv = bf2f(p.x[(size_t)r * p.H + d + q]);
            o[q] = f2bf(xv + rnd(0, bf2f(c)));
        }
    }
    const uint2 ov = {pack2(o[0], o[1]), pack2(o[2], o[3])};
    *(uint2 *)((p.L ? p.comb + (size_t)r * p.D : p.out + (size_t)r * p.H) + d) = ov;
}

template __global__ void pf_route_kernel<256>(LayerParams);
template __global__ void pf_route_kernel<MAX_EXPERTS>(LayerParams);
template __global__ void pf_gate_kernel<false>(LayerParams);
template __global__ void pf_gate_kernel<true>(LayerParams);

}  // namespace moe
