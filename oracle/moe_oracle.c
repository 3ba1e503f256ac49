/*
 * moe_oracle.c -- plain, slow CPU oracle of one latent mixture-of-experts decode layer.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may link, load or call this
 * file: only the tests, the smoke check and the benchmark's CPU-baseline leg use it.
 * It shares no code, header or table with the HIP library.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -shared -fPIC (no FTZ, no contraction:
 * every a*b+c below is two rounded IEEE operations unless fmaf() is written out).
 *
 * What it computes (TensorFold pull request 1038, «What's in it», the latent MoE bullet:
 * gate gemv -> route top-k -> fc1_latent_proj -> routed experts -> combine ->
 * fc2_latent_proj -> + shared -> + residual), one row at a time:
 *
 *   O1  z = rnd(C64(x . Wg))            gate logits; fp32 and fmaf for an fp32 router
 *   O2  s = fp32(1 / (1 + exp(-z)))     sigmoid, evaluated in binary64, rounded once
 *   O3  b = s + c                        correction bias (selection only)
 *   O4  gamma_g = top1(b) + top2(b)      per contiguous group of E/G experts
 *   O5  keep the topk_group best groups (ties -> lower group id)
 *   O6  pick top_k experts of kept groups by (b desc, id asc); NaN ranks lowest
 *   O7  S = sum of s over picks in pick order; w_j = (s_j / S) * rho
 *   O8  u = rnd(W1 . x)                  fc1_latent_proj (u = x when non-latent)
 *   O9  h = rnd(U_e . u), a = rnd(relu(h)^2), y_j = rnd(D_e . a)
 *       with U_e[i][k] = q * scale + bias (b-bit affine codes, b = 4 in the Bolt-like
 *       layer and 2, 3, 5, 6 or 8 for the other widths of the affine family; groups of
 *       group_size (64; 32 or 128) along k)
 *   O10 c = rnd(8-lane combine of fp32(w_j * y_j))
 *   O11 m = rnd(W2 . c)                  fc2_latent_proj (m = c when non-latent)
 *   O12 sh = rnd(Sd . rnd(relu(rnd(Su . x))^2)), or +0 without a shared expert
 *   O13 out = rnd(x + rnd(m + sh))
 *
 * rnd() rounds to the activation dtype (bf16, or fp16 for the fp16 family of
 * TensorFold pull request 1295, «What this changes»: fp16 activations, fp32 sums),
 * round to nearest even, no flush to zero. Every dot product accumulates in fp32.
 * Apart from the gate (whose order is fixed, see oracle_gate_c64), each dot product
 * here is a plain left-to-right sum from k = 0: the layer fixes no order for them.
 *
 * Readings of what the pages leave open (group score, bias use, tie and NaN rules,
 * the combine lane order, rounding points, the 4-bit layout) follow the text above;
 * each is stated at the function that takes it.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_BF16 1
#define ORC_F16 2
#define ORC_F32 3

typedef struct {
    int32_t hidden, latent, n_experts, n_group, topk_group, top_k;
    int32_t expert_inter, shared_inter, group_size;
    int32_t act_dtype;    /* ORC_BF16 or ORC_F16 */
    int32_t router_dtype; /* ORC_BF16 (bf16 weights, bf16 logits) or ORC_F32 */
    int32_t has_bias, norm_topk;
    float routed_scaling;
    int32_t quant_bits;   /* code width of the routed experts: 2, 3, 4, 5, 6 or 8 (0: 4) */
} orc_cfg;

typedef struct {
    const uint16_t *gate_w16; /* [E][H] bf16, router_dtype == ORC_BF16 */
    const float *gate_w32;    /* [E][H] fp32, router_dtype == ORC_F32 */
    const float *corr_bias;   /* [E] fp32 or NULL */
    const uint16_t *fc1_w;    /* [L][H] bf16 */
    const uint16_t *fc2_w;    /* [H][L] bf16 */
    const uint32_t *up_q;     /* [E][I][D/8]: nibble n of word w is code k = 8w + n */
    const uint16_t *up_s, *up_b;     /* [E][I][D/64] bf16 */
    const uint32_t *dn_q;     /* [E][D][I/8] */
    const uint16_t *dn_s, *dn_b;     /* [E][D][I/64] bf16 */
    const uint16_t *sh_up;    /* [SI][H] bf16 */
    const uint16_t *sh_dn;    /* [H][SI] bf16 */
} orc_weights;

/* Optional per-row intermediates (any pointer may be NULL). Values are stored as the
 * float value of what the layer holds at that point (already rounded where rnd applies). */
typedef struct {
    float *z;    /* [E] gate logits */
    float *s;    /* [E] sigmoid scores */
    float *u;    /* [D] expert input (latent) */
    float *a;    /* [k][I] expert activations */
    float *y;    /* [k][D] expert outputs */
    float *c;    /* [D] combine */
    float *m;    /* [H] fc2 output (or c) */
    float *sh;   /* [H] shared expert output */
} orc_stages;

/* ---------------------------------------------------------------- number formats */

static float f_from_bits(uint32_t b) { float f; memcpy(&f, &b, 4); return f; }
static uint32_t bits_from_f(float f) { uint32_t b; memcpy(&b, &f, 4); return b; }

float oracle_bf16_to_f32(uint16_t h) { return f_from_bits((uint32_t)h << 16); }

/* fp32 -> bf16, round to nearest even; NaN stays a quiet NaN. */
uint16_t oracle_f32_to_bf16(float f)
{
    uint32_t b = bits_from_f(f);
    if ((b & 0x7F800000u) == 0x7F800000u && (b & 0x007FFFFFu))
        return (uint16_t)((b >> 16) | 0x0040u);
    uint32_t lsb = (b >> 16) & 1u;
    return (uint16_t)((b + 0x7FFFu + lsb) >> 16);
}

/* IEEE binary16 -> fp32 (exact). */
float oracle_f16_to_f32(uint16_t h)
{
    uint32_t sign = (uint32_t)(h >> 15) << 31;
    int exp = (h >> 10) & 0x1F;
    uint32_t man = h & 0x3FFu;
    if (exp == 0x1F) return f_from_bits(sign | 0x7F800000u | (man << 13));
    if (exp == 0) {
        /* subnormal: man * 2^-24, exact in fp32 */
        float v = (float)man * 5.9604644775390625e-08f;
        return sign ? -v : v;
    }
    return f_from_bits(sign | ((uint32_t)(exp - 15 + 127) << 23) | (man << 13));
}

/* fp32 -> IEEE binary16, round to nearest even, overflow to infinity, with
 * subnormals. Written from the format definition: the value is scaled to an integer
 * number of units of the target's last place and rounded once. */
uint16_t oracle_f32_to_f16(float f)
{
    uint32_t b = bits_from_f(f);
    uint16_t sign = (uint16_t)((b >> 16) & 0x8000u);
    uint32_t absb = b & 0x7FFFFFFFu;
    if (absb >= 0x7F800000u) /* inf or NaN */
        return (uint16_t)(sign | 0x7C00u | (absb > 0x7F800000u ? 0x200u : 0u));
    double a = (double)f_from_bits(absb);
    /* unit in the last place of the binade holding a (binary16: 10 fraction bits,
     * minimum exponent -14, so the smallest ulp is 2^-24) */
    int e;
    frexp(a, &e);              /* a = m * 2^e, m in [0.5, 1) */
    int ulp_exp = e - 1 - 10;  /* a in [2^(e-1), 2^e) */
    if (ulp_exp < -24) ulp_exp = -24;
    double units = ldexp(a, -ulp_exp);       /* exact: a has 24 bits */
    double r = nearbyint(units);             /* default rounding: nearest even */
    double v = ldexp(r, ulp_exp);            /* rounded magnitude */
    if (v > 65504.0) return (uint16_t)(sign | 0x7C00u);   /* beyond the largest finite */
    if (v == 0.0) return sign;
    int ve;
    frexp(v, &ve);
    int ebits = ve - 1 + 15;                 /* biased exponent of v */
    if (ebits <= 0) {                        /* subnormal: v = man * 2^-24 */
        uint32_t man = (uint32_t)ldexp(v, 24);
        return (uint16_t)(sign | man);
    }
    uint32_t man = (uint32_t)(ldexp(v, -(ve - 1) + 10)) - 1024u; /* drop hidden bit */
    return (uint16_t)(sign | ((uint32_t)ebits << 10) | man);
}

static float act_load(const orc_cfg *cfg, uint16_t v)
{
    return cfg->act_dtype == ORC_F16 ? oracle_f16_to_f32(v) : oracle_bf16_to_f32(v);
}

static uint16_t act_store(const orc_cfg *cfg, float v)
{
    return cfg->act_dtype == ORC_F16 ? oracle_f32_to_f16(v) : oracle_f32_to_bf16(v);
}

/* rnd(): round to the activation dtype and return the value as fp32 */
static float rnd(const orc_cfg *cfg, float v) { return act_load(cfg, act_store(cfg, v)); }

/* ---------------------------------------------------------------- O1 gate */

/* C64, the gate's fixed summation order (the pages pin routing to one reference
 * kernel's bits, TensorFold pull request 1038, «Per operator and row invariance»; the
 * order itself is the reading taken here): 64 lane partials, lane t accumulating, in
 * order, the terms at k = 512 j + 8 t + i for j = 0, 1, ... and i = 0..7, starting from
 * +0; then for d = 32, 16, 8, 4, 2, 1 every lane t replaces P[t] by P[t] + P[t ^ d];
 * the result is P[0]. Each term is fmaf(x_k, w_k, P): for bf16 x bf16 the product is
 * exact, so this equals a multiply then an add. K must be a multiple of 512. */
float oracle_gate_c64(const float *x, const float *w, int K)
{
    float P[64], Q[64];
    for (int t = 0; t < 64; ++t) {
        float acc = 0.0f;
        for (int j = 0; j < K / 512; ++j)
            for (int i = 0; i < 8; ++i) {
                int k = 512 * j + 8 * t + i;
                acc = fmaf(x[k], w[k], acc);
            }
        P[t] = acc;
    }
    for (int d = 32; d >= 1; d >>= 1) {
        for (int t = 0; t < 64; ++t) Q[t] = P[t] + P[t ^ d];
        memcpy(P, Q, sizeof P);
    }
    return P[0];
}

/* ---------------------------------------------------------------- O2 sigmoid */

/* Exact logistic function rounded to fp32: evaluated in binary64, rounded once. */
float oracle_sigmoid(float z)
{
    return (float)(1.0 / (1.0 + exp(-(double)z)));
}

/* ---------------------------------------------------------------- O3-O7 route */

/* Total order used for every selection: larger value first, NaN below every number
 * (NaNs among themselves by id), -0 equal to +0, then the lower id first. Returns 1
 * when (va, ia) ranks before (vb, ib). */
static int ranks_before(float va, int ia, float vb, int ib)
{
    int na = isnan(va), nb = isnan(vb);
    if (na != nb) return nb;       /* the number ranks before the NaN */
    if (!na) {
        if (va > vb) return 1;
        if (va < vb) return 0;
    }
    return ia < ib;
}

/* Group-limited top-k selection, one row (TensorFold pull request 1038, «What's in
 * it»: gate gemv then tf_route_topk; «Per operator and row invariance» names it
 * group_expert_select at k = 9). Readings: sigmoid scores; the correction bias enters
 * the selection only; a group's score is the sum of its two best biased scores; the
 * best topk_group groups are kept and the others excluded; top_k experts of the kept
 * groups are picked, in rank order; the weights are the unbiased scores divided by
 * their sum (summed in pick order), times the routed scaling factor.
 * z: [E] logits; bias: [E] or NULL. Writes idx[top_k], w[top_k]; s[E] if not NULL.
 * Returns 0, or -1 for an invalid configuration. */
int oracle_route(const orc_cfg *cfg, const float *z, const float *bias,
                 int32_t *idx, float *w, float *s_out)
{
    enum { MAXE = 4096, MAXG = 256 };
    int E = cfg->n_experts, G = cfg->n_group, TG = cfg->topk_group, K = cfg->top_k;
    if (E <= 0 || E > MAXE || G <= 0 || G > MAXG || E % G || TG < 1 || TG > G) return -1;
    int per = E / G;
    if (K < 1 || K > E || TG * per < K || (G > 1 && per < 2)) return -1;
    float s[MAXE], b[MAXE], gam[MAXG];
    char keep[MAXG], taken[MAXE];

    for (int e = 0; e < E; ++e) {                       /* O2, O3 */
        s[e] = oracle_sigmoid(z[e]);
        b[e] = (cfg->has_bias && bias) ? s[e] + bias[e] : s[e];
        taken[e] = 0;
    }
    for (int g = 0; g < G; ++g) {                       /* O4 */
        int i1 = -1, i2 = -1;
        for (int e = g * per; e < (g + 1) * per; ++e) {
            if (i1 < 0 || ranks_before(b[e], e, b[i1], i1)) { i2 = i1; i1 = e; }
            else if (i2 < 0 || ranks_before(b[e], e, b[i2], i2)) i2 = e;
        }
        gam[g] = (i2 >= 0) ? b[i1] + b[i2] : b[i1];
        keep[g] = 0;
    }
    for (int r = 0; r < TG; ++r) {                      /* O5 */
        int best = -1;
        for (int g = 0; g < G; ++g)
            if (!keep[g] && (best < 0 || ranks_before(gam[g], g, gam[best], best))) best = g;
        keep[best] = 1;
    }
    for (int j = 0; j < K; ++j) {                       /* O6 */
        int best = -1;
        for (int e = 0; e < E; ++e) {
            if (taken[e] || !keep[e / per]) continue;
            if (best < 0 || ranks_before(b[e], e, b[best], best)) best = e;
        }
        taken[best] = 1;
        idx[j] = best;
    }
    float S = s[idx[0]];                                /* O7 */
    for (int j = 1; j < K; ++j) S = S + s[idx[j]];
    for (int j = 0; j < K; ++j) {
        float v = cfg->norm_topk ? s[idx[j]] / S : s[idx[j]];
        w[j] = v * cfg->routed_scaling;
    }
    if (s_out) memcpy(s_out, s, sizeof(float) * E);
    return 0;
}

/* ---------------------------------------------------------------- dense and 4-bit dot products */

/* sum_k x[k] * W[n][k] for a bf16 weight row, left to right in fp32 from +0 */
static float dot_bf16_row(const uint16_t *wrow, const float *x, int K)
{
    float acc = 0.0f;
    for (int k = 0; k < K; ++k) acc = acc + oracle_bf16_to_f32(wrow[k]) * x[k];
    return acc;
}

/* One 4-bit affine weight (a format of the affine family on the mlx-bun decode-speed
 * page, §7.4 experiment axes: affine 2..8-bit with groups of 32/64/128): code q in
 * 0..15 at position k of a row, w = q * scale + bias with the row's bf16 scale and bias
 * of group k / 64. Both operations are exact in fp32 for these operands. */
float oracle_dequant(uint32_t q, uint16_t scale_bits, uint16_t bias_bits)
{
    float sc = oracle_bf16_to_f32(scale_bits), bi = oracle_bf16_to_f32(bias_bits);
    return (float)q * sc + bi;
}

/* Code k of a row of b-bit codes: bits [k b, (k + 1) b) of the row read as one little-endian
 * bit string over its u32 words (bit j of the string is bit j % 32 of word j / 32), the
 * lowest bit first. For b = 4 this is nibble k % 8 of word k / 8, the lowest nibble first;
 * a code of 3, 5 or 6 bits may straddle two words. (The pages fix no packing; this is ours.) */
uint32_t oracle_code(const uint32_t *qrow, int k, int bits)
{
    uint32_t q = 0;
    for (int i = 0; i < bits; ++i) {
        long j = (long)k * bits + i;
        q |= ((qrow[j / 32] >> (j % 32)) & 1u) << i;
    }
    return q;
}

/* sum_k U[n][k] * x[k] for one row of a b-bit expert matrix (codes `qrow` [K b / 32] words,
 * scales and biases [K/gs]), left to right in fp32 from +0 */
static float dot_qb_row(const uint32_t *qrow, const uint16_t *srow, const uint16_t *brow,
                        const float *x, int K, int gs, int bits)
{
    float acc = 0.0f;
    for (int k = 0; k < K; ++k) {
        uint32_t q = oracle_code(qrow, k, bits);
        float wq = oracle_dequant(q, srow[k / gs], brow[k / gs]);
        acc = acc + wq * x[k];
    }
    return acc;
}

/* fp32 value of W . x for every output n of a bf16 matrix [N][K] (exposed for tests) */
void oracle_dense(const uint16_t *W, const float *x, int N, int K, float *out)
{
    for (int n = 0; n < N; ++n) out[n] = dot_bf16_row(W + (size_t)n * K, x, K);
}

/* fp32 value of U . x for every output n of a b-bit matrix (exposed for tests); rows of
 * K b / 32 code words */
void oracle_qb_matvec(const uint32_t *Q, const uint16_t *S, const uint16_t *B,
                      const float *x, int N, int K, int gs, int bits, float *out)
{
    size_t rw = (size_t)K * bits / 32;
    for (int n = 0; n < N; ++n)
        out[n] = dot_qb_row(Q + (size_t)n * rw, S + (size_t)n * (K / gs),
                            B + (size_t)n * (K / gs), x, K, gs, bits);
}

/* the same for 4-bit codes */
void oracle_q4_matvec(const uint32_t *Q, const uint16_t *S, const uint16_t *B,
                      const float *x, int N, int K, int gs, float *out)
{
    oracle_qb_matvec(Q, S, B, x, N, K, gs, 4, out);
}

static float relu_sq(const orc_cfg *cfg, float h)
{
    float r = h > 0.0f ? h : 0.0f;   /* relu of the rounded pre-activation; NaN -> +0 */
    return rnd(cfg, r * r);
}

/* ---------------------------------------------------------------- O10 combine */

/* Weighted sum over the picks (TensorFold pull request 1038, «What's in it»: the
 * combine follows a column reduction's lane order past 8 picks, 8 lanes with pick 8
 * added onto pick 0). Lane t sums, from +0 and in increasing j, the fp32 products
 * w_j * y_j of the picks j = t, t + 8, ...; the lanes are then joined as
 * ((T0 + T4) + (T2 + T6)) + ((T1 + T5) + (T3 + T7)). y: [k][D] values, w: [k].
 * Writes the fp32 sum (before rounding) to out[D]. */
void oracle_combine(const float *y, const float *w, int k, int D, float *out)
{
    for (int d = 0; d < D; ++d) {
        float T[8];
        for (int t = 0; t < 8; ++t) {
            float acc = 0.0f;
            for (int j = t; j < k; j += 8) acc = acc + w[j] * y[(size_t)j * D + d];
            T[t] = acc;
        }
        out[d] = ((T[0] + T[4]) + (T[2] + T[6])) + ((T[1] + T[5]) + (T[3] + T[7]));
    }
}

/* ---------------------------------------------------------------- stages of the layer */

enum { ORC_ST_LATENT = 2, ORC_ST_EXPERT_ACT = 3, ORC_ST_EXPERT_OUT = 4, ORC_ST_COMBINE = 5,
       ORC_ST_SHARED_ACT = 6, ORC_ST_SHARED_OUT = 7, ORC_ST_FC2 = 8, ORC_ST_FINAL = 9 };

/* One stage of one row, from that stage's own input (fp32 values of what the layer holds):
 *   ORC_ST_LATENT      in = x [H]        -> u = rnd(W1 . x) [L]
 *   ORC_ST_EXPERT_ACT  in = u [D], e     -> a = rnd(relu(rnd(U_e . u))^2) [I]
 *   ORC_ST_EXPERT_OUT  in = a [I], e     -> y = rnd(D_e . a) [D]
 *   ORC_ST_SHARED_ACT  in = x [H]        -> a' = rnd(relu(rnd(Su . x))^2) [SI]
 *   ORC_ST_SHARED_OUT  in = a' [SI]      -> sh = rnd(Sd . a') [H]
 *   ORC_ST_FC2         in = c [L]        -> m = rnd(W2 . c) [H]
 *   ORC_ST_FINAL       in = x, in2 = m, in3 = sh (NULL: +0) [H] -> out = rnd(x + rnd(m + sh))
 * out gets the rounded values, pre (if not NULL) the fp32 value before the last rounding.
 * Returns 0, or -1 for a stage this configuration does not have. */
int oracle_stage(const orc_cfg *cfg, const orc_weights *W, int stage, int e, const float *in,
                 const float *in2, const float *in3, float *out, float *pre)
{
    int H = cfg->hidden, L = cfg->latent, I = cfg->expert_inter, SI = cfg->shared_inter;
    int gs = cfg->group_size, D = L ? L : H, nb = cfg->quant_bits ? cfg->quant_bits : 4;
    int n = 0;
    float *tmp = NULL;
    switch (stage) {
    case ORC_ST_LATENT:
        if (!L) return -1;
        n = L;
        tmp = malloc(sizeof(float) * n);
        oracle_dense(W->fc1_w, in, L, H, tmp);
        for (int i = 0; i < n; ++i) out[i] = rnd(cfg, tmp[i]);
        break;
    case ORC_ST_EXPERT_ACT:
        n = I;
        tmp = malloc(sizeof(float) * n);
        oracle_qb_matvec(W->up_q + (size_t)e * I * ((size_t)D * nb / 32), W->up_s + (size_t)e * I * (D / gs),
                         W->up_b + (size_t)e * I * (D / gs), in, I, D, gs, nb, tmp);
        for (int i = 0; i < n; ++i) out[i] = relu_sq(cfg, rnd(cfg, tmp[i]));
        break;
    case ORC_ST_EXPERT_OUT:
        n = D;
        tmp = malloc(sizeof(float) * n);
        oracle_qb_matvec(W->dn_q + (size_t)e * D * ((size_t)I * nb / 32), W->dn_s + (size_t)e * D * (I / gs),
                         W->dn_b + (size_t)e * D * (I / gs), in, D, I, gs, nb, tmp);
        for (int i = 0; i < n; ++i) out[i] = rnd(cfg, tmp[i]);
        break;
    case ORC_ST_SHARED_ACT:
        if (!SI) return -1;
        n = SI;
        tmp = malloc(sizeof(float) * n);
        oracle_dense(W->sh_up, in, SI, H, tmp);
        for (int i = 0; i < n; ++i) out[i] = relu_sq(cfg, rnd(cfg, tmp[i]));
        break;
    case ORC_ST_SHARED_OUT:
        if (!SI) return -1;
        n = H;
        tmp = malloc(sizeof(float) * n);
        oracle_dense(W->sh_dn, in, H, SI, tmp);
        for (int i = 0; i < n; ++i) out[i] = rnd(cfg, tmp[i]);
        break;
    case ORC_ST_FC2:
        if (!L) return -1;
        n = H;
        tmp = malloc(sizeof(float) * n);
        oracle_dense(W->fc2_w, in, H, L, tmp);
        for (int i = 0; i < n; ++i) out[i] = rnd(cfg, tmp[i]);
        break;
    case ORC_ST_FINAL:
        n = H;
        tmp = malloc(sizeof(float) * n);
        for (int i = 0; i < n; ++i) tmp[i] = in[i] + rnd(cfg, in2[i] + (in3 ? in3[i] : 0.0f));
        for (int i = 0; i < n; ++i) out[i] = rnd(cfg, tmp[i]);
        break;
    default:
        return -1;
    }
    if (pre) memcpy(pre, tmp, sizeof(float) * n);
    free(tmp);
    return 0;
}

/* ---------------------------------------------------------------- the layer, one row */

/* x_bits: [H] activation bits. Writes out_bits[H] (rounded), out_f32[H] (the value
 * before the final rounding, may be NULL), idx[top_k], w[top_k]. st may be NULL.
 * Returns 0, -1 for an invalid configuration, -2 when out of memory. */
int oracle_forward_row(const orc_cfg *cfg, const orc_weights *W, const uint16_t *x_bits,
                       uint16_t *out_bits, float *out_f32, int32_t *idx, float *w,
                       const orc_stages *st)
{
    int H = cfg->hidden, L = cfg->latent, E = cfg->n_experts, K = cfg->top_k;
    int I = cfg->expert_inter, SI = cfg->shared_inter, gs = cfg->group_size;
    int D = L ? L : H, nb = cfg->quant_bits ? cfg->quant_bits : 4;
    if (H <= 0 || H % 512 || D % gs || I % gs || gs % 8 || K > 64) return -1;
    if (nb < 2 || nb > 8 || nb == 7 || (D * nb) % 32 || (I * nb) % 32) return -1;
    int rc = -2;
    float *x = malloc(sizeof(float) * H), *z = malloc(sizeof(float) * E);
    float *u = malloc(sizeof(float) * D);
    float *a = malloc(sizeof(float) * (size_t)K * I), *y = malloc(sizeof(float) * (size_t)K * D);
    float *c = malloc(sizeof(float) * D), *m = malloc(sizeof(float) * H);
    float *sh = malloc(sizeof(float) * H), *tmp = malloc(sizeof(float) * (H > D ? H : D));
    float *gsh = SI ? malloc(sizeof(float) * SI) : NULL;
    float *wrow = malloc(sizeof(float) * H), *outv = malloc(sizeof(float) * H);
    if (!x || !z || !u || !a || !y || !c || !m || !sh || !tmp || !wrow || !outv || (SI && !gsh))
        goto done;

    for (int k = 0; k < H; ++k) x[k] = act_load(cfg, x_bits[k]);

    /* O1 gate logits */
    for (int e = 0; e < E; ++e) {
        if (cfg->router_dtype == ORC_F32) {
            z[e] = oracle_gate_c64(x, W->gate_w32 + (size_t)e * H, H);
        } else {
            for (int k = 0; k < H; ++k) wrow[k] = oracle_bf16_to_f32(W->gate_w16[(size_t)e * H + k]);
            z[e] = oracle_bf16_to_f32(oracle_f32_to_bf16(oracle_gate_c64(x, wrow, H)));
        }
    }
    /* O2-O7 */
    rc = oracle_route(cfg, z, W->corr_bias, idx, w, st ? st->s : NULL);
    if (rc) goto done;
    rc = -2;
    /* O8 latent projection */
    if (L) oracle_stage(cfg, W, ORC_ST_LATENT, 0, x, NULL, NULL, u, NULL);
    else memcpy(u, x, sizeof(float) * H);
    /* O9 routed experts */
    for (int j = 0; j < K; ++j) {
        oracle_stage(cfg, W, ORC_ST_EXPERT_ACT, idx[j], u, NULL, NULL, a + (size_t)j * I, NULL);
        oracle_stage(cfg, W, ORC_ST_EXPERT_OUT, idx[j], a + (size_t)j * I, NULL, NULL, y + (size_t)j * D, NULL);
    }
    /* O10 combine */
    oracle_combine(y, w, K, D, tmp);
    for (int d = 0; d < D; ++d) c[d] = rnd(cfg, tmp[d]);
    /* O11 back to hidden */
    if (L) oracle_stage(cfg, W, ORC_ST_FC2, 0, c, NULL, NULL, m, NULL);
    else memcpy(m, c, sizeof(float) * H);
    /* O12 shared expert on the layer input */
    if (SI) {
        oracle_stage(cfg, W, ORC_ST_SHARED_ACT, 0, x, NULL, NULL, gsh, NULL);
        oracle_stage(cfg, W, ORC_ST_SHARED_OUT, 0, gsh, NULL, NULL, sh, NULL);
    } else {
        for (int n = 0; n < H; ++n) sh[n] = 0.0f;
    }
    /* O13 + shared, + residual */
    oracle_stage(cfg, W, ORC_ST_FINAL, 0, x, m, sh, outv, out_f32);
    for (int n = 0; n < H; ++n) out_bits[n] = act_store(cfg, outv[n]);
    if (st) {
        if (st->z) memcpy(st->z, z, sizeof(float) * E);
        if (st->u) memcpy(st->u, u, sizeof(float) * D);
        if (st->a) memcpy(st->a, a, sizeof(float) * (size_t)K * I);
        if (st->y) memcpy(st->y, y, sizeof(float) * (size_t)K * D);
        if (st->c) memcpy(st->c, c, sizeof(float) * D);
        if (st->m) memcpy(st->m, m, sizeof(float) * H);
        if (st->sh) memcpy(st->sh, sh, sizeof(float) * H);
    }
    rc = 0;
done:
    free(x); free(z); free(u); free(a); free(y); free(c); free(m); free(sh);
    free(tmp); free(gsh); free(wrow); free(outv);
    return rc;
}

/* rows independent rows: x_bits [rows][H] -> out_bits [rows][H], out_f32 [rows][H] (or
 * NULL), idx [rows][top_k], w [rows][top_k]. */
int oracle_forward(const orc_cfg *cfg, const orc_weights *W, int rows, const uint16_t *x_bits,
                   uint16_t *out_bits, float *out_f32, int32_t *idx, float *w)
{
    int H = cfg->hidden, K = cfg->top_k;
    for (int r = 0; r < rows; ++r) {
        int rc = oracle_forward_row(cfg, W, x_bits + (size_t)r * H, out_bits + (size_t)r * H,
                                    out_f32 ? out_f32 + (size_t)r * H : NULL,
                                    idx + (size_t)r * K, w + (size_t)r * K, NULL);
        if (rc) return rc;
    }
    return 0;
}

/* ---------------------------------------------------------------- array helpers for the tests */

void oracle_sigmoid_n(const float *z, float *s, long n)
{
    for (long i = 0; i < n; ++i) s[i] = oracle_sigmoid(z[i]);
}

void oracle_f32_to_bf16_n(const float *f, uint16_t *h, long n)
{
    for (long i = 0; i < n; ++i) h[i] = oracle_f32_to_bf16(f[i]);
}

void oracle_f32_to_f16_n(const float *f, uint16_t *h, long n)
{
    for (long i = 0; i < n; ++i) h[i] = oracle_f32_to_f16(f[i]);
}

void oracle_f16_to_f32_n(const uint16_t *h, float *f, long n)
{
    for (long i = 0; i < n; ++i) f[i] = oracle_f16_to_f32(h[i]);
}

/* gate logits of `rows` rows: x [rows][H] fp32 values, w [E][H] fp32 values -> z [rows][E]
 * fp32 (the C64 sum, before any rounding to the logit dtype) */
void oracle_gate_c64_rows(const float *x, const float *w, int rows, int E, int H, float *z)
{
    for (int r = 0; r < rows; ++r)
        for (int e = 0; e < E; ++e)
            z[(size_t)r * E + e] = oracle_gate_c64(x + (size_t)r * H, w + (size_t)e * H, H);
}
