// layer_plan.h -- what the host hands the layer kernel: sizes, pointers and the work-item
// table of one forward. Internal to the library (host and device code of the HIP build).
#pragma once
#include <stdint.h>

namespace moe {

// Stages of one forward, in dependency order (TensorFold pull request 1038, «What's in
// it»: gate gemv -> route -> fc1_latent_proj -> routed experts -> combine -> fc2_latent_proj
// -> + shared -> + residual). A stage only reads what earlier stages wrote.
enum Stage : int {
    ST_GATE = 0,   // gate logits, one wave per expert, fixed 64-lane order
    ST_FC1,        // u = rnd(W1 . x), 16 outputs per item (MFMA)
    ST_SHUP,       // shared expert up + relu^2, 16 outputs per item
    ST_ROUTE,      // one row per item: sigmoid, group-limited top-k, weights (and, for a
                   // one-row pass, the schedule)
    ST_SHDN,       // shared expert down, 16 outputs per item
    ST_SCHED,      // one item: distinct picked experts and their (row, pick) lists
    ST_UP,         // routed expert up + relu^2: (slot, block of outputs) per item
    ST_DOWN,       // routed expert down: (slot, block of outputs) per item
    ST_COMBINE,    // weighted sum over the picks: (row, 256 latent outputs) per item
    ST_FC2,        // m = rnd(W2 . c), out = rnd(x + rnd(m + sh)), 16 outputs per item (for a
                   // one-row pass each item first forms the combine c itself)
    NSTAGE
};

enum : int {
    MAX_EXPERTS = 1024,
    MAX_TOPK = 16,
    MAX_ROWS = 256,
};

// schedule block (int32) in the workspace: [0] = U (distinct experts picked),
// [SCH_EXPERT + u] = expert of slot u (increasing expert id), [SCH_OFF + u] = first pair
// of slot u (U + 1 entries), [SCH_PAIRS + i] = pair row * top_k + pick, sorted by
// (expert, row).
enum : int {
    SCH_U = 0,
    SCH_EXPERT = 1,
    SCH_OFF = SCH_EXPERT + MAX_EXPERTS,
    SCH_PAIRS = SCH_OFF + MAX_EXPERTS + 1,
    SCH_COUNT = SCH_PAIRS + MAX_ROWS * MAX_TOPK,
};

constexpr int WG_THREADS = 256;   // 4 waves of 64 (schedule, expert and combine items)
constexpr int DENSE_THREADS = 512;  // 8 waves (gate, route, dense projections)
constexpr int EXPERT_LDS_CODES = 16384;   // LDS bytes for one expert item's codes
constexpr int EXPERT_LDS_SCALES = 1024;   // ... and for its scales (and again its biases)
constexpr int EXPERT_MAX_BLOCK = 32;      // output rows of one expert item at most
constexpr int COMBINE_BLOCK = 256;
constexpr int DENSE_TILE = 16;    // outputs per dense item

struct LayerParams {
    // sizes
    int H, L, D, E, G, TG, K, I, SI, rows;
    int act_f16, router_f32, has_bias, norm_topk;
    float rho;
    // weights (device, borrowed)
    const uint16_t *gate_w16;
    const float *gate_w32;
    const float *bias;
    const uint16_t *fc1, *fc2;
    const uint32_t *up_q;
    const uint16_t *up_s, *up_b;
    const uint32_t *dn_q;
    const uint16_t *dn_s, *dn_b;
    const uint16_t *su, *sd;
    // input / output (device, caller's)
    const uint16_t *x;
    uint16_t *out;
    // workspace (device, library-owned)
    void *logits;          // [rows][E] bf16 or fp32
    int32_t *idx;          // [rows][K]
    float *wts;            // [rows][K]
    int32_t *sched;        // SCH_COUNT
    uint16_t *u;           // [rows][D] latent (unused when non-latent: experts read x)
    uint16_t *shact;       // [rows][SI]
    uint16_t *eact;        // [rows*K][I]
    uint16_t *eout;        // [rows*K][D]
    uint16_t *comb;        // [rows][D]
    uint16_t *shout;       // [rows][H]
    uint32_t *err;         // device error flag (bit 1: a route found no candidate, bit 2: an
                           // invalid schedule; neither happens for a valid configuration)
    // work-item table: items of stage s are [item_base[s], item_base[s + 1])
    int item_base[NSTAGE + 1];
    int umax;              // slots enumerated by ST_UP / ST_DOWN items
    int up_nb, dn_nb;      // output rows of one routed up / down item
    int up_blocks, dn_blocks, comb_blocks;
    int single_row;        // rows == 1: route writes the schedule, fc2 items combine inline
};

}  // namespace moe
