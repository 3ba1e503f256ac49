// layer_plan.h -- what the host hands the layer kernel: sizes, pointers and the work-item
// table of one forward. Internal to the library (host and device code of the HIP build).
#pragma once
#include <stdint.h>

namespace moe {

// Stages of one forward, in dependency order (TensorFold pull request 1038, «What's in
// it»: gate gemv -> route -> fc1_latent_proj -> routed experts -> combine -> fc2_latent_proj
// -> + shared -> + residual). A stage only reads what earlier launches wrote, or what a
// "last arriver" of the same launch reads after every item it depends on has counted itself
// done. Only the route items wait: for the logits of the gate items dispatched before them
// in the same launch (bounded; see ctr_hand).
enum Stage : int {
    ST_GATE = 0,   // gate logits, one wave per expert, fixed 64-lane order; with the logit
                   // hand-off (LayerParams::hand) the last `rows` items are the route items,
                   // which wait for their row's logits
    ST_FC1,        // u = rnd(W1 . x), 16 outputs per item (MFMA)
    ST_SHUP,       // shared expert up + relu^2, 16 outputs per item
    ST_ROUTE,      // without the hand-off: one row per item; in either place, the last route item
                   // of a multi-row pass builds the schedule (distinct experts and their (row,
                   // pick) lists)
    ST_SHDN_A,     // shared expert down, first half of the outputs
    ST_UP,         // routed expert up + relu^2: (slot, block of outputs) per item
    ST_SHDN_B,     // shared expert down, second half of the outputs
    ST_DOWN,       // routed expert down: (slot, block of outputs) per item; the last item of
                   // each block to finish combines that block (and, non-latent, adds x)
    ST_FC2,        // m = rnd(W2 . c), out = rnd(x + rnd(m + sh)), 16 outputs per item
    NSTAGE
};

enum : int {
    MAX_EXPERTS = 1024,
    MAX_TOPK = 16,
    MAX_ROWS = 256,            // rows of a decode pass
    MAX_PREFILL_ROWS = 4096,   // rows of a prefill pass (and of a handle's workspace)
    // completion counters (uint32) of the last-arriver steps; the dense projections' tile
    // counters follow (offsets in LayerParams)
    CTR_ROUTE = 1,
    CTR_BLOCK = 2,         // CTR_BLOCK + b: down items of output block b done
    CTR_DENSE = 2048,
};

// schedule block (int32) in the workspace: [SCH_U] = U (distinct experts picked); the
// record of slot u at [SCH_REC + SCH_RECW u] = {expert, offset of its pairs, number of pairs,
// first pair, second pair (or -1), 0, 0, 0} (slots in increasing expert id; a slot past U
// holds expert -1), so that an item reads its slot, and the input rows of its first two
// pairs, with two adjacent 16-byte loads; [SCH_PAIRS + i] = pair row * top_k + pick, sorted
// by (expert, row).
enum : int {
    SCH_U = 0,
    SCH_RECW = 8,
    SCH_REC = 8,
    SCH_PAIRS = SCH_REC + SCH_RECW * MAX_EXPERTS,
    SCH_COUNT = SCH_PAIRS + MAX_ROWS * MAX_TOPK,
};

constexpr int WG_THREADS = 256;   // 4 waves of 64 in every item (three items per CU at once)
constexpr int EXPERT_LDS_CODES = 32768;   // LDS bytes for one expert item's codes
constexpr int EXPERT_LDS_SCALES = 2048;   // ... and for its scales (and again its biases)
constexpr int EXPERT_MAX_BLOCK = 64;      // output rows of one expert item at most
constexpr int DENSE_TILE = 16;    // outputs per dense item
constexpr int DENSE_XLDS = 8192;  // input elements a dense item stages in LDS at most

// Waves a dense item splits its part of K over, in contiguous slices that are each a multiple
// of 128 inputs: nw, halved while the part does not divide evenly.
__host__ __device__ inline int dense_nsplit(int kpart, int nw) {
    int n = nw;
    while (n > 1 && kpart % (128 * n)) n >>= 1;
    return n;
}

// The first launch of a one-row pass (the front kernel): blocks of whole output rows of fc1
// and the shared up projection, one workgroup each, FRONT_SW waves taking one K slice each (a
// slice: the K range one wave of a dense item takes), and a gate wave; after them one
// workgroup routes the row.
constexpr int FRONT_SW = 8;
constexpr int FRONT_THREADS = (FRONT_SW + 1) * 64;
constexpr int FRONT_ROWS_MAX = 24;   // rows of a block at most (two MFMA row tiles, the second partial)
constexpr int FRONT_U_MAX = 16;      // K slices at most (each wave takes at most two)
constexpr int FRONT_KW_MAX = 512;   // inputs of a slice at most (one 16-byte load per lane)

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
    uint32_t *ctr;         // completion counters, zero between forwards
    int ctr_fc1, ctr_shup, ctr_shdn, ctr_fc2;   // first counter of each dense projection's tiles
    int ks_fc1, ks_shup, ks_shdn, ks_fc2;       // items (K splits) per 16-output tile
    float *part_fc1, *part_shup, *part_shdn, *part_fc2;   // split-K partial sums [tile][split][row][16]
    uint32_t *err;         // device error flag (bit 1: a route found no candidate, bit 2: an
                           // invalid schedule; neither happens for a valid configuration)
    // work-item table: items of stage s are [item_base[s], item_base[s + 1])
    int item_base[NSTAGE + 1];
    int umax;              // slots enumerated by ST_UP / ST_DOWN items
    int up_nb, dn_nb;      // output rows of one routed up / down item
    int qbits;             // routed expert code width (2, 3, 4, 5, 6, 8)
    int gs_log2;           // log2 of the quantization group (32, 64, 128 inputs)
    int generic;           // not 4-bit codes in groups of 64: the width-generic expert kernels
    int up_blocks, dn_blocks;
    int single_row;        // rows == 1: the route item (first gate item) routes and writes the schedule
    int gate_rc;           // rows of one gate item (the whole pass unless its rows are staged)
    int inline_comb;       // one-row latent pass: fc2 items compute the combine themselves
    // hand != 0: the route items run in the gate launch, after its gate items (the last
    // `rows` items of the gate stage); each gate item hands its logits to them through 64-bit
    // words [rows][E] in the counter block at ctr_hand (bit 32: present), which a route item
    // polls for at most wait_ticks ticks of the 100 MHz real-time counter
    int hand;
    int ctr_hand;
    uint32_t wait_ticks;
    // front_wgs > 0: a one-row pass may run its first launch as the front kernel: an empty
    // workgroup, front_wgs row blocks, then the route workgroup
    int front_wgs;
    int cus;               // compute units of the device
    // the lm_head gemv (a separate entry point sharing the dense tiles): out [rows][lm_n],
    // fp32 (lm_f32) or bf16
    void *lm_out;
    int lm_n, lm_f32;
    // the prefill's per-expert lists of picks (workspace)
    int32_t *pf_count;     // [E] picks of each expert (zeroed before the route)
    int32_t *pf_slot;      // [rows * K] place of each pick in its expert's list
    int32_t *pf_off;       // [E + 1] start of each expert's list
    int32_t *pf_tile;      // [E + 1] first row tile of each expert (tiles of 64 picks)
    int32_t *pf_pairs;     // [rows * K] pick ids (row * K + j), grouped by expert
    int32_t *pf_tmap;      // [row tiles] (expert << 8) | the tile's place among the expert's
};

}  // namespace moe
