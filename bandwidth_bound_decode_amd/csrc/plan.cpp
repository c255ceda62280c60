// plan.cpp - host-only planning for the decode GEMV: split count, tile, unroll, grid,
// workspace and the summation-depth bound. Pure integer/float arithmetic, no HIP calls.
//
// The rule follows the decode-GEMV page ("Decode GEMV at half of HBM bandwidth",
// "A strong answer"):
//   - cause 1: a skinny output gives too few workgroups to cover the machine, so the
//     reduction dimension is split as well until every CU has several workgroups;
//   - the reversal paragraph: a shape whose row blocks alone already cover the machine
//     several times (the LM head, gate_up) gets no split, because split-K costs extra
//     partial-sum traffic and a second pass; the split count is chosen per shape;
//   - cause 2 / Little's law: each lane keeps U independent 16-byte loads outstanding per
//     row, and the plan reports the bytes that puts in flight per CU next to what
//     bandwidth x latency demands.
// The wave quantization chain of the GPU performance chains page is why the target is a
// whole number of workgroups per CU rather than "just over one wave".
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <new>

#include "plan.h"

namespace bbd {

bool variant_supported(int m, int r, int u)
{
    for (const Variant &v : kVariants)
        if (v.m == m && v.r == r && v.u == u)
            return true;
    return false;
}

}  // namespace bbd

using namespace bbd;

namespace {

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

// Default tile per batch size and shape: (rows per wave R, unroll U, waves per workgroup).
// At M = 1 every wave owns one row (measured on MI355X: single-row waves beat two- and
// four-row waves at every Llama-8B shape once the resident-wave cap below is applied).
//   - Rows of more than 8 wave steps (K > 4096) are read in bursts of 4 steps.
//   - Shorter rows are read in one burst when the grid needs more than one round of
//     waves (of up to 4 steps when rows are that short); when it fits in one round, in
//     the shortest burst (2, 4 or 8 steps, at most the row) that keeps kBurstTargetBytes
//     in flight per CU. Beyond one round (and for single-step rows from
//     kShortRowBlockMinRows rows) kShortRowWaves of them share a workgroup.
// Larger M spends VGPRs on X vectors and accumulators, so the W unroll shrinks. Every
// choice gives bitwise the same result.
void default_tile(int m, int64_t n, int64_t k, int cus, int *r, int *u, int *waves)
{
    int64_t steps = (k + kWaveStep - 1) / kWaveStep;
    if (m == 1) {
        *r = 1;
        const bool many = n > (int64_t)kOneRoundWavesPerCU * cus;
        *waves = steps < 8 && (many || (steps == 1 && n >= kShortRowBlockMinRows))
                     ? kShortRowWaves
                     : 1;
        const int64_t per_cu = ceil_div(n, (int64_t)cus);   // one row per wave
        if (steps > 8) {
            *u = 4;
        } else if (!many) {
            *u = 2;
            while (*u < 8 && *u < steps && per_cu * *u * kWaveStep * 2 < kBurstTargetBytes)
                *u *= 2;
        } else if (steps <= 2) {
            *u = 2;
        } else if (steps <= 4) {
            *u = 4;
        } else {
            *u = 8;
        }
    } else if (m == 2) {
        // 2 <= M <= 16: the tiles of the LDS-staged batch kernel (batch.hip), measured on
        // MI355X at 4096 x 14336; each is also a compiled tile of the general kernel, which
        // runs any call the batch kernel does not take.
        *r = 1;
        *u = 4;
        *waves = 8;
    } else if (m <= 8) {
        *r = 2;
        *u = 2;
        *waves = 4;
    } else {
        *r = 2;
        *u = 1;
        *waves = 8;
    }
}

// Automatic resident-wave cap per CU (0: none) for a batch-1 unsplit launch of `waves_total`
// single-wave workgroups (multi-wave workgroups measured faster uncapped). Measured on MI355X (down_proj 4096 x 14336: 18.36 us capped at 8
// in two equal rounds, 18.97 us uncapped in one round of 16, 20.1 us at 12 in unequal
// rounds; gate_up, QKV and the LM head: best near 12). A cap makes the workgroups of later
// rounds start wherever a CU frees up, which evens out the finish times of the CUs; the cap
// is spread so that all rounds are equally full.
int auto_cap(int m, int s, int waves, int64_t k, int64_t waves_total, int cus)
{
    if (m != 1 || s != 1 || waves != 1)
        return 0;
    const int64_t steps = (k + kWaveStep - 1) / kWaveStep;
    const int64_t per_cu = ceil_div(waves_total, cus);
    int limit;
    if (steps > 8)
        limit = kCapLongRows;
    else if (per_cu > kOneRoundWavesPerCU)
        limit = kCapShortRows;
    else
        return 0;
    if (per_cu <= limit)
        return 0;
    const int64_t rounds = ceil_div(per_cu, limit);
    return (int)ceil_div(per_cu, rounds);
}

// LDS bytes per workgroup that let at most `blocks` workgroups share one CU's LDS, with
// allocations in units of `granule` bytes; 0 if no such size exists.
int lds_for_blocks(int blocks, int granule)
{
    if (blocks < 1)
        return 0;
    const int bytes = kLdsPerCU / blocks / granule * granule;
    if (bytes < granule || (int64_t)(blocks + 1) * bytes <= kLdsPerCU)
        return 0;
    return bytes;
}

// K elements per split for S splits: wave-step aligned when a slice spans more than one
// wave-wide step, so every lane of every slice but the last walks the same vectors.
int64_t slice_for(int64_t k, int s)
{
    int64_t per = ceil_div(k, s);
    return per > kWaveStep ? round_up(per, kWaveStep) : round_up(per, kVecElems);
}

// The most fp32 roundings any product passes through: 4 chained dot2 steps per 16-byte
// vector a lane accumulates (+1 inside the first dot2), 1 for a scalar head and 1 for a
// scalar tail element, 6 levels of the wave64 reduction tree, and S-1 combine additions.
int depth_for(int64_t slice, int s)
{
    int64_t vecs = ceil_div(slice, kVecElems);
    int64_t per_lane = ceil_div(vecs, kWaveLanes);
    return (int)(4 * per_lane + 1 + 2 + 6 + (s - 1));
}

// The same bound for the matrix-core kernel. The instruction's internal summation order is
// not documented, so a product is charged 32 roundings inside the MFMA it enters (as if the
// 32 products of a 16x16x32 step were added one at a time) and the running accumulator one
// rounding per later MFMA of the wave's chain (chunk / 32 per chunk); then the 7 adds of
// the other waves' partial tiles and S-1 combine additions.
int mfma_depth_for(int64_t slice, int s, int chunk)
{
    int64_t chunks = ceil_div(slice, chunk);
    int64_t turns = ceil_div(chunks, kMfmaWaves);
    return (int)(32 + (chunk / 32) * turns + (kMfmaWaves - 1) + (s - 1));
}

// The matrix-core kernel for unaligned rows: a wave's chain holds the MFMAs of at most one
// edge or ragged chunk and of its share of the streamed whole chunks (32 roundings in the
// first MFMA, then one per MFMA), then the 7 wave additions, then the addition of the fp32
// sum of the <= 15 head and tail elements (a shorter chain).
int mfma_unaligned_depth_for(int64_t k)
{
    const int64_t chunks = k / kMfmaUnalignedChunk;
    const int64_t turns = ceil_div(chunks, kMfmaWaves) + 1;
    return (int)(32 + (kMfmaUnalignedChunk / 32) * turns + (kMfmaWaves - 1) + 1);
}

bool valid_waves(int w) { return w == 1 || w == 2 || w == 4 || w == 8; }

// INT4 weights, unsplit. A product of a 32-weight vector passes through its 16-step dot2
// chain (+1 inside the first dot2), the scaled addition into the lane's accumulator, one
// more such addition per later vector of the lane, and the 6 levels of the wave reduction.
int int4_depth_for(int64_t k)
{
    int64_t vecs = ceil_div(k, kInt4VecElems);
    return (int)(17 + 1 + ceil_div(vecs, kWaveLanes) + 6);
}

bool int4_tile_supported(int u, int r)
{
    return (r == 1 && (u == 1 || u == 2 || u == 4 || u == 7)) || (r == 2 && (u == 1 || u == 2));
}

// Tiles measured on MI355X (sweep of U, R, waves per workgroup, grid cap and the x staging
// form at the six Llama shapes, graph replays of rotated weights). With x in LDS:
//   - the burst is the whole row where the row's vectors per lane allow it (7 at K = 14336,
//     2 at K = 4096), else 4, 2 or 1 vectors per lane;
//   - one row per wave, one workgroup per row block: 8 waves per workgroup for rows of four
//     or more vectors per lane, 4 for short rows below 16384 outputs;
//   - short rows from 16384 outputs on: two rows per wave sharing every x vector, 4 waves
//     per workgroup, at most 32 waves per CU, the workgroups looping over row blocks;
//   - the fp16 form of x only when a workgroup covers at least kInt4Fp16MinRows rows (the
//     LM head), since its staging is paid once per workgroup.
// Without LDS (x longer than 64 KiB staged), two rows per single-wave workgroup.
gemv_status plan_int4(gemv_plan_t *out, int64_t n, int64_t k, int m,
                      const gemv_device_desc *dev, const gemv_plan_opts &o)
{
    if (m != 1 || k % kInt4VecElems != 0 || o.splits > 1 || o.mfma > 0 || o.waves_per_cu < 0 ||
        o.waves_per_cu > kMaxWavesPerCU || o.int4_fp16 < -1 || o.int4_fp16 > 1)
        return GEMV_ERR_INVALID_ARG;
    const int64_t vecs = k / kInt4VecElems;
    const int64_t steps = ceil_div(vecs, kWaveLanes);
    // x staged in LDS: 64 bytes of pairs and a 4-byte multiplier per 32-element vector
    const int64_t x_lds = vecs * (64 + 4);
    const bool xlds = x_lds <= kInt4MaxLdsX;
    int r, u, waves, cap = 0;
    if (xlds) {
        u = steps == 7 ? 7 : steps >= 4 ? 4 : steps >= 2 ? 2 : 1;
        if (steps < 4 && n >= kInt4TwoRowsFrom) {
            r = 2;
            u = u > 2 ? 2 : u;
            waves = 4;
            cap = kInt4ShortRowsCap;
        } else {
            // rows of fewer than 4 vectors per lane in 4-wave workgroups: twice the grid, so
            // the short shapes reach every CU (k_proj 2.72 -> 2.48 us, QKV 4.78 -> 4.66 us)
            r = 1;
            waves = steps < 4 ? 4 : 8;
        }
    } else {
        r = 2;
        u = 2;
        waves = 1;
    }
    if (o.rows_per_wave)
        r = o.rows_per_wave;
    if (o.unroll)
        u = o.unroll;
    if (o.waves_per_block)
        waves = o.waves_per_block;
    if (!int4_tile_supported(u, r) || !(valid_waves(waves) || waves == 16) ||
        (!xlds && u == 7 && waves > 8))
        return GEMV_ERR_INVALID_ARG;
    const int depth = int4_depth_for(k);
    if (depth > kMaxDepth)
        return GEMV_ERR_INVALID_ARG;
    gemv_plan_s *p = new (std::nothrow) gemv_plan_s;
    if (!p)
        return GEMV_ERR_INVALID_ARG;
    memset(p, 0, sizeof *p);
    p->n = n;
    p->k = k;
    p->m = 1;
    p->device = -1;
    p->dev = *dev;
    p->splits = 1;
    p->rows_per_wave = r;
    p->waves_per_block = waves;
    p->unroll = u;
    p->slice = k;
    // One workgroup per row block, or (waves_per_cu) at most that many resident waves' worth
    // of workgroups per CU, each looping over row blocks so that its x staging serves them.
    const int64_t row_blocks = ceil_div(n, (int64_t)r * waves);
    int64_t grid = row_blocks;
    const int waves_cap = o.waves_per_cu > 0 ? o.waves_per_cu : cap;
    if (waves_cap > 0) {
        const int64_t most = ceil_div((int64_t)dev->compute_units * waves_cap, waves);
        if (most < grid)
            grid = most;
    }
    p->grid_x = (int)grid;
    p->grid_y = 1;
    p->block_threads = kWaveLanes * waves;
    p->depth_bound = depth;
    p->weights = GEMV_WEIGHTS_INT4;
    p->lds_bytes = xlds ? (int)x_lds : 0;   // the staged x
    p->waves_per_cu = waves_cap;
    // The fp16 form of the staged x costs its conversion once per workgroup and saves about
    // a quarter of the unpacking per row: tried when a workgroup covers enough rows.
    const int64_t rows_per_group = (int64_t)r * waves * ceil_div(row_blocks, grid);
    p->int4_fp16 = xlds && (o.int4_fp16 > 0 ||
                            (o.int4_fp16 == 0 && rows_per_group >= kInt4Fp16MinRows));
    int64_t per_cu = ceil_div((int64_t)p->grid_x * waves, dev->compute_units);
    if (per_cu > kMaxWavesPerCU)
        per_cu = kMaxWavesPerCU;
    p->bif_per_cu = (double)per_cu * u * r * kWaveLanes * 16.0;
    p->bif_needed = gemv_bytes_in_flight(dev->hbm_bytes_per_s, dev->latency_s) / dev->compute_units;
    *out = p;
    return GEMV_OK;
}

// RMSNorm prologue, batch 1, unsplit, one row per wave. A product W * hi (or W * lo)
// passes through its lane's chain (four dot2 per vector, +1 inside the first), the one
// addition of the two chains, the 6 wave levels and the final scaling; rms_inv carries
// half the relative error of sum h^2 (per-thread dot2 chains of four per vector, +1, the
// 6 wave levels and waves - 1 adds) plus the division, square root and reciprocal. The
// bound adds both (with the final product) as roundings.
int rmsnorm_depth_for(int64_t k, int waves)
{
    const int64_t vecs = ceil_div(k, kVecElems);
    const int64_t dot = 4 * ceil_div(vecs, kWaveLanes) + 1 + 1 + 6;
    const int64_t sq = 4 * ceil_div(vecs, (int64_t)kWaveLanes * waves) + 1 + 6 + (waves - 1);
    return (int)(dot + ceil_div(sq, 2) + 4);
}

gemv_status plan_rmsnorm(gemv_plan_t *out, int64_t n, int64_t k, int m,
                         const gemv_device_desc *dev, const gemv_plan_opts &o)
{
    if (m != 1 || k % kVecElems != 0 || k > kNormMaxK || o.splits > 1 || o.mfma > 0 ||
        o.rows_per_wave > 1)
        return GEMV_ERR_INVALID_ARG;
    const int64_t vecs = k / kVecElems;
    const int64_t steps = ceil_div(vecs, kWaveLanes);
    // Measured (sweep of U, waves per workgroup and grid size at QKV and gate_up): rows of
    // 8 or more wave steps in one burst of 8, shorter in the largest burst that fits.
    int u = o.unroll ? o.unroll : (steps >= 8 ? 8 : steps >= 4 ? 4 : steps >= 2 ? 2 : 1);
    int waves = o.waves_per_block ? o.waves_per_block : 8;
    if (!(u == 1 || u == 2 || u == 4 || u == 8) || !valid_waves(waves))
        return GEMV_ERR_INVALID_ARG;
    const int depth = rmsnorm_depth_for(k, waves);
    if (depth > kMaxDepth)
        return GEMV_ERR_INVALID_ARG;
    gemv_plan_s *p = new (std::nothrow) gemv_plan_s;
    if (!p)
        return GEMV_ERR_INVALID_ARG;
    memset(p, 0, sizeof *p);
    p->n = n;
    p->k = k;
    p->m = 1;
    p->device = -1;
    p->dev = *dev;
    p->splits = 1;
    p->rows_per_wave = 1;
    p->waves_per_block = waves;
    p->unroll = u;
    p->slice = k;
    // Up to four row blocks per CU the workgroups loop over row blocks, two per CU, so the
    // staging is paid once per workgroup rather than once per block (measured: QKV 9.3 us
    // against 10.1 us with one workgroup per block). Beyond that every block gets a workgroup
    // of its own and the dispatcher hands them to whichever CU frees up, where looping
    // workgroups would each own a fixed share (gate_up 35.5-36.0 against 36.1-36.8 us with
    // four looping workgroups per CU, lm_head 149-152 against 163 us). opts.waves_per_cu
    // sets the looping grid's workgroups per CU instead, -1 one workgroup per block.
    const int64_t blocks = ceil_div(n, waves);
    const bool many = blocks > (int64_t)kNormManyBlocksPerCU * dev->compute_units;
    int64_t per_cu_blocks = kNormBlocksPerCU;
    if (o.waves_per_cu > 0)
        per_cu_blocks = o.waves_per_cu >= waves ? o.waves_per_cu / waves : 1;
    const int64_t most = o.waves_per_cu < 0 || (many && o.waves_per_cu == 0)
                             ? blocks
                             : per_cu_blocks * dev->compute_units;
    p->grid_x = (int)(blocks < most ? blocks : most);
    p->grid_y = 1;
    p->block_threads = kWaveLanes * waves;
    p->depth_bound = depth;
    p->prologue = GEMV_PROLOGUE_RMSNORM;
    p->lds_bytes = (int)(32 * vecs + 4 * waves);
    int64_t per_cu = ceil_div((int64_t)p->grid_x * waves, dev->compute_units);
    if (per_cu > kMaxWavesPerCU)
        per_cu = kMaxWavesPerCU;
    p->bif_per_cu = (double)per_cu * u * kWaveLanes * 16.0;
    p->bif_needed = gemv_bytes_in_flight(dev->hbm_bytes_per_s, dev->latency_s) / dev->compute_units;
    *out = p;
    return GEMV_OK;
}

}  // namespace

extern "C" double gemv_bytes_in_flight(double bytes_per_s, double latency_s)
{
    return bytes_per_s * latency_s;
}

extern "C" gemv_status gemv_plan_for(gemv_plan_t *out, int64_t n, int64_t k, int m,
                                     const gemv_device_desc *dev, const gemv_plan_opts *opts)
{
    if (!out)
        return GEMV_ERR_INVALID_ARG;
    *out = nullptr;
    if (!dev || dev->compute_units < 1 || !(dev->hbm_bytes_per_s > 0) || !(dev->latency_s > 0))
        return GEMV_ERR_INVALID_ARG;
    if (n < 1 || k < 1 || m < 1 || m > GEMV_MAX_M)
        return GEMV_ERR_INVALID_ARG;
    // Row indices and grid sizes are held in 32 bits on the device.
    if (n > (int64_t)1 << 30 || k > (int64_t)1 << 30)
        return GEMV_ERR_INVALID_ARG;
    gemv_plan_opts o = {0, 0, 0, 0, 0, 0, 0, 0, 0};
    if (opts)
        o = *opts;
    if (o.splits < 0 || o.rows_per_wave < 0 || o.waves_per_block < 0 || o.unroll < 0 ||
        o.waves_per_cu < -1 || o.waves_per_cu > kMaxWavesPerCU || o.mfma < -1 || o.mfma > 1 ||
        (o.int4_fp16 != 0 && o.weights != GEMV_WEIGHTS_INT4))
        return GEMV_ERR_INVALID_ARG;
    if (o.prologue == GEMV_PROLOGUE_RMSNORM && o.weights == GEMV_WEIGHTS_BF16)
        return plan_rmsnorm(out, n, k, m, dev, o);
    if (o.prologue != 0)
        return GEMV_ERR_INVALID_ARG;
    if (o.weights == GEMV_WEIGHTS_INT4)
        return plan_int4(out, n, k, m, dev, o);
    if (o.weights != GEMV_WEIGHTS_BF16)
        return GEMV_ERR_INVALID_ARG;

    int r, u, waves;
    default_tile(m, n, k, dev->compute_units, &r, &u, &waves);
    if (o.rows_per_wave)
        r = o.rows_per_wave;
    if (o.unroll)
        u = o.unroll;
    if (o.waves_per_block)
        waves = o.waves_per_block;
    if (!valid_waves(waves) || !variant_supported(m, r, u))
        return GEMV_ERR_INVALID_ARG;

    // The split count depends on N, K and the machine only - not on M - so that every
    // row of a batched result is summed in the same order as the batch-1 result. It is
    // decided on the batch-1 tile's wave count: one wave per R rows.
    int r1, u1, w1;
    default_tile(1, n, k, dev->compute_units, &r1, &u1, &w1);
    int64_t waves_s1 = ceil_div(n, o.rows_per_wave ? r : r1);

    int s;
    int64_t slice;
    if (o.splits) {
        // A forced split count gets slices aligned to 8 elements only, so that any count
        // that leaves no slice empty is accepted.
        s = o.splits;
        if (s > kMaxSplits)
            return GEMV_ERR_INVALID_ARG;
        slice = round_up(ceil_div(k, s), kVecElems);
        if (ceil_div(k, slice) != s)   // some slice would be empty
            return GEMV_ERR_INVALID_ARG;
    } else {
        // No split while the rows alone give every CU a few waves: a split adds a dependent
        // chain of memory round trips (partial store, ticket, partial loads) to the tail.
        // Below that, split until every CU has kTargetWavesPerCU waves.
        int64_t floor_waves = (int64_t)kMinWavesPerCU * dev->compute_units;
        int64_t target = (int64_t)kTargetWavesPerCU * dev->compute_units;
        int64_t want = waves_s1 >= floor_waves ? 1 : ceil_div(target, waves_s1);
        int64_t cap = k / kMinSlice > 1 ? k / kMinSlice : 1;
        if (want > cap)
            want = cap;
        if (want > kMaxSplits)
            want = kMaxSplits;
        // Take the first candidate count, from `want` up, whose slices meet the
        // summation-depth bound (the realised count can be lower than the candidate when
        // slices round up to whole wave steps).
        s = 0;
        slice = 0;
        for (int cand = (int)want; cand <= kMaxSplits; ++cand) {
            slice = slice_for(k, cand);
            s = (int)ceil_div(k, slice);
            if (depth_for(slice, s) <= kMaxDepth)
                break;
        }
        // K beyond ~720k elements cannot meet the bound with 64 slices: refuse rather than
        // return a plan whose result may miss the tolerance.
        if (depth_for(slice, s) > kMaxDepth)
            return GEMV_ERR_INVALID_ARG;
    }

    // Resident-wave cap, enforced per workgroup: a whole number of workgroups per CU.
    int cap_blocks = 0, cap_lds = 0;
    {
        const int64_t total = ceil_div(n, (int64_t)r * waves) * s * waves;
        const int cap = o.waves_per_cu > 0   ? o.waves_per_cu
                        : o.waves_per_cu < 0 ? 0
                                             : auto_cap(m, s, waves, k, total, dev->compute_units);
        if (cap > 0) {
            cap_blocks = cap / waves;
            cap_lds = lds_for_blocks(cap_blocks, kLdsGranule);
            if (!cap_lds) {
                if (o.waves_per_cu > 0)   // a forced cap that cannot be enforced
                    return GEMV_ERR_INVALID_ARG;
                cap_blocks = 0;
            }
        }
    }

    // Matrix-core launch for batches: 16-row workgroups with 128-element chunks (K a
    // multiple of 128) for M <= 8, and for larger M while 32-row workgroups would not cover
    // the CUs and M K stays within kMfmaNarrowMaxMK; else 32-row workgroups with 64-element
    // chunks. Split over K (with the same deterministic combine) only while the row blocks
    // alone leave CUs without one.
    int mf = 0, mf_s = 1, mf_depth = 0;
    int64_t mf_slice = k;
    const bool wide_splits = ceil_div(n, (int64_t)kMfmaRowsPerBlock) < dev->compute_units;
    const bool narrow = k % kMfmaNarrowChunk == 0 &&
                        (m <= kMfmaNarrowShortX || (wide_splits && (int64_t)m * k <= kMfmaNarrowMaxMK));
    const int mf_rows = narrow ? kMfmaNarrowRows : kMfmaRowsPerBlock;
    const int mf_chunk = narrow ? kMfmaNarrowChunk : kMfmaChunk;
    const int64_t mf_grid = ceil_div(n, mf_rows);
    {
        const bool forced = o.splits || o.rows_per_wave || o.waves_per_block || o.unroll ||
                            o.waves_per_cu;
        const bool want_mf = o.mfma > 0 ? m >= 2 : o.mfma == 0 && m >= kMfmaMinBatch && !forced;
        if (want_mf && k % mf_chunk == 0) {
            int64_t want = mf_grid >= dev->compute_units ? 1 : ceil_div(dev->compute_units, mf_grid);
            int64_t cap = k / mf_chunk / kMfmaWaves;   // every wave keeps a chunk per slice
            if (want > cap)
                want = cap > 1 ? cap : 1;
            if (want > kMaxSplits)
                want = kMaxSplits;
            for (int cand = (int)want; cand <= kMaxSplits; ++cand) {
                mf_slice = round_up(ceil_div(k, cand), mf_chunk);
                mf_s = (int)ceil_div(k, mf_slice);
                mf_depth = mfma_depth_for(mf_slice, mf_s, mf_chunk);
                if (mf_depth <= kMaxDepth)
                    break;
            }
            mf = mf_depth <= kMaxDepth;
            if (mf && mf_s > 1 && o.mfma == 0 && (int64_t)m * k <= kMfmaSplitMinMK)
                mf = 0;   // a split this small runs faster on the VALU kernels
        }
    }

    // Unaligned single-matrix calls on the matrix cores (decided per call: the layout is
    // the call's): from kMfmaUnalignedMinBatch by default (kMfmaUnalignedStagedMinBatch
    // where the VALU kernel stages x whole over many rows per CU), with every tile option
    // left to the plan, rows enough for the CUs and the kernel's chain within the depth bound.
    int mf_unal = 0;
    {
        const bool forced = o.splits || o.rows_per_wave || o.waves_per_block || o.unroll ||
                            o.waves_per_cu;
        const bool x_whole = (k / kVecElems) * m * 16 <= kShiftMaxLds;
        const bool many_rows = n >= kMfmaUnalignedManyRowsPerCU * dev->compute_units;
        const int min_m = x_whole && many_rows ? kMfmaUnalignedStagedMinBatch : kMfmaUnalignedMinBatch;
        const bool want = o.mfma > 0 ? m >= 2 : o.mfma == 0 && m >= min_m && !forced;
        const int depth = mfma_unaligned_depth_for(k);
        if (want && n >= (int64_t)kMfmaUnalignedRowsPerCU * dev->compute_units &&
            depth <= kMaxDepth)
            mf_unal = depth;
    }

    gemv_plan_s *p = new (std::nothrow) gemv_plan_s;
    if (!p)
        return GEMV_ERR_INVALID_ARG;
    memset(p, 0, sizeof *p);
    p->n = n;
    p->k = k;
    p->m = m;
    p->device = -1;
    p->dev = *dev;
    p->splits = s;
    p->mfma_unaligned_depth = mf_unal;
    p->rows_per_wave = r;
    p->waves_per_block = waves;
    p->unroll = u;
    p->slice = slice;
    p->grid_x = (int)ceil_div(n, (int64_t)r * waves);
    p->grid_y = s;
    p->block_threads = kWaveLanes * waves;
    p->depth_bound = depth_for(slice, s);
    p->mfma = mf;
    p->mfma_splits = mf ? mf_s : 0;
    p->mfma_slice = mf ? mf_slice : 0;
    p->mfma_grid_x = mf ? (int)mf_grid : 0;
    p->mfma_depth = mf ? mf_depth : 0;
    p->mfma_rows = mf ? mf_rows : 0;
    const int ws_splits = mf && mf_s > s ? mf_s : s;
    if (ws_splits > 1) {
        // One arrival ticket per row block (in a fixed-size region), then S x M x N fp32
        // partial sums, for whichever launch splits more.
        int64_t slots = p->grid_x > kTicketSlots ? p->grid_x : kTicketSlots;
        if (mf && mf_grid > slots)
            slots = mf_grid;
        p->partial_offset = (size_t)round_up(slots * (int64_t)sizeof(unsigned), 256);
        p->workspace =
            p->partial_offset + (size_t)ws_splits * (size_t)m * (size_t)n * sizeof(float);
    }

    int64_t total_waves = (int64_t)p->grid_x * p->grid_y * waves;
    p->waves_per_cu = cap_blocks * waves;
    p->lds_bytes = cap_lds;
    int64_t per_cu = ceil_div(total_waves, dev->compute_units);
    if (per_cu > kMaxWavesPerCU)
        per_cu = kMaxWavesPerCU;
    if (p->waves_per_cu && per_cu > p->waves_per_cu)
        per_cu = p->waves_per_cu;
    p->bif_per_cu = (double)per_cu * u * r * kWaveLanes * 16.0;
    p->bif_needed = gemv_bytes_in_flight(dev->hbm_bytes_per_s, dev->latency_s) / dev->compute_units;
    *out = p;
    return GEMV_OK;
}

extern "C" size_t gemv_workspace_size(gemv_plan_t p) { return p ? p->workspace : 0; }

extern "C" gemv_status gemv_plan_query(gemv_plan_t p, gemv_plan_info *info)
{
    if (!p || !info)
        return GEMV_ERR_INVALID_ARG;
    info->splits = p->splits;
    info->rows_per_wave = p->rows_per_wave;
    info->waves_per_block = p->waves_per_block;
    info->unroll = p->unroll;
    info->grid_x = p->grid_x;
    info->grid_y = p->grid_y;
    info->block_threads = p->block_threads;
    info->slice = p->slice;
    info->depth_bound = p->depth_bound;
    info->bytes_in_flight_per_cu = p->bif_per_cu;
    info->bytes_in_flight_needed = p->bif_needed;
    info->waves_per_cu = p->waves_per_cu;
    info->lds_bytes = p->lds_bytes;
    info->mfma = p->mfma;
    info->mfma_splits = p->mfma_splits;
    info->mfma_slice = p->mfma_slice;
    info->mfma_grid_x = p->mfma_grid_x;
    info->mfma_depth_bound = p->mfma_depth;
    info->mfma_rows = p->mfma_rows;
    info->weights = p->weights;
    info->prologue = p->prologue;
    info->int4_fp16 = p->int4_fp16;
    info->mfma_unaligned_depth = p->mfma_unaligned_depth;
    return GEMV_OK;
}

extern "C" void gemv_plan_destroy(gemv_plan_t p) { delete p; }

extern "C" const char *gemv_status_string(gemv_status s)
{
    switch (s) {
    case GEMV_OK: return "ok";
    case GEMV_ERR_INVALID_ARG: return "invalid argument";
    case GEMV_ERR_MISALIGNED: return "misaligned pointer";
    case GEMV_ERR_WORKSPACE: return "workspace missing or too small";
    case GEMV_ERR_DEVICE: return "device error or unsupported device";
    case GEMV_ERR_CAPTURE: return "graph capture error";
    case GEMV_ERR_TIMEOUT: return "chain dependency wait exceeded its spin limit";
    }
    return "unknown status";
}
