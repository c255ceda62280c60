// plan.h - internal: the plan object and the table of compiled kernel variants.
//
// Shared by plan.cpp (host arithmetic only, no HIP headers) and gemv.hip (launches).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "gemv.h"

namespace bbd {

// Architectural facts the plan sizes launches for (CDNA4 / gfx950).
constexpr int kWaveLanes = 64;          // lanes per wavefront
constexpr int kVecElems = 8;            // bf16 elements per 16-byte load
constexpr int kWaveStep = kWaveLanes * kVecElems;   // K elements one wave-wide load covers
constexpr int kMaxWavesPerCU = 32;      // 4 SIMDs x 8 waves
constexpr int kMaxSplits = 64;
constexpr int kLdsPerCU = 160 * 1024;   // LDS bytes per CU
constexpr int kLdsGranule = 512;        // LDS allocation unit assumed when planning offline

// Planning constants (tunable, see the plan rule in plan.cpp).
constexpr int kMinWavesPerCU = 1;       // no split while N / R gives this many waves per CU
constexpr int kTargetWavesPerCU = 4;    // a split aims for this many waves per CU
constexpr int64_t kMinSlice = 1024;     // never split K finer than this many elements
constexpr int kMaxDepth = 160;          // gamma_160 (u = 2^-24) = 9.54e-6 < 1e-5
// Loaded HBM latency on MI355X, measured with the pure-read stream (gemv_read_stream):
// bytes in flight / rate is 0.40 us with 1 KiB in flight per CU and rises to ~0.66 us where
// the rate reaches its ceiling (16-24 KiB per CU); the plans report Little's law with it.
constexpr double kDefaultLatency = 0.65e-6;
// Batch-1 resident-wave caps per CU (measured on MI355X, see the plan rule in plan.cpp):
// rows longer than 8 wave steps stream best with at most 8 single-row waves per CU, in
// equal rounds; short rows with more waves than one round holds, with at most 12.
constexpr int kCapLongRows = 8;
constexpr int kCapShortRows = 12;
constexpr int kOneRoundWavesPerCU = 16;   // short rows: up to this many waves per CU run
// Batch-1 rows shorter than 8 wave steps (K < 4096) run in uncapped workgroups of
// kShortRowWaves waves when the rows need more than one round of kOneRoundWavesPerCU
// single-wave workgroups per CU, or are a single wave step long (K <= 512) and number at
// least kShortRowBlockMinRows: single-wave workgroups that stream a few KiB each are then
// handed out slower than they finish (measured on MI355X: 8192 x 1024 5.98 -> 4.46 us,
// 16384 x 2048 13.8 -> 11.3 us, 4096 x 512 2.93 -> 2.54 us, 2048 x 512 2.44 -> 2.27 us;
// within one round at 2-7 steps, 4096 x 1024..3584, between -4 % and +3 %, so those keep
// single-wave workgroups, as do 1024 rows and K = 4096).
constexpr int64_t kShortRowBlockMinRows = 2048;
// Batch-1 grids of one round (at most kOneRoundWavesPerCU single-wave workgroups per CU)
// take the shortest burst that keeps this many bytes in flight per CU: the read ceiling's
// knee (measured on MI355X: K = 4096 at 1-4 waves per CU fastest with bursts of 8, at 6-8
// with 4, at 12-16 with 2; e.g. 768 x 4096 3.10 -> 2.87 us, 4096 x 4096 6.75 -> 6.54 us).
constexpr int64_t kBurstTargetBytes = 24 * 1024;
constexpr int kShortRowWaves = 8;
// Ticket counters sit at the start of a split plan's workspace in a region of at least this
// many slots, so that plans with up to this many row blocks can share one workspace in any
// order without one plan's partial sums landing on another plan's tickets.
constexpr int64_t kTicketSlots = 4096;
// Matrix-core kernel (mfma.hip): workgroups of 8 waves that take K in chunks; used by
// default from this batch size on (at 4096 x 14336 it is faster than the VALU kernels from
// M = 2 on: 19.4 against 19.8 us, and 19.8 against 24.4 us at M = 8). Two forms: 32-row
// blocks with 64-element chunks, whose two 16-row tiles share every X fragment, and 16-row
// blocks with 128-element chunks, twice the row blocks (4096 rows fill 256 CUs without
// splitting K). The 16-row form is taken (K a multiple of 128) for M <= 8, where it stages
// 8 X vectors per chunk, and for M = 9..16 when the 32-row blocks would leave CUs without
// one (so K would be split) and M K is at most kMfmaNarrowMaxMK: it then reads X twice as
// often per weight byte but needs no split and no combine. Measured on MI355X, M = 9..16:
// 4096 x 4096 7.3-7.8 against 9.2 us, 6144 x 4096 11.9-12.7 against 14.7-15.1 us, 1024 x
// 4096 6.7 against 8.0-8.2 us, 4096 x 14336 20.2-21.6 against 21.5-21.7 us up to M = 14;
// the forms tie at M = 15 there and the split 32-row form wins at M = 16 (22.1 against
// 22.3 us). With enough row blocks for the 32-row form (14336 x 4096) it is as fast or
// faster at every M from 9.
constexpr int kMfmaRowsPerBlock = 32;
constexpr int kMfmaChunk = 64;
constexpr int kMfmaNarrowRows = 16;
constexpr int kMfmaNarrowChunk = 128;
constexpr int kMfmaNarrowShortX = 8;                    // X vectors staged for M <= 8
constexpr int64_t kMfmaNarrowMaxMK = 14 * 14336;
constexpr int kMfmaWaves = 8;
// An automatic matrix-core plan that has to split K (too few row blocks for the CUs) gives
// way to the VALU kernels up to this M K: the split's combine is then most of the time
// (measured on MI355X, each shape warmed up: at M = 2 / 4, 1024 x 4096 4.39 / 5.80 us on the
// VALU kernels against 6.43 / 6.58 us split, 2048 x 4096 5.39 / 6.40 against 6.95 / 7.13 us,
// 3072 x 4096 6.77 / 7.80 against 8.85 / 9.01 us; M = 8 at K = 4096 (7.18 against 7.92 us
// at 2048 rows) and M = 4 at K = 14336 (12.0 against 14.9 us) stay on the matrix cores).
constexpr int64_t kMfmaSplitMinMK = 16384;
constexpr int kMfmaMinBatch = 2;
// Unaligned single-matrix calls (W or x rows off the 16-byte grid) run on the matrix cores
// from this batch size (measured on MI355X against the class-staged VALU kernel, odd row
// strides: 4097 x 14337 at M = 9 / 10 / 12 / 13 42.1 / 43.9 / 47.6 / 48.6 us against
// 40.6 / 44.4 / 51.0 / 54.6, and 52.4 against 67.4 us at M = 16; 14337 x 4097 at M = 9 / 10
// 39.8 / 41.3 against 40.1 / 43.0 us; 4099 x 4097 ahead from M = 8), with at least
// kMfmaUnalignedRowsPerCU rows per CU so that its 16-row tiles cover the CUs.
constexpr int kMfmaUnalignedMinBatch = 10;
constexpr int kMfmaUnalignedRowsPerCU = 16;
// ...but from kMfmaUnalignedStagedMinBatch where the class-staged VALU kernel stages the M
// shifted x rows whole (within kShiftMaxLds) and has at least kMfmaUnalignedManyRowsPerCU rows
// per CU to amortize that staging over (measured at 28673 x 4097: M = 10 71.7 us on the
// matrix cores against 67.4 us, 12 76.1 against 76.7, 14 78.1 against 100.6).
constexpr int kMfmaUnalignedStagedMinBatch = 12;
constexpr int64_t kMfmaUnalignedManyRowsPerCU = 64;
// x staged in LDS by the class-staged unaligned kernel: the whole rows up to this many bytes,
// in chunks beyond.
constexpr int64_t kShiftMaxLds = 128 * 1024;
constexpr int kMfmaUnalignedChunk = 128;
// INT4 weights (int4.hip): 32 weights per 16-byte vector, one bf16 scale per 128.
constexpr int kInt4VecElems = 32;
constexpr int kInt4Group = 128;
constexpr int kInt4MaxLdsX = 64 * 1024;   // x staged in LDS up to this many bytes (2K)
constexpr int64_t kInt4TwoRowsFrom = 16384;   // short INT4 rows: two per wave from this N
constexpr int kInt4ShortRowsCap = 32;         // waves per CU for two-row short INT4 rows
constexpr int64_t kInt4Fp16MinRows = 32;      // fp16 staging when a workgroup covers this
                                              // many rows or more

// One compiled (M, R, U) combination of the aligned fast-path kernel. The unaligned path
// exists for every M and takes R at run time.
struct Variant {
    int m, r, u;
};

// The fast-path kernels gemv.hip instantiates. Keep in sync with its dispatch table.
constexpr Variant kVariants[] = {
    {1, 1, 2}, {1, 1, 4}, {1, 1, 7}, {1, 1, 8}, {1, 1, 14}, {1, 2, 2}, {1, 2, 4}, {1, 2, 7},
    {1, 2, 8}, {1, 4, 2}, {1, 4, 4}, {1, 4, 7}, {1, 4, 8},
    {2, 1, 2}, {2, 1, 4}, {2, 2, 2}, {2, 2, 4},
    {3, 1, 2}, {3, 1, 4}, {3, 2, 2}, {3, 2, 4},
    {4, 1, 2}, {4, 1, 4}, {4, 2, 2}, {4, 2, 4},
    {5, 1, 2}, {5, 2, 2}, {6, 1, 2}, {6, 2, 2}, {7, 1, 2}, {7, 2, 2}, {8, 1, 2}, {8, 2, 2},
    {9, 1, 2}, {9, 2, 2}, {10, 1, 2}, {10, 2, 2}, {11, 1, 2}, {11, 2, 2}, {12, 1, 2},
    {12, 2, 2}, {13, 1, 2}, {13, 2, 2}, {14, 1, 2}, {14, 2, 2}, {15, 1, 2}, {15, 2, 2},
    {16, 1, 2}, {16, 2, 2},
    {9, 2, 1}, {10, 2, 1}, {11, 2, 1}, {12, 2, 1}, {13, 2, 1}, {14, 2, 1}, {15, 2, 1},
    {16, 2, 1},
};

bool variant_supported(int m, int r, int u);

// Launch a validated batch-1 call on the whole-row kernels (whole.hip) when it qualifies;
// *done tells whether it did.
gemv_status launch_whole(gemv_plan_t p, const gemv_segment *segs, int nseg, const void *X,
                         void *stream, bool *done);

// Launch a validated 2 <= M <= 16 call on the LDS-staged batch kernel (batch.hip) when it
// qualifies; *done tells whether it did.
gemv_status launch_batch(gemv_plan_t p, const gemv_segment *segs, int nseg, const void *X,
                         int64_t ldx, void *stream, bool *done);

// Launch a validated call on the matrix-core kernel (mfma.hip) when the plan chose it and
// the call qualifies; *done tells whether it did. A split launch takes its arrival tickets
// and partial sums from `tickets` and `partial` (see the workspace layout in gemv.h).
gemv_status launch_mfma(gemv_plan_t p, const gemv_segment *segs, int nseg, const void *X,
                        int64_t ldx, unsigned *tickets, float *partial, void *stream,
                        bool *done);

// Launch a validated unaligned single-matrix call on the matrix-core kernel for unaligned
// rows (mfma.hip) when the plan allows it; *done tells whether it did.
gemv_status launch_mfma_unaligned(gemv_plan_t p, const gemv_segment &seg, const void *X,
                                  int64_t ldx, void *stream, bool *done);

// RMSNorm-prologue launch (norm.hip) of a validated call; the plan's unroll picks the kernel.
gemv_status launch_rmsnorm(gemv_plan_t p, const gemv_segment *segs, int nseg, const void *H,
                           const void *gamma, float eps, void *stream);
constexpr int64_t kNormMaxK = 16368;   // 4K + 64 bytes of LDS (hi and lo halves, wave sums)
constexpr int kNormBlocksPerCU = 2;       // RMSNorm-prologue workgroups per CU in the grid,
constexpr int kNormManyBlocksPerCU = 4;   // or one per row block beyond this many blocks per CU

// INT4-weight launch (int4.hip) of a validated call; the plan's unroll, rows per wave and
// LDS size pick the kernel.
gemv_status launch_int4(gemv_plan_t p, const void *Wq, int64_t ldq, const void *S, int64_t lds,
                        const void *X, float *Y, void *stream);

// Record the HIP error code behind a GEMV_ERR_DEVICE / GEMV_ERR_CAPTURE for
// gemv_last_hip_error() (thread-local) and return `status`.
gemv_status record_hip_error(int hip_error, gemv_status status);

}  // namespace bbd

struct gemv_plan_s {
    int64_t n, k;
    int m;
    int device;                 // HIP device id, or -1 for a plan made by gemv_plan_for
    gemv_device_desc dev;
    int splits;                 // S
    int rows_per_wave;          // R
    int waves_per_block;
    int unroll;                 // U
    int64_t slice;              // K elements per split (multiple of 8)
    int grid_x, grid_y, block_threads;
    int depth_bound;
    size_t workspace;           // ticket counters, then the split partials
    size_t partial_offset;      // byte offset of the partial sums in the workspace
    double bif_per_cu, bif_needed;
    int waves_per_cu;           // resident-wave cap per CU (0: none)
    int lds_bytes;              // LDS reserved per workgroup to enforce the cap
    int mfma;                   // aligned single-matrix calls run the matrix-core kernel
    int mfma_splits;
    int64_t mfma_slice;
    int mfma_grid_x;
    int mfma_depth;
    int mfma_rows;              // rows per matrix-core workgroup: 32 or 16
    int weights;                // GEMV_WEIGHTS_BF16 or GEMV_WEIGHTS_INT4
    int prologue;               // 0 or GEMV_PROLOGUE_RMSNORM
    int int4_fp16;              // INT4 with x in LDS: the workgroups try the fp16 staging
    int mfma_unaligned_depth;   // unaligned single-matrix calls run on the matrix cores (> 0)
};
