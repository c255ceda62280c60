/*
 * gemv.h - C ABI of the MI355X (gfx950) decode GEMV library, libbbd_gemv.so.
 *
 * The operation is the memory-bound decode GEMV of the decode-GEMV page ("Decode GEMV at
 * half of HBM bandwidth", inferenceinterviews.com): a row-major [N, K] bf16 weight W times
 * a bf16 vector x, one fp32-accumulated output per row,
 *
 *     Y[m][n] = sum_{k<K} W[n][k] * X[m][k]      for m < M, n < N,
 *
 * with M = 1 at decode batch 1 and M <= 16 for the skinny batches of the page's follow-up
 * on batch 16 ("What interviewers probe next"). bf16 inputs are widened and every
 * product-sum is accumulated in fp32 (tiled-GEMM page, "What interviewers probe next",
 * the bf16 question). Y is overwritten, never accumulated into.
 *
 * Conventions for every entry point:
 *   - Every tensor pointer (W, X, Y, workspace) is a DEVICE pointer on the plan's device.
 *     Streams are hipStream_t passed as void* (NULL = the legacy default stream, which
 *     cannot be captured into a graph).
 *   - Ownership: the caller owns W, X, Y, the workspace and the stream. A plan owns host
 *     memory only; a segment array is read during the call and not kept. A captured graph
 *     refers to the caller's buffers, which must outlive it.
 *   - Errors: every call returns a status; nothing aborts, throws or prints. Arguments are
 *     validated before any HIP call, so a rejected call enqueues nothing. Launch failures
 *     come back as GEMV_ERR_DEVICE with the HIP error code in gemv_last_hip_error().
 *     Faults inside a kernel surface at the caller's next synchronisation.
 *   - gemv_run and gemv_fused_run allocate nothing and never synchronise with the host, so
 *     they can be captured into a graph. Calls that share a workspace must not overlap.
 *   - Results are bitwise reproducible for a fixed plan, fixed inputs and a fixed alignment
 *     class (see gemv_run): split partial sums are combined in a fixed order, never with
 *     atomics (decode-GEMV page, "What interviewers probe next", the last-bit question).
 */
#ifndef BBD_GEMV_H
#define BBD_GEMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GEMV_OK = 0,
    GEMV_ERR_INVALID_ARG = 1, /* a size, count, leading dimension, option or pointer is bad */
    GEMV_ERR_MISALIGNED = 2,  /* W/X not 2-byte aligned, or Y/workspace not 4-byte aligned */
    GEMV_ERR_WORKSPACE = 3,   /* workspace missing or smaller than gemv_workspace_size()   */
    GEMV_ERR_DEVICE = 4,      /* not a gfx950 device, or a HIP call failed                  */
    GEMV_ERR_CAPTURE = 5,     /* graph capture misuse (legacy stream, not capturing, ...)   */
    GEMV_ERR_TIMEOUT = 6      /* a chain's dependency wait exceeded its spin limit          */
} gemv_status;

/* Largest batch a plan accepts (the skinny-batch range of the decode-GEMV page). */
#define GEMV_MAX_M 16
/* Largest number of segments gemv_fused_run accepts (QKV uses 3, gate_up 2). */
#define GEMV_MAX_SEGMENTS 4

typedef struct gemv_plan_s *gemv_plan_t;

/*
 * Plan overrides; 0 in a field means "choose automatically".
 *   splits          S, the number of K slices (split-K; decode-GEMV page, "A strong
 *                   answer", cause 1). 1 <= S <= 64 and every slice must be non-empty.
 *   rows_per_wave   R, output rows one 64-lane wave reduces together (1, 2 or 4).
 *   waves_per_block waves in a workgroup (1, 2, 4 or 8).
 *   unroll          U, independent 16-byte W loads per row each lane issues before using
 *                   any of them (cause 2 of the same section): 2, 4, 7, 8 or 14 (7 and 14
 *                   divide the 28 wave steps of a 14336-element row); 1 for batches of 9-16.
 *   waves_per_cu    most waves of the launch resident on one CU at a time: 1..32, or -1
 *                   for no cap. A cap below what registers allow makes later workgroups
 *                   start as earlier ones finish, on whichever CU frees up first; it is
 *                   enforced by reserving LDS per workgroup (the kernels use none).
 *   mfma            the matrix-core kernel for batches (decode-GEMV page: past a handful of
 *                   vectors the work stops being a matrix-vector product and matrix units
 *                   start to pay; on MI355X they do from M = 2): 0 = automatic (M >= 2
 *                   with no tile, split or cap forced, except where the matrix-core launch
 *                   would have to split K and M*K <= 16384: there the split's combine costs
 *                   more than the VALU kernels' extra vectors), 1 = for any M >= 2,
 *                   -1 = never. It
 *                   needs K to be a multiple of 64 (of 128 for the 16-row form).
 *                   It runs only for 16-byte-aligned single-matrix calls; other calls of
 *                   the same plan take the VALU kernels the fields above describe. The
 *                   VALU kernels sum every output in the same order at every M, so with
 *                   -1 each row of a batched result is bitwise equal to its batch-1 result;
 *                   the matrix-core kernel meets the same tolerance in another order.
 * Not every (M, R, U) combination is compiled; an unsupported one is GEMV_ERR_INVALID_ARG.
 */
typedef struct {
    int splits;
    int rows_per_wave;
    int waves_per_block;
    int unroll;
    int waves_per_cu;
    int mfma;
    int weights;        /* GEMV_WEIGHTS_BF16 (0) or GEMV_WEIGHTS_INT4; see gemv_int4_run */
    int prologue;       /* 0, or GEMV_PROLOGUE_RMSNORM; see gemv_rmsnorm_run */
    int int4_fp16;      /* INT4 plans whose x is staged in LDS: 1 = try the fp16 form of the
                           staged x, -1 = bf16 only, 0 = automatic (see gemv_int4_run) */
} gemv_plan_opts;

/* Input prologues a plan can be made for. */
#define GEMV_PROLOGUE_RMSNORM 1

/* Weight formats a plan can be made for. */
#define GEMV_WEIGHTS_BF16 0
#define GEMV_WEIGHTS_INT4 1

/*
 * The device a plan is sized for. gemv_plan fills it from the runtime; gemv_plan_for takes
 * it from the caller and makes no HIP call (host-only planning and testing).
 *   compute_units    CUs the grid is sized to fill (256 on MI355X).
 *   hbm_bytes_per_s  peak HBM bandwidth (8.0e12 on MI355X).
 *   latency_s        assumed loaded memory latency for Little's law.
 */
typedef struct {
    int compute_units;
    double hbm_bytes_per_s;
    double latency_s;
} gemv_device_desc;

/* What a plan chose, for tests, tuning and the bench. */
typedef struct {
    int splits;             /* S */
    int rows_per_wave;      /* R */
    int waves_per_block;
    int unroll;             /* U */
    int grid_x;             /* row blocks: ceil(N / (R * waves_per_block)) */
    int grid_y;             /* = S */
    int block_threads;      /* 64 * waves_per_block */
    int64_t slice;          /* K elements per split; a multiple of 8; the last may be short */
    int depth_bound;        /* h: the most fp32 roundings any product passes through */
    double bytes_in_flight_per_cu;   /* 16-byte W loads outstanding per CU at full residency */
    double bytes_in_flight_needed;   /* Little's law per CU: bandwidth * latency / CUs     */
    int waves_per_cu;       /* resident-wave cap per CU, 0 when the launch has none */
    int lds_bytes;          /* LDS reserved per workgroup to enforce that cap (0: none) */
    /* The matrix-core launch, when mfma is 1 (aligned single-matrix calls run it; the
       fields above then describe the kernels every other call of the plan takes). */
    int mfma;
    int mfma_splits;        /* K slices; > 1 uses the workspace like a VALU split */
    int64_t mfma_slice;     /* K elements per slice, a multiple of the chunk */
    int mfma_grid_x;        /* row blocks: ceil(N / mfma_rows); 8 waves per workgroup */
    int mfma_depth_bound;   /* h for that kernel, counting 32 roundings per MFMA */
    int weights;            /* the plan's weight format */
    int prologue;           /* the plan's input prologue (0: none) */
    int int4_fp16;          /* INT4: 1 when the workgroups try the fp16 form of staged x */
    int mfma_rows;          /* rows per matrix-core workgroup: 16 (K a multiple of 128, and
                               M <= 8 or, for M = 9..16, 32-row blocks too few for the
                               CUs with M K <= 14 * 14336; chunks of 128 K elements) or 32
                               (chunks of 64); 0 without the matrix-core launch */
    int mfma_unaligned_depth;   /* > 0 when single-matrix calls whose W or x rows are off the
                               16-byte grid run on the matrix cores (M >= 10 by default, or
                               M >= 12 where the M x rows fit 128 KiB and N >= 64 rows per
                               CU; M >= 2 with mfma = 1; N >= 16 rows per CU; no tile
                               option forced): h for that kernel; 0 when they take the
                               VALU kernels */
} gemv_plan_info;

/*
 * Little's law for memory (decode-GEMV page, "A strong answer"; GPU performance chains
 * page, "Bytes in flight to reach bandwidth"): the bytes that must be outstanding to sustain
 * `bytes_per_s` when each request takes `latency_s`. Pure arithmetic.
 */
double gemv_bytes_in_flight(double bytes_per_s, double latency_s);

/*
 * Create a plan for Y[M][N] = X[M][K] . W[N][K]^T on HIP device `device`.
 * n >= 1, k >= 1, 1 <= m <= GEMV_MAX_M. `opts` may be NULL.
 * Returns GEMV_ERR_DEVICE if the device is not gfx950 (the only architecture compiled).
 * On success *out owns a host allocation released by gemv_plan_destroy.
 */
gemv_status gemv_plan(gemv_plan_t *out, int64_t n, int64_t k, int m, int device,
                      const gemv_plan_opts *opts);

/* Same as gemv_plan for an explicit device description; makes no HIP call. */
gemv_status gemv_plan_for(gemv_plan_t *out, int64_t n, int64_t k, int m,
                          const gemv_device_desc *dev, const gemv_plan_opts *opts);

/*
 * Bytes of workspace gemv_run needs: 0 when S == 1; otherwise a ticket region of
 * 4 * max(grid_x, 4096) bytes (one 32-bit arrival counter per row block) followed by the
 * S*M*N fp32 partial sums. A plan with both a split VALU launch and a split matrix-core
 * launch needs the larger of the two. 0 for a NULL plan.
 */
size_t gemv_workspace_size(gemv_plan_t p);

gemv_status gemv_plan_query(gemv_plan_t p, gemv_plan_info *info);

/* Release a plan (NULL is allowed). Plans are immutable after creation. */
void gemv_plan_destroy(gemv_plan_t p);

/*
 * Y[m][n] = sum_k W[n][k] * X[m][k] on `stream`, asynchronously.
 *   W   bf16 [n][ldw], ldw >= k, 2-byte aligned.
 *   X   bf16 [m][ldx], ldx >= k, 2-byte aligned (ldx is ignored when m == 1).
 *   Y   fp32 [m][ldy], ldy >= n, 4-byte aligned; overwritten.
 *   Leading dimensions above 2^31 - 1 elements are GEMV_ERR_INVALID_ARG.
 *   workspace  device buffer of at least gemv_workspace_size(p) bytes, 4-byte aligned
 *              (NULL allowed when that size is 0). It holds the split partial sums and
 *              the tickets that pick, per row block, the workgroup that adds them up.
 *              It must be zero-filled before its first use; every call that completes
 *              leaves its tickets at zero again. One workspace can therefore be shared,
 *              without clearing, by any plans with at most 4096 row blocks (grid_x), in
 *              any order, as long as their calls do not overlap; every automatically
 *              chosen split plan on MI355X has fewer than 4096 row blocks.
 * With S > 1 the S partial sums of each output are added in slice order 0..S-1 by the last
 * workgroup of its row block to finish, inside the same launch (no second kernel).
 * When W and X are 16-byte aligned with ldw and ldx multiples of 8 the fast path runs
 * (one 16-byte load per lane per row step); any other layout runs the unaligned path,
 * which gives a result within the same tolerance but not bitwise equal to the fast path
 * (for a plan with mfma_unaligned_depth > 0, on the matrix cores: rows c, c + C, ... with
 * C = 8 / gcd(ldw, 8) share one offset from the 16-byte grid and are tiled as one aligned
 * matrix).
 */
gemv_status gemv_run(gemv_plan_t p,
                     const void *W, int64_t ldw,
                     const void *X, int64_t ldx,
                     float *Y, int64_t ldy,
                     void *workspace, size_t ws_bytes, void *stream);

/*
 * gemv_run with no workspace argument, for callers that cannot allocate device memory:
 * code being captured into a graph, tight serving loops, harnesses that forbid hipMalloc.
 * The split launches' arrival tickets and partial sums live in a static device array
 * inside the library, GEMV_STATIC_SCRATCH_BYTES per GPU (held on every GPU the library
 * runs on until the process ends): the first GEMV_STATIC_TICKET_SLOTS 32-bit words are
 * tickets, the rest fp32 partial sums. Arguments, validation and the result are those of
 * gemv_run; with the same plan and inputs the result is bitwise equal to gemv_run's.
 *   - A plan that splits (the VALU or the matrix-core launch) and needs more than
 *     GEMV_STATIC_TICKET_SLOTS row blocks, or more partial-sum bytes than the array holds
 *     after the tickets, is refused with GEMV_ERR_WORKSPACE before any HIP call. Unsplit
 *     plans use no scratch.
 *   - Every call on a GPU shares that GPU's array and it keeps the last call's contents:
 *     calls that overlap on one GPU (other streams, other threads) race and give wrong
 *     results. Calls issued in order on one stream never overlap.
 *   - The first call on a device looks the array up (hipGetSymbolAddress, on the plan's
 *     device) and enqueues on `stream` one small kernel that zeroes the tickets; every
 *     completed call leaves them at zero. No call allocates or synchronises with the host.
 */
#define GEMV_STATIC_SCRATCH_BYTES (4u << 20)
#define GEMV_STATIC_TICKET_SLOTS 16384

gemv_status gemv_run_static(gemv_plan_t p,
                            const void *W, int64_t ldw,
                            const void *X, int64_t ldx,
                            float *Y, int64_t ldy, void *stream);

/*
 * One GEMV over several weight matrices that share X: the fused QKV and gate_up
 * projections (decode-GEMV page, "A strong answer", cause 3). Segment i holds rows
 * [sum_{j<i} n_j, sum_{j<=i} n_j) of the plan's N rows:
 *   W    bf16 [n][ldw], ldw >= k;   Y  fp32 [m][ldy], ldy >= n.
 * 1 <= nseg <= GEMV_MAX_SEGMENTS and sum n_i == the plan's n. The result is bitwise equal
 * to gemv_run on the row-concatenation of the segments (same plan, same alignment class).
 */
typedef struct {
    const void *W;
    int64_t n;
    int64_t ldw;
    float *Y;
    int64_t ldy;
} gemv_segment;

gemv_status gemv_fused_run(gemv_plan_t p, const gemv_segment *segs, int nseg,
                           const void *X, int64_t ldx,
                           void *workspace, size_t ws_bytes, void *stream);

/*
 * Batch-1 GEMV with INT4 weights (decode-GEMV page, the follow-up in which the weights
 * become INT4: a quarter of the bytes, unpacked in registers while the next loads are in
 * flight). The page fixes no format; this library's:
 *   - weight v in [-8, 7] stored as a two's-complement nibble; row n of Wq starts at
 *     Wq + n*ldq bytes, and element k is the low nibble of byte k/2 when k is even and
 *     the high nibble when k is odd;
 *   - one bf16 scale per run of 128 consecutive elements of a row: scale[n][k/128] at
 *     S + n*lds (elements);
 *   - the weight's value is v * scale, and Y[n] = sum_k (v_nk * scale[n][k/128]) * X[k],
 *     accumulated in fp32 and overwritten, within the same tolerance as gemv_run.
 * The plan must come from gemv_plan / gemv_plan_for with opts.weights = GEMV_WEIGHTS_INT4,
 * m = 1 and k a multiple of 32 (whole 16-byte vectors; the last group may be short); it
 * never splits K, and opts.splits > 1 and mfma = 1 are GEMV_ERR_INVALID_ARG. rows_per_wave
 * (1 or 2), unroll (1, 2, 4 or 7; 1 or 2 with two rows), waves_per_block (1, 2, 4, 8 or 16)
 * and int4_fp16 may be forced; waves_per_cu > 0 caps the grid at that many waves per CU,
 * each workgroup then looping over row blocks.
 * When x fits in LDS (68 bytes per 32 elements, up to 64 KiB) the workgroup stages it once.
 * With the fp16 form (int4_fp16) each 32-element vector of x is staged as fp16 x * 2^s, s
 * its own power of two; a workgroup in which any element does not convert exactly (or x
 * holds an inf or NaN) falls back to bf16. Both forms form every product exactly and meet
 * the same tolerance, but round in a different order, so their results may differ in the
 * last bits; for a fixed plan and x the result is reproducible.
 * Wq and X must be 16-byte aligned with ldq a multiple of 16 (>= k/2), S 2-byte and Y
 * 4-byte aligned (else GEMV_ERR_MISALIGNED); lds >= ceil(k/128); leading dimensions up
 * to 2^31 - 1. No workspace; no allocation or host synchronisation (capture-safe).
 * gemv_run and gemv_fused_run reject INT4 plans, and this call rejects bf16 plans
 * (GEMV_ERR_INVALID_ARG).
 */
gemv_status gemv_int4_run(gemv_plan_t p, const void *Wq, int64_t ldq, const void *S,
                          int64_t lds, const void *X, float *Y, void *stream);

/*
 * Batch-1 GEMV of the RMS-normalised input (GPU performance chains page, "Fused RMSNorm
 * traffic": at decode a normalisation's bytes are trivial and its launch is the cost, so
 * the projections that consume it compute it themselves):
 *   rms_inv = 1 / sqrt( sum_k H[k]^2 / K + eps ),
 *   Y_i[n]  = rms_inv * sum_k W_i[n][k] * (gamma[k] * H[k])
 * for every segment i (one launch; QKV and gate_up pass their matrices as segments, as in
 * gemv_fused_run), with no rounding between the norm and the GEMV; within the gemv_run
 * tolerance, with s_abs = rms_inv * sum_k |W[n][k] gamma[k] H[k]|.
 * The plan must come from gemv_plan / gemv_plan_for with opts.prologue =
 * GEMV_PROLOGUE_RMSNORM, m = 1 and k a multiple of 8 up to 16368 (the numerator gamma*H is
 * staged in LDS); it never splits K. H and gamma are bf16 [k], 16-byte aligned; every W_i
 * is 16-byte aligned with one shared ldw, a multiple of 8 (else GEMV_ERR_MISALIGNED /
 * GEMV_ERR_INVALID_ARG); each Y_i is fp32 [n_i] (the segments' ldy is not used); eps >= 0
 * and finite. No workspace; no allocation or host synchronisation (capture-safe).
 * gemv_run and gemv_fused_run reject these plans, and this call rejects any other plan.
 */
gemv_status gemv_rmsnorm_run(gemv_plan_t p, const gemv_segment *segs, int nseg, const void *H,
                             const void *gamma, float eps, void *stream);

/*
 * Graph capture of a GEMV sequence, so a whole decode step crosses the host-device boundary
 * once (decode-GEMV page, cause 3; GPU performance chains page, "Launch gaps in a decode
 * step"). begin starts a thread-local capture on `stream` (not the legacy default stream);
 * gemv_run / gemv_fused_run calls on that stream are recorded, not executed; end stops the
 * capture and instantiates an executable graph owned by *out; launch replays it on `stream`.
 */
typedef struct gemv_graph_s *gemv_graph_t;

gemv_status gemv_graph_begin(void *stream);
gemv_status gemv_graph_end(void *stream, gemv_graph_t *out);
gemv_status gemv_graph_launch(gemv_graph_t g, void *stream);
void gemv_graph_destroy(gemv_graph_t g);

/*
 * A chain: a decode step's dependent GEMVs run by ONE persistent launch (decode-GEMV page,
 * "A strong answer", cause 3: launch and ramp-up cost rivals the transfer of a small
 * matrix; GPU performance chains page, "Launch gaps in a decode step").
 *
 * Link i is one GEMV (batch 1) whose input may be the previous link's output: no wave
 * computes with link i's input before every output of link i-1 has been stored and made
 * visible device-wide. The launch is one workgroup per CU: worker waves stream weights and
 * keep several bursts of loads in flight across link boundaries (weights never depend on
 * the previous result), and one controller wave per workgroup stages x into LDS, writes the
 * workgroup's outputs and takes part in the grid-wide wait between links - so HBM keeps
 * streaming across link boundaries instead of draining and refilling once per GEMV.
 * Each output row is summed exactly as gemv_run / gemv_fused_run sum it with an unsplit
 * plan, so a chain's results are bitwise equal to running its links one by one.
 *
 * Every wait is bounded by a spin limit; a wait that runs out sets an error flag and the
 * launch finishes early (never hangs). gemv_chain_check reports it. Two runs of one chain
 * must not execute concurrently (they share its counters); runs on one stream never do.
 */
typedef struct {
    const gemv_segment *segs;   /* 1..GEMV_MAX_SEGMENTS weights and outputs sharing X; the
                                   segment ldy fields are ignored (batch 1) */
    int nseg;
    const void *X;              /* bf16 [k], 16-byte aligned */
    int64_t k;                  /* reduction length of every segment, >= 8; x of the
                                   longest link must fit in one CU's LDS (k up to ~80K) */
} gemv_chain_link;

typedef struct {
    int waves_per_cu;           /* worker waves per CU, 1..11 (0 = 8); one controller wave
                                   per CU comes on top */
    unsigned spin_limit;        /* polls before a wait gives up (0 = auto, ~1 s) */
} gemv_chain_opts;

typedef struct gemv_chain_s *gemv_chain_t;

/*
 * Build a chain on HIP device `device` from `nlinks` >= 1 links (read during the call only).
 * Every weight must be 16-byte aligned with ldw a multiple of 8 and every X 16-byte aligned
 * (the fast-path layout; anything else is GEMV_ERR_MISALIGNED). Allocates the chain's
 * device-side descriptor table and counters here, once; gemv_chain_run allocates nothing.
 * The weights, inputs and outputs stay owned by the caller and must outlive the chain.
 */
gemv_status gemv_chain_create(gemv_chain_t *out, const gemv_chain_link *links, int nlinks,
                              int device, const gemv_chain_opts *opts);

/* One launch that runs every link in order on `stream`; asynchronous and capturable. */
gemv_status gemv_chain_run(gemv_chain_t c, void *stream);

/*
 * Synchronise with the device and report GEMV_ERR_TIMEOUT if a dependency wait of an
 * earlier run gave up (that run's outputs are then incomplete); clears the flag. Not for
 * use during graph capture.
 */
gemv_status gemv_chain_check(gemv_chain_t c);

/* Release a chain and its device memory (NULL is allowed). */
void gemv_chain_destroy(gemv_chain_t c);

/*
 * Measurement support, not part of the GEMV: read `rows` rows of `row_bytes` bytes from the
 * device buffer `buf` (row r at buf + r * row_bytes) with the batch-1 GEMV's weight stream
 * and nothing else - one single-wave workgroup per row, each lane issuing `unroll` (1, 2, 4
 * or 8) nontemporal 16-byte loads before using any, lanes 16 bytes apart - with at most
 * `waves_per_cu` (1..31; 0 or 32: no cap) such workgroups resident on a CU. Over a buffer
 * much larger than the caches its rate is the achievable read ceiling; a sweep of unroll
 * and waves_per_cu gives bandwidth against bytes in flight, whose linear part has the
 * loaded latency as its slope (Little's law: decode-GEMV page, "A strong answer"; GPU
 * performance chains page, "Bytes in flight to reach bandwidth"). row_bytes must be a
 * multiple of 1024 * unroll, buf 16-byte and sink 4-byte aligned; the words read are
 * folded together and the fold is stored to *sink only if it equals one fixed value, which
 * keeps the loads from being dropped. Asynchronous on `stream`; allocates nothing.
 */
gemv_status gemv_read_stream(const void *buf, int64_t rows, int64_t row_bytes, int unroll,
                             int waves_per_cu, unsigned *sink, void *stream);

/* A static description of a status code ("unknown status" for anything else). */
const char *gemv_status_string(gemv_status s);

/* The hipError_t behind this thread's last GEMV_ERR_DEVICE / GEMV_ERR_CAPTURE (0 if none). */
int gemv_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* BBD_GEMV_H */
