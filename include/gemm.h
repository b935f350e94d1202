/*
 * gemm.h — C ABI of a software-pipelined, persistent, tiled GEMM for AMD Instinct MI355X (gfx950).
 *
 *     C = A · Bᵀ      A[M, K] and B[N, K] K-major (row-major with leading dimensions lda, ldb),
 *                     fp16 or bf16 inputs, fp32 accumulation, C[M, N] row-major (ldc) in fp16,
 *                     bf16 or fp32.
 *
 * The operation is the tiled GEMM of the tutorial "GEMM II — pipelining with TMA" (Step 4: the
 * A tile at {m, k} and the B tile at {n, k}, fp32 accumulate; Step 5: a ring of stages fed ahead
 * of the math; Step 6: a persistent pool of workgroups walking a grouped tile raster; the
 * TMA-store epilogue: cast the fp32 accumulator to the output type and store). The stage ring
 * follows "Multi-Stage Software Pipelining" (Prefill / Main loop, num_stages 2..4); the operand
 * staging layout follows the 128-byte swizzle of "Async Data Movement: TMA".
 *
 * Element (i, j) of C is  sum_{k<K} A[i*lda + k] * B[j*ldb + k],  accumulated in fp32 and rounded
 * to nearest-even into the output type. C is overwritten; there is no alpha, beta or bias.
 *
 * Ownership and threading.
 *   - A plan is created by gemm_plan_create, owned by the caller, immutable after creation, and
 *     freed by gemm_plan_destroy.
 *   - A plan owns a device workspace, allocated on the current device by gemm_plan_create and
 *     freed by gemm_plan_destroy, when its configuration splits K (fp32 partial planes: splits x
 *     M x roundup(N, 8) x 4 bytes) or stages its operands (load_path GEMM_LOAD_STAGED: copies of
 *     A and B with rows of roundup(K, 8) elements); otherwise it holds no device memory.
 *     gemm_plan_workspace_bytes reports the size.
 *   - A, B and C are caller-owned device pointers; they must stay valid until the work enqueued
 *     by gemm_run has completed on its stream. C must not overlap A or B (they are read while C
 *     is written); A and B are only read and may overlap, or be one matrix (C = A·Aᵀ).
 *   - gemm_run only enqueues kernels on `stream` (a hipStream_t; NULL is the default stream). It
 *     neither allocates nor synchronises. A plan without a workspace may be run concurrently on
 *     several streams; runs of a plan with a workspace share it and must not overlap (run them on
 *     one stream, or order them with events, or make one plan per stream).
 *
 * Errors. Every entry point returns a gemm_status_t; nothing aborts or throws across the ABI.
 * A failed kernel launch returns GEMM_ERR_HIP. Misalignment is never an error: it only selects
 * the register-staged load path.
 */
#ifndef SPT_GEMM_H
#define SPT_GEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { GEMM_F16 = 0, GEMM_BF16 = 1, GEMM_F32 = 2 } gemm_dtype_t;

typedef enum {
  GEMM_OK = 0,
  GEMM_ERR_INVALID = -1,     /* a null out-pointer, negative size, ld too small, bad config */
  GEMM_ERR_UNSUPPORTED = -2, /* dtype combination or size this library does not handle */
  GEMM_ERR_HIP = -3,         /* a HIP runtime call or kernel launch failed */
  GEMM_ERR_NOMEM = -4        /* allocating the plan or its device workspace failed */
} gemm_status_t;

/* How the K-loop stages operand tiles into LDS. */
typedef enum {
  GEMM_LOAD_AUTO = 0, /* DMA when pointers, lda/ldb and K allow it, else REG */
  GEMM_LOAD_DMA = 1,  /* direct global->LDS buffer loads (16-byte chunks, needs alignment) */
  GEMM_LOAD_REG = 2,  /* global->VGPR->LDS copies with per-element K masking (any alignment) */
  GEMM_LOAD_STAGED = 3 /* copy A and B into workspace rows of roundup(K, 8) elements (zero
                          padded), then DMA; any alignment. AUTO takes it when DMA is not
                          possible, the copies fit in 3 GiB and each source operand spans
                          under 2 GiB (M rows of lda, N rows of ldb) */
} gemm_load_path_t;

/*
 * Kernel configuration. gemm_plan_create takes an optional override (NULL = heuristic);
 * gemm_plan_describe reports the configuration a plan will launch.
 *   bm, bn, bk   output tile (bm x bn) and K-tile depth; bk is 32, 64 or 128
 *   stages       S, LDS ring depth (1 = serial: wait for a tile, compute it, then load the next).
 *                With bk 64 and a square tile, 5 means a split ring of five operand slots, each
 *                holding one A or one B K-tile (two and a half stages)
 *   waves        wavefronts per workgroup (64 lanes each); 8 selects the two-wave-group kernel
 *                (256x256, bk 64, stages 2 or 5), where one group of four waves runs MFMAs while
 *                the other issues loads, alternating at workgroup barriers
 *   mfma         MFMA shape: 16 = v_mfma_f32_16x16x32_{f16,bf16}; 32 = v_mfma_f32_32x32x16_{f16,bf16}
 *                (two-wave-group kernel with the split ring only: 256x256, bk 64, stages 5, waves 8)
 *   persistent   1: launch min(#tiles, grid) workgroups that loop over tiles in static rounds;
 *                0: one workgroup per tile; 2: as 1, but after its first tile each workgroup takes
 *                the next tile nobody has taken from an atomic counter in the plan's workspace
 *                (4-wave DMA kernels whose ring leaves 16 bytes of the 160 KiB of LDS, else
 *                GEMM_ERR_UNSUPPORTED). The counters are zero
 *                when a launch starts and the launch leaves them at zero, so the plan needs no
 *                reset between runs or graph replays; like every plan with a workspace it must
 *                not run on two streams at once
 *   group_m      grouped raster height, in tiles (tiles sharing A row bands run back to back)
 *   load_path    gemm_load_path_t
 *   grid         workgroups launched (describe only; 0 in an override means "from the device")
 *   lds_bytes    LDS per workgroup (describe only)
 *   splits       split-K: K ranges per output tile, 1..16 (0 in an override means 1). Each range
 *                of ceil(ceil(K/bk)/splits) K-tiles is a work unit of its own writing an fp32
 *                partial plane; a second kernel adds the planes in range order and rounds once.
 *                The built-in choice splits when the output tiles alone leave workgroup slots of
 *                the device idle. DMA and staged paths only
 *   stream       cache hint for an operand that only one workgroup reads: 0 none, 1 A, 2 B. The
 *                hinted operand is loaded non-temporally (streaming replacement, not kept in L2
 *                or the MALL for a later launch), which leaves the cache to the shared operand.
 *                Only the 32x32 tiles (bk 128, waves 2) have these variants; others with a
 *                nonzero value are GEMM_ERR_UNSUPPORTED. The built-in choice streams B when all
 *                of M fits one tile row and B spans at least 64 MiB (A likewise when N fits one
 *                tile column), with the 8-deep ring. Results are identical with and without it
 */
typedef struct {
  int bm, bn, bk;
  int stages;
  int waves;
  int mfma;
  int persistent;
  int group_m;
  int load_path;
  int grid;
  int lds_bytes;
  int splits;
  int stream;
} gemm_config_t;

typedef struct gemm_plan_s* gemm_plan_t;

/*
 * Create a plan for C[M,N] = A[M,K]·B[N,K]ᵀ on the current HIP device.
 *   out       receives the plan (set to NULL on failure)
 *   M, N, K   sizes, each in [0, 2^31 - 1]; M or N == 0 makes gemm_run a no-op, K == 0 writes zeros
 *   a_dtype, b_dtype   GEMM_F16 or GEMM_BF16, and equal
 *   c_dtype   GEMM_F16, GEMM_BF16 or GEMM_F32
 *   lda >= K, ldb >= K, ldc >= N   leading dimensions in elements
 *   config    NULL for the built-in choice, else an explicit configuration (validated)
 * An override is validated (against 256 CUs and 160 KiB of LDS) before the device is queried.
 * Errors: GEMM_ERR_INVALID (null out, bad sizes or ld, invalid override),
 *         GEMM_ERR_UNSUPPORTED (dtype pair, a tile whose row span exceeds 2^31 bytes, an override
 *         whose workspace exceeds the caps: 1 GiB of partial planes, 3 GiB of staged operands,
 *         or a staged override whose source operand spans 2 GiB or more),
 *         GEMM_ERR_HIP (no usable gfx950 device), GEMM_ERR_NOMEM (host or device allocation).
 */
gemm_status_t gemm_plan_create(gemm_plan_t* out, int64_t M, int64_t N, int64_t K,
                               gemm_dtype_t a_dtype, gemm_dtype_t b_dtype, gemm_dtype_t c_dtype,
                               int64_t lda, int64_t ldb, int64_t ldc, const gemm_config_t* config);

/*
 * Enqueue C = A·Bᵀ on `stream` (hipStream_t, NULL = default stream).
 *   A: M rows of lda elements, B: N rows of ldb elements, C: M rows of ldc elements; only
 *   C[i*ldc + j] with i < M, j < N is written (the ldc padding is never touched).
 *   If A or B is not 16-byte aligned the register-staged path runs instead of the DMA path
 *   (a staged plan copies the operands and needs no alignment). C needs only its element's
 *   alignment (2 bytes for F16/BF16, 4 for F32): the 16-byte stores take any byte offset.
 *   A staged plan launches the staging copy first; a split plan launches the mainloop into its
 *   partial planes and then the reduction, all on `stream`.
 * Errors: GEMM_ERR_INVALID (null plan; null A, B or C while M, N > 0), GEMM_ERR_HIP (launch).
 */
gemm_status_t gemm_run(gemm_plan_t plan, const void* A, const void* B, void* C, void* stream);

/* Free a plan and its workspace. NULL is accepted and returns GEMM_OK. Work enqueued with the
 * plan must have completed. GEMM_ERR_HIP if freeing the workspace failed (the plan is freed). */
gemm_status_t gemm_plan_destroy(gemm_plan_t plan);

/* Bytes of device workspace the plan owns (0 when none). Errors: GEMM_ERR_INVALID on NULL. */
gemm_status_t gemm_plan_workspace_bytes(gemm_plan_t plan, int64_t* out);

/* Copy the configuration `plan` launches into *out (for a plan in two parts, part 0's, with this
 * plan's load path). Errors: GEMM_ERR_INVALID on NULL. */
gemm_status_t gemm_plan_describe(gemm_plan_t plan, gemm_config_t* out);

/*
 * How a plan covers the output. Without an override, a plan may cut the problem in two when one
 * tile size would leave the last round of workgroups mostly idle (wave quantisation): part 0 takes
 * whole rounds of its tiles, part 1 is planned on its own by the same model (smaller tiles, or K
 * split), and gemm_run launches them one after the other on the same stream, over the same
 * operands (after the staging copy, when the plan stages).
 *   *dim     -1: one part; 1: the output's columns are cut at *at (part 0: columns [0, at),
 *            part 1: [at, N)); 0: its rows are cut at *at
 *   first    part 0's configuration (the plan's own when *dim is -1); may be NULL
 *   second   part 1's configuration (untouched when *dim is -1); may be NULL
 * Errors: GEMM_ERR_INVALID (null plan, dim or at).
 */
gemm_status_t gemm_plan_parts(gemm_plan_t plan, int* dim, int64_t* at, gemm_config_t* first, gemm_config_t* second);

/* Static, human-readable name of a status code ("GEMM_OK", ...). Never NULL. */
const char* gemm_status_string(gemm_status_t status);

/*
 * For callers that cannot allocate device memory (work recorded under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): plan and enqueue C = A·Bᵀ in one call that
 * calls no allocating routine (no hipMalloc, hipFree or host heap). Arguments and result are those
 * of gemm_plan_create with a NULL config followed by gemm_run: the same built-in choice, the same
 * kernels, the same bits. The plan lives on this call's stack. A plan that needs a workspace (a
 * staged operand copy, split-K partial planes) takes it from a static device array of
 * GEMM_NOALLOC_SCRATCH_BYTES, which each device holds from the library's first use there until the
 * process ends; the first call on a device looks up that device's copy (hipGetSymbolAddress), so
 * make one call outside graph capture before capturing. Every launch writes whatever part of the
 * array it later reads, so no state carries over from one call to the next.
 *   The array is shared by every call on a device: calls that overlap on one device (on different
 *   streams, or from different threads without ordering) race on it and must be ordered by the
 *   caller. Calls on different devices do not interact.
 * Errors: those of gemm_plan_create and gemm_run; GEMM_ERR_UNSUPPORTED when the plan's workspace
 *   exceeds GEMM_NOALLOC_SCRATCH_BYTES (64 MiB: for example a staged copy of more than 64 MiB of
 *   operands, or split-K partial planes of more than 64 MiB). Nothing is enqueued on an error.
 */
#define GEMM_NOALLOC_SCRATCH_BYTES ((int64_t)64 << 20)
gemm_status_t gemm_run_noalloc(int64_t M, int64_t N, int64_t K, gemm_dtype_t a_dtype, gemm_dtype_t b_dtype,
                               gemm_dtype_t c_dtype, int64_t lda, int64_t ldb, int64_t ldc, const void* A,
                               const void* B, void* C, void* stream);

/* ------------------------------------------------------------------------------------------
 * Host-only introspection (no device work). They expose the exact functions the kernels use,
 * so their invariants can be tested without a GPU.
 * ---------------------------------------------------------------------------------------- */

/*
 * The configuration gemm_plan_create would launch for this problem on a device with `cu_count`
 * compute units and `lds_bytes` of LDS per workgroup, assuming 16-byte aligned pointers: the
 * built-in choice when `config` is NULL, else the override after the same validation (so every
 * override error can be checked without a GPU). Same argument checks and errors as
 * gemm_plan_create (minus GEMM_ERR_HIP and GEMM_ERR_NOMEM).
 */
gemm_status_t gemm_select_config(int64_t M, int64_t N, int64_t K, gemm_dtype_t a_dtype,
                                 gemm_dtype_t b_dtype, gemm_dtype_t c_dtype, int64_t lda,
                                 int64_t ldb, int64_t ldc, int cu_count, int lds_bytes,
                                 const gemm_config_t* config, gemm_config_t* out);

/*
 * The cut gemm_plan_create would make without an override (see gemm_plan_parts), on a device with
 * `cu_count` compute units and `lds_bytes` of LDS per workgroup: *dim -1 (and *first the single
 * configuration), or the cut and both parts' configurations. Same argument checks and errors as
 * gemm_select_config; dim and at must not be NULL.
 */
gemm_status_t gemm_select_parts(int64_t M, int64_t N, int64_t K, gemm_dtype_t a_dtype, gemm_dtype_t b_dtype,
                                gemm_dtype_t c_dtype, int64_t lda, int64_t ldb, int64_t ldc, int cu_count,
                                int lds_bytes, int* dim, int64_t* at, gemm_config_t* first, gemm_config_t* second);

/*
 * Work unit handled by workgroup `wg` (0 <= wg < grid) on its `round`-th pass of the persistent
 * loop, for a tiles_m x tiles_n tile grid with `splits` K ranges per tile, grouped raster of
 * height group_m, and `grid` workgroups (dispatched round-robin over the 8 XCDs): output tile
 * (*tm, *tn), K range *split. Units are numbered range by range (all tiles of range 0 in raster
 * order, then range 1, ...). Returns 1, or 0 when that workgroup has no unit in that round.
 * Invalid arguments return -1.
 */
int gemm_schedule_tile(int64_t tiles_m, int64_t tiles_n, int splits, int group_m, int grid, int wg,
                       int round, int64_t* tm, int64_t* tn, int* split);

/*
 * The pipeline protocol's counts for the DMA kernel with this tile (bm, bn, bk), ring depth and wave
 * count, as the kernel uses them ("GEMM II — pipelining with TMA", Step 5; "Multi-Stage Software
 * Pipelining", Prefill and Main loop): out[0..9] = loads per wave of an A operand tile, of a B
 * operand tile, of a stage; 1 for the split ring of five operand slots; the vmcnt threshold after the
 * prologue and at each hand-over; the refill loads issued in the hand-over k-step and in k-step 0 of
 * the next K-tile; and, for the two-group kernel (waves 8), the first group's threshold after its
 * prologue and the second group's after a memory phase in which it loaded. Returns 10, or -1 when
 * no DMA kernel has this shape or out is NULL or n_out < 10.
 */
int gemm_pipeline_protocol(int bm, int bn, int bk, int stages, int waves, int* out, int n_out);

/*
 * Byte offset, inside one LDS operand tile of `rows` rows and depth bk (32, 64 or 128), of the
 * 16-byte chunk holding elements [8*chunk, 8*chunk + 8) of tile row `row` (the XOR swizzle:
 * 128-byte rows with chunk XOR (row mod 8) for bk 64 and 128, 64-byte rows with chunk XOR
 * ((row / 4) mod 4) for bk 32). Returns -1 for invalid arguments.
 */
int64_t gemm_lds_chunk_offset(int rows, int bk, int row, int chunk);

/* ------------------------------------------------------------------------------------------
 * Measurement aids (device work on `stream`; the caller times them with events).
 * ---------------------------------------------------------------------------------------- */

/*
 * Launch a dense-MFMA throughput kernel: every wave issues `iters` x 16 independent
 * v_mfma_f32_16x16x32_bf16 on register operands, `waves_per_simd` waves per SIMD on every CU.
 * *flops receives the floating-point operations the launch performs (2·16·16·32 per MFMA).
 * Errors: GEMM_ERR_INVALID (iters < 1, waves_per_simd not in 1..2, null flops), GEMM_ERR_HIP.
 */
gemm_status_t gemm_probe_mfma_peak(int64_t iters, int waves_per_simd, void* stream, double* flops);

/*
 * Launch a streaming copy of `bytes` (a multiple of 16) from src to dst with 16-byte loads and
 * stores; used to read the HBM bandwidth and to scale memory-traffic counters.
 * Errors: GEMM_ERR_INVALID (null pointer, bytes not a multiple of 16), GEMM_ERR_HIP.
 */
gemm_status_t gemm_probe_copy(const void* src, void* dst, int64_t bytes, void* stream);

/*
 * Launch an LDS read-pattern kernel (one workgroup of 4 waves per CU, `iters` x 8 ds_read_b128
 * per lane). swizzle -1: lane l reads 16*l (the conflict-free reference); 0..4: lane l reads row
 * l%16, 16-byte chunk l/16 of a 128-byte-row tile, with the physical chunk XOR-ed by
 * 0: nothing, 1: row%8, 2: (row%8) XOR bit3(row), 3: (row/2)%8, 4: (row%4) XOR (bit2(row)<<2).
 * Read with the SQ_LDS_BANK_CONFLICT counter to compare LDS layouts.
 * Errors: GEMM_ERR_INVALID (swizzle outside -1..4, iters < 1), GEMM_ERR_HIP.
 */
gemm_status_t gemm_probe_lds_read(int swizzle, int64_t iters, void* stream);

/*
 * Launch a read-only streaming kernel over `bytes` (a multiple of 16) at src: 16-byte loads, eight
 * in flight per thread, nothing written but one word that no input selects. Over a buffer larger
 * than the 256 MB MALL it measures the HBM read bandwidth, the ceiling of a memory-bound GEMM's
 * operand stream ("Multi-Stage Software Pipelining", Performance: DRAM throughput is the figure
 * the pages read for a load-bound loop). The caller times it with events.
 * Errors: GEMM_ERR_INVALID (null src, bytes negative or not a multiple of 16), GEMM_ERR_HIP.
 */
gemm_status_t gemm_probe_read(const void* src, int64_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPT_GEMM_H */
