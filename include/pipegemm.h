/*
 * pipegemm.h -- C ABI of the software-pipelined tiled GEMM for AMD Instinct
 * MI355X (gfx950).
 *
 * Operation.  gemm_run computes C = A * B,
 *     C[i][j] = sum_{k=0}^{K-1} A[i][k] * B[k][j],   0 <= i < M, 0 <= j < N,
 * the product the "CUDA Kernel Study: Pipelining" README benchmarks (Example
 * Code: "C = A x B") and that "Part 4 -- Pipelining and Occupancy"
 * (gpucourse.com) writes out as the triple loop of section 4.3.  The K loop
 * runs over BK-wide tiles restructured into prologue / main loop / epilogue
 * so that the global->LDS copy of the next tile overlaps the matrix-core
 * work on the current one ("pipeline-gpu-kernel", step 3; the README's
 * ping-pong and multi-stage cases).  Pipelining reorders loads only; the
 * arithmetic is that of the unpipelined loop ("pipeline-gpu-kernel", step 5).
 *
 * Element types (input -> accumulator -> output):
 *   GEMM_I8   int8  -> int32 (exact; wraps modulo 2^32 like the uint32_t
 *                     reference at the end of the gpucourse section 4.3)
 *   GEMM_F16  fp16  -> fp32  -> fp16 (round to nearest even)
 *   GEMM_BF16 bf16  -> fp32  -> bf16 (round to nearest even)
 *   GEMM_F32  fp32  -> fp32  -> fp32
 *
 * Layouts (leading dimensions are in elements):
 *   A is always row-major M x K:  A(i,k) = A[i*lda + k], lda >= K.
 *   GEMM_LAYOUT_RR: B row-major K x N:     B(k,j) = B[k*ldb + j], ldb >= N.
 *   GEMM_LAYOUT_RC: B column-major K x N:  B(k,j) = B[j*ldb + k], ldb >= K.
 *   C is always row-major M x N:  C(i,j) = C[i*ldc + j], ldc >= N.
 *
 * Alignment:
 *   C: 16-byte aligned, ldc a multiple of 4 elements.  Layout RR: N a
 *     multiple of 16 bytes worth of elements.
 *   A and B, GEMM_VARIANT_DIRECT: 16-byte aligned, lda and ldb times the
 *     element size multiples of 16 bytes, K a multiple of 16 bytes worth of
 *     elements (its copies move whole aligned 16-byte chunks).
 *   A and B, GEMM_VARIANT_REG: aligned to their element size; any K, lda and
 *     ldb.  When K is not a multiple of 16 bytes worth of elements the chunk
 *     holding column K-1 of each row is read in exact 8/4/2/1-byte pieces
 *     (the bounds-checked fallback for the last tile that "pipeline-gpu-kernel"
 *     names under its pitfalls, cp.async boundary handling): no byte past
 *     column K-1 of a row is read.  Rows and pointers that are not 16-byte
 *     aligned are read with unaligned 16-byte loads.
 *
 * Pipeline depth and load path:
 *   stages in [1, 4].
 *   GEMM_VARIANT_DIRECT: global -> LDS copies that bypass registers (the
 *     README's cp.async case; here the LDS-DMA form of buffer loads).  An
 *     LDS ring of `stages` slots with stages-1 tiles in flight; stages = 1 is
 *     the serial load-sync-compute-sync loop of the README's Background.
 *     The 256x256 tiles keep their full K-tile at stages = 3 by splitting
 *     the ring by operand: three slots for A (two tiles in flight), two for
 *     B (one in flight), 160 KiB in all; at stages = 4 they halve the
 *     K-tile (four whole slots).
 *   GEMM_VARIANT_REG: global -> VGPR -> LDS (the README's ping-pong case).
 *     min(stages, 2) LDS slots and max(1, stages-1) register staging sets,
 *     each a tile in flight; stages = 1 is the skill's register-only prefetch
 *     into a single buffer (step 1, "if it fails"), stages = 2 the classic
 *     double buffer.
 *   For a fixed dtype, layout and tile every (stages, variant) pair adds
 *   the same products in the same k order (the instances built from 16x16
 *   matrix-core blocks as well as those built from 32x32 ones), so all of
 *   them return bit-identical C.
 *
 * Memory ownership.  The caller allocates, owns and frees A, B, C and the
 * stream; they are device pointers (hipMalloc or torch CUDA tensors) on the
 * handle's device.  The library allocates no device memory; its code object
 * holds one static array of GEMM_NOALLOC_SCRATCH_BYTES per device, the
 * workspace of gemm_run_splitk_noalloc.  A and B are only read.  C must not
 * overlap A or B.
 *
 * Errors.  Every entry point returns GEMM_OK (0) or one of the codes below;
 * nothing is thrown across the ABI.  Argument checks run before any HIP call,
 * so a rejected call has no side effect.  gemm_run, gemm_run_splitk,
 * gemm_run_streamk and gemm_run_splitk_noalloc are asynchronous: each
 * enqueues one kernel launch on `stream` (and nothing else, so a graph can
 * capture it) and returns; faults during execution surface at the caller's
 * next synchronisation of that stream.
 */
#ifndef PIPEGEMM_H
#define PIPEGEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { GEMM_I8 = 0, GEMM_F16 = 1, GEMM_BF16 = 2, GEMM_F32 = 3 } gemm_dtype_t;
typedef enum { GEMM_LAYOUT_RR = 0, GEMM_LAYOUT_RC = 1 } gemm_layout_t;
typedef enum { GEMM_VARIANT_REG = 0, GEMM_VARIANT_DIRECT = 1 } gemm_variant_t;

enum {
    GEMM_OK = 0,
    GEMM_ERR_INVALID_ARG = 1,  /* NULL handle/pointer, negative size, bad enum,
                                  leading dimension too small, stages not in [1,4] */
    GEMM_ERR_ALIGNMENT = 2,    /* an alignment rule above is broken: C's, RR's N,
                                  A/B not element-aligned, or (direct variant
                                  only) A/B rows or K not whole 16-byte chunks */
    GEMM_ERR_UNSUPPORTED = 3,  /* no kernel instance fits the LDS budget, an
                                  operand tile row span exceeds 2^31 bytes, or
                                  (gemm_run_splitk) more than one split with
                                  more than 16384 C tiles */
    GEMM_ERR_HIP = 4,          /* a HIP runtime call failed (no device, launch
                                  failure); see gemm_last_hip_error */
    GEMM_ERR_SCRATCH = 5       /* gemm_run_splitk_noalloc: the split-K workspace
                                  the call needs exceeds
                                  GEMM_NOALLOC_SCRATCH_BYTES */
};

/* Size of the library's static scratch buffer (one per device), the
 * workspace of gemm_run_splitk_noalloc: 32 MiB. */
#define GEMM_NOALLOC_SCRATCH_BYTES (32 * 1024 * 1024)

/* Tile classes selectable with gemm_set_tile.  GEMM_TILE_256x256_W8 is the
 * 256x256 tile run by 8 waves (2 per SIMD) instead of 4; it is never chosen
 * automatically (its register-staged instances spill a few registers).
 * GEMM_TILE_AUTO lets the library choose the largest of the 4-wave tiles
 * that still gives at least one workgroup per compute unit. */
enum { GEMM_TILE_AUTO = -1, GEMM_TILE_256x256 = 0, GEMM_TILE_128x128 = 1, GEMM_TILE_32x64 = 2,
       GEMM_TILE_256x256_W8 = 3 };

typedef struct gemm_handle_s *gemm_handle_t;

/* What gemm_run would launch for a given call (see gemm_query). */
typedef struct {
    int32_t tile;            /* GEMM_TILE_* actually chosen */
    int32_t block_m, block_n, block_k;
    int32_t waves_m, waves_n;
    int32_t threads;         /* per workgroup */
    int32_t lds_slots;       /* slots of the LDS ring (the split ring of
                                the 256x256 tiles at 3 direct stages: 3 for
                                A, 2 for B) */
    int32_t reg_sets;        /* VGPR staging sets (0 for the direct variant) */
    int32_t tiles_in_flight; /* K-tiles loading while one is multiplied
                                (split ring: 2 for A, 1 for B) */
    int32_t lds_bytes;       /* LDS per workgroup */
    int32_t loads_per_tile;  /* 16-byte loads per lane per K-tile */
    int64_t grid;            /* workgroups launched */
    int64_t k_tiles;         /* ceil(K / block_k) */
    int32_t k_tail;          /* K mod block_k; 0 means no ragged last tile */
    int32_t c_tiles;         /* C tiles; above grid when each workgroup of a
                                256x256 tile computes several in turn (then
                                grid = one workgroup per CU) */
    int32_t splits;          /* K splits per C tile (1: none); see gemm_run_splitk */
    int32_t mfma_block;      /* edge of the MFMA blocks the kernel uses: 16
                                (4-wave 256x256 tile, 2-3 direct stages, either
                                layout, int8/fp16/bf16) or 32; both give the
                                same bits */
    int64_t workspace_bytes; /* workspace gemm_run_splitk needs (0 when splits = 1),
                                or gemm_run_streamk (see there) */
    int32_t waves_k;         /* waves sharing each C block, each taking its own
                                run of every K-tile's k-steps; their partial
                                sums are added in LDS after the K loop (1: none) */
    int32_t sk_tiles;        /* gemm_run_streamk: C tiles shared out stream-K
                                (the last sk_tiles of the c_tiles); the others
                                run data-parallel.  0 otherwise */
} gemm_config_info_t;

/* Bind a handle to HIP device `device`.  Allocates host memory for the
 * handle only.  The first call for a device also sets up that device's copy
 * of the static scratch buffer of gemm_run_splitk_noalloc: it looks up its
 * address and clears its arrival counters with one small kernel on the null
 * stream, waiting for it (so call it outside any graph capture).  Returns
 * GEMM_ERR_INVALID_ARG for a NULL `out` or a negative device, GEMM_ERR_HIP
 * when the device does not exist or that set-up fails. */
int gemm_create(gemm_handle_t *out, int device);

/* C = A * B on `stream` (a hipStream_t; NULL is the null stream).  Argument
 * checks as described above; M, N or K may be 0 (M or N = 0 does nothing,
 * K = 0 writes C = 0).  Launches on the handle's device. */
int gemm_run(gemm_handle_t h, int64_t M, int64_t N, int64_t K,
             int dtype, int layout, int stages, int variant,
             const void *A, int64_t lda, const void *B, int64_t ldb,
             void *C, int64_t ldc, void *stream);

/* C = A * B with K split over `splits` workgroups per C tile, for shapes with
 * fewer C tiles than compute units (a partial wave: skinny or small M x N
 * with a long K).  The split count is the analogue, across workgroups, of
 * what the pages do within one: more independent loads in flight per unit of
 * C; "CUDA Kernel Study: Pipelining" (Detailed Analysis) and "Part 4 --
 * Pipelining and Occupancy" (gpucourse.com) tie the gain of pipelining to
 * the occupancy it leaves.
 *   splits >= 1 asks for that many (1 = gemm_run); 0 lets the library take
 *   the smallest that gives every CU a workgroup, but at most 8 and with at
 *   least two K units per split (the last split reads every partial tile,
 *   so the final sum grows with the count).  The count used is clamped
 *   to [1, min(64, K / largest K-tile of the tile class)] and reported by
 *   gemm_query_splitk.  Each split takes whole units of the class's largest
 *   K-tile (the ragged rest goes to the last split), so for a given split
 *   count every (stages, variant) pair still returns bit-identical C.
 *   Each split writes its fp32 (int32 for GEMM_I8) accumulators to the
 *   workspace and counts itself in an arrival counter; the split that
 *   arrives last adds the partial tiles in split order 0, 1, ..., rounds
 *   once and stores C.  No workgroup waits for another, and the result does
 *   not depend on which one arrives last.  int8 stays exact.
 * Workspace: caller-owned device memory of at least
 *   info.workspace_bytes = 65536 + c_tiles * splits * block_m * block_n * 4
 *   bytes, 256-byte aligned, overlapping none of A, B, C.  Its first 65536
 *   bytes hold the arrival counters and must be zero before its first use;
 *   every call that completes leaves them zero again, so one workspace
 *   serves any later call, of any shape, on the same stream.  Calls that
 *   share a workspace must not run concurrently (two streams race).
 *   NULL / 0 is accepted when the split count used is 1.
 * Errors: as gemm_run; also GEMM_ERR_INVALID_ARG for splits < 0, a NULL or
 * too small workspace when splits > 1 are used, GEMM_ERR_ALIGNMENT for a
 * workspace not 256-byte aligned, GEMM_ERR_UNSUPPORTED for splits > 1 with
 * more than 16384 C tiles. */
int gemm_run_splitk(gemm_handle_t h, int64_t M, int64_t N, int64_t K,
                    int dtype, int layout, int stages, int variant, int splits,
                    const void *A, int64_t lda, const void *B, int64_t ldb,
                    void *C, int64_t ldc, void *workspace, int64_t workspace_bytes,
                    void *stream);

/* C = A * B with the tiles shared out stream-K over `grid` workgroups
 * (0: one per compute unit), for shapes whose C tiles do not fill a whole
 * number of rounds of the grid (a partial last wave: e.g. 400 tiles of
 * 256 x 256 on 256 CUs take two rounds of gemm_run, the second 56% full).
 * This is the other half of the split-K / stream-K pair "CUDA Kernel Study:
 * Pipelining" (Detailed Analysis) and "Part 4 -- Pipelining and Occupancy"
 * (gpucourse.com, section 4.2: occupancy and waves of blocks) point to.
 *   Every full round of `grid` tiles but the last runs as in gemm_run (one
 *   tile per workgroup at a time).  The remaining sk_tiles tiles (between
 *   one and two rounds' worth, or all of them when there are fewer than two
 *   rounds) are cut into units of the tile class's largest K-tile, numbered
 *   tile by tile, and workgroup g takes the g-th of `grid` equal runs of
 *   units (sizes differ by at most one).  A tile covered by one workgroup is
 *   stored as in gemm_run; a tile split between several is summed from
 *   their fp32 (int32 for GEMM_I8) partial tiles by whichever arrives last,
 *   in K order, so the result does not depend on arrival order, every
 *   (stages, variant) pair returns bit-identical C for a given grid, and
 *   int8 stays exact.  Float results may differ from gemm_run's in the last
 *   bits (the partial sums are grouped differently).
 *   The grid used is min(grid, sk_tiles x units); gemm_query_streamk
 *   reports it, sk_tiles and the workspace size.
 * Workspace: caller-owned device memory of at least info.workspace_bytes =
 *   65536 + 2 x grid x block_m x block_n x 4 bytes, 256-byte aligned,
 *   overlapping none of A, B, C; its first 65536 bytes are arrival counters
 *   that must be zero before the first use and are zero again after every
 *   completed call (as for gemm_run_splitk, whose workspace it may share).
 *   Calls that share a workspace must not run concurrently.  NULL / 0 is
 *   accepted when sk_tiles is 0 (M or N = 0).
 * Errors: as gemm_run; also GEMM_ERR_INVALID_ARG for grid < 0 or a NULL or
 * too small workspace, GEMM_ERR_ALIGNMENT for a workspace not 256-byte
 * aligned, GEMM_ERR_UNSUPPORTED for more than 16384 C tiles or a grid whose
 * partial tiles would pass 2 GiB. */
int gemm_run_streamk(gemm_handle_t h, int64_t M, int64_t N, int64_t K,
                     int dtype, int layout, int stages, int variant, int grid,
                     const void *A, int64_t lda, const void *B, int64_t ldb,
                     void *C, int64_t ldc, void *workspace, int64_t workspace_bytes,
                     void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * gemm_run_splitk with the library's own static scratch buffer as its
 * workspace, so the caller passes no workspace and nothing is allocated.
 *   Same arguments, checks and results as gemm_run_splitk (bit for bit:
 * same kernels, same split count), without `workspace` / `workspace_bytes`.
 * The buffer is a file-scope device array of GEMM_NOALLOC_SCRATCH_BYTES per
 * device, held until the process ends; gemm_create sets it up for its
 * device.  A call whose split-K workspace (info.workspace_bytes of
 * gemm_query_splitk) exceeds that size returns GEMM_ERR_SCRATCH before any
 * HIP call; with one split (splits = 1, or the automatic choice taking one)
 * no scratch is used.  The call calls no hipMalloc, hipFree or allocating
 * routine and enqueues one kernel launch on `stream`.
 *   Every call on a device shares that device's buffer, which keeps the
 * last call's contents; its arrival counters are zero after every completed
 * call.  Calls that overlap on one device (e.g. on two streams) race on the
 * buffer and must not be issued. */
int gemm_run_splitk_noalloc(gemm_handle_t h, int64_t M, int64_t N, int64_t K,
                            int dtype, int layout, int stages, int variant, int splits,
                            const void *A, int64_t lda, const void *B, int64_t ldb,
                            void *C, int64_t ldc, void *stream);

/* Release a handle.  NULL is a no-op.  Does not synchronise any stream. */
int gemm_destroy(gemm_handle_t h);

/* Force a tile class for later gemm_run calls on this handle
 * (GEMM_TILE_AUTO restores the automatic choice). */
int gemm_set_tile(gemm_handle_t h, int tile);

/* The configuration gemm_run would use, after the same argument checks, with
 * no HIP call and no device access.  Pointers are never dereferenced: a
 * non-NULL pointer is checked for alignment, a NULL one is taken as "not
 * given" and skipped.  The tile is chosen for a 256-CU device (MI355X).
 * `tile` is a GEMM_TILE_* value. */
int gemm_query(int64_t M, int64_t N, int64_t K, int dtype, int layout, int stages,
               int variant, int tile, const void *A, int64_t lda, const void *B,
               int64_t ldb, const void *C, int64_t ldc, gemm_config_info_t *info);

/* gemm_query for gemm_run_splitk: the same, with the split count (and the
 * workspace size) that call would use. */
int gemm_query_splitk(int64_t M, int64_t N, int64_t K, int dtype, int layout, int stages,
                      int variant, int tile, int splits, const void *A, int64_t lda,
                      const void *B, int64_t ldb, const void *C, int64_t ldc,
                      gemm_config_info_t *info);

/* gemm_query for gemm_run_streamk: the tile, grid, sk_tiles and workspace
 * size that call would use (for a 256-CU device when grid = 0). */
int gemm_query_streamk(int64_t M, int64_t N, int64_t K, int dtype, int layout, int stages,
                       int variant, int tile, int grid, const void *A, int64_t lda,
                       const void *B, int64_t ldb, const void *C, int64_t ldc,
                       gemm_config_info_t *info);

/* Resources and occupancy of the kernel instance gemm_run would launch for a
 * call (see gemm_occupancy), the figures the "Part 4 -- Pipelining and
 * Occupancy" page (section 4.2) reads from the occupancy calculator. */
typedef struct {
    int32_t blocks_per_cu;   /* hipOccupancyMaxActiveBlocksPerMultiprocessor at
                                the instance's block size (no dynamic LDS) */
    int32_t waves_per_cu;    /* blocks_per_cu x waves per block (4 SIMDs per CU) */
    int32_t num_regs;        /* hipFuncGetAttributes numRegs: vector registers
                                per lane as the runtime reports them */
    int32_t lds_bytes;       /* static LDS per workgroup (sharedSizeBytes) */
    int32_t scratch_bytes;   /* private scratch per lane (localSizeBytes; 0 =
                                no register spill) */
    int32_t threads;         /* per workgroup */
} gemm_occupancy_t;

/* The occupancy of the instance gemm_run would launch on this handle (its
 * tile override, its device) for a call of this shape, dtype, layout,
 * stages and variant; pointers are not needed (the checks of gemm_query).
 * Makes HIP calls (function attributes, occupancy) on the handle's device;
 * launches nothing.  Errors: those of gemm_query, GEMM_ERR_INVALID_ARG for a
 * NULL handle or `out`, GEMM_ERR_HIP when a HIP call fails. */
int gemm_occupancy(gemm_handle_t h, int64_t M, int64_t N, int64_t K, int dtype, int layout,
                   int stages, int variant, gemm_occupancy_t *out);

/* Static text for a status code (never NULL). */
const char *gemm_status_string(int status);

/* The last hipError_t seen by this thread's failing call (0 if none). */
int gemm_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PIPEGEMM_H */
