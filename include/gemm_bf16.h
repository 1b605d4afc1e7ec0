/*
 * gemm_bf16.h -- C ABI of the MI355X (gfx950) pipelined, persistent bf16 GEMM.
 *
 * The operation is the matmul the reference pages build their pipelines
 * around: C = A * B with bf16 operands, fp32 accumulation and the fp32
 * results converted to bf16 in the epilogue ("Allow separate sub-DAG for load
 * and compute warp groups with warp-specialized circular buffering", section
 * "Pseudo-code").  Element by element:
 *
 *     C[i*ldc + j] = bf16_rne( sum_{k<K} A[i*lda + k] * B(k, j) )      (i<M, j<N)
 *
 * with B(k, j) = B[k*ldb + j] for gemm_bf16 (B stored K x N, row-major) and
 * B(k, j) = B[j*ldb + k] for gemm_bf16_bt (B stored N x K, row-major).  The
 * sum is accumulated in fp32 by the matrix cores; the order of the fp32
 * additions is the library's, so results may differ from an exactly rounded
 * product by the fp32 rounding of the partial sums (well under one bf16 ulp
 * for K up to ~10^5 at unit-size inputs).  Bit identity: calls whose plans
 * agree on the MFMA block (plan.mfma_block: 16 x 16 x 32 or 32 x 32 x 16
 * MFMAs) and on the k split (plan.k_splits, plan.tail_tiles,
 * plan.tail_splits, and the tile plan.bm x plan.bn whenever a split is
 * present) run the same chain of MFMA accumulations for every element and
 * give the same bits, whatever the sync mode, stage count or B layout.
 * Calls whose plans differ in any of these may differ by fp32 rounding.
 * There is no alpha/beta: C is overwritten.
 *
 * How the work is done (none of this changes the result):
 *   - a persistent grid walks the output tiles grid-stride ("Allow separate
 *     sub-DAG ...", sections "Context" and "Scheduling Proposal");
 *   - operand tiles stream through an S-stage LDS ring (circular buffer)
 *     filled by direct global-to-LDS loads ("Use mbarrier for WAR for
 *     circular buffering", both code listings);
 *   - the ring is synchronised either by one workgroup barrier per k-step
 *     (GEMM_SYNC_BARRIER, that page's first listing), or by separate per-stage
 *     "loaded" (RAW) and "fully read" (WAR) counters (GEMM_SYNC_FLAGS, that
 *     page's second listing), or by the same counters between dedicated
 *     loader waves and MFMA waves (GEMM_SYNC_WAVESPEC, the producer/consumer
 *     split of "Allow separate sub-DAG ...", section "Pseudo-code"), or by
 *     those counters between loader waves and two groups of MFMA waves that
 *     take the output tiles in turn (GEMM_SYNC_PINGPONG, the ping-pong matmul
 *     that page's section "Why?" names).
 *
 * Memory ownership: A, B and C are device pointers owned by the caller, on
 * the HIP device that is current when the call is made.  The library never
 * allocates, frees or retains them.  A and B are only read.  C must not
 * overlap A or B.
 *
 * Split k range: a shape with at most half as many output tiles as pipelines
 * (compute units x plan.pipelines, in the chosen configuration's tile, see
 * gemm_bf16_plan) and a long k range -- K a multiple of 64 * s
 * and K / s >= 512 for some s >= 2 -- is computed as s chunks of k (s <= 16)
 * so that the GPU fills.  Each output tile's chunks are summed in fp32, in
 * chunk order, after one fp32 chain per chunk; the result differs from the
 * unsplit sum only by fp32 rounding, is the same for every sync mode and
 * stage count with the same tile, MFMA block and split (plan.bm, plan.bn,
 * plan.mfma_block, plan.k_splits), and is deterministic.  The fp32 partial tiles
 * (plan.workspace_bytes) live in temporary device memory the library keeps
 * (see "Temporary memory" below).  Not a section of the pages: the
 * persistent schedule there assumes enough output tiles.
 *
 * Split tail: when the output tiles (in the chosen configuration's tile) do
 * not fill whole rounds of the persistent grid and the last round would hold
 * at most half the compute units' worth, the last r tiles of the schedule
 * run as a second launch with the k range split into s chunks (K a multiple
 * of 64 * s, K / s >= 1024, K - K / s >= 2048, 2 <= s <= min(16,
 * compute units / r)), then
 * reduced as above.  The
 * tiles of that tail differ from an unsplit result by fp32 rounding only,
 * and deterministically; since the tail depends on the tile, modes with
 * different tiles (see gemm_bf16_plan) can differ there in the last bit.
 * plan.tail_tiles and plan.tail_splits report it.
 *
 * Asynchrony: a call validates its arguments on the host, enqueues its work
 * on `stream` (a hipStream_t; NULL means the null stream) and returns.  A
 * return of GEMM_OK means "enqueued"; faults during execution surface at the
 * next synchronisation with the stream, as for any HIP kernel.
 *
 * Thread safety: calls may be made from several host threads.
 */
#ifndef GEMM_BF16_H
#define GEMM_BF16_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Ring synchronisation schemes. */
enum {
    GEMM_SYNC_BARRIER = 0,  /* one s_barrier per k-step covers RAW and WAR */
    GEMM_SYNC_FLAGS = 1,    /* per-stage full/empty LDS counters, every wave loads and computes */
    GEMM_SYNC_WAVESPEC = 2, /* per-stage counters between loader waves and MFMA waves */
    GEMM_SYNC_PINGPONG = 3  /* as GEMM_SYNC_WAVESPEC, with two MFMA wave groups taking output
                               tiles in turn: one group's epilogue overlaps the other's MFMAs.
                               With 2 stages each group has a ring of its own and both
                               groups compute at once (plan.pipelines = 2) */
};

/*
 * The `stages` value that selects the split-window ring (GEMM_SYNC_BARRIER
 * only): instead of whole stages, the LDS holds five windows of one operand
 * tile each (256 x 64 bf16, 32 KiB).  A k-step's A tile and B tile sit in two
 * windows; when a k-step's windows are drained, one takes the B tile of the
 * k-step after next and the other the A tile of the one after that, so A
 * tiles get two k-steps to land and B tiles one.  The output tile's epilogue
 * is staged in a drained window, so the whole 160 KiB serves the ring.  The
 * split follows the shared-memory reduction strategies of "[WIP] SM120 fused
 * backward kernel: exploratory shared-memory reduction" (section
 * "Shared-memory reduction strategies": buffer aliasing, and a producer that
 * streams one half of an operand while the consumer computes on the other).
 * Results follow the bit-identity rule above (its plan has 16 x 16 MFMA
 * blocks and the 256 x 256 tile).
 */
enum { GEMM_STAGES_WINDOWS = 5 };

/* Status codes.  Every entry point returns GEMM_OK (0) or one of these. */
enum {
    GEMM_OK = 0,
    GEMM_ERR_INVALID_VALUE = -1,     /* negative size, NULL pointer with a nonzero extent,
                                        leading dimension too small, NULL output struct */
    GEMM_ERR_MISALIGNED = -2,        /* a pointer not 2-byte aligned */
    GEMM_ERR_UNSUPPORTED_SHAPE = -3, /* N or K above 2^22, M above 2^31 - 1, or more work
                                        items than the schedule indexes */
    GEMM_ERR_STAGES = -4,            /* stages not 0 (default), 2..4, or GEMM_STAGES_WINDOWS
                                        with GEMM_SYNC_BARRIER */
    GEMM_ERR_SYNC_MODE = -5,         /* sync_mode not one of GEMM_SYNC_* */
    GEMM_ERR_DEVICE = -6,            /* no HIP device, or the current device is not gfx950 */
    GEMM_ERR_LAUNCH = -7,            /* the kernel launch was rejected by the runtime */
    GEMM_ERR_ALIAS = -8,             /* C overlaps A or B */
    GEMM_ERR_SCRATCH = -9            /* gemm_bf16_noalloc only: the call needs more temporary
                                        memory than its scratch region holds */
};

/* Size of gemm_bf16_noalloc's per-device scratch region, in bytes. */
enum { GEMM_NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024 };

/* The tiling and launch shape chosen for a problem (see gemm_bf16_plan). */
typedef struct gemm_bf16_plan {
    int32_t bm, bn, bk;       /* output tile BM x BN, k-step BK */
    int32_t stages;           /* depth of the LDS ring (GEMM_STAGES_WINDOWS: the split-window ring) */
    int32_t sync_mode;        /* GEMM_SYNC_* */
    int32_t b_transposed;     /* 1 for gemm_bf16_bt */
    int32_t mfma_waves;       /* waves that run the matrix-core loop */
    int32_t producer_waves;   /* dedicated loader waves (GEMM_SYNC_WAVESPEC, GEMM_SYNC_PINGPONG), else 0 */
    int32_t threads;          /* threads per workgroup */
    int32_t lds_bytes;        /* LDS per workgroup */
    int64_t tiles;            /* output tiles: ceil(M/bm) * ceil(N/bn) */
    int64_t k_steps;          /* k-steps per work item: ceil((K / k_splits) / bk) */
    int64_t grid;             /* persistent workgroups of the main launch:
                                 min((tiles - tail_tiles) * k_splits, compute units) */
    int64_t k_splits;         /* chunks the k range is split into (1: no split) */
    int64_t workspace_bytes;  /* fp32 partial tiles of a split call or a split tail (0 without either) */
    int64_t tail_tiles;       /* split tail: the last tail_tiles tiles of the raster run as a second
                                 launch with the k range split in tail_splits chunks (0: none) */
    int64_t tail_splits;      /* chunks of the split tail (0 without one) */
    int64_t pad_bytes;        /* zero-padded operand copies when N or K is not a multiple of 8 (0 otherwise);
                                 the plan's other fields then describe the padded problem */
    int64_t mfma_block;       /* MFMA block edge: 16 (v_mfma_f32_16x16x32_bf16, 32 k per instruction) or 32
                                 (v_mfma_f32_32x32x16_bf16, 16 k per instruction).  Calls whose plans agree
                                 on it and on the k split (k_splits, tail_tiles, tail_splits, bm, bn) run
                                 the same chain of MFMAs for every element and give the same bits. */
    int64_t pipelines;        /* independent LDS rings per workgroup: 2 where each MFMA group has its own
                                 ring and takes every other work item (GEMM_SYNC_PINGPONG, 2 stages), else 1.
                                 The k split fills compute units x pipelines work items. */
} gemm_bf16_plan_t;

/*
 * gemm_bf16: C[M,N] = A[M,K] * B[K,N]; A row-major (lda >= K), B row-major
 * K x N (ldb >= N), C row-major (ldc >= N).  Sizes and leading dimensions are
 * in elements.
 *
 * Requirements: M, N, K >= 0; N and K at most 2^22; A, B, C 2-byte aligned
 * (checked only for operands that are read or written).  M == 0 or N == 0 is
 * a no-op.  K == 0 writes +0 to every element of C.
 *
 * Fast path: N and K multiples of 8, lda, ldb, ldc multiples of 8 and at most
 * 2^22, A, B, C 16-byte aligned.  Any other call copies A and B, zero-padded
 * to multiples of 8 elements, into compact buffers (plan.pad_bytes, temporary
 * memory as below), runs the fast path on them and copies the N valid columns
 * of the result into C.  The zero padding
 * along K contributes only zero products, so results are those of the
 * unpadded problem.
 *
 * stages: 0 picks the default for the sync mode (GEMM_STAGES_WINDOWS for
 * GEMM_SYNC_BARRIER, 3 for GEMM_SYNC_PINGPONG, 2 for the others); otherwise
 * 2, 3 or 4 whole stages, or GEMM_STAGES_WINDOWS (barrier sync only).
 * sync_mode: GEMM_SYNC_BARRIER, GEMM_SYNC_FLAGS, GEMM_SYNC_WAVESPEC or
 * GEMM_SYNC_PINGPONG.
 * stream: a hipStream_t (NULL for the null stream).
 *
 * Temporary memory (split workspaces, padded copies): the library keeps
 * blocks of device memory per device and reuses them; a call allocates only
 * when no kept block fits, and frees nothing (gemm_bf16_release_workspaces
 * does, on request).  A block is reused by a later call on the stream of its
 * last use (stream order makes that safe), or on any stream once the event
 * it recorded after that use has completed.  So repeated calls on one stream
 * reuse one block per size, and each stream that runs such calls
 * concurrently with another holds its own.  New blocks are sized to a power
 * of two of at least 1 MiB and allocated stream-ordered
 * (hipMallocFromPoolAsync from a pool the library creates per device;
 * hipMallocAsync if it could not be created).  The calls never wait for the
 * GPU: a stream-ordered free (hipFreeAsync) returns only after the stream's
 * queued work has finished, which is why they keep their blocks.  Under
 * graph capture the memory is allocated and freed inside the captured graph
 * instead.  A failed allocation returns GEMM_ERR_DEVICE.
 * gemm_bf16_workspace_info reports what is kept.
 *
 * Returns GEMM_OK once the work is enqueued, else a negative status.
 * Validation that does not need the device happens before any HIP call; after
 * a validation error nothing was enqueued.  A failed allocation or launch
 * later in the call may leave earlier steps enqueued, and C is then
 * unspecified.
 */
int gemm_bf16(int64_t M, int64_t N, int64_t K,
              const void* A, int64_t lda,
              const void* B, int64_t ldb,
              void* C, int64_t ldc,
              int stages, int sync_mode, void* stream);

/*
 * gemm_bf16_bt: as gemm_bf16, but B is stored transposed: N x K row-major
 * (ldb >= K), so that C[i][j] = sum_k A[i][k] * B[j*ldb + k].
 */
int gemm_bf16_bt(int64_t M, int64_t N, int64_t K,
                 const void* A, int64_t lda,
                 const void* B, int64_t ldb,
                 void* C, int64_t ldc,
                 int stages, int sync_mode, void* stream);

/*
 * gemm_bf16_noalloc: gemm_bf16 for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments, results and bits as gemm_bf16 (B stored
 * K x N); it calls no hipMalloc, hipFree or allocating library routine.
 *
 * Where gemm_bf16 takes temporary memory the library keeps -- the fp32
 * partial tiles of a split k range or split tail (plan.workspace_bytes) and
 * the zero-padded operand copies of a call off the 8-element grid
 * (plan.pad_bytes, or less when only some operands need copying) -- this entry
 * point uses a fixed scratch region of GEMM_NOALLOC_SCRATCH_BYTES (64 MiB)
 * per device instead: a static device array the library's code object
 * carries, present on every GPU the library runs on until the process ends.
 * 64 MiB holds every split workspace on a device with up to 256 compute units
 * (one 256 x 256 fp32 partial tile per compute unit at most); padded copies
 * must fit beside it.  A call whose needs exceed the region returns
 * GEMM_ERR_SCRATCH before anything is enqueued.
 *
 * The region is shared by every call on one GPU and keeps the last call's
 * contents (nothing in it needs to start at zero: every byte a call reads
 * from it was written earlier in the same call).  Calls that overlap in time
 * on one GPU -- on different streams, or from different host threads --
 * race on it and give undefined results; order them on one stream, or use
 * gemm_bf16.  Nothing here records a hipMemsetAsync.
 */
int gemm_bf16_noalloc(int64_t M, int64_t N, int64_t K,
                      const void* A, int64_t lda,
                      const void* B, int64_t ldb,
                      void* C, int64_t ldc,
                      int stages, int sync_mode, void* stream);

/*
 * gemm_bf16_plan: the plan gemm_bf16 (b_transposed == 0) or gemm_bf16_bt
 * (b_transposed != 0) would use for this shape, stage count and sync mode.
 * Writes *out and returns GEMM_OK, or returns a negative status (sizes,
 * stages and sync mode are validated as in gemm_bf16; pointers and leading
 * dimensions are not involved).  Queries the current device for its compute
 * unit count.
 */
int gemm_bf16_plan(int64_t M, int64_t N, int64_t K, int b_transposed,
                   int stages, int sync_mode, gemm_bf16_plan_t* out);

/*
 * gemm_bf16_plan_cus: gemm_bf16_plan for a device with `compute_units`
 * compute units, without querying any device (host code only; usable where
 * no GPU is present).  gemm_bf16 on a device with that many compute units
 * uses exactly this plan.  Returns GEMM_ERR_INVALID_VALUE for a null `out`
 * or compute_units < 1, otherwise as gemm_bf16_plan.
 */
int gemm_bf16_plan_cus(int64_t M, int64_t N, int64_t K, int b_transposed,
                       int stages, int sync_mode, int compute_units, gemm_bf16_plan_t* out);

/*
 * gemm_bf16_strerror: a static, NUL-terminated description of a status code
 * (never NULL; unknown codes give "unknown status").
 */
const char* gemm_bf16_strerror(int status);

/*
 * Failed synchronisation.  The counter-synchronised modes (GEMM_SYNC_FLAGS,
 * GEMM_SYNC_WAVESPEC, GEMM_SYNC_PINGPONG) wait on LDS counters with bounded
 * polls, so a protocol failure -- a counter that never reaches its target --
 * cannot hang the GPU: the wave gives up and runs its finite loops to the
 * end.  Such a call still returns GEMM_OK (the failure happens after it
 * returned).  The caller learns of it in two ways:
 *   - C: every output tile whose computation may have used data the failure
 *     let through is written as NaN (bf16 quiet NaN) in full.  Tiles of other
 *     workgroups, and tiles a workgroup stored before its failure, hold
 *     correct values.  A result without NaN where the inputs have none is
 *     therefore trustworthy.
 *   - gemm_bf16_sync_timeouts below counts the waits that gave up.
 * GEMM_SYNC_BARRIER uses the hardware barrier only and cannot fail this way.
 */

/*
 * gemm_bf16_sync_timeouts: the number of bounded waits on ring counters that
 * gave up since the library was loaded on the current device.  Zero in
 * correct operation.  Synchronises the device.  If reset != 0 the counter is
 * cleared after reading.  Returns the count (>= 0) or a negative status.
 */
int64_t gemm_bf16_sync_timeouts(int reset);

/*
 * gemm_bf16_set_sync_spin_limit: the number of unsuccessful polls after which
 * a ring counter wait gives up, for calls made from now on (process-wide).
 * polls == 0 restores the default (2^22 polls, about 0.3 s of waiting);
 * polls must be at most 2^32 - 1.  Returns the previous limit, or
 * GEMM_ERR_INVALID_VALUE.  A tiny limit makes waits give up while the data is
 * merely late, which exercises the failure handling above on purpose; the
 * kernels still terminate normally.
 */
int64_t gemm_bf16_set_sync_spin_limit(int64_t polls);

/*
 * gemm_bf16_workspace_info: the temporary memory the library keeps on the
 * current device for split and padded calls ("Temporary memory" above):
 * *blocks the number of blocks, *bytes their total size, *busy how many are
 * taken by a call that is being enqueued right now (0 between calls).  Host
 * memory, three int64_t; host-side only, does not synchronise.  Returns
 * GEMM_OK, GEMM_ERR_INVALID_VALUE for a null pointer, or GEMM_ERR_DEVICE.
 */
int gemm_bf16_workspace_info(int64_t* blocks, int64_t* bytes, int64_t* busy);

/*
 * gemm_bf16_release_workspaces: frees the temporary memory the library keeps
 * on the current device ("Temporary memory" above) and returns it from the
 * library's pool to the device.  Synchronises the device first; calls made
 * from other threads meanwhile wait for it.  A block that another thread's
 * call holds at that moment stays kept.  Later split and padded calls
 * allocate again as needed.  Not for use under graph capture.  Returns
 * GEMM_OK or GEMM_ERR_DEVICE.
 */
int gemm_bf16_release_workspaces(void);

/*
 * Clock sampling, for measurement.  Under load the clock of these boards is
 * set by the power limit and depends on the kernel and the data, so a
 * throughput alone does not say how busy the matrix cores were; profiler
 * counter passes change the power state themselves.  While sampling is on,
 * thread 0 of every GEMM workgroup that has work adds its elapsed shader-clock
 * ticks (s_memtime), its elapsed constant-rate ticks (s_memrealtime) and a
 * count of one to per-device sums when it finishes.  Sampling costs a few
 * scalar instructions and three atomic adds per workgroup and leaves results
 * unchanged bit for bit.  The split reduction, zero-fill and padding kernels
 * take no samples.
 *
 * gemm_bf16_set_clock_sampling: on (enable != 0) or off for calls made from
 * now on (process-wide, default off).  Returns the previous setting (0 or 1).
 */
int gemm_bf16_set_clock_sampling(int enable);

/*
 * gemm_bf16_clock_samples: the current device's sums since the library was
 * loaded or last reset: out[0] shader-clock ticks, out[1] constant-rate
 * ticks, out[2] samples (workgroups), and out[3] the constant rate in Hz.
 * The mean clock in Hz is out[0] / out[1] * out[3].  `out` is host memory of
 * four uint64_t.  Synchronises the device (not for use under graph capture);
 * if reset != 0 the sums are cleared after reading.  Returns GEMM_OK,
 * GEMM_ERR_INVALID_VALUE for a null `out`, or GEMM_ERR_DEVICE.
 */
int gemm_bf16_clock_samples(uint64_t* out, int reset);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_BF16_H */
