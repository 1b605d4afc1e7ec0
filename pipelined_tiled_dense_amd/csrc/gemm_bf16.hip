// Pipelined, persistent, tiled bf16 GEMM for MI355X (gfx950 / CDNA4).
//
//   C[M,N] = bf16_rne( A[M,K] * B )   with fp32 accumulation on the matrix cores,
//   B stored K x N (gemm_bf16) or N x K (gemm_bf16_bt).
//
// The pages this follows describe the method for other hardware; what is kept
// and how it maps onto gfx950:
//
// * Circular buffer ("Use mbarrier for WAR for circular buffering", both code
//   listings).  Operand tiles stream through an S-stage ring in LDS.  A stage
//   is filled by direct global-to-LDS loads (buffer_load_dwordx4 ... lds): each
//   lane's 16 bytes land at a fixed slot of a 1 KiB LDS window, so the XOR
//   swizzle that keeps the later fragment reads free of bank conflicts is
//   applied on the global side (each lane fetches the chunk that belongs in its
//   slot).  gfx950 has no bulk-copy engine or transaction-counting barrier:
//   every loading wave issues its own share and learns that its data has
//   landed from its vector-memory counter (s_waitcnt vmcnt).
//
// * Ring synchronisation.  GEMM_SYNC_BARRIER: one workgroup
//   s_barrier per k-step, after each wave's own loads for the stage landed and
//   its reads of the previous stage completed, covers both the read-after-write
//   and the write-after-read hazard (the page's first listing, whose WAR guard
//   is a block-wide barrier).  GEMM_SYNC_FLAGS: two monotonic counters per
//   stage in LDS -- "full" (every loading wave's data for this use has landed)
//   and "empty" (every reading wave has finished with it) -- the page's two
//   signals per stage (the second listing).  A wave releases a stage as soon as
//   its fragment reads have landed, ahead of its last MFMAs on them; the reads
//   of both counters go out together and their round trip overlaps MFMAs.
//
// * Wave specialisation ("Allow separate sub-DAG for load and compute warp
//   groups with warp-specialized circular buffering", section "Pseudo-code").
//   GEMM_SYNC_WAVESPEC runs loader waves over one flat stream of (tile, k-step)
//   positions and MFMA waves over tile { k-step { ... } epilogue } loop nests,
//   talking only through the full/empty counters.  The empty counters start at
//   zero and are read as "free" for a stage's first use, which is what the
//   consumer's initial arrive on every empty barrier achieves there.  gfx950
//   cannot move registers between roles, so all waves get one register budget:
//   either one MFMA wave per SIMD next to the loaders (256 x 128 tiles,
//   double-buffered fragments) or two (256 x 256 tiles, one fragment set per
//   wave, the other wave covering its reads).
//
// * Ping-pong (same page, section "Why?", which names ping-pong matmul
//   kernels as a goal).  GEMM_SYNC_PINGPONG keeps the loader waves and splits
//   the MFMA waves into two groups that take the workgroup's output tiles in
//   turn; each position is released by the group that computes it, so one
//   group's epilogue overlaps the other's main loop.  With 3 and 4 stages the
//   groups share one ring and their main loops alternate; with 2 stages each
//   group has a pipeline of its own (ring, counters, two loader waves), and
//   the groups compute side by side, two MFMA waves per SIMD.
//
// * Split windows ("[WIP] SM120 fused backward kernel: exploratory
//   shared-memory reduction", section "Shared-memory reduction strategies":
//   buffer aliasing, and streaming one half of an operand while the other is
//   computed on).  With barrier sync the ring can instead be five windows of
//   one operand tile each: a k-step's A tile and B tile live in separate
//   windows, the B tile of the k-step after next refills a drained window
//   first, and the epilogue stages through a drained window.
//
// * Persistent scheduling (same page, sections "Context" and "Scheduling
//   Proposal").  A grid of min(tiles, CUs) workgroups walks the output tiles
//   grid-stride; the load side sees the merged (tile, k-step) stream, so the
//   ring keeps prefetching across tile boundaries while the compute side runs
//   separate tile and k loops.  Tile ids are remapped so that the tiles the
//   hardware places on one XCD at the same time are neighbours (shared L2).
//
// * Epilogue (same page, "Pseudo-code": convert fp32 to bf16, registers to
//   shared memory, store).  Accumulators are converted with round-to-nearest-
//   even, written to a wave-private LDS strip, read back as whole 128-byte row
//   segments and stored with 16-byte buffer stores; being wave-private, the
//   strip needs no block-wide sync.
//
// * Split k range and split tail (not sections of the pages, whose persistent
//   schedule assumes enough output tiles).  Shapes with few output tiles, and
//   the last few tiles of a mostly empty last round, run as k chunks; each
//   chunk's fp32 partial tile is stored in register order and a reduction
//   kernel adds the chunks in chunk order, then rounds once.
//
// * Counter initialisation happens before any wave can arrive on a counter
//   ("[Tutorial] Fix race condition in 2SM TMEM alloc ...", sections
//   "Problem" and "Fix"): counters are zeroed, then one workgroup barrier,
//   then the first arrive or poll.  Every counter wait is bounded: a wait that
//   gives up is counted (gemm_bf16_sync_timeouts), marks its workgroup, and
//   the wave finishes its loops instead of hanging; the workgroup then writes
//   every output tile its reads may have corrupted as NaN.
//
// Edges: buffer resources range-check every load and store.  Rows past M or
// N, and the k tail of the last k-step, are read as zeros (the lane's offset is
// pushed past the resource); stores past M or N are dropped the same way.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <type_traits>
#include <utility>
#include <vector>

#include "gemm_bf16.h"

namespace {

#define LDS_AS __attribute__((address_space(3)))
typedef LDS_AS char lds_char;
typedef LDS_AS uint32_t lds_u32;
typedef LDS_AS uint64_t lds_u64;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) short i16x4_t;
typedef __attribute__((ext_vector_type(8))) short i16x8_t;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2_t;

// A byte offset no resource covers: loads there return zeros, stores vanish.
constexpr uint32_t kOOB = 0x80000000u;
// Cache policies of buffer stores: the default, and non-temporal (the nt bit).
constexpr int kStoreDefault = 0;
constexpr int kStoreNonTemporal = 2;
constexpr uint32_t kMaxRecords = 0x7FFFFFF0u;
// Raw buffer resource, 32-bit data format (third descriptor word for gfx9).
constexpr int kRsrcWord3 = 0x00020000;
// Bounded spin on ring counters: ~0.3 s at s_sleep(1) per poll (the default;
// gemm_bf16_set_sync_spin_limit changes it for later launches).
constexpr uint32_t kSpinLimit = 1u << 22;

__device__ unsigned long long g_sync_timeouts;

// Sums of the kernels' clock samples (clock_begin / clock_end): per slot,
// shader-clock ticks, constant-rate ticks, samples.  Workgroup b adds to slot
// b mod kClockSlots; each slot has a 128-byte line of its own, so the atomics
// of one launch's workgroups do not queue on one address (same-address
// device-wide atomics from all XCDs cost several percent of a 100 us call).
constexpr int kClockSlots = 256;
__device__ __align__(128) unsigned long long g_clock_sums[kClockSlots][16];

// s_waitcnt immediates (gfx9 layout: vmcnt[3:0] + [15:14], expcnt[6:4],
// lgkmcnt[11:8]); counters not named are left at their maximum.
constexpr int waitcnt_vm(int n) { return (n & 0xF) | (((n >> 4) & 3) << 14) | (0x7 << 4) | (0xF << 8); }
constexpr int kWaitLgkm0 = 0xF | (0x3 << 14) | (0x7 << 4);

#define COMPILER_FENCE() asm volatile("" ::: "memory")

// A value the optimiser must treat as unknown at this point.  Used inside
// loops for per-lane address bases, so that the many addresses derived from
// them are recomputed (a VALU op or two) instead of being hoisted out of the
// tile loop and kept live next to 256 accumulator registers.
__device__ __forceinline__ uint32_t opaque(uint32_t x)
{
    asm volatile("" : "+v"(x));
    return x;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes)
{
    uint32_t n = bytes <= 0 ? 0u : (bytes > (int64_t)kMaxRecords ? kMaxRecords : (uint32_t)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, kRsrcWord3);
}

// Byte count for a resource that starts `rem` bytes (rem > 0) before the end
// of its operand.  Counts of 2^31 and more are capped at kMaxRecords; the cap
// never cuts off an access the kernel makes, whose offsets stay below
// 2^31 - 2^23 (leading dimensions are at most 2^22 elements).
__device__ __forceinline__ uint32_t records(uint64_t rem)
{
    return (rem >> 31) ? kMaxRecords : (uint32_t)rem;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_n(const void* base, uint32_t nrec)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nrec, kRsrcWord3);
}

// One 16-byte-per-lane global-to-LDS load at byte offset voff + soff of the
// resource.  The hardware range check counts both offsets: a lane whose 16
// bytes start at or past the resource's byte count writes zeros.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, lds_char* dst, uint32_t voff, uint32_t soff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LDS_AS void*)dst, 16, voff, (int)soff, 0, 0);
}

enum {
    SYNC_BARRIER = GEMM_SYNC_BARRIER,
    SYNC_FLAGS = GEMM_SYNC_FLAGS,
    SYNC_WAVESPEC = GEMM_SYNC_WAVESPEC,
    SYNC_PINGPONG = GEMM_SYNC_PINGPONG
};

// ---------------------------------------------------------------------------
// Compile-time configuration of one kernel instance.
// ---------------------------------------------------------------------------
template <int BM_, int BN_, int BK_, int S_, int WM_, int WN_, int SYNC_, bool BT_, int NP_, bool WIN_ = false,
          int MF_ = 32, bool DUAL_ = false, int SPREAD_ = 0>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, S = S_, WM = WM_, WN = WN_;
    static constexpr int SYNC = SYNC_;
    static constexpr bool BT = BT_;                 // B stored N x K
    // Split-window ring: the LDS holds NWIN windows of one operand tile each
    // (a position's A tile and its B tile occupy two windows), instead of S
    // whole stages; the epilogue stages through a drained window.
    static constexpr bool WIN = WIN_;
    static constexpr int NWIN = WIN ? 5 : 0;
    // Dedicated loader waves in the wave-specialised and ping-pong modes.
    static constexpr bool PRODUCERS = SYNC == SYNC_WAVESPEC || SYNC == SYNC_PINGPONG;
    static constexpr int GROUPS = (SYNC == SYNC_PINGPONG) ? 2 : 1; // MFMA wave groups taking tiles in turn
    static constexpr int NCWG = WM * WN;            // MFMA waves per group: one output tile
    static constexpr int NCW = GROUPS * NCWG;       // MFMA waves
    static constexpr int NP = PRODUCERS ? NP_ : 0;  // dedicated loader waves
    // Ping-pong with one pipeline per MFMA group: each group has its own
    // ring of S stages, its own counters and NP / GROUPS loader waves.
    static constexpr bool DUAL = DUAL_;
    static constexpr int PIPES = DUAL ? GROUPS : 1;
    static constexpr int NLW = PRODUCERS ? NP / PIPES : NCW; // waves that load one position
    static constexpr int NW = NCW + NP;
    static constexpr int THREADS = NW * 64;
    // Cache policy of the stores of C.  C is written once and never read back
    // by the GEMM, and each XCD writes as much C per round of output tiles as
    // its L2 holds; stored normally those lines displace operand lines that
    // the XCD's other workgroups are still reading, so C goes out
    // non-temporal (measured +1-6% on the barrier and flag kernels, level on
    // the wave-specialised ones).  Ping-pong over one shared ring, where one
    // group's epilogue runs beside the other group's main loop, measured
    // 3-5% slower with it and keeps the default.  Operand loads keep the
    // default policy (non-temporal loads lost 10-40%: their lines are reused
    // across the XCD's workgroups within a few k-steps), and so do fp32
    // partial tiles, which the reduction reads right back.
    static constexpr int STORE_C = (SYNC == SYNC_PINGPONG && !DUAL) ? kStoreDefault : kStoreNonTemporal;
    static constexpr int TM = BM / WM, TN = BN / WN;                 // wave tile
    // MFMA block edge.  32: v_mfma_f32_32x32x16_bf16, one 16-wide k-step per
    // MFMA region.  16: v_mfma_f32_16x16x32_bf16, whose 32-wide k-step takes
    // two regions, each over half of the wave's block rows.  At equal LDS
    // bytes per FLOP the 16 x 16 form moves half the accumulator register
    // traffic per FLOP and sustains a higher clock under the power limit.
    static constexpr int MF = MF_;
    using Acc = std::conditional_t<MF == 16, f32x4_t, f32x16_t>;
    static constexpr int FM = TM / MF, FN = TN / MF;                 // MFMA blocks per wave
    static constexpr int KK = BK / 16;                               // MFMA regions (16 k each) per stage
    static constexpr int A_BYTES = BM * BK * 2;
    static constexpr int B_BYTES = BN * BK * 2;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    static constexpr int A_LOADS = A_BYTES / 1024 / NLW;            // 1 KiB DMA instructions per loading wave
    static constexpr int B_LOADS = B_BYTES / 1024 / NLW;
    static constexpr int LOADS = A_LOADS + B_LOADS;
    static constexpr int CPR_K = BK / 8;                             // 16-byte chunks per K-contiguous row
    static constexpr int CPR_N = BN / 8;                             // chunks per row of a K x N B tile
    static constexpr int RING_BYTES = WIN ? NWIN * A_BYTES : PIPES * S * STAGE_BYTES;
    // Ring counters (2 x S 32-bit words, or S 64-bit signal words) and the
    // workgroup's poison word (SyncState), padded to 8 bytes.
    static constexpr int FLAG_BYTES = (SYNC != SYNC_BARRIER) ? PIPES * 2 * S * 4 + 8 : 0;
    // Epilogue strip per MFMA wave: 32 rows x 64 columns of bf16 when that
    // fits next to the ring (or, with windows, inside one window).  Else,
    // with 16 x 16 blocks, 16 rows x 64 columns: the same bytes as 32 x 32,
    // but every row the strip hands to the stores is a whole 128-byte line
    // of C (64-byte rows wrote 35-40% more bytes to HBM than C holds, and
    // slowed the epilogue where all workgroups store at once); with 32 x 32
    // blocks, 32 rows x 32 columns.
    static constexpr bool EPI_FULL =
        WIN ? NCW * 32 * 64 * 2 <= A_BYTES : RING_BYTES + NCW * 32 * 64 * 2 + FLAG_BYTES <= 160 * 1024;
    static constexpr int EPI_W = (EPI_FULL || MF_ == 16) ? 64 : 32;
    static constexpr int EPI_H = (EPI_FULL || MF_ != 16) ? 32 : 16;
    static constexpr int EPI_WAVE_BYTES = EPI_H * EPI_W * 2;
    static constexpr int EPI_OFFSET = RING_BYTES;
    static constexpr int FLAG_OFFSET = WIN ? RING_BYTES : EPI_OFFSET + NCW * EPI_WAVE_BYTES;
    static constexpr int LDS_BYTES = FLAG_OFFSET + FLAG_BYTES;
    // Where the all-wave kernel steps its load cursor: inside the second MFMA
    // region of a k-step when there are three or more regions, else after
    // the k-step (one position further ahead).  The branch-free cursor needs
    // at least this many k-steps per tile.
    static constexpr bool PREP_IN_REGION = KK >= 3;
    static constexpr int LONGK_MIN_KT = WIN ? 3 : S + (PREP_IN_REGION ? 1 : 2);
    // Loader waves: s_sleep argument (units of 64 cycles) between pairs of
    // a position's DMA instructions, 0 for one burst.  When every workgroup
    // of an XCD issues the same panel slice at the same moment, their
    // requests for a line reach the L2 while its first miss is still
    // outstanding, and each of them misses and fetches the line again;
    // spread over part of the position's compute time, the later requests
    // find it.  Chosen per configuration by measurement (Pick below).
    static constexpr int SPREAD_SLEEP = PRODUCERS ? SPREAD_ : 0;

    static_assert(BK == 32 || BK == 64, "BK");
    static_assert(KK % 2 == 0, "fragment double buffering assumes an even number of MFMA k-steps");
    static_assert(FM >= 1 && FN >= 2 && FN % 2 == 0, "wave tile");
    static_assert(MF == 32 || (MF == 16 && FM % 2 == 0 && (BK == 64 || !PRODUCERS)),
                  "16 x 16 blocks: 64-wide stages, or 32-wide stages in the all-wave kernels");
    static_assert(A_BYTES % (1024 * NLW) == 0 && B_BYTES % (1024 * NLW) == 0, "DMA split");
    static_assert(64 % CPR_K == 0, "a DMA window covers whole K-contiguous rows");
    static_assert(CPR_N == 16 || CPR_N == 32, "a DMA window covers whole K x N rows of B");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
    static_assert(S >= 2 && S <= 4, "stages");
    static_assert(SPREAD_ >= 0 && SPREAD_ <= 8 && (SPREAD_ == 0 || PRODUCERS), "loader spread");
    static_assert(!DUAL || (SYNC == SYNC_PINGPONG && NP % GROUPS == 0), "one pipeline per ping-pong group");
    static_assert(!WIN || (SYNC == SYNC_BARRIER && S == 2 && KK == 4 && A_BYTES == B_BYTES &&
                           NCW * EPI_WAVE_BYTES <= A_BYTES),
                  "the window ring runs the barrier kernel on equal A and B tiles");
};

// A work item is one output tile and one chunk of the k range.  Without a
// split (splits == 1) the chunk is all of K and work items are output tiles.
// A launch covers the `span` output tiles that start at raster position
// `tile_base`: all tiles, or, for a split tail, the last few.
struct Params {
    const char* A;
    const char* B;
    char* C;
    float* partial;                   // fp32 partial tiles, splits > 1 only
    int64_t M, N, K, lda, ldb, ldc;   // elements
    int64_t ksplit;                   // k elements per chunk (K when splits == 1)
    int32_t tiles_m, tiles_n, tiles_mn, splits;
    int32_t tiles;                    // work items of this launch: span * splits
    int32_t span, tile_base;          // the launch's output tiles: raster positions tile_base .. + span - 1
    int32_t k_steps;                  // k-steps per work item
    int32_t group_m;
    int32_t small_span;               // A and B each span fewer than kMaxRecords bytes
    uint32_t spin_limit;              // polls before a ring counter wait gives up
    uint32_t clock_on;                // nonzero: workgroups add clock samples to g_clock_sums
};

// Optional clock sampling.  With p.clock_on set, thread 0 of every workgroup
// that has work adds its elapsed shader-clock ticks (s_memtime), its elapsed
// constant-rate ticks (s_memrealtime) and a count of one to its slot of
// g_clock_sums.
// The ratio of the two sums times the constant rate is the clock the kernels
// ran at, measured without a profiler (whose counter passes change the power
// state).  Nothing stays live in between: the start subtracts its stamps from
// the sums and the end adds its own (unsigned sums wrap, so they hold the sum
// of the elapsed ticks once every workgroup has ended).  Wave 0, which takes
// the samples, is an MFMA wave in every kernel.
__device__ __forceinline__ void clock_begin(const Params& p)
{
    if (p.clock_on && threadIdx.x == 0) {
        const uint64_t c = __builtin_amdgcn_s_memtime(), r = __builtin_amdgcn_s_memrealtime();
        unsigned long long* slot = g_clock_sums[blockIdx.x % kClockSlots];
        atomicAdd(&slot[0], (unsigned long long)(0 - c));
        atomicAdd(&slot[1], (unsigned long long)(0 - r));
    }
}

__device__ __forceinline__ void clock_end(const Params& p)
{
    if (p.clock_on && threadIdx.x == 0) {
        const uint64_t c = __builtin_amdgcn_s_memtime(), r = __builtin_amdgcn_s_memrealtime();
        unsigned long long* slot = g_clock_sums[blockIdx.x % kClockSlots];
        atomicAdd(&slot[0], (unsigned long long)c);
        atomicAdd(&slot[1], (unsigned long long)r);
        atomicAdd(&slot[2], 1ull);
    }
}

// Swizzles.  The LDS has 64 four-byte banks (256 bytes per cycle); a 16-byte
// read is served 16 lanes at a time, an 8-byte read 32 lanes at a time.
//
// K-contiguous tiles (A, and B stored N x K) hold rows of BK elements.  A
// fragment read has lanes 0..15 on 16 consecutive rows at one logical chunk;
// those rows span 8 (BK = 64, 128-byte rows) or 4 (BK = 32, 64-byte rows)
// bank windows, so XORing the chunk with (row / 2) mod 8, respectively
// (row / 4) mod 4, puts the 16 lanes on 16 different 16-byte bank groups.
template <int BK>
__device__ __forceinline__ int swz_k(int row)
{
    return BK == 64 ? ((row >> 1) & 7) : ((row >> 2) & 3);
}

// K-contiguous tiles with 32-wide k-steps read by 16 x 16 x 32 MFMAs.  A
// fragment read then covers one 16-row x 64-byte block (1 KiB, the span of one
// DMA instruction): lane l (bits l5..l0) takes row r = l % 16 and chunk
// h = l / 16.  With 64-byte rows the bank window of a row is set by the row's
// place in the block, so XORing the chunk alone left 2-way conflicts under
// the LDS's grouping of lanes into cycles (measured: half of all LDS cycles
// were conflict stalls, with or without the DMA running; the 64-wide swizzle
// above measures conflict-free).  So the rows of each block are permuted as
// well: row r (bits r3..r0) goes to the 64-byte segment
//     seg(r) = (r2, r1, r3, r0)
// and its chunk h to position h ^ (r2, r1) in the segment.  The bank slot of
// a read is then (r3, r0, h1 ^ r2, h0 ^ r1), which spreads the lanes of every
// cycle over distinct slots for every grouping of lanes under which the
// 64-wide swizzle is conflict-free.  A row keeps its 4 chunks in one 64-byte
// segment, so each DMA instruction still fetches whole 64-byte row pieces.
__device__ __forceinline__ int kperm_seg(int r)
{
    return (r & 1) | (((r >> 3) & 1) << 1) | (((r >> 1) & 1) << 2) | (((r >> 2) & 1) << 3);
}

// Inverse of kperm_seg: the row held in segment k.
__device__ __forceinline__ int kperm_row(int k)
{
    return (k & 1) | (((k >> 2) & 1) << 1) | (((k >> 3) & 1) << 2) | (((k >> 1) & 1) << 3);
}

// The 16-byte slot, within its block, of reading lane l's (row, chunk).
__device__ __forceinline__ int kperm_slot(int l)
{
    const int r = l & 15;
    return kperm_seg(r) * 4 + ((l >> 4) ^ ((r >> 1) & 3));
}

// K x N tiles of B hold rows of BN elements (512 or 256 bytes, so every row
// starts on the same bank).  With 32 x 32 blocks a transposing read has lanes
// 0..31 on 4 consecutive k-rows x 4 chunks; XORing chunk bits 2-3 with
// (k mod 4) spreads the 16 (row, chunk) pairs over all 16 bank groups.  With
// 16 x 16 blocks lanes 0..31 cover k-rows r and r + 8 (r = 0..3) x 2 chunks,
// so chunk bit 1 is also XORed with k-row bit 3.
template <int MF>
__device__ __forceinline__ int swz_n(int krow)
{
    return MF == 16 ? (((krow & 3) << 2) | (((krow >> 3) & 1) << 1)) : ((krow & 3) << 2);
}

// Output tile at raster position Lt (0 <= Lt < tiles_mn): a grouped raster,
// runs of group_m tile rows walked column by column, so a run of consecutive
// positions covers a compact block of output tiles.
__device__ __forceinline__ void raster_tile(const Params& p, int32_t Lt, int32_t& tm, int32_t& tn)
{
    const int32_t per_group = p.group_m * p.tiles_n;
    const int32_t grp = Lt / per_group;
    const int32_t first_m = grp * p.group_m;
    const int32_t gm = min(p.tiles_m - first_m, p.group_m);
    const int32_t in = Lt - grp * per_group;
    const int32_t col = in / gm;
    tm = first_m + (in - col * gm);
    tn = col;
}

// Output tile (tm, tn), k chunk sp and the tile's index u within the launch's
// span, of work item t, for a grid of G persistent workgroups (workgroup b
// takes ids b, b + G, b + 2G, ...).  Branch-free scalar code.
__device__ __forceinline__ void tile_coords(const Params& p, int32_t t, int32_t G, int32_t& tm, int32_t& tn,
                                            int32_t& sp, int32_t& u)
{
    // The hardware deals workgroups to the 8 XCDs round-robin; within every
    // full round of G ids, give XCD x a contiguous run of G/8 ids.
    const int32_t round = t / G;
    const int32_t b = t - round * G;
    const int32_t remapped = round * G + (b & 7) * (G >> 3) + (b >> 3);
    const int32_t L = ((G & 7) == 0 && (round + 1) * G <= p.tiles) ? remapped : t;
    // Chunk-major: consecutive ids share a k chunk and walk the raster.
    sp = L / p.span;
    u = L - sp * p.span;
    raster_tile(p, p.tile_base + u, tm, tn);
}

// The ring counters live in their own LDS words, apart from every stage.  Their
// loads and atomic adds are written as inline assembly: issued as ordinary
// LDS operations, the compiler's wait-count insertion cannot tell them apart
// from the stages that in-flight global-to-LDS DMAs write, and waits for all
// of the wave's outstanding loads before each one, which drains the ring.
__device__ __forceinline__ uint32_t lds_addr(const lds_u32* p)
{
    return (uint32_t)(uintptr_t)p;
}

// The counter's current value (all lanes read the same word); the read is
// complete when this returns.
__device__ __forceinline__ uint32_t load_counter(const lds_u32* ctr)
{
    uint32_t v;
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_addr(ctr)) : "memory");
    return __builtin_amdgcn_readfirstlane(v);
}

// A wave's state for the bounded waits on ring counters.  A wait that gives
// up (after `limit` unsuccessful polls) is counted in g_sync_timeouts, sets
// the wave's sticky `failed` flag -- once set, later waits return at once, so
// the wave runs its finite loops to the end without blocking and the kernel
// always terminates -- and sets the workgroup's poison word in LDS, waiting
// until that write has landed.  Only after that can the wave go on to refill
// a stage early or read one before its data landed, so any wave of the
// workgroup that reads data corrupted by the failure reads it after the
// poison word was set; every wave checks the word before it stores a tile
// (poison_tile) and then writes NaN instead of values.  A workgroup's tiles
// stored before the failure are correct; other workgroups are unaffected.
struct SyncState {
    bool failed = false;
    lds_u32* poison = nullptr;   // one 32-bit LDS word per workgroup, zeroed before the first wait
    uint32_t limit = kSpinLimit;
};

__device__ __forceinline__ void give_up(SyncState& st)
{
    if ((threadIdx.x & 63) == 0) {
        atomicAdd(&g_sync_timeouts, 1ull);
        asm volatile("ds_write_b32 %0, %1" ::"v"(lds_addr(st.poison)), "v"(1u) : "memory");
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    st.failed = true;
}

// Bounded wait until *ctr >= target.
__device__ __forceinline__ void wait_counter(const lds_u32* ctr, uint32_t target, SyncState& st)
{
    uint32_t spins = 0;
    while (!st.failed && load_counter(ctr) < target) {
        if (++spins > st.limit)
            give_up(st);
        // The first polls go back to back (one LDS round trip each); a wait
        // that lasts longer sleeps between polls.
        if (spins > 8)
            __builtin_amdgcn_s_sleep(1);
    }
    COMPILER_FENCE();
}

// The all-wave FLAGS kernel packs two signals into one 64-bit word per stage s:
// the low half counts announcements of the position held in stage s ("full",
// RAW), the high half counts releases of the position held in the stage
// before it, s - 1 mod S ("empty", WAR).  Each wave moves from position c to
// c + 1 by releasing c and announcing c + 1 in one atomic add, and one read
// checks both signals.  Neither half carries into the other: each counts what
// a separate 32-bit counter would, NW per use of a stage, which stays far
// below 2^32 for every launch the host accepts.
constexpr uint64_t kAnnounce = 1ull;
constexpr uint64_t kRelease = 1ull << 32;

__device__ __forceinline__ uint32_t lds_addr(const lds_u64* p)
{
    return (uint32_t)(uintptr_t)p;
}

__device__ __forceinline__ void arrive_pair(lds_u64* word, uint64_t inc)
{
    COMPILER_FENCE();
    if ((threadIdx.x & 63) == 0)
        asm volatile("ds_add_u64 %0, %1" ::"v"(lds_addr(word)), "v"(inc) : "memory");
    COMPILER_FENCE();
}

// The read goes out now; wait_pair_issued, called after unrelated work,
// completes it and polls again until both halves reach their targets.
__device__ __forceinline__ uint64_t pair_read_issue(const lds_u64* word)
{
    uint64_t v;
    asm volatile("ds_read_b64 %0, %1" : "=v"(v) : "v"(lds_addr(word)) : "memory");
    return v;
}

__device__ __forceinline__ bool pair_reached(uint64_t v, uint32_t full_target, uint32_t empty_target)
{
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return lo >= full_target && hi >= empty_target;
}

// Bounded like wait_counter.
__device__ __forceinline__ void wait_pair(const lds_u64* word, uint32_t full_target, uint32_t empty_target,
                                          SyncState& st)
{
    uint32_t spins = 0;
    for (;;) {
        uint64_t v;
        asm volatile("ds_read_b64 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_addr(word)) : "memory");
        if (st.failed || pair_reached(v, full_target, empty_target))
            break;
        if (++spins > st.limit)
            give_up(st);
        if (spins > 8)
            __builtin_amdgcn_s_sleep(1);
    }
    COMPILER_FENCE();
}

// Completes a read from pair_read_issue; polls on only if it came back short.
__device__ __forceinline__ void wait_pair_issued(uint64_t v, const lds_u64* word, uint32_t full_target,
                                                 uint32_t empty_target, SyncState& st)
{
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(v) : : "memory");
    if (!pair_reached(v, full_target, empty_target))
        wait_pair(word, full_target, empty_target, st);
    COMPILER_FENCE();
}

// A poll split in two: the read goes out now; wait_counter_issued, called
// after unrelated work, completes it and falls back to wait_counter if the
// value is still short of the target.
__device__ __forceinline__ uint32_t counter_read_issue(const lds_u32* ctr)
{
    uint32_t v;
    asm volatile("ds_read_b32 %0, %1" : "=v"(v) : "v"(lds_addr(ctr)) : "memory");
    return v;
}

__device__ __forceinline__ void wait_counter_issued(uint32_t v, const lds_u32* ctr, uint32_t target, SyncState& st)
{
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(v) : : "memory");
    if ((uint32_t)__builtin_amdgcn_readfirstlane(v) < target)
        wait_counter(ctr, target, st);
    COMPILER_FENCE();
}

// wait_counter for a wait that usually lasts long (a ping-pong group waiting
// through the other group's tile): after the first polls it sleeps longer,
// so a waiting wave takes fewer issue slots from the waves computing on its
// SIMD.  Still bounded: st.limit polls of at most 512 cycles' sleep.
__device__ __forceinline__ void wait_counter_long(const lds_u32* ctr, uint32_t target, SyncState& st)
{
    uint32_t spins = 0;
    while (!st.failed && load_counter(ctr) < target) {
        if (++spins > st.limit)
            give_up(st);
        if (spins > 64)
            __builtin_amdgcn_s_sleep(8);
        else if (spins > 8)
            __builtin_amdgcn_s_sleep(1);
    }
    COMPILER_FENCE();
}

// One arrival (lane 0 adds 1).
__device__ __forceinline__ void arrive(lds_u32* ctr)
{
    COMPILER_FENCE();
    if ((threadIdx.x & 63) == 0)
        asm volatile("ds_add_u32 %0, %1" ::"v"(lds_addr(ctr)), "v"(1u) : "memory");
    COMPILER_FENCE();
}

__device__ __forceinline__ void block_barrier()
{
    COMPILER_FENCE();
    __builtin_amdgcn_s_barrier();
    COMPILER_FENCE();
}

template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    COMPILER_FENCE();
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(N));
    COMPILER_FENCE();
}

__device__ __forceinline__ void wait_lgkm0()
{
    COMPILER_FENCE();
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    COMPILER_FENCE();
}

// ---------------------------------------------------------------------------
// Load side: one loading wave's share of the (tile, k-step) stream.
//
// Slot s of an operand's stage region (16 bytes; s = (t*NLW + lw)*64 + lane
// for the wave's t-th 1 KiB DMA instruction) holds row s / CPR and physical
// chunk s % CPR; the lane fetches the logical chunk that the swizzle places
// there.  These per-lane byte offsets do not depend on the tile, so they are
// computed once.  Per position only scalar values move.  A resource's byte
// count ends at the last element of the operand, so rows past M (A), past N
// (B stored N x K) and k-rows past K (B stored K x N) read as zeros by
// themselves.  The two edges a byte count cannot express -- the k tail inside
// a row, and columns past N of a K x N B tile -- are masked per lane with a
// select.
//
// Every call emits exactly LOADS DMA instructions, also for a position past the
// end of the stream (it gets resources of zero bytes, so it writes zeros and
// touches no memory).  That keeps the vector-memory counter arithmetic of the
// waits exact.
//
// Two cursors.  The stepping cursor (LONGK: at least LONGK_MIN_KT k-steps per
// tile, and each operand spanning less than kMaxRecords bytes) keeps both
// resources at the tile origin for the whole tile and moves through the k
// range with the loads' scalar offset, which the range check counts as well:
// a step is three scalar adds.  The compute loop computes the next tile's
// resources once per tile (prefetch_next_tile) and switches the cursor to
// them at a fixed k-step (enter_next_tile, a uniform branch at the top of the
// k-step), so the scheduled MFMA regions stay free of branches.  A tile past
// the end gets resources of zero bytes.  The other cursor rebuilds the
// resources at every position from its origin and enters a new tile itself
// (a uniform branch); it serves short k ranges, where the cursor can cross
// several tiles during one compute tile, and operands of 2 GiB or more.
// ---------------------------------------------------------------------------
// First DMA instruction of part `part` when a wave's `loads` instructions
// for one position are cut into `nparts` contiguous runs.
constexpr int part_begin(int part, int nparts, int loads) { return part * loads / nparts; }

// EDGE: the loads mask the k tail inside a row and the columns past N of a
// K x N B tile per lane.  Without EDGE every position is whole (K a multiple
// of BK, and N of BN for a K x N B), so there is nothing to mask.
template <class C, bool LONGK, bool EDGE = true>
struct Loader {
    int32_t total;                // positions in this workgroup's stream
    int32_t n_tiles;
    int32_t t_first = 0, t_stride = 1;   // the stream's tiles: t_first + t * t_stride
    uint32_t voffA[C::A_LOADS];
    uint32_t voffB[C::B_LOADS];
    // One past the last byte of A and of B.  Each operand's resource runs from
    // the position's origin to here, which excludes rows past M (A), rows past
    // N (B stored N x K) and k-rows past K (B stored K x N).
    const char* a_end;
    const char* b_end;

    __device__ __forceinline__ static int slot(int t, int lw, int lane) { return (t * C::NLW + lw) * 64 + lane; }
    // K-contiguous tiles with 32-wide k-steps and 16 x 16 blocks permute the
    // rows of each 1 KiB block as well as their chunks (kperm_seg); otherwise
    // rows stay in place and only the chunk is swizzled.
    static constexpr bool KPERM = C::MF == 16 && C::BK == 32;
    // Logical row (within the tile) of a K-contiguous slot.
    __device__ __forceinline__ static int krow(int s)
    {
        if constexpr (KPERM)
            return (s >> 6) * 16 + kperm_row((s & 63) >> 2);
        else
            return s / C::CPR_K;
    }
    // Logical k offset (elements) of a K-contiguous slot.
    __device__ __forceinline__ static int kofs_k(int s)
    {
        if constexpr (KPERM)
            return ((s & 3) ^ (((s & 63) >> 4) & 3)) * 8;
        else
            return ((s % C::CPR_K) ^ swz_k<C::BK>(s / C::CPR_K)) * 8;
    }
    // Logical column offset (elements) of a slot in a K x N tile of B.
    __device__ __forceinline__ static int nofs_n(int s)
    {
        const int row = s / C::CPR_N;
        return ((s % C::CPR_N) ^ swz_n<C::MF>(row)) * 8;
    }

    __device__ __forceinline__ void init(const Params& p, int32_t ntiles, int lw, int lane, int32_t first = 0,
                                         int32_t stride = 1)
    {
        t_first = first;
        t_stride = stride;
        const uint32_t lda2 = (uint32_t)p.lda * 2u, ldb2 = (uint32_t)p.ldb * 2u;
#pragma unroll
        for (int t = 0; t < C::A_LOADS; ++t) {
            const int s = slot(t, lw, lane);
            voffA[t] = (uint32_t)krow(s) * lda2 + (uint32_t)kofs_k(s) * 2u;
        }
#pragma unroll
        for (int t = 0; t < C::B_LOADS; ++t) {
            const int s = slot(t, lw, lane);
            if constexpr (C::BT)
                voffB[t] = (uint32_t)krow(s) * ldb2 + (uint32_t)kofs_k(s) * 2u;
            else
                voffB[t] = (uint32_t)(s / C::CPR_N) * ldb2 + (uint32_t)nofs_n(s) * 2u;
        }
        a_end = p.A + ((p.M - 1) * p.lda + p.K) * 2;
        b_end = C::BT ? p.B + ((p.N - 1) * p.ldb + p.K) * 2 : p.B + ((p.K - 1) * p.ldb + p.N) * 2;
        n_tiles = ntiles;
        total = ntiles * p.k_steps;
        if constexpr (LONGK) {
            bstep = C::BT ? (uint32_t)C::BK * 2u : (uint32_t)C::BK * 2u * (uint32_t)p.ldb;
            cur = tile_prep(p, 0);
            prefetch_next_tile(p, 1);
        } else {
            q = 0;
            kt = 0;
            ti = 0;
            tile_origin(p, 0, pa, pb, nrem, krem);
        }
    }

    // Origin of the workgroup's t-th work item: its tile at the first k of
    // its chunk (t is clamped to the last item; positions past the end are
    // never read), and the n and k extents left from there for the masks.
    __device__ __forceinline__ void tile_origin(const Params& p, int32_t t, const char*& a, const char*& b,
                                                int32_t& n_left, int32_t& k_left) const
    {
        int32_t tm = 0, tn = 0, sp = 0, u = 0;
        tile_coords(p, (int32_t)blockIdx.x + (t_first + min(t, n_tiles - 1) * t_stride) * (int32_t)gridDim.x,
                    (int32_t)gridDim.x, tm, tn, sp, u);
        const int64_t m0 = (int64_t)tm * C::BM, n0 = (int64_t)tn * C::BN, k0 = (int64_t)sp * p.ksplit;
        a = p.A + (m0 * p.lda + k0) * 2;
        b = C::BT ? p.B + (n0 * p.ldb + k0) * 2 : p.B + (k0 * p.ldb + n0) * 2;
        n_left = (int32_t)(p.N - n0);
        k_left = (int32_t)(p.K - k0);
    }

    // Scalar part of issuing one position: the two buffer resources, the
    // scalar offsets of the position within them, and the remaining k / n
    // extents used by the edge masks.
    struct Prep {
        __amdgpu_buffer_rsrc_t ra, rb;
        int32_t krem, nrem;
        uint32_t soa, sob;
    };

    // Stepping cursor: the resources of the workgroup's t-th work item at its
    // origin, or of zero bytes for t >= n_tiles.  Each operand spans less than
    // kMaxRecords bytes, so the byte counts are exact.
    __device__ __forceinline__ Prep tile_prep(const Params& p, int32_t t) const
    {
        const char* a;
        const char* b;
        Prep r;
        tile_origin(p, t, a, b, r.nrem, r.krem);
        const bool live = t < n_tiles;
        r.ra = rsrc_n(a, live ? (uint32_t)(a_end - a) : 0u);
        r.rb = rsrc_n(b, live ? (uint32_t)(b_end - b) : 0u);
        r.soa = 0;
        r.sob = 0;
        return r;
    }

    // Stepping cursor: the resources of the tile the cursor enters next.
    // Called at the start of compute tile t with t + 1; enter_next_tile then
    // switches to them inside compute tile t.
    __device__ __forceinline__ void prefetch_next_tile(const Params& p, int32_t t)
    {
        nxt = tile_prep(p, t);
    }

    // Stepping cursor: move onto the prefetched tile's origin.  The compute
    // loop calls this at the top of the k-step whose preparation is the first
    // position of the next tile.
    __device__ __forceinline__ void enter_next_tile() { cur = nxt; }

    // Stepping cursor: the current position and the next tile's origin, and
    // the scalar-offset step of B per k-step.
    Prep cur, nxt;
    uint32_t bstep;

    // Rebuilding cursor: position q, k-step kt within its tile, the operand
    // origins at that position, and the k / n extents left for the edge masks.
    int32_t q, kt, ti;
    int32_t krem, nrem;
    const char* pa;
    const char* pb;

    // The cursor's position prepared for issue, then the cursor steps on.
    // Positions at or past the end of the stream get empty resources.
    __device__ __forceinline__ Prep prepare_and_advance(const Params& p)
    {
        constexpr uint32_t kstep = (uint32_t)C::BK * 2u;
        if constexpr (LONGK) {
            const Prep r = cur;
            cur.soa += kstep;
            cur.sob += bstep;
            cur.krem -= C::BK;
            return r;
        } else {
            const bool live = q < total;
            Prep r;
            r.krem = krem;
            r.nrem = nrem;
            r.ra = rsrc_n(pa, live ? records((uint64_t)(a_end - pa)) : 0u);
            r.rb = rsrc_n(pb, live ? records((uint64_t)(b_end - pb)) : 0u);
            r.soa = 0;
            r.sob = 0;
            ++q;
            if (++kt == p.k_steps) {
                kt = 0;
                tile_origin(p, ++ti, pa, pb, nrem, krem);
            } else {
                krem -= C::BK;
                pa += kstep;
                pb += C::BT ? (int64_t)kstep : (int64_t)kstep * p.ldb;
            }
            return r;
        }
    }

    // DMA instruction t (0 <= t < LOADS; A first, then B) of this wave for a
    // prepared position, into the A tile at a_tile or the B tile at b_tile.
    __device__ __forceinline__ void fire_one(const Prep& r, int t, lds_char* a_tile, lds_char* b_tile, int lw,
                                             int lane) const
    {
        if (t < C::A_LOADS) {
            const bool ok = !EDGE || kofs_k(slot(t, lw, lane)) < r.krem;
            lds_dma16(r.ra, a_tile + (t * C::NLW + lw) * 1024, ok ? voffA[t] : kOOB, r.soa);
        } else {
            const int tb = t - C::A_LOADS;
            const int s = slot(tb, lw, lane);
            const bool ok = !EDGE || (C::BT ? (kofs_k(s) < r.krem) : (nofs_n(s) < r.nrem));
            lds_dma16(r.rb, b_tile + (tb * C::NLW + lw) * 1024, ok ? voffB[tb] : kOOB, r.sob);
        }
    }

    // The same into a whole stage (A tile, then B tile).
    __device__ __forceinline__ void fire_one(const Prep& r, int t, lds_char* stage, int lw, int lane) const
    {
        fire_one(r, t, stage, stage + C::A_BYTES, lw, lane);
    }

    // Part `part` of NPARTS of the wave's DMA instructions for a prepared
    // position: the LOADS instructions cut into NPARTS contiguous runs.
    template <int NPARTS>
    __device__ __forceinline__ void fire(const Prep& r, int part, lds_char* stage, int lw, int lane) const
    {
        static_assert(NPARTS >= 1 && NPARTS <= C::LOADS, "parts");
#pragma unroll
        for (int t = 0; t < C::LOADS; ++t)
            if (t >= part_begin(part, NPARTS, C::LOADS) && t < part_begin(part + 1, NPARTS, C::LOADS))
                fire_one(r, t, stage, lw, lane);
    }

    // Issue all of this wave's DMA for the cursor's position into `stage`
    // and step the cursor.
    __device__ __forceinline__ void issue_next(const Params& p, lds_char* stage, int lw, int lane)
    {
        fire<1>(prepare_and_advance(p), 0, stage, lw, lane);
    }
};

// ---------------------------------------------------------------------------
// Compute side: fragment reads and the MFMA chain of one MFMA wave.
// ---------------------------------------------------------------------------
template <class C>
struct Frags {
    bf16x8_t a[C::FM];
    bf16x8_t b[C::FN];       // B stored N x K
    i16x4_t bh[C::FN][2];    // B stored K x N: the two transposing reads per block
};

template <class C>
constexpr int frag_reads() { return C::FM + (C::BT ? 1 : 2) * C::FN; }

// The frag_reads<C>() LDS read instructions of MFMA k-step kk, one at a time.
// The MFMA runs with the B fragment as its first operand, so accumulator
// block (i, j) holds C^T: lane l owns column m = l%32 and rows
// n = 8*(r/4) + 4*(l/32) + r%4 (32 x 32 blocks), or column m = l%16 and rows
// n = 4*(l/16) + r (16 x 16 blocks).
//
// 16 x 16 blocks (32-wide k-step kk): lane l reads row (base + 16*i + l%16),
// logical chunk 4*kk + l/16; with B stored K x N, group g = l/16 of a
// transposing read takes k-rows 32*kk + 8*g + 4*hh + r and the chunk of
// column 16*J + 4*q, 2*J + q/2, which the swizzle XORs with 4*r + 2*(g%2):
// it becomes 2*(J ^ (2*r + g%2)) + q/2.  The reads go A block 0, then B,
// then the other A blocks: the first MFMAs of a k-step need A block 0 and
// every B block.
//
// K-contiguous tiles: lane l reads row (base + 32*i + l%32), logical chunk
// 2*kk + l/32.  Every block starts on a multiple of 8 rows, so the swizzle
// term depends on l only and the block index moves the address by a
// constant.
//
// B stored K x N, ds_read_b64_tr_b16: within each 16-lane group, lane 4r+q
// addresses k-row r, columns 4q..4q+3 of a 4 x 16 block; lane i receives
// column i for the 4 k-rows.  Two reads give the 8 k values of the operand.
// The k-row of lane (r, q) is 16*kk + 8*(l/32) + 4*hh + r, so its swizzle
// term is 4*r; the logical chunk of block j is 4*(wn*TN/32 + j) +
// 2*((l>>4)&1) + q/2, and the XOR only touches the 4*(wn*TN/32 + j) part:
// it becomes 4*((wn*TN/32 + j) ^ r).
template <class C>
struct FragReader {
    uint32_t a_off, b_off;
    int r;

    __device__ __forceinline__ FragReader(int wm, int wn, int lane, int kk)
    {
        if constexpr (C::MF == 16) {
            const int h = lane >> 4, r16 = lane & 15;
            // 64-wide k-steps: row r16 in place, chunk swizzled; 32-wide: the
            // lane's (row, chunk) at kperm_slot(lane) of the 1 KiB block.
            const uint32_t in_block = (C::BK == 32) ? (uint32_t)kperm_slot(lane) << 4
                                                     : (uint32_t)(r16 * (C::BK * 2)) +
                                                           (uint32_t)(((4 * kk + h) ^ swz_k<C::BK>(r16)) << 4);
            a_off = opaque((uint32_t)(wm * C::TM * (C::BK * 2)) + in_block);
            if constexpr (C::BT) {
                b_off = opaque((uint32_t)(wn * C::TN * (C::BK * 2)) + in_block);
                r = 0;
            } else {
                const int q = r16 & 3, rr = r16 >> 2;
                r = 2 * rr + (h & 1);
                // With one fragment set per wave (two MFMA waves per SIMD
                // beside loader waves, 168 registers each) the four B block
                // offsets derived from r would stay live through the k-step
                // loop and push it into spills; an opaque r makes them be
                // recomputed (two VALU operations per read) at every k-step.
                if constexpr (C::PRODUCERS && C::NCW == 8)
                    r = (int)opaque((uint32_t)r);
                const uint32_t krow0 = (uint32_t)(32 * kk + 8 * h + rr);
                b_off = opaque(krow0 * (C::BN * 2) + (uint32_t)((q >> 1) * 16 + (q & 1) * 8));
            }
        } else {
            init32(wm, wn, lane, kk);
        }
    }

    // Offsets for 32 x 32 blocks (16-wide k-step kk).
    __device__ __forceinline__ void init32(int wm, int wn, int lane, int kk)
    {
        const int h = lane >> 5;
        const int r32 = lane & 31;
        const uint32_t xk = (uint32_t)(((2 * kk + h) ^ swz_k<C::BK>(r32)) << 4);
        a_off = opaque((uint32_t)((wm * C::TM + r32) * (C::BK * 2)) + xk);
        if constexpr (C::BT) {
            b_off = opaque((uint32_t)((wn * C::TN + r32) * (C::BK * 2)) + xk);
            r = 0;
        } else {
            const int g = lane >> 4, i16 = lane & 15, q = i16 & 3;
            r = i16 >> 2;
            const int low = 2 * (g & 1) + (q >> 1);
            const uint32_t krow0 = (uint32_t)(16 * kk + 8 * (g >> 1) + r);
            b_off = opaque(krow0 * (C::BN * 2) + (uint32_t)(low * 16 + (q & 1) * 8));
        }
    }

    // Read instruction d, from the A tile at a_tile and the B tile at b_tile:
    // with 16 x 16 blocks A block 0, the B reads, then the other A blocks;
    // with 32 x 32 blocks the A blocks, then the B reads (read32).
    __device__ __forceinline__ void read(Frags<C>& f, const lds_char* a_tile, const lds_char* b_tile, int wn,
                                         int d) const
    {
        if constexpr (C::MF == 16) {
            constexpr int NB = (C::BT ? 1 : 2) * C::FN;   // B reads
            if (d == 0 || d > NB) {
                const int i = (d == 0) ? 0 : d - NB;
                f.a[i] = *(const LDS_AS bf16x8_t*)(a_tile + a_off + i * (16 * C::BK * 2));
            } else if constexpr (C::BT) {
                f.b[d - 1] = *(const LDS_AS bf16x8_t*)(b_tile + b_off + (d - 1) * (16 * C::BK * 2));
            } else {
                const int j = (d - 1) >> 1, hh = (d - 1) & 1;
                const int J = wn * C::FN + j;
                const uint32_t jchunk = (uint32_t)(2 * (J ^ r)) * 16u;
                const lds_char* addr = b_tile + b_off + (uint32_t)(4 * hh * (C::BN * 2)) + jchunk;
                f.bh[j][hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4_t*)addr);
            }
        } else {
            read32(f, a_tile, b_tile, wn, d);
        }
    }

    __device__ __forceinline__ void read32(Frags<C>& f, const lds_char* a_tile, const lds_char* b_tile, int wn,
                                           int d) const
    {
        if (d < C::FM) {
            f.a[d] = *(const LDS_AS bf16x8_t*)(a_tile + a_off + d * (32 * C::BK * 2));
        } else if constexpr (C::BT) {
            const int j = d - C::FM;
            f.b[j] = *(const LDS_AS bf16x8_t*)(b_tile + b_off + j * (32 * C::BK * 2));
        } else {
            const int j = (d - C::FM) >> 1, hh = (d - C::FM) & 1;
            const int J = wn * (C::TN / 32) + j;
            const uint32_t jchunk = (uint32_t)(4 * (J ^ r)) * 16u;
            const lds_char* addr = b_tile + b_off + (uint32_t)(4 * hh * (C::BN * 2)) + jchunk;
            f.bh[j][hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4_t*)addr);
        }
    }

    // The same from a whole stage (A tile, then B tile).
    __device__ __forceinline__ void read(Frags<C>& f, const lds_char* stage, int wn, int d) const
    {
        read(f, stage, stage + C::A_BYTES, wn, d);
    }

    // With 16 x 16 blocks: A block i of a whole stage into f.a[slot].
    __device__ __forceinline__ void read_a_into(Frags<C>& f, const lds_char* stage, int i, int slot) const
    {
        static_assert(C::MF == 16, "16 x 16 blocks");
        f.a[slot] = *(const LDS_AS bf16x8_t*)(stage + a_off + i * (16 * C::BK * 2));
    }
};

template <class C>
__device__ __forceinline__ void read_frags(Frags<C>& f, const lds_char* stage, int wm, int wn, int lane, int kk)
{
    const FragReader<C> rd(wm, wn, lane, kk);
#pragma unroll
    for (int d = 0; d < frag_reads<C>(); ++d)
        rd.read(f, stage, wn, d);
}

// Slots of one MFMA k-step region of M MFMAs, D LDS fragment reads and V
// global-to-LDS DMA issues.  Slot i holds MFMA i, LDS read i while reads
// remain (they are for the next k-step, so they have the rest of this
// k-step's MFMAs to land), and the DMA issues that fall on it, V spread
// evenly from the first slot on.  The texture path of a CU drains one 1 KiB
// DMA issue in tens of cycles; bunching the issues of all waves (they leave
// the barrier together) fills its queue and stalls every wave's instruction
// issue, MFMAs included.
//
// DMA writes to and reads from LDS keep their program order (the compiler
// cannot tell the ring stages apart), so emit_memops issues them in slot
// order, and sched_slots then only has to place the MFMAs between them.
template <int M, int V, int I>
constexpr int slot_dma_begin() { return (I * V + M - 1) / M; }

template <int M, int D, int V, int I = 0, class RD, class FR>
__device__ __forceinline__ void emit_memops(RD&& rd, FR&& fr)
{
    if constexpr (I < M || I < D) {
        if constexpr (I < D)
            rd(I);
        if constexpr (I < M) {
#pragma unroll
            for (int v = slot_dma_begin<M, V, I>(); v < slot_dma_begin<M, V, I + 1>(); ++v)
                fr(v);
        }
        emit_memops<M, D, V, I + 1>(rd, fr);
    }
}

// The memory operations of one region: D fragment reads from stage `src`
// and DMA instructions t0 .. t0 + V - 1 of a prepared position into stage
// `dst`.  The two stages always differ, and saying so (restrict) lets the
// compiler keep the reads apart from the in-flight DMA writes: without it,
// every read that follows a DMA in program order waits for all of the wave's
// outstanding loads.
template <int M, int D, int V, int OFF = 0, class C, class LD>
__device__ __forceinline__ void region_memops(const FragReader<C>& rdr, Frags<C>& f, const lds_char* __restrict__ src,
                                              int wn, const LD& ld, const typename LD::Prep& prep, int t0,
                                              lds_char* __restrict__ dst, int w, int lane)
{
    emit_memops<M, D, V>([&](int d) { rdr.read(f, src, wn, d + OFF); },
                         [&](int v) { ld.fire_one(prep, t0 + v, dst, w, lane); });
}

// The same for the window ring: fragment reads from the A and B windows of
// one position, DMA instructions t0 .. t0 + V - 1 (all of them A, or all B)
// into a third window.
template <int M, int D, int V, int OFF = 0, class C, class LD>
__device__ __forceinline__ void region_memops_win(const FragReader<C>& rdr, Frags<C>& f,
                                                  const lds_char* __restrict__ a_src,
                                                  const lds_char* __restrict__ b_src, int wn, const LD& ld,
                                                  const typename LD::Prep& prep, int t0, lds_char* __restrict__ dst,
                                                  int w, int lane)
{
    emit_memops<M, D, V>([&](int d) { rdr.read(f, a_src, b_src, wn, d + OFF); },
                         [&](int v) { ld.fire_one(prep, t0 + v, dst, dst, w, lane); });
}

// SALU scalar instructions may follow each MFMA (the load cursor's step, in
// the region that carries it).
template <int M, int D, int V, int SALU = 0, int I = 0>
__device__ __forceinline__ void sched_slots()
{
    if constexpr (I < M) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          // MFMA
        if constexpr (I < D)
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);      // LDS read
        // Scalar work before the DMA issue: a DMA's LDS address (M0) is
        // itself set by a scalar instruction.
        if constexpr (SALU > 0)
            __builtin_amdgcn_sched_group_barrier(0x004, SALU, 0);   // SALU
        constexpr int nv = slot_dma_begin<M, V, I + 1>() - slot_dma_begin<M, V, I>();
        if constexpr (nv > 0)
            __builtin_amdgcn_sched_group_barrier(0x020, nv, 0);     // VMEM read
        sched_slots<M, D, V, SALU, I + 1>();
    } else if constexpr (D > M) {
        __builtin_amdgcn_sched_group_barrier(0x100, D - M, 0);
    }
}

template <class C>
__device__ __forceinline__ bf16x8_t b_frag(const Frags<C>& f, int j)
{
    if constexpr (C::BT)
        return f.b[j];
    const i16x8_t v = __builtin_shufflevector(f.bh[j][0], f.bh[j][1], 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8_t, v);
}

// MFMAs LO .. HI-1 of one k-step (block x = i * FN + j).
template <class C, int LO, int HI>
__device__ __forceinline__ void mfma_range(f32x16_t (&acc)[C::FM][C::FN], const Frags<C>& f)
{
#pragma unroll
    for (int x = LO; x < HI; ++x)
        acc[x / C::FN][x % C::FN] =
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(b_frag<C>(f, x % C::FN), f.a[x / C::FN], acc[x / C::FN][x % C::FN], 0, 0, 0);
}

// MFMA region kk of a stage in the all-wave kernels.  32 x 32 blocks: the
// region is 16-wide k-step kk over every block, from fragment buffer kk & 1.
// 16 x 16 blocks: the region is half of 32-wide k-step kk / 2, block rows
// (kk & 1) * FM/2 .. + FM/2 - 1 (MFMA x = i' * FN + j), from buffer
// (kk / 2) & 1.
template <class C>
constexpr int region_mfmas() { return C::MF == 16 ? C::FM * C::FN / 2 : C::FM * C::FN; }

template <class C, int KKI, int LO, int HI>
__device__ __forceinline__ void region_mfma(typename C::Acc (&acc)[C::FM][C::FN], const Frags<C> (&fr)[2])
{
    if constexpr (C::MF == 16) {
        const Frags<C>& f = fr[(KKI >> 1) & 1];
        constexpr int I0 = (KKI & 1) * (C::FM / 2);
#pragma unroll
        for (int x = LO; x < HI; ++x)
            acc[I0 + x / C::FN][x % C::FN] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                b_frag<C>(f, x % C::FN), f.a[I0 + x / C::FN], acc[I0 + x / C::FN][x % C::FN], 0, 0, 0);
    } else {
        mfma_range<C, LO, HI>(acc, fr[KKI & 1]);
    }
}

// The fragment reads that region kk (not the last of its stage) issues for
// the next k-step of the same stage: that k-step, the number of reads, the
// first read's index and the buffer.  A 32 x 32 region reads all of k-step
// kk + 1.  The two regions of a 16 x 16 k-step each read half of the next
// one; the last k-step's first region reads nothing, since the next
// stage's fragments are readable only after the synchronisation in the
// stage's last region.
struct RegionReads {
    int ks, d, off, buf;
};

// Reads the last region of a stage issues for the next stage's first k-step,
// after the synchronisation.  Normally all of them, into buffer 0.  With one
// 16 x 16 k-step per stage (32-wide stages) buffer 0 is still in use by the
// last region's MFMAs: the reads for the first half (A blocks 0 .. FM/2 - 1
// and the B blocks) go to buffer 1 and are copied into buffer 0 at the end of
// the stage (take_next_stage); the compiler needs real moves only for the B
// blocks, whose registers the last region still reads.
template <class C>
constexpr int next_stage_reads()
{
    constexpr int NB = (C::BT ? 1 : 2) * C::FN;
    return (C::MF == 16 && C::KK == 2) ? NB + C::FM / 2 : frag_reads<C>();
}

template <class C>
__device__ __forceinline__ void take_next_stage(Frags<C> (&fr)[2])
{
    if constexpr (C::MF == 16 && C::KK == 2) {
#pragma unroll
        for (int i = 0; i < C::FM / 2; ++i)
            fr[0].a[i] = fr[1].a[i];
#pragma unroll
        for (int j = 0; j < C::FN; ++j) {
            if constexpr (C::BT) {
                fr[0].b[j] = fr[1].b[j];
            } else {
                fr[0].bh[j][0] = fr[1].bh[j][0];
                fr[0].bh[j][1] = fr[1].bh[j][1];
            }
        }
    }
}

template <class C, int KKI>
constexpr RegionReads region_reads()
{
    constexpr int D = frag_reads<C>();
    if constexpr (C::MF == 16 && C::KK == 2) {
        // A 32-wide stage is one 16 x 16 k-step: its first region reads the
        // A blocks of the second half (the last region of the previous stage
        // read the rest, see next_stage_reads).
        constexpr int NB = (C::BT ? 1 : 2) * C::FN;
        return RegionReads{0, C::FM / 2, NB + C::FM / 2, 0};
    } else if constexpr (C::MF == 16) {
        static_assert(D % 2 == 0, "two halves of a k-step's reads");
        constexpr int ks = (KKI >> 1) + 1;
        if constexpr (ks < C::KK / 2)
            return RegionReads{ks, D / 2, (KKI & 1) * (D / 2), ks & 1};
        else
            return RegionReads{0, 0, 0, 0};
    } else {
        return RegionReads{KKI + 1, D, 0, (KKI + 1) & 1};
    }
}

typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

// Two fp32 values -> two bf16 (round to nearest even) in one 32-bit word.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    const bf16x2_t v = __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t);
    return __builtin_bit_cast(uint32_t, v);
}

// fp32 accumulators -> bf16 (RNE) -> wave-private LDS strip -> 16-byte stores.
// The strip is 32 rows (m) x 64 columns (n) with 128-byte rows.  Writes: lane
// l holds row l%32 and, per 4 accumulator registers, 4 consecutive columns
// (8 bytes); the 32 lanes of one write cycle cover 32 rows at one column
// position, so the chunk is XORed with (row / 2) mod 8 and the two 8-byte
// halves of a chunk are swapped for rows 16..31, which gives 32 different
// 8-byte bank slots.  Reads: 8 lanes cover one 128-byte row segment of C (16
// lanes, two rows, per cycle), so each store instruction writes 8 full row
// segments; reads of rows 16..31 swap the halves back.
template <class C>
__device__ __forceinline__ void epilogue(const Params& p, f32x16_t (&acc)[C::FM][C::FN], lds_char* strip,
                                         int32_t m0, int32_t n0, int wm, int wn, int lane_in)
{
    const int lane = (int)opaque((uint32_t)lane_in);
    const __amdgpu_buffer_rsrc_t rc =
        make_rsrc(p.C + ((int64_t)m0 * p.ldc + n0) * 2, ((p.M - m0 - 1) * p.ldc + (p.N - n0)) * 2);
    const int row_w = lane & 31, half = lane >> 5;
    const int32_t mrem = (int32_t)min(p.M - m0, (int64_t)C::BM);
    const int32_t nrem = (int32_t)min(p.N - n0, (int64_t)C::BN);
    const uint32_t ldc2 = (uint32_t)p.ldc * 2u;
    const uint32_t wbase = opaque((uint32_t)(row_w * 128 + (half ^ (row_w >> 4)) * 8));
    const int rrow = lane >> 3, rc8 = lane & 7;          // read slot u adds 8*u rows
    const uint32_t rbase = opaque((uint32_t)(rrow * 128 + ((rc8 ^ (rrow >> 1)) * 16)));
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
#pragma unroll
        for (int jp = 0; jp < C::FN / 2; ++jp) {
            // Keep each pass's conversions next to its own stores.
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                // Keep this block in AGPRs up to here, so its copy to VGPRs
                // happens now rather than for all blocks at once.
                if constexpr (C::FM * C::FN * 16 > 128)
                    asm volatile("" : "+a"(acc[i][2 * jp + jj]));
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const f32x16_t& a = acc[i][2 * jp + jj];
                    u32x2_t v;
                    v.x = pack_bf16x2(a[4 * g + 0], a[4 * g + 1]);
                    v.y = pack_bf16x2(a[4 * g + 2], a[4 * g + 3]);
                    const uint32_t chunk = (uint32_t)(((4 * jj + g) ^ ((row_w >> 1) & 7)) * 16);
                    *(LDS_AS u32x2_t*)(strip + wbase + chunk) = v;
                }
            }
            wait_lgkm0();
            const int gr0 = wm * C::TM + 32 * i + rrow;            // tile row of read slot 0
            const int gc = wn * C::TN + 64 * jp + 8 * rc8;         // tile column of this lane's chunk
            const uint32_t obase = opaque((uint32_t)gr0 * ldc2 + (uint32_t)gc * 2u);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                // row rrow + 8u: (row / 2) mod 8 equals (rrow / 2) + 4u mod 8, i.e.
                // the XOR term gains 4 for odd u; halves are swapped for u >= 2.
                u32x4_t v = *(const LDS_AS u32x4_t*)(strip + ((rbase + u * 8 * 128) ^ ((u & 1) ? 64u : 0u)));
                if (u >= 2)
                    v = u32x4_t{v.z, v.w, v.x, v.y};
                const bool ok = (gr0 + 8 * u < mrem) && (gc < nrem);
                __builtin_amdgcn_raw_buffer_store_b128(v, rc, ok ? obase + (uint32_t)(8 * u) * ldc2 : kOOB, 0, C::STORE_C);
            }
            wait_lgkm0();
        }
    }
}

// The same with a 32 x 32 strip (64-byte rows, one MFMA block per pass),
// used when LDS is short.  Writes: the chunk (4 per row) is XORed with
// (row / 4) mod 4 and halves are swapped for rows 16..31, so the 32 lanes of
// a write cycle (32 rows, 4 rows per 256-byte bank window) hit 32 different
// 8-byte slots.  Reads: 4 lanes cover one 64-byte row segment, 16 lanes (4
// rows) per cycle on 16 different 16-byte slots.
template <class C>
__device__ __forceinline__ void epilogue_narrow(const Params& p, f32x16_t (&acc)[C::FM][C::FN], lds_char* strip,
                                                int32_t m0, int32_t n0, int wm, int wn, int lane_in)
{
    const int lane = (int)opaque((uint32_t)lane_in);
    const __amdgpu_buffer_rsrc_t rc =
        make_rsrc(p.C + ((int64_t)m0 * p.ldc + n0) * 2, ((p.M - m0 - 1) * p.ldc + (p.N - n0)) * 2);
    const int row_w = lane & 31, half = lane >> 5;
    const int32_t mrem = (int32_t)min(p.M - m0, (int64_t)C::BM);
    const int32_t nrem = (int32_t)min(p.N - n0, (int64_t)C::BN);
    const uint32_t ldc2 = (uint32_t)p.ldc * 2u;
    const uint32_t wbase = opaque((uint32_t)(row_w * 64 + (half ^ (row_w >> 4)) * 8));
    const int rrow = lane >> 2, rc4 = lane & 3;          // read slot u adds 16*u rows
    const uint32_t rbase = opaque((uint32_t)(rrow * 64 + ((rc4 ^ ((rrow >> 2) & 3)) * 16)));
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
#pragma unroll
        for (int j = 0; j < C::FN; ++j) {
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (C::FM * C::FN * 16 > 128)
                asm volatile("" : "+a"(acc[i][j]));
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x16_t& a = acc[i][j];
                u32x2_t v;
                v.x = pack_bf16x2(a[4 * g + 0], a[4 * g + 1]);
                v.y = pack_bf16x2(a[4 * g + 2], a[4 * g + 3]);
                const uint32_t chunk = (uint32_t)((g ^ ((row_w >> 2) & 3)) * 16);
                *(LDS_AS u32x2_t*)(strip + wbase + chunk) = v;
            }
            wait_lgkm0();
            const int gr0 = wm * C::TM + 32 * i + rrow;
            const int gc = wn * C::TN + 32 * j + 8 * rc4;
            const uint32_t obase = opaque((uint32_t)gr0 * ldc2 + (uint32_t)gc * 2u);
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                u32x4_t v = *(const LDS_AS u32x4_t*)(strip + rbase + u * 16 * 64);
                if (u == 1)
                    v = u32x4_t{v.z, v.w, v.x, v.y};
                const bool ok = (gr0 + 16 * u < mrem) && (gc < nrem);
                __builtin_amdgcn_raw_buffer_store_b128(v, rc, ok ? obase + (uint32_t)(16 * u) * ldc2 : kOOB, 0, C::STORE_C);
            }
            wait_lgkm0();
        }
    }
}

// 16 x 16 blocks: lane l of block (i, j) holds row 16i + l%16 and columns
// 16j + 4*(l/16) + 0..3.  A pass converts EH/16 block rows (EH rows, the
// strip's height: 32, or 16 when LDS is short) by 4 blocks (the strip's 64
// columns, 128-byte rows) into the strip, then stores it.  Writes: the 32
// lanes of a write cycle cover 16 rows at one chunk (both 8-byte halves);
// the chunk is XORed with (row / 2) mod 8 (two rows per 256-byte bank
// window), which puts them on 32 different 8-byte bank slots.  Reads: 8
// lanes cover one 128-byte row segment of C, 16 lanes (2 rows) per cycle on
// 16 different 16-byte slots.
template <class C>
__device__ __forceinline__ void epilogue16(const Params& p, f32x4_t (&acc)[C::FM][C::FN], lds_char* strip,
                                           int32_t m0, int32_t n0, int wm, int wn, int lane_in)
{
    constexpr int W = C::EPI_W, RB = 2 * W, JB = W / 16;   // columns, row bytes and blocks per pass
    constexpr int EH = C::EPI_H, IB = EH / 16;              // rows and block rows per pass
    constexpr int LPR = RB / 16, RPI = 64 / LPR;           // lanes per strip row, rows per read
    static_assert(W == 64 && C::FN % JB == 0 && C::FM % IB == 0, "whole passes of 128-byte rows");
    const int lane = (int)opaque((uint32_t)lane_in);
    const __amdgpu_buffer_rsrc_t rc =
        make_rsrc(p.C + ((int64_t)m0 * p.ldc + n0) * 2, ((p.M - m0 - 1) * p.ldc + (p.N - n0)) * 2);
    const int32_t mrem = (int32_t)min(p.M - m0, (int64_t)C::BM);
    const int32_t nrem = (int32_t)min(p.N - n0, (int64_t)C::BN);
    const uint32_t ldc2 = (uint32_t)p.ldc * 2u;
    auto swz = [](int row) { return (row >> 1) & 7; };
    const int wrow = lane & 15, wq = lane >> 4;
    const int rrow = lane / LPR, rchunk = lane % LPR;
#pragma unroll
    for (int i2 = 0; i2 < C::FM / IB; ++i2) {
#pragma unroll
        for (int jp = 0; jp < C::FN / JB; ++jp) {
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ii = 0; ii < IB; ++ii) {
#pragma unroll
                for (int jj = 0; jj < JB; ++jj) {
                    const f32x4_t& a = acc[IB * i2 + ii][JB * jp + jj];
                    u32x2_t v;
                    v.x = pack_bf16x2(a[0], a[1]);
                    v.y = pack_bf16x2(a[2], a[3]);
                    const int row = 16 * ii + wrow;
                    const int cb = 32 * jj + 8 * wq;             // byte column in the strip row
                    const uint32_t off = opaque((uint32_t)(row * RB + (((cb >> 4) ^ swz(row)) << 4) + (cb & 15)));
                    *(LDS_AS u32x2_t*)(strip + off) = v;
                }
            }
            wait_lgkm0();
            const int gr0 = wm * C::TM + EH * i2 + rrow;         // tile row of read slot 0
            const int gc = wn * C::TN + W * jp + 8 * rchunk;     // tile column of this lane's chunk
            const uint32_t obase = opaque((uint32_t)gr0 * ldc2 + (uint32_t)gc * 2u);
#pragma unroll
            for (int u = 0; u < EH / RPI; ++u) {
                const int row = rrow + RPI * u;
                const u32x4_t v = *(const LDS_AS u32x4_t*)(strip + row * RB + ((rchunk ^ swz(row)) << 4));
                const bool ok = (gr0 + RPI * u < mrem) && (gc < nrem);
                __builtin_amdgcn_raw_buffer_store_b128(v, rc, ok ? obase + (uint32_t)(RPI * u) * ldc2 : kOOB, 0, C::STORE_C);
            }
            wait_lgkm0();
        }
    }
}

template <class C>
__device__ __forceinline__ void store_tile(const Params& p, typename C::Acc (&acc)[C::FM][C::FN], lds_char* strip,
                                           int32_t m0, int32_t n0, int wm, int wn, int lane)
{
    if constexpr (C::MF == 16)
        epilogue16<C>(p, acc, strip, m0, n0, wm, wn, lane);
    else if constexpr (C::EPI_W == 64)
        epilogue<C>(p, acc, strip, m0, n0, wm, wn, lane);
    else
        epilogue_narrow<C>(p, acc, strip, m0, n0, wm, wn, lane);
}

// Split k range: the work item's fp32 accumulators go, unrounded, to its
// partial tile (BM x BN fp32 in the workspace); k_reduce_splits adds the
// chunks later.  The partial tile keeps the registers' order: 16-byte unit
// (((wave * FM + i) * FN + j) * NG + g) * 64 + lane holds registers
// 4g..4g+3 of lane `lane` in block (i, j) of MFMA wave `wave` (wm * WN + wn),
// NG = MF * MF / 256 groups per block (4 or 1), so each store instruction writes 1 KiB
// contiguously.  Those registers hold row wm*TM + MF*i + lane%MF and four
// consecutive columns from unit_col<C>(j, g, lane).
template <class C>
__device__ __forceinline__ int unit_col(int j, int g, int lane)
{
    return C::MF == 16 ? 16 * j + 4 * (lane >> 4) : 32 * j + 8 * g + 4 * (lane >> 5);
}

template <class C>
__device__ __forceinline__ void store_partial(const Params& p, typename C::Acc (&acc)[C::FM][C::FN], int32_t widx,
                                              int wm, int wn, int lane_in)
{
    constexpr int NG = C::MF * C::MF / 256;
    const int lane = (int)opaque((uint32_t)lane_in);
    const __amdgpu_buffer_rsrc_t rp = rsrc_n(p.partial + (int64_t)widx * (C::BM * C::BN), C::BM * C::BN * 4u);
    const int wave = wm * C::WN + wn;
    const uint32_t base = opaque((uint32_t)(wave * C::FM * C::FN * NG * 1024 + lane * 16));
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
#pragma unroll
        for (int j = 0; j < C::FN; ++j) {
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (C::MF == 32 && C::FM * C::FN * 16 > 128)
                asm volatile("" : "+a"(acc[i][j]));
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                const typename C::Acc& a = acc[i][j];
                // Whole vectors only: a bit cast of a single vector element
                // is not what this needs.
                const f32x4_t v = {a[4 * g + 0], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]};
                const uint32_t off = base + (uint32_t)(((i * C::FN + j) * NG + g) * 1024);
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), rp, off, 0, 0);
            }
        }
    }
}

// C = bf16_rne(sum of the partial tiles over the k chunks, in chunk order),
// for the launch's span of output tiles.  The partial tile of chunk sp and
// of the launch's u-th tile (raster position tile_base + u) is number
// sp * span + u.  One thread per 16-byte unit of the partial tiles' register
// order (4 consecutive output columns), so reads are contiguous across
// lanes; units outside the matrix are skipped (N % 8 == 0 keeps a unit
// whole).
template <class C>
__global__ void __launch_bounds__(256) k_reduce_splits(Params p)
{
    constexpr int64_t UNITS = (int64_t)C::BM * C::BN / 4;   // 16-byte units per tile
    const int64_t total = (int64_t)p.span * UNITS;
    const int64_t chunk_stride = (int64_t)p.span * C::BM * C::BN;
    for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < total;
         q += (int64_t)gridDim.x * blockDim.x) {
        const int32_t u = (int32_t)(q / UNITS);
        const int32_t unit = (int32_t)(q - (int64_t)u * UNITS);
        constexpr int NG = C::MF * C::MF / 256;
        const int lane = unit & 63;
        int rest = unit >> 6;
        const int g = rest % NG;
        rest /= NG;
        const int j = rest % C::FN;
        rest /= C::FN;
        const int i = rest % C::FM;
        const int wave = rest / C::FM;
        const int wm = wave / C::WN, wn = wave % C::WN;
        int32_t tm, tn;
        raster_tile(p, p.tile_base + u, tm, tn);
        const int64_t r = (int64_t)tm * C::BM + wm * C::TM + C::MF * i + (lane % C::MF);
        const int64_t c0 = (int64_t)tn * C::BN + wn * C::TN + unit_col<C>(j, g, lane);
        if (r >= p.M || c0 >= p.N)
            continue;
        const f32x4_t* src = (const f32x4_t*)(p.partial + (int64_t)u * C::BM * C::BN) + unit;
        f32x4_t sum = {0.f, 0.f, 0.f, 0.f};
        for (int32_t sp = 0; sp < p.splits; ++sp) {
            const f32x4_t v = src[sp * chunk_stride / 4];
            sum.x += v.x;
            sum.y += v.y;
            sum.z += v.z;
            sum.w += v.w;
        }
        u32x2_t out;
        out.x = pack_bf16x2(sum.x, sum.y);
        out.y = pack_bf16x2(sum.z, sum.w);
        *(u32x2_t*)(p.C + (r * p.ldc + c0) * 2) = out;
    }
}

// Before a tile is stored: if this wave gave up a ring wait, or another wave
// of the workgroup did (the poison word, see SyncState), every element of the
// wave's part of the tile becomes NaN, so the output shows where it cannot be
// trusted.  A uniform branch; the LDS read costs one round trip per tile.
template <class C>
__device__ __forceinline__ void poison_tile(typename C::Acc (&acc)[C::FM][C::FN], const SyncState& st)
{
    if (st.failed || load_counter(st.poison) != 0u) {
        const float nan = __builtin_nanf("");
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
            for (int j = 0; j < C::FN; ++j)
#pragma unroll
                for (int r = 0; r < (int)(sizeof(typename C::Acc) / sizeof(float)); ++r)
                    acc[i][j][r] = nan;
    }
}

// ---------------------------------------------------------------------------
// Kernel: every wave loads and computes (GEMM_SYNC_BARRIER, GEMM_SYNC_FLAGS).
// ---------------------------------------------------------------------------
template <class C, bool LONGK, bool EDGE>
__global__ void __launch_bounds__(C::THREADS) k_gemm(Params p)
{
    static_assert(!C::PRODUCERS, "configs with loader waves use k_gemm_ws / k_gemm_pp");
    __shared__ __attribute__((aligned(1024))) char smem_raw[C::LDS_BYTES];
    lds_char* smem = (lds_char*)smem_raw;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = w / C::WN, wn = w % C::WN;
    static_assert(C::FLAG_OFFSET % 8 == 0, "64-bit signal words");
    lds_u64* sig = (lds_u64*)(smem + C::FLAG_OFFSET);

    lds_u32* poison = (lds_u32*)(sig + C::S);
    if constexpr (C::SYNC == SYNC_FLAGS) {
        if (threadIdx.x < C::S)
            sig[threadIdx.x] = 0ull;
        if (threadIdx.x == 0)
            *poison = 0u;
    }
    __syncthreads();   // counters are initialised before any wave can arrive

    const int32_t G = gridDim.x, b = blockIdx.x;
    const int32_t n_tiles = (b < p.tiles) ? (p.tiles - 1 - b) / G + 1 : 0;
    const int32_t KT = p.k_steps;
    const int32_t total = n_tiles * KT;

    if (total == 0)
        return;
    clock_begin(p);
    Loader<C, LONGK, EDGE> ld;
    ld.init(p, n_tiles, w, lane);
#pragma unroll
    for (int q = 0; q < C::S - 1; ++q)
        ld.issue_next(p, smem + q * C::STAGE_BYTES, w, lane);

    Frags<C> fr[2];
    lds_char* strip = smem + C::EPI_OFFSET + w * C::EPI_WAVE_BYTES;
    auto stage_at = [&](int s) { return smem + s * C::STAGE_BYTES; };

    // Ring bookkeeping for the position c being computed: its stage s_cur,
    // the stage s_prev of position c - 1 (which the load of position
    // c + S - 1 refills), and its generation gen = c / S.
    int s_cur = 0, s_prev = C::S - 1;
    uint32_t gen = 0;
    SyncState st;
    st.poison = poison;
    st.limit = p.spin_limit;

    // Make position c + 1 (stage s_nxt, generation g_nxt) readable.  This
    // wave's DMA groups for positions c+1 .. c+S-1 are outstanding (S-1
    // groups of LOADS; positions past the end of the stream are issued too, as
    // empty loads), possibly followed by younger epilogue stores.  Waiting
    // until at most LOADS*(S-2) vector-memory operations are outstanding
    // leaves at most that many loads outstanding; loads complete in order, so
    // the oldest group has landed however the younger operations complete.
    // BARRIER: one s_barrier then covers the other waves' loads (RAW) and
    // every wave's reads of the stage being refilled next (WAR).
    auto sync_next = [&](int s_nxt, uint32_t g_nxt) {
        wait_vmcnt<C::LOADS * (C::S - 2)>();
        if constexpr (C::SYNC == SYNC_BARRIER) {
            block_barrier();
        } else {
            arrive_pair(sig + s_nxt, kAnnounce);
            wait_pair_issued(pair_read_issue(sig + s_nxt), sig + s_nxt, (g_nxt + 1) * C::NW, 0u, st);
        }
    };

    // A position's DMA is issued in parts, spread over the MFMA regions of the
    // following stage, so the texture path never receives a burst of every
    // wave's loads at once: part 0 right after the synchronisation that frees
    // its stage, the others with the next stage's first MFMA regions.  With
    // three or more stages there is one part per region (KK).  With two stages
    // the data is needed one stage later, so there are two parts: after the
    // synchronisation and in the next stage's first region.  Both sync modes
    // share this schedule; they differ only in how the workgroup synchronises.
    constexpr int NPARTS = (C::S == 2) ? 2 : C::KK;
    //
    // The load cursor's step is several dozen scalar instructions, and all
    // waves reach it together; they queue for the CU's one scalar unit.  With
    // three or more MFMA regions per k-step (PREP_IN_REGION), the cursor
    // prepares position c + S inside region 1 of k-step c, its instructions
    // spread between the MFMAs; next_prep (position c + S - 1) becomes
    // fire_prep at the top of the k-step.  With two regions that pattern
    // cannot be scheduled next to the region's DMA issues, so the cursor
    // prepares position c + S + 1 after the k-step instead (ahead of the
    // barrier its instructions would delay every wave's arrival).
    constexpr bool PIR = C::PREP_IN_REGION;
    sync_next(0, 0);
    typename Loader<C, LONGK, EDGE>::Prep fire_prep = ld.prepare_and_advance(p);      // position S - 1
    ld.template fire<NPARTS>(fire_prep, 0, stage_at(C::S - 1), w, lane);
    typename Loader<C, LONGK, EDGE>::Prep next_prep = fire_prep;
    if constexpr (!PIR)
        next_prep = ld.prepare_and_advance(p);                                  // position S
    read_frags<C>(fr[0], smem, wm, wn, lane, 0);

    for (int32_t it = 0; it < n_tiles; ++it) {
        int32_t tm, tn;
        int32_t sp, u;
        tile_coords(p, b + it * G, G, tm, tn, sp, u);
        if constexpr (LONGK)
            ld.prefetch_next_tile(p, it + 1);
        typename C::Acc acc[C::FM][C::FN];
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
            for (int j = 0; j < C::FN; ++j)
                acc[i][j] = typename C::Acc{};

        for (int32_t kt = 0; kt < KT; ++kt) {
            // The cursor prepares position c + S (or c + S + 1) during
            // k-step c: from this k-step on, that is the next tile.
            if constexpr (LONGK) {
                if (kt == KT - (PIR ? C::S : C::S + 1))
                    ld.enter_next_tile();
            }
            const lds_char* stage = stage_at(s_cur);
            const int s_nxt = (s_cur + 1 == C::S) ? 0 : s_cur + 1;
            const uint32_t g_nxt = gen + (s_nxt == 0 ? 1u : 0u);
            if constexpr (PIR)
                fire_prep = next_prep;
            // MFMA k-step region kk of this stage (kk is a constant).
            auto region = [&]<int kk>() {
                constexpr int M = region_mfmas<C>();
                constexpr int SALU = (PIR && kk == 1) ? 6 : 0;
                if constexpr (PIR && kk == 1)
                    next_prep = ld.prepare_and_advance(p);
                if constexpr (kk + 1 < C::KK) {
                    // Fragments of k-step kk + 1; part kk + 1 of the load of
                    // position c + S - 1 into the stage of position c - 1
                    // (part 0 went out right after the last synchronisation).
                    constexpr int part = kk + 1;
                    constexpr int t0 = part < NPARTS ? part_begin(part, NPARTS, C::LOADS) : 0;
                    constexpr int V = part < NPARTS ? part_begin(part + 1, NPARTS, C::LOADS) - t0 : 0;
                    constexpr RegionReads rr = region_reads<C, kk>();
                    const FragReader<C> rdr(wm, wn, lane, rr.ks);
                    region_memops<M, rr.d, V, rr.off>(rdr, fr[rr.buf], stage, wn, ld, fire_prep, t0, stage_at(s_prev),
                                                      w, lane);
                    region_mfma<C, kk, 0, M>(acc, fr);
                    sched_slots<M, rr.d, V, SALU>();
                } else {
                    // Last MFMA k-step of this stage: the workgroup hands the
                    // stage back and makes the next position readable; then
                    // part 0 of the load of position c + S refills this stage
                    // and the next stage's first fragments are read.  At the
                    // end of the stream this runs once more on an empty
                    // position, which keeps the block free of branches.  The
                    // first MFMAs (their fragments are in registers) keep the
                    // pipe busy while the workgroup gathers.
                    //
                    // BARRIER: PRE MFMAs, then one s_barrier.
                    //
                    // FLAGS: after one MFMA the wave waits for its fragment
                    // reads of position c (it may release the stage) and its
                    // loads of position c + 1 (it may announce them), does
                    // both in one atomic add, and sends out the read of the
                    // signal word; two more MFMAs (three with 32-wide k-steps,
                    // measured) cover its round trip.  The refill needs the
                    // stage released by every wave (WAR) and the next
                    // position announced by every wave (RAW): both halves of
                    // the word reach their targets together.
                    constexpr int PRE = (C::SYNC == SYNC_FLAGS) ? (C::S == 2 ? 3 : 4) : 2;
                    if constexpr (C::SYNC == SYNC_FLAGS) {
                        region_mfma<C, kk, 0, 1>(acc, fr);
                        __builtin_amdgcn_sched_barrier(0);
                        wait_lgkm0();
                        wait_vmcnt<C::LOADS * (C::S - 2)>();
                        arrive_pair(sig + s_nxt, kAnnounce | kRelease);
                        const uint64_t v = pair_read_issue(sig + s_nxt);
                        __builtin_amdgcn_sched_barrier(0);
                        region_mfma<C, kk, 1, PRE>(acc, fr);
                        __builtin_amdgcn_sched_barrier(0);
                        wait_pair_issued(v, sig + s_nxt, (g_nxt + 1) * C::NW, (gen + 1) * C::NW, st);
                    } else {
                        region_mfma<C, kk, 0, PRE>(acc, fr);
                        __builtin_amdgcn_sched_barrier(0);
                        wait_lgkm0();
                        sync_next(s_nxt, g_nxt);
                    }
                    constexpr int V = part_begin(1, NPARTS, C::LOADS);
                    constexpr int DN = next_stage_reads<C>();
                    constexpr int NBUF = (C::MF == 16 && C::KK == 2) ? 1 : 0;
                    const FragReader<C> rdr(wm, wn, lane, 0);
                    region_memops<M - PRE, DN, V>(rdr, fr[NBUF], stage_at(s_nxt), wn, ld, next_prep, 0,
                                                  stage_at(s_cur), w, lane);
                    region_mfma<C, kk, PRE, M>(acc, fr);
                    sched_slots<M - PRE, DN, V>();
                    take_next_stage<C>(fr);
                }
                __builtin_amdgcn_sched_barrier(0);
            };
            [&]<int... KS>(std::integer_sequence<int, KS...>) {
                (region.template operator()<KS>(), ...);
            }(std::make_integer_sequence<int, C::KK>{});
            if constexpr (!PIR) {
                fire_prep = next_prep;
                next_prep = ld.prepare_and_advance(p);
            }
            s_prev = s_cur;
            s_cur = s_nxt;
            gen = g_nxt;
        }
        if constexpr (C::SYNC == SYNC_FLAGS)
            poison_tile<C>(acc, st);
        if (p.splits > 1)
            store_partial<C>(p, acc, sp * p.span + u, wm, wn, lane);
        else
            store_tile<C>(p, acc, strip, tm * C::BM, tn * C::BN, wm, wn, lane);
    }
    clock_end(p);
}

// ---------------------------------------------------------------------------
// Kernel: barrier sync over the split-window ring.
//
// The LDS is five windows of one operand tile (32 KiB at 256 x 64 bf16).
// Position c keeps its A tile in window 2c mod 5 and its B tile in window
// 2c+1 mod 5.  The barrier of k-step c (in its last MFMA region) frees the two
// windows of position c, and they take the B tile of position c+2 and the A
// tile of position c+3.  So every B tile has one k-step to land (as in a
// two-stage ring) but every A tile has two, and the barrier only waits for
// the B tile of the next position: the loads in flight at a barrier are
// spread over twice the time.  The epilogue stages through the window that
// held the tile's last B tile; the A load that reuses it is issued after a
// barrier that follows the epilogue.
//
// Per k-step c (DMA parts are halves of one operand tile per wave):
//   region 0: second half of B(c+1); the cursor prepares position c+2
//   region 1: first half of A(c+2)
//   region 2: second half of A(c+2)
//   region 3: PRE MFMAs; wait until B(c+1) has landed (only the A(c+2)
//             loads may still be outstanding); barrier; first half of
//             B(c+2); fragments of k-step 0 of position c+1
// ---------------------------------------------------------------------------
template <class C, bool LONGK, bool EDGE>
__global__ void __launch_bounds__(C::THREADS) k_gemm_win(Params p)
{
    static_assert(C::WIN && C::SYNC == SYNC_BARRIER, "window-ring configs only");
    __shared__ __attribute__((aligned(1024))) char smem_raw[C::LDS_BYTES];
    lds_char* smem = (lds_char*)smem_raw;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = w / C::WN, wn = w % C::WN;

    const int32_t G = gridDim.x, b = blockIdx.x;
    const int32_t n_tiles = (b < p.tiles) ? (p.tiles - 1 - b) / G + 1 : 0;
    const int32_t KT = p.k_steps;
    if (n_tiles == 0 || KT == 0)
        return;
    clock_begin(p);

    constexpr int AH = C::A_LOADS / 2, BH = C::B_LOADS / 2;   // DMA instructions per half tile
    auto win = [&](int i) { return smem + i * C::A_BYTES; };
    auto step5 = [](int i, int d) { return i + d >= 5 ? i + d - 5 : i + d; };
    using Prep = typename Loader<C, LONGK, EDGE>::Prep;

    Loader<C, LONGK, EDGE> ld;
    ld.init(p, n_tiles, w, lane);
    // Prologue: positions 0 and 1 whole except the second half of B(1),
    // which region 0 of k-step 0 issues like any other.
    Prep prep_b = ld.prepare_and_advance(p);
#pragma unroll
    for (int t = 0; t < C::LOADS; ++t)
        ld.fire_one(prep_b, t, win(0), win(1), w, lane);
    prep_b = ld.prepare_and_advance(p);
#pragma unroll
    for (int t = 0; t < C::A_LOADS + BH; ++t)
        ld.fire_one(prep_b, t, win(2), win(3), w, lane);
    wait_vmcnt<C::A_LOADS + BH>();
    block_barrier();

    Frags<C> fr[2];
    read_frags<C>(fr[0], win(0), wm, wn, lane, 0);   // A at window 0, B at window 1
    int wa = 0;                                      // A window of the position being computed
    Prep prep_a = prep_b;

    for (int32_t it = 0; it < n_tiles; ++it) {
        int32_t tm, tn;
        int32_t sp, u;
        tile_coords(p, b + it * G, G, tm, tn, sp, u);
        if constexpr (LONGK)
            ld.prefetch_next_tile(p, it + 1);
        typename C::Acc acc[C::FM][C::FN];
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
            for (int j = 0; j < C::FN; ++j)
                acc[i][j] = typename C::Acc{};

        for (int32_t kt = 0; kt < KT; ++kt) {
            // Region 0 prepares position c + 2: from this k-step on, that is
            // the next tile.
            if constexpr (LONGK) {
                if (kt == KT - 2)
                    ld.enter_next_tile();
            }
            const lds_char* a_cur = win(wa);
            const lds_char* b_cur = win(step5(wa, 1));
            auto region = [&]<int kk>() {
                constexpr int M = region_mfmas<C>(), D = frag_reads<C>();
                if constexpr (kk < 3) {
                    constexpr int SALU = (kk == 0) ? 6 : 0;
                    if constexpr (kk == 0)
                        prep_a = ld.prepare_and_advance(p);                     // position c + 2
                    constexpr RegionReads rr = region_reads<C, kk>();
                    const FragReader<C> rdr(wm, wn, lane, rr.ks);
                    if constexpr (kk == 0)
                        region_memops_win<M, rr.d, C::B_LOADS - BH, rr.off>(rdr, fr[rr.buf], a_cur, b_cur, wn, ld,
                                                                            prep_b, C::A_LOADS + BH,
                                                                            win(step5(wa, 3)), w, lane);
                    else
                        region_memops_win<M, rr.d, (kk == 1) ? AH : C::A_LOADS - AH, rr.off>(
                            rdr, fr[rr.buf], a_cur, b_cur, wn, ld, prep_a, (kk == 1) ? 0 : AH,
                            win(step5(wa, 4)), w, lane);
                    region_mfma<C, kk, 0, M>(acc, fr);
                    sched_slots<M, rr.d, (kk == 0) ? C::B_LOADS - BH : (kk == 1) ? AH : C::A_LOADS - AH, SALU>();
                } else {
                    constexpr int PRE = 2;
                    region_mfma<C, kk, 0, PRE>(acc, fr);
                    __builtin_amdgcn_sched_barrier(0);
                    wait_lgkm0();
                    wait_vmcnt<C::A_LOADS>();
                    block_barrier();
                    const FragReader<C> rdr(wm, wn, lane, 0);
                    region_memops_win<M - PRE, D, BH>(rdr, fr[0], win(step5(wa, 2)), win(step5(wa, 3)), wn, ld,
                                                      prep_a, C::A_LOADS, win(wa), w, lane);
                    region_mfma<C, kk, PRE, M>(acc, fr);
                    sched_slots<M - PRE, D, BH>();
                }
                __builtin_amdgcn_sched_barrier(0);
            };
            [&]<int... KS>(std::integer_sequence<int, KS...>) {
                (region.template operator()<KS>(), ...);
            }(std::make_integer_sequence<int, C::KK>{});
            prep_b = prep_a;
            wa = step5(wa, 2);
        }
        if (p.splits > 1) {
            store_partial<C>(p, acc, sp * p.span + u, wm, wn, lane);
        } else {
            // The window of the last position's B tile is free until region 1
            // of the next k-step reloads it.
            store_tile<C>(p, acc, win(step5(wa, 4)) + w * C::EPI_WAVE_BYTES, tm * C::BM, tn * C::BN, wm, wn, lane);
            wait_lgkm0();
            block_barrier();
        }
    }
    clock_end(p);
}

// ---------------------------------------------------------------------------
// Loader waves of the wave-specialised and ping-pong kernels.
// ---------------------------------------------------------------------------
template <class C>
__device__ __forceinline__ void producer_loop(const Params& p, lds_char* smem, lds_u32* full, lds_u32* empty,
                                              int32_t n_tiles, int lw, int lane, SyncState& st, int32_t first = 0,
                                              int32_t stride = 1)
{
    const int32_t total = n_tiles * p.k_steps;
    // Loader wave: one flat loop over (tile, k-step) positions.  The data
    // of position q is announced on full[] once it has landed, D positions
    // later (the wave keeps D + 1 positions of loads in flight).  Issuing
    // position q waits for the release of position q - S, so announcing
    // q - D then depends on the consumers having finished q - S; D = S - 2
    // leaves them one computed stage of slack (a larger lag would make
    // every stage wait for that release-issue-announce chain).
    constexpr int D = (C::S - 2 < 2) ? C::S - 2 : 2;
    Loader<C, false> ld;
    ld.init(p, n_tiles, lw, lane, first, stride);
    for (int32_t q = 0; q < total; ++q) {
        const int s = q % C::S;
        // Each use of a stage is released by the NCWG MFMA waves of the one
        // group that computes the position.
        if (q >= C::S)
            wait_counter(empty + s, (uint32_t)(q / C::S) * C::NCWG, st);
        if constexpr (C::SPREAD_SLEEP > 0) {
            const auto pr = ld.prepare_and_advance(p);
#pragma unroll
            for (int t = 0; t < C::LOADS; ++t) {
                ld.fire_one(pr, t, smem + s * C::STAGE_BYTES, lw, lane);
                if (t % 2 == 1 && t + 1 < C::LOADS)
                    __builtin_amdgcn_s_sleep(C::SPREAD_SLEEP);
            }
        } else {
            ld.issue_next(p, smem + s * C::STAGE_BYTES, lw, lane);
        }
        if (q >= D) {
            wait_vmcnt<C::LOADS * D>();
            arrive(full + (q - D) % C::S);
        }
    }
    wait_vmcnt<0>();
    for (int32_t q = (total > D ? total - D : 0); q < total; ++q)
        arrive(full + q % C::S);
}

// Last MFMA k-step of a position in an MFMA wave of the loader/MFMA kernels.
// The wave releases the stage (its fragment reads have landed) and sends out
// the read of the next position's announcement counter; PRE MFMAs, whose
// fragments are in registers, cover its round trip.  Once every loader has
// announced, the next position's first fragments are read beside the
// remaining MFMAs.  Without a next position (has_next false) only the MFMAs
// run.
//
// With 16 x 16 blocks the last region is the second half of the last 32-wide
// k-step; half of its MFMAs go before the wait, so that the other half can
// cover the next position's fragment reads.
template <class C>
__device__ __forceinline__ void consumer_last_kstep(typename C::Acc (&acc)[C::FM][C::FN], Frags<C> (&fr)[2],
                                                    lds_u32* empty_cur, const lds_u32* full_next,
                                                    uint32_t next_target, bool has_next, const lds_char* next_stage,
                                                    int wm, int wn, int lane, SyncState& st)
{
    constexpr int M = region_mfmas<C>();
    constexpr int PRE = (C::MF == 16) ? M / 2 : (M > 4) ? M - 3 : M / 2;
    wait_lgkm0();
    arrive(empty_cur);
    const uint32_t v = counter_read_issue(full_next);
    __builtin_amdgcn_sched_barrier(0);
    region_mfma<C, C::KK - 1, 0, PRE>(acc, fr);
    __builtin_amdgcn_sched_barrier(0);
    wait_counter_issued(v, full_next, has_next ? next_target : 0u, st);
    if (has_next)
        read_frags<C>(fr[0], next_stage, wm, wn, lane, 0);
    region_mfma<C, C::KK - 1, PRE, M>(acc, fr);
    sched_slots<M - PRE, frag_reads<C>(), 0>();
}

// ---------------------------------------------------------------------------
// Kernel: dedicated loader waves and MFMA waves (GEMM_SYNC_WAVESPEC).
// ---------------------------------------------------------------------------
template <class C>
__global__ void __launch_bounds__(C::THREADS) k_gemm_ws(Params p)
{
    static_assert(C::SYNC == SYNC_WAVESPEC, "k_gemm_ws");
    __shared__ __attribute__((aligned(1024))) char smem_raw[C::LDS_BYTES];
    lds_char* smem = (lds_char*)smem_raw;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    lds_u32* full = (lds_u32*)(smem + C::FLAG_OFFSET);
    lds_u32* empty = full + C::S;
    if (threadIdx.x < 2 * C::S + 1)
        full[threadIdx.x] = 0u;   // full[], empty[] and the poison word
    __syncthreads();   // counters are initialised before the roles split
    SyncState st;
    st.poison = full + 2 * C::S;
    st.limit = p.spin_limit;

    const int32_t G = gridDim.x, b = blockIdx.x;
    const int32_t n_tiles = (b < p.tiles) ? (p.tiles - 1 - b) / G + 1 : 0;
    const int32_t KT = p.k_steps;
    const int32_t total = n_tiles * KT;

    if (w >= C::NCW) {
        producer_loop<C>(p, smem, full, empty, n_tiles, w - C::NCW, lane, st);
        return;
    }

    // MFMA wave: tile { k-step { wait full; read; release; MFMA } epilogue }.
    const int wm = w / C::WN, wn = w % C::WN;
    lds_char* strip = smem + C::EPI_OFFSET + w * C::EPI_WAVE_BYTES;
    if constexpr (C::NCW == 8) {
        // Two MFMA waves per SIMD and one fragment set each (Pick above):
        // read, wait, MFMAs; while one wave waits for its reads the other
        // wave's MFMAs keep the SIMD's matrix core busy.  The stage is handed
        // back once its last fragment reads have landed, before the MFMAs on
        // them, which read registers only.
        if (total == 0)
            return;
        clock_begin(p);
        int32_t c = 0;
        for (int32_t it = 0; it < n_tiles; ++it) {
            int32_t tm, tn;
            int32_t sp, u;
            tile_coords(p, b + it * G, G, tm, tn, sp, u);
            typename C::Acc acc[C::FM][C::FN];
#pragma unroll
            for (int i = 0; i < C::FM; ++i)
#pragma unroll
                for (int j = 0; j < C::FN; ++j)
                    acc[i][j] = typename C::Acc{};
            for (int32_t kt = 0; kt < KT; ++kt, ++c) {
                const int s = c % C::S;
                const lds_char* stage = smem + s * C::STAGE_BYTES;
                wait_counter(full + s, (uint32_t)(c / C::S + 1) * C::NP, st);
                if constexpr (C::MF == 32) {
                    // Per 16-wide k-step: all fragments, then its MFMAs.
#pragma unroll
                    for (int kk = 0; kk < C::KK; ++kk) {
                        Frags<C> f;
                        read_frags<C>(f, stage, wm, wn, lane, kk);
                        wait_lgkm0();
                        if (kk == C::KK - 1)
                            arrive(empty + s);
                        mfma_range<C, 0, C::FM * C::FN>(acc, f);
                    }
                } else {
                    // Per 32-wide k-step: the B blocks and A blocks
                    // 0 .. FM/2 - 1 (read order of FragReader), their MFMAs,
                    // then A blocks FM/2 .. FM - 1 into the same A registers
                    // and theirs.  No wait for all of a batch's reads: each
                    // MFMA waits (lgkmcnt) only for its own fragments, so the
                    // first MFMAs start once A block 0 and B block 0 are in
                    // (measured +0.4-2%); the stage is released after a wait
                    // for every read of its last k-step.
                    constexpr int H = (C::BT ? 1 : 2) * C::FN + C::FM / 2;
#pragma unroll
                    for (int ks = 0; ks < C::BK / 32; ++ks) {
                        const FragReader<C> rd(wm, wn, lane, ks);
                        Frags<C> f;
#pragma unroll
                        for (int d = 0; d < H; ++d)
                            rd.read(f, stage, wn, d);
#pragma unroll
                        for (int i = 0; i < C::FM / 2; ++i)
#pragma unroll
                            for (int j = 0; j < C::FN; ++j)
                                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b_frag<C>(f, j), f.a[i],
                                                                                   acc[i][j], 0, 0, 0);
#pragma unroll
                        for (int i = 0; i < C::FM / 2; ++i)
                            rd.read_a_into(f, stage, C::FM / 2 + i, i);
                        if (ks == C::BK / 32 - 1) {
                            wait_lgkm0();
                            arrive(empty + s);
                        }
#pragma unroll
                        for (int i = 0; i < C::FM / 2; ++i)
#pragma unroll
                            for (int j = 0; j < C::FN; ++j)
                                acc[C::FM / 2 + i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                    b_frag<C>(f, j), f.a[i], acc[C::FM / 2 + i][j], 0, 0, 0);
                    }
                }
            }
            poison_tile<C>(acc, st);
            if (p.splits > 1)
                store_partial<C>(p, acc, sp * p.span + u, wm, wn, lane);
            else
                store_tile<C>(p, acc, strip, tm * C::BM, tn * C::BN, wm, wn, lane);
        }
        clock_end(p);
        return;
    }
    Frags<C> fr[2];
    if (total == 0)
        return;
    clock_begin(p);
    wait_counter(full, (uint32_t)C::NP, st);
    read_frags<C>(fr[0], smem, wm, wn, lane, 0);

    int32_t c = 0;
    for (int32_t it = 0; it < n_tiles; ++it) {
        int32_t tm, tn;
        int32_t sp, u;
        tile_coords(p, b + it * G, G, tm, tn, sp, u);
        typename C::Acc acc[C::FM][C::FN];
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
            for (int j = 0; j < C::FN; ++j)
                acc[i][j] = typename C::Acc{};
        for (int32_t kt = 0; kt < KT; ++kt, ++c) {
            const lds_char* stage = smem + (c % C::S) * C::STAGE_BYTES;
            // MFMA region kk of the stage: the next k-step's fragment reads
            // (region_reads) beside this region's MFMAs; the last region
            // hands the stage back.
            auto region = [&]<int kk>() {
                constexpr int M = region_mfmas<C>();
                if constexpr (kk + 1 < C::KK) {
                    constexpr RegionReads rr = region_reads<C, kk>();
                    const FragReader<C> rdr(wm, wn, lane, rr.ks);
#pragma unroll
                    for (int d = 0; d < rr.d; ++d)
                        rdr.read(fr[rr.buf], stage, wn, d + rr.off);
                    region_mfma<C, kk, 0, M>(acc, fr);
                    sched_slots<M, rr.d, 0>();
                } else {
                    const int s1 = (c + 1) % C::S;
                    consumer_last_kstep<C>(acc, fr, empty + c % C::S, full + s1,
                                           (uint32_t)((c + 1) / C::S + 1) * C::NP, c + 1 < total,
                                           smem + s1 * C::STAGE_BYTES, wm, wn, lane, st);
                }
                __builtin_amdgcn_sched_barrier(0);
            };
            [&]<int... KS>(std::integer_sequence<int, KS...>) {
                (region.template operator()<KS>(), ...);
            }(std::make_integer_sequence<int, C::KK>{});
        }
        poison_tile<C>(acc, st);
        if (p.splits > 1)
            store_partial<C>(p, acc, sp * p.span + u, wm, wn, lane);
        else
            store_tile<C>(p, acc, strip, tm * C::BM, tn * C::BN, wm, wn, lane);
    }
    clock_end(p);
}

// ---------------------------------------------------------------------------
// Kernel: loader waves and two MFMA wave groups that take the output tiles in
// turn (GEMM_SYNC_PINGPONG).
//
// One shared ring (3 and 4 stages).  The loader waves stream the
// workgroup's (tile, k-step) positions in order,
// exactly as in the wave-specialised kernel.  MFMA group g computes the
// workgroup's tiles g, g + 2, ...: it waits for and releases only the
// positions of its own tiles, and each position is released by the one
// group that computes it.  While group g converts and stores its tile, the
// other group is already computing the next tile from the positions the
// loaders keep streaming, so the epilogue overlaps MFMA work; the two
// groups' main loops alternate.  A group's first wait for a tile lasts about
// one tile of the other group (far inside the bounded wait).
//
// One pipeline per group (C::DUAL, 2 stages).  Only one group computing at a
// time leaves one MFMA wave per SIMD issuing.  Here group g has a ring, full
// and empty counters and two loader waves of its own and streams its tiles
// g, g + 2, ... with the wave-specialised MFMA loop, so both groups compute
// at once; each group's epilogue overlaps the other group's main loop.
// ---------------------------------------------------------------------------
template <class C>
__global__ void __launch_bounds__(C::THREADS) k_gemm_pp(Params p)
{
    static_assert(C::SYNC == SYNC_PINGPONG && C::GROUPS == 2, "k_gemm_pp");
    __shared__ __attribute__((aligned(1024))) char smem_raw[C::LDS_BYTES];
    lds_char* smem = (lds_char*)smem_raw;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    constexpr int NCTR = C::PIPES * 2 * C::S;     // full[] and empty[] of every pipeline
    lds_u32* full = (lds_u32*)(smem + C::FLAG_OFFSET);
    lds_u32* empty = full + C::S;
    if (threadIdx.x < NCTR + 1)
        full[threadIdx.x] = 0u;   // the counters and the poison word
    __syncthreads();   // counters are initialised before the roles split
    SyncState st;
    st.poison = full + NCTR;
    st.limit = p.spin_limit;

    if constexpr (C::DUAL) {
        // One pipeline per group: group g owns ring g, counters g, loader
        // waves g * NLG .. + NLG - 1 and the workgroup's tiles g, g + 2, ...
        // The groups run side by side, each on its own tiles; the stagger
        // of their epilogues comes from the other group's work.
        constexpr int NLG = C::NP / C::GROUPS;
        const int32_t G = gridDim.x, b = blockIdx.x;
        const int32_t n_tiles = (b < p.tiles) ? (p.tiles - 1 - b) / G + 1 : 0;
        const int32_t KT = p.k_steps;
        const int g = (w < C::NCW) ? w / C::NCWG : (w - C::NCW) / NLG;
        const int32_t n_g = n_tiles > g ? (n_tiles - g + C::GROUPS - 1) / C::GROUPS : 0;
        lds_char* ring = smem + g * C::S * C::STAGE_BYTES;
        lds_u32* full_g = full + g * 2 * C::S;
        lds_u32* empty_g = full_g + C::S;
        if (w >= C::NCW) {
            producer_loop<C>(p, ring, full_g, empty_g, n_g, (w - C::NCW) % NLG, lane, st, g, C::GROUPS);
            return;
        }
        const int wg = w % C::NCWG;
        const int wm = wg / C::WN, wn = wg % C::WN;
        lds_char* strip = smem + C::EPI_OFFSET + w * C::EPI_WAVE_BYTES;
        const int32_t total = n_g * KT;
        if (total == 0)
            return;
        clock_begin(p);
        Frags<C> fr[2];
        wait_counter(full_g, (uint32_t)NLG, st);
        read_frags<C>(fr[0], ring, wm, wn, lane, 0);
        int32_t c = 0;
        for (int32_t j = 0; j < n_g; ++j) {
            int32_t tm, tn;
            int32_t sp, u;
            tile_coords(p, b + (g + C::GROUPS * j) * G, G, tm, tn, sp, u);
            typename C::Acc acc[C::FM][C::FN];
#pragma unroll
            for (int i = 0; i < C::FM; ++i)
#pragma unroll
                for (int jj = 0; jj < C::FN; ++jj)
                    acc[i][jj] = typename C::Acc{};
            for (int32_t kt = 0; kt < KT; ++kt, ++c) {
                const lds_char* stage = ring + (c % C::S) * C::STAGE_BYTES;
                auto region = [&]<int kk>() {
                    constexpr int M = region_mfmas<C>();
                    if constexpr (kk + 1 < C::KK) {
                        constexpr RegionReads rr = region_reads<C, kk>();
                        const FragReader<C> rdr(wm, wn, lane, rr.ks);
#pragma unroll
                        for (int d = 0; d < rr.d; ++d)
                            rdr.read(fr[rr.buf], stage, wn, d + rr.off);
                        region_mfma<C, kk, 0, M>(acc, fr);
                        sched_slots<M, rr.d, 0>();
                    } else {
                        const int s1 = (c + 1) % C::S;
                        consumer_last_kstep<C>(acc, fr, empty_g + c % C::S, full_g + s1,
                                               (uint32_t)((c + 1) / C::S + 1) * NLG, c + 1 < total,
                                               ring + s1 * C::STAGE_BYTES, wm, wn, lane, st);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                };
                [&]<int... KS>(std::integer_sequence<int, KS...>) {
                    (region.template operator()<KS>(), ...);
                }(std::make_integer_sequence<int, C::KK>{});
            }
            poison_tile<C>(acc, st);
            if (p.splits > 1)
                store_partial<C>(p, acc, sp * p.span + u, wm, wn, lane);
            else
                store_tile<C>(p, acc, strip, tm * C::BM, tn * C::BN, wm, wn, lane);
        }
        clock_end(p);
        return;
    }

    const int32_t G = gridDim.x, b = blockIdx.x;
    const int32_t n_tiles = (b < p.tiles) ? (p.tiles - 1 - b) / G + 1 : 0;
    const int32_t KT = p.k_steps;

    if (w >= C::NCW) {
        producer_loop<C>(p, smem, full, empty, n_tiles, w - C::NCW, lane, st);
        return;
    }

    // MFMA wave of group g: its tiles { wait full; read; release; MFMA } epilogue.
    const int g = w / C::NCWG, wg = w % C::NCWG;
    const int wm = wg / C::WN, wn = wg % C::WN;
    lds_char* strip = smem + C::EPI_OFFSET + w * C::EPI_WAVE_BYTES;
    auto stage_of = [&](int32_t q) { return smem + (q % C::S) * C::STAGE_BYTES; };
    Frags<C> fr[2];
    if (n_tiles > 0)
        clock_begin(p);
    for (int32_t it = g; it < n_tiles; it += 2) {
        int32_t tm, tn;
        int32_t sp, u;
        tile_coords(p, b + it * G, G, tm, tn, sp, u);
        int32_t c = it * KT;
        wait_counter_long(full + c % C::S, (uint32_t)(c / C::S + 1) * C::NP, st);
        read_frags<C>(fr[0], stage_of(c), wm, wn, lane, 0);
        typename C::Acc acc[C::FM][C::FN];
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
            for (int j = 0; j < C::FN; ++j)
                acc[i][j] = typename C::Acc{};
        for (int32_t kt = 0; kt < KT; ++kt, ++c) {
            const lds_char* stage = stage_of(c);
            auto region = [&]<int kk>() {
                constexpr int M = region_mfmas<C>();
                if constexpr (kk + 1 < C::KK) {
                    constexpr RegionReads rr = region_reads<C, kk>();
                    const FragReader<C> rdr(wm, wn, lane, rr.ks);
#pragma unroll
                    for (int d = 0; d < rr.d; ++d)
                        rdr.read(fr[rr.buf], stage, wn, d + rr.off);
                    region_mfma<C, kk, 0, M>(acc, fr);
                    sched_slots<M, rr.d, 0>();
                } else {
                    // The group's next position within this tile; the next
                    // tile's first position is waited for after the epilogue.
                    consumer_last_kstep<C>(acc, fr, empty + c % C::S, full + (c + 1) % C::S,
                                           (uint32_t)((c + 1) / C::S + 1) * C::NP, kt + 1 < KT, stage_of(c + 1),
                                           wm, wn, lane, st);
                }
                __builtin_amdgcn_sched_barrier(0);
            };
            [&]<int... KS>(std::integer_sequence<int, KS...>) {
                (region.template operator()<KS>(), ...);
            }(std::make_integer_sequence<int, C::KK>{});
        }
        poison_tile<C>(acc, st);
        if (p.splits > 1)
            store_partial<C>(p, acc, sp * p.span + u, wm, wn, lane);
        else
            store_tile<C>(p, acc, strip, tm * C::BM, tn * C::BN, wm, wn, lane);
    }
    if (n_tiles > 0)
        clock_end(p);
}

// C = 0 for K == 0 (16-byte stores, range-checked like the epilogue).
__global__ void __launch_bounds__(256) k_zero_fill(char* C, int64_t M, int64_t N, int64_t ldc)
{
    const int64_t chunks_per_row = N / 8;
    const int64_t total = M * chunks_per_row;
    for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < total;
         q += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = q / chunks_per_row, cch = q - r * chunks_per_row;
        *(u32x4_t*)(C + (r * ldc + cch * 8) * 2) = u32x4_t{0u, 0u, 0u, 0u};
    }
}

// dst[r][c] = src[r][c] inside the src_rows x src_cols source, 0 outside it,
// for the dst_rows x dst_cols destination (2-byte elements, any leading
// dimensions and 2-byte alignment).  Pads operands to multiples of 8 elements
// and copies a padded result back.  One thread per group of 8 destination
// columns: a 16-byte load or store where the address is 16-byte aligned and
// the whole group lies inside the matrix, element accesses otherwise.
__global__ void __launch_bounds__(256) k_pad_copy(const uint16_t* src, int64_t src_rows, int64_t src_cols,
                                                  int64_t ld_src, uint16_t* dst, int64_t dst_rows,
                                                  int64_t dst_cols, int64_t ld_dst)
{
    const int64_t groups_per_row = (dst_cols + 7) / 8;
    const int64_t total = dst_rows * groups_per_row;
    for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < total;
         q += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = q / groups_per_row, c0 = (q - r * groups_per_row) * 8;
        uint16_t v[8];
        const uint16_t* s = src + r * ld_src + c0;
        if (r < src_rows && c0 + 8 <= src_cols && ((uintptr_t)s & 15) == 0) {
            const u32x4_t x = *(const u32x4_t*)s;
            __builtin_memcpy(v, &x, 16);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                v[e] = (r < src_rows && c0 + e < src_cols) ? s[e] : (uint16_t)0;
        }
        uint16_t* d = dst + r * ld_dst + c0;
        if (c0 + 8 <= dst_cols && ((uintptr_t)d & 15) == 0) {
            u32x4_t x;
            __builtin_memcpy(&x, v, 16);
            *(u32x4_t*)d = x;
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (c0 + e < dst_cols)
                    d[e] = v[e];
        }
    }
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
// The kernel instance used for each (sync mode, stage count).  All-wave modes
// use a 256 x 256 tile over 8 waves (2 x 4, each 128 x 64, two waves per SIMD
// so that one can issue MFMAs while the other waits on a load) with 16 x 16
// MFMA blocks.  The wave-specialised 3-stage ring uses 4 MFMA waves (2 x 2
// over 256 x 128, one per SIMD, double-buffered fragments, 16 x 16 blocks)
// and 4 loader waves; the 2- and 4-stage rings are specialised below.  The
// k-step width follows the LDS budget (see BK below).
template <int SYNC, int S>
struct Pick {
    // 64-wide k-steps (128-byte rows per DMA instruction) wherever the ring
    // fits: two stages of 256 x 256, three of the wave-specialised 256 x 128.
    static constexpr int BK = (S == 2 || (SYNC == SYNC_WAVESPEC && S == 3)) ? 64 : 32;
    static_assert(SYNC != SYNC_WAVESPEC || S == 3, "the other wave-specialised rings are specialised below");
    template <bool BT>
    using type = Cfg<256, (SYNC == SYNC_WAVESPEC) ? 128 : 256, BK, S, 2, (SYNC == SYNC_WAVESPEC) ? 2 : 4, SYNC, BT,
                     (SYNC == SYNC_WAVESPEC) ? 4 : 0, false, 16>;
};

// The wave-specialised 2- and 4-stage rings: 8 MFMA waves (two per SIMD,
// 128 x 64 each) over a 256 x 256 tile next to 4 loader waves.  Three waves
// per SIMD leave each 168 registers: 128 accumulators and one fragment set of
// 32 x 32 blocks (24 registers) fit, two sets do not, so these MFMA waves run
// k_gemm_ws's single-buffered loop and rely on the other MFMA wave of their
// SIMD to cover their fragment reads.  Two 64-wide stages or four 32-wide
// ones fill 128 KiB.  The 2-stage ring uses 16 x 16 blocks instead, half a
// 32-wide k-step of fragments at a time (32 registers); with a K x N B that
// fits only because FragReader recomputes the lane-dependent offsets of the
// transposing B reads at every k-step instead of keeping them live.  The
// 3-stage ring keeps the 256 x 128 tile with one MFMA wave per SIMD and
// double-buffered fragments.
//
// The loaders' spread (the last Cfg argument, s_sleep units between pairs of
// DMA instructions) was measured per configuration on the three large
// workloads: 2 for the 2-stage ring (+1-8%; L2 misses per call 3.8 -> 2.1
// GB at 8192^3), 3 for the 4-stage ring (+3-4%).  The 3-stage ring keeps
// one burst (with a spread it measured up to 1% slower).
template <>
struct Pick<SYNC_WAVESPEC, 2> {
    template <bool BT>
    using type = Cfg<256, 256, 64, 2, 2, 4, SYNC_WAVESPEC, BT, 4, false, 16, false, 2>;
};

template <>
struct Pick<SYNC_WAVESPEC, 4> {
    template <bool BT>
    using type = Cfg<256, 256, 32, 4, 2, 4, SYNC_WAVESPEC, BT, 4, false, 32, false, 3>;
};

// Ping-pong: each of the two MFMA groups needs a wave on every SIMD, so
// with the loader waves a SIMD holds three waves and each has about a third
// of the register file: the groups' tiles are 128 x 128 (4 waves of 64 x 64).
// A stage is 32 KiB at 64-wide k-steps, so up to 4 stages fit in one shared
// ring, or two per group in the 2-stage instance's per-group rings.  The
// loaders sleep one unit between pairs of DMA instructions (measured 0-6%
// faster than one burst; longer sleeps starve these smaller stages).
template <int S>
struct Pick<SYNC_PINGPONG, S> {
    template <bool BT>
    using type = Cfg<128, 128, 64, S, 2, 2, SYNC_PINGPONG, BT, 4, false, 16, false, 1>;
};

template <>
struct Pick<SYNC_PINGPONG, 2> {
    template <bool BT>
    using type = Cfg<128, 128, 64, 2, 2, 2, SYNC_PINGPONG, BT, 4, false, 16, true, 1>;
};

// The split-window ring: the two-stage barrier instance's tile, waves and
// k-step over five windows (stages == GEMM_STAGES_WINDOWS).
template <>
struct Pick<SYNC_BARRIER, GEMM_STAGES_WINDOWS> {
    template <bool BT>
    using type = Cfg<256, 256, 64, 2, 2, 4, SYNC_BARRIER, BT, 0, true, 16>;
};

template <class C>
int launch(const Params& p, int64_t grid, hipStream_t stream)
{
    // Whole positions only (no per-lane edge masks) when K is a multiple of
    // the k-step and, for a K x N B, N of the tile width.  Split chunks are
    // multiples of 64 elements, so they split K evenly.
    const bool edge = (p.ksplit % C::BK != 0) || (!C::BT && p.N % C::BN != 0);
    const bool longk = p.k_steps >= C::LONGK_MIN_KT && p.small_span;
    const dim3 g((unsigned)grid), b(C::THREADS);
    if constexpr (C::SYNC == SYNC_WAVESPEC)
        hipLaunchKernelGGL(k_gemm_ws<C>, g, b, 0, stream, p);
    else if constexpr (C::SYNC == SYNC_PINGPONG)
        hipLaunchKernelGGL(k_gemm_pp<C>, g, b, 0, stream, p);
    else if constexpr (C::WIN) {
        if (longk && !edge)
            hipLaunchKernelGGL(HIP_KERNEL_NAME(k_gemm_win<C, true, false>), g, b, 0, stream, p);
        else if (longk)
            hipLaunchKernelGGL(HIP_KERNEL_NAME(k_gemm_win<C, true, true>), g, b, 0, stream, p);
        else
            hipLaunchKernelGGL(HIP_KERNEL_NAME(k_gemm_win<C, false, true>), g, b, 0, stream, p);
    } else {
        if (longk && !edge)
            hipLaunchKernelGGL(HIP_KERNEL_NAME(k_gemm<C, true, false>), g, b, 0, stream, p);
        else if (longk)
            hipLaunchKernelGGL(HIP_KERNEL_NAME(k_gemm<C, true, true>), g, b, 0, stream, p);
        else
            hipLaunchKernelGGL(HIP_KERNEL_NAME(k_gemm<C, false, true>), g, b, 0, stream, p);
    }
    return hipGetLastError() == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
}

struct Shape {
    int bm, bn, bk, mfma_waves, producer_waves, threads, lds_bytes, mfma_block, pipes;
};

template <class C>
Shape shape_of()
{
    return Shape{C::BM, C::BN, C::BK, C::NCW, C::NP, C::THREADS, C::LDS_BYTES, C::MF, C::PIPES};
}

// Calls f.template operator()<Cfg>() for the instance of (sync, stages, bt).
template <class F>
auto with_cfg(int sync_mode, int stages, bool bt, F&& f)
{
#define PTD_PICK(SY, ST)                                                            \
    if (sync_mode == SY && stages == ST)                                            \
        return bt ? f.template operator()<typename Pick<SY, ST>::template type<true>>() \
                  : f.template operator()<typename Pick<SY, ST>::template type<false>>();
    PTD_PICK(SYNC_BARRIER, 2) PTD_PICK(SYNC_BARRIER, 3) PTD_PICK(SYNC_BARRIER, 4)
    PTD_PICK(SYNC_BARRIER, GEMM_STAGES_WINDOWS)
    PTD_PICK(SYNC_FLAGS, 2) PTD_PICK(SYNC_FLAGS, 3) PTD_PICK(SYNC_FLAGS, 4)
    PTD_PICK(SYNC_WAVESPEC, 2) PTD_PICK(SYNC_WAVESPEC, 3)
    PTD_PICK(SYNC_PINGPONG, 2) PTD_PICK(SYNC_PINGPONG, 3) PTD_PICK(SYNC_PINGPONG, 4)
#undef PTD_PICK
    return bt ? f.template operator()<typename Pick<SYNC_WAVESPEC, 4>::template type<true>>()
              : f.template operator()<typename Pick<SYNC_WAVESPEC, 4>::template type<false>>();
}

// 64-wide k-steps: each DMA instruction then covers 8 rows of 128 bytes
// instead of 16 rows of 64, which the texture path serves markedly faster.
// The LDS holds two such stages of a 256 x 256 tile and three of the
// wave-specialised mode's 256 x 128.
// stages == 0: the split-window ring with barrier sync (level with the
// 2-stage ring at 8192^3, ahead of it by up to 4.5% on the other large
// shapes, same bits), 3 stages for ping-pong, 2 for the others.
int default_stages(int sync_mode)
{
    if (sync_mode == GEMM_SYNC_BARRIER)
        return GEMM_STAGES_WINDOWS;
    return sync_mode == GEMM_SYNC_PINGPONG ? 3 : 2;
}

// The allocation-free entry point's temporary memory: one region per GPU the
// library runs on, held until the process ends.  Its size covers every split
// workspace on a device of up to 256 compute units (a split has at most one
// 256 x 256 fp32 partial tile per compute unit); padded operand copies must
// fit beside it.  In host code `scratch` names a host-side stand-in: the
// device address is taken once per device with hipGetSymbolAddress (with
// that device current) and only that address is ever passed to a kernel.
constexpr int64_t kScratchBytes = GEMM_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];

// A block of temporary device memory (split workspace, padded operand
// copies) that the library keeps for later calls.
struct WsBlock {
    char* ptr = nullptr;
    int64_t bytes = 0;
    hipStream_t stream = nullptr;  // stream of the block's last use
    hipEvent_t done = nullptr;     // recorded on `stream` right after that use
    bool busy = false;             // taken by a call that has not handed it back
};

struct DeviceInfo {
    bool probed = false;
    int status = GEMM_OK;
    int cus = 0;
    // New temporary blocks are allocated from this stream-ordered pool (the
    // default pool if it could not be created).
    hipMemPool_t pool = nullptr;
    // The blocks kept for reuse (guarded by g_dev_mutex).  None is ever
    // freed: the runtime's stream-ordered free returns only once the
    // stream's queued work has finished, which would stall the caller for
    // the whole GPU time of every call that needs temporary memory.
    std::vector<WsBlock> blocks;
    // This device's copy of `scratch` (null if its address could not be
    // taken: the allocation-free entry point then returns GEMM_ERR_DEVICE).
    char* scratch_ptr = nullptr;
};

// Polls before a ring counter wait gives up, for every launch from now on.
std::atomic<uint32_t> g_spin_limit{kSpinLimit};

// Clock sampling (clock_begin / clock_end) for every launch from now on.
std::atomic<bool> g_clock_on{false};

constexpr int kMaxDevices = 64;
std::mutex g_dev_mutex;
DeviceInfo g_dev[kMaxDevices];

int device_info(int* cus, hipMemPool_t* pool = nullptr, char** scratch_ptr = nullptr, DeviceInfo** info = nullptr)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return GEMM_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(g_dev_mutex);
    DeviceInfo& d = g_dev[dev];
    if (!d.probed) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
            d.status = GEMM_ERR_DEVICE;
        } else {
            d.status = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? GEMM_OK : GEMM_ERR_DEVICE;
            d.cus = prop.multiProcessorCount;
        }
        if (d.status == GEMM_OK) {
            hipMemPoolProps props;
            memset(&props, 0, sizeof props);
            props.allocType = hipMemAllocationTypePinned;
            props.handleTypes = hipMemHandleTypeNone;
            props.location.type = hipMemLocationTypeDevice;
            props.location.id = dev;
            hipMemPool_t pl = nullptr;
            if (hipMemPoolCreate(&pl, &props) == hipSuccess && pl) {
                uint64_t keep = UINT64_MAX;
                if (hipMemPoolSetAttribute(pl, hipMemPoolAttrReleaseThreshold, &keep) == hipSuccess)
                    d.pool = pl;
                else
                    (void)hipMemPoolDestroy(pl);
            }
            void* sp = nullptr;
            if (hipGetSymbolAddress(&sp, HIP_SYMBOL(scratch)) == hipSuccess && sp)
                d.scratch_ptr = (char*)sp;
            else
                (void)hipGetLastError();   // leave no sticky error behind for the caller's next call
        }
        d.probed = true;
    }
    *cus = d.cus;
    if (info)
        *info = &d;
    if (pool)
        *pool = d.pool;
    if (scratch_ptr)
        *scratch_ptr = d.scratch_ptr;
    return d.status;
}

// Where a call's temporary device memory (split workspaces, padded operand
// copies) comes from.  Kept (fixed == nullptr): the device's reusable blocks
// (temp_take).  Fixed: consecutive pieces of this device's scratch region,
// taken in order and never released; nothing is allocated or freed.
struct TempMem {
    DeviceInfo* info = nullptr;
    hipMemPool_t pool = nullptr;
    char* fixed = nullptr;
    int64_t fixed_left = 0;
};

int64_t align256(int64_t b)
{
    return (b + 255) & ~(int64_t)255;
}

hipError_t pool_alloc(const TempMem& t, void** p, int64_t bytes, hipStream_t s)
{
    return t.pool ? hipMallocFromPoolAsync(p, (size_t)bytes, t.pool, s) : hipMallocAsync(p, (size_t)bytes, s);
}

// Temporary memory of `bytes` for one call on stream s, handed back with
// temp_give once the call's work on it is enqueued.
//
// Kept blocks: the smallest free block that is large enough and either was
// last used on s (stream order puts that use before this one) or whose
// completion event has fired.  Without one, a new block -- the size rounded
// up to a power of two, at least 1 MiB, so that one block serves a range of
// calls -- is allocated stream-ordered on s and kept.  Calls on one stream
// therefore reuse one block per size they need at once, and each stream that
// runs such calls at the same time as another holds its own.
//
// Under graph capture the memory is allocated and freed inside the graph
// instead (nothing runs at capture, so the free does not stall), as each
// replay's own allocation.
int temp_take(TempMem& t, int64_t bytes, hipStream_t s, void** p, hipEvent_t* done = nullptr)
{
    *p = nullptr;
    if (done)
        *done = nullptr;
    if (t.fixed) {
        const int64_t need = align256(bytes);
        if (need > t.fixed_left)
            return GEMM_ERR_SCRATCH;
        *p = t.fixed;
        t.fixed += need;
        t.fixed_left -= need;
        return GEMM_OK;
    }
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) != hipSuccess) {
        (void)hipGetLastError();
        return GEMM_ERR_DEVICE;
    }
    if (cs != hipStreamCaptureStatusNone) {
        const hipError_t e = pool_alloc(t, p, bytes, s);
        return (e == hipSuccess && *p) ? GEMM_OK : GEMM_ERR_DEVICE;
    }
    std::lock_guard<std::mutex> lock(g_dev_mutex);
    std::vector<WsBlock>& v = t.info->blocks;
    int best = -1;
    for (int i = 0; i < (int)v.size(); ++i) {
        const WsBlock& b = v[i];
        if (b.busy || b.bytes < bytes || (best >= 0 && v[best].bytes <= b.bytes))
            continue;
        if (b.stream != s && hipEventQuery(b.done) != hipSuccess) {
            (void)hipGetLastError();   // not finished yet: no error for the caller's next call
            continue;
        }
        best = i;
    }
    if (best < 0) {
        int64_t size = (int64_t)1 << 20;
        while (size < bytes)
            size <<= 1;
        WsBlock b;
        if (hipEventCreateWithFlags(&b.done, hipEventDisableTiming) != hipSuccess) {
            (void)hipGetLastError();
            return GEMM_ERR_DEVICE;
        }
        void* q = nullptr;
        if (pool_alloc(t, &q, size, s) != hipSuccess || !q) {
            (void)hipEventDestroy(b.done);
            (void)hipGetLastError();
            return GEMM_ERR_DEVICE;
        }
        b.ptr = (char*)q;
        b.bytes = size;
        v.push_back(b);
        best = (int)v.size() - 1;
    }
    v[best].busy = true;
    v[best].stream = s;
    *p = v[best].ptr;
    if (done)
        *done = v[best].done;
    return GEMM_OK;
}

// Hands back what temp_take gave: a kept block becomes free once its
// completion event is recorded on s after the call's work on it -- here, or,
// with `recorded`, already by the launch of the last kernel that uses it
// (as that kernel's completion, with no separate marker on the stream);
// memory taken under graph capture is freed in the graph.
int temp_give(const TempMem& t, void* p, hipStream_t s, bool recorded = false)
{
    if (t.fixed || !p)
        return GEMM_OK;
    {
        std::lock_guard<std::mutex> lock(g_dev_mutex);
        for (WsBlock& b : t.info->blocks)
            if (b.busy && b.ptr == (char*)p) {
                if (!recorded && hipEventRecord(b.done, s) != hipSuccess) {
                    // Its last use has no event to wait on: it stays taken.
                    (void)hipGetLastError();
                    return GEMM_ERR_DEVICE;
                }
                b.busy = false;
                return GEMM_OK;
            }
    }
    return hipFreeAsync(p, s) == hipSuccess ? GEMM_OK : GEMM_ERR_DEVICE;
}

bool overlaps(const void* a, int64_t a_bytes, const void* b, int64_t b_bytes)
{
    if (a_bytes <= 0 || b_bytes <= 0)
        return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + (uintptr_t)b_bytes && b0 < a0 + (uintptr_t)a_bytes;
}

int64_t span_bytes(int64_t rows, int64_t cols, int64_t ld)
{
    return (rows <= 0 || cols <= 0) ? 0 : ((rows - 1) * ld + cols) * 2;
}

constexpr int64_t kMaxLd = (int64_t)1 << 22;
constexpr int64_t kMaxSplits = 16;

int validate_shape(int64_t M, int64_t N, int64_t K, int stages, int sync_mode)
{
    if (sync_mode != GEMM_SYNC_BARRIER && sync_mode != GEMM_SYNC_FLAGS && sync_mode != GEMM_SYNC_WAVESPEC &&
        sync_mode != GEMM_SYNC_PINGPONG)
        return GEMM_ERR_SYNC_MODE;
    if (stages != 0 && (stages < 2 || stages > 4) &&
        !(stages == GEMM_STAGES_WINDOWS && sync_mode == GEMM_SYNC_BARRIER))
        return GEMM_ERR_STAGES;
    if (M < 0 || N < 0 || K < 0)
        return GEMM_ERR_INVALID_VALUE;
    // Leading dimensions of at least N and K, rounded up to 8, must fit the
    // loads' 2^22-element row stride.
    if (M > ((int64_t)1 << 31) - 1 || N > kMaxLd || K > kMaxLd)
        return GEMM_ERR_UNSUPPORTED_SHAPE;
    return GEMM_OK;
}

int64_t round8(int64_t x)
{
    return (x + 7) & ~(int64_t)7;
}

// Which operands a call copies into zero-padded compact buffers.  K off the
// 8-element grid pads A and B along k; N off the grid pads B's n extent and
// C's columns; otherwise an operand is copied only if its own leading
// dimension or pointer does not suit the kernels' 16-byte row segments.
struct PadSet {
    bool a, b, c;
};

PadSet pad_set(int64_t N, int64_t K, bool a_ok, bool b_ok, bool c_ok)
{
    const bool k_off = K % 8 != 0, n_off = N % 8 != 0;
    return PadSet{k_off || !a_ok, k_off || n_off || !b_ok, n_off || !c_ok};
}

// Bytes of those copies (256-byte aligned parts): A as M x K8, B as N8 x K8
// (stored N x K) or K8 x N8, C as M x N8.
int64_t pad_bytes(int64_t M, int64_t N, int64_t K, PadSet ps)
{
    auto up = [](int64_t b) { return (b + 255) & ~(int64_t)255; };
    const int64_t N8 = round8(N), K8 = round8(K);
    const int64_t a = (ps.a && K > 0) ? M * K8 * 2 : 0;
    const int64_t b = (ps.b && K > 0) ? N8 * K8 * 2 : 0;
    const int64_t c = ps.c ? M * N8 * 2 : 0;
    return up(a) + up(b) + up(c);
}

// Number of k chunks.  Shapes with at most half as many output tiles (in
// the configuration's tile) as pipelines and a long k range are split into
// equal chunks of a multiple of 64 elements, each at least 512 long, so that
// tiles x chunks work items can fill the GPU.  `cus` counts pipelines: the
// compute units times the independent pipelines one workgroup runs (two where
// each MFMA group has its own ring and takes every other work item).
// Configurations with different tiles or pipeline counts may therefore split
// a shape differently.
int64_t choose_splits(int64_t tiles, int64_t K, int cus)
{
    if (tiles <= 0 || 2 * tiles > cus)
        return 1;
    int64_t s = cus / tiles;
    if (s > kMaxSplits)
        s = kMaxSplits;
    for (; s >= 2; --s)
        if (K % (64 * s) == 0 && K / s >= 512)
            return s;
    return 1;
}

// Split tail.  When the output tiles do not fill whole rounds of the
// persistent grid and the last round would leave at least half the compute
// units idle, the last r tiles of the raster become a second launch whose k
// range is split into s chunks: that round then takes about 1/s of a tile's
// time, plus one fp32 partial tile per chunk and a reduction.  A nearly idle
// last round runs at a raised clock under the board's power limit, so the
// split only pays when it removes much work from that round: chunks of at
// least 1024 elements (a multiple of 64), and at least 2048 elements of the
// k range taken off each tail tile (measured: K = 2048 lost with 2 or 4
// chunks, K = 4096 gained 3-14%).  Returns s (0: no split tail) and sets r.
int64_t choose_tail_splits(int64_t tiles, int64_t K, int cus, int64_t& r)
{
    r = 0;
    if (tiles <= cus)
        return 0;
    const int64_t rem = tiles % cus;
    if (rem == 0 || 2 * rem > cus)
        return 0;
    int64_t s = cus / rem;
    if (s > kMaxSplits)
        s = kMaxSplits;
    for (; s >= 2; --s)
        if (K % (64 * s) == 0 && K / s >= 1024 && K - K / s >= 2048) {
            r = rem;
            return s;
        }
    return 0;
}

// The plan of the kernels' launch.  N or K that is not a multiple of 8 is
// run on zero-padded copies (N and K rounded up to 8), so the plan is that of
// the padded problem.
int fill_plan(int64_t M, int64_t N_in, int64_t K_in, int b_transposed, int stages, int sync_mode, int cus,
              gemm_bf16_plan_t* out)
{
    const int64_t N = round8(N_in), K = round8(K_in);
    const int st = stages == 0 ? default_stages(sync_mode) : stages;
    const Shape v = with_cfg(sync_mode, st, b_transposed != 0, []<class C>() { return shape_of<C>(); });
    gemm_bf16_plan_t pl;
    memset(&pl, 0, sizeof pl);
    pl.bm = v.bm;
    pl.bn = v.bn;
    pl.bk = v.bk;
    pl.stages = st;
    pl.sync_mode = sync_mode;
    pl.b_transposed = b_transposed ? 1 : 0;
    pl.mfma_waves = v.mfma_waves;
    pl.producer_waves = v.producer_waves;
    pl.threads = v.threads;
    pl.lds_bytes = v.lds_bytes;
    pl.mfma_block = v.mfma_block;
    pl.pipelines = v.pipes;
    const int64_t tm = (M + v.bm - 1) / v.bm, tn = (N + v.bn - 1) / v.bn;
    pl.tiles = tm * tn;
    pl.k_splits = choose_splits(pl.tiles, K, cus * v.pipes);
    pl.k_steps = (K / pl.k_splits + v.bk - 1) / v.bk;
    if (pl.k_splits == 1)
        pl.tail_splits = choose_tail_splits(pl.tiles, K, cus, pl.tail_tiles);
    const int64_t items = (pl.tiles - pl.tail_tiles) * pl.k_splits;
    pl.grid = items < cus ? items : cus;
    pl.workspace_bytes = pl.k_splits > 1 ? items * v.bm * v.bn * 4 : pl.tail_tiles * pl.tail_splits * v.bm * v.bn * 4;
    if (items > ((int64_t)1 << 30) || items * pl.k_steps > ((int64_t)1 << 30))
        return GEMM_ERR_UNSUPPORTED_SHAPE;
    pl.pad_bytes = (N != N_in || K != K_in)
                       ? pad_bytes(M, N_in, K_in, pad_set(N_in, K_in, true, true, true))
                       : 0;
    *out = pl;
    return GEMM_OK;
}

int gemm_direct(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb, void* C,
                int64_t ldc, int stages, int sync_mode, hipStream_t s, bool bt, int cus, TempMem& tm);

int launch_pad_copy(const void* src, int64_t src_rows, int64_t src_cols, int64_t ld_src, void* dst, int64_t dst_rows,
                    int64_t dst_cols, int64_t ld_dst, hipStream_t s)
{
    const int64_t total = dst_rows * ((dst_cols + 7) / 8);
    if (total == 0)
        return GEMM_OK;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536)
        blocks = 65536;
    hipLaunchKernelGGL(k_pad_copy, dim3((unsigned)blocks), dim3(256), 0, s, (const uint16_t*)src, src_rows, src_cols,
                       ld_src, (uint16_t*)dst, dst_rows, dst_cols, ld_dst);
    return hipGetLastError() == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
}

// Shapes, leading dimensions or pointers the kernels cannot address directly:
// the operands pad_set names are copied, zero-padded, into compact buffers
// whose rows are multiples of 8 elements (N and K rounded up to 8), the GEMM
// runs on those (and on the operands used in place), and the valid N columns
// of a padded result are copied into C.  Zero k-columns add only zero
// products, so the result is that of the unpadded problem.  The copies live
// in temporary memory taken for this call (see TempMem).
int gemm_padded(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb, void* C,
                int64_t ldc, int stages, int sync_mode, hipStream_t s, bool bt, int cus, TempMem& tm, PadSet ps)
{
    const int64_t N8 = round8(N), K8 = round8(K);
    const int64_t b_rows = bt ? N8 : K8, b_cols = bt ? K8 : N8;
    const int64_t a_bytes = (ps.a && K > 0) ? M * K8 * 2 : 0;
    const int64_t b_bytes = (ps.b && K > 0) ? b_rows * b_cols * 2 : 0;
    const int64_t bytes = pad_bytes(M, N, K, ps);
    void* ws = nullptr;
    int rc = temp_take(tm, bytes, s, &ws);
    if (rc != GEMM_OK)
        return rc;
    char* a2 = (char*)ws;
    char* b2 = a2 + align256(a_bytes);
    char* c2 = b2 + align256(b_bytes);
    const void* a_use = A;
    const void* b_use = B;
    void* c_use = ps.c ? (void*)c2 : C;
    int64_t lda_use = lda, ldb_use = ldb, ldc_use = ps.c ? N8 : ldc;
    if (K > 0 && ps.a) {
        rc = launch_pad_copy(A, M, K, lda, a2, M, K8, K8, s);
        a_use = a2;
        lda_use = K8;
    }
    if (K > 0 && ps.b && rc == GEMM_OK) {
        rc = launch_pad_copy(B, bt ? N : K, bt ? K : N, ldb, b2, b_rows, b_cols, b_cols, s);
        b_use = b2;
        ldb_use = b_cols;
    }
    if (rc == GEMM_OK)
        rc = gemm_direct(M, N8, K8, K > 0 ? a_use : nullptr, lda_use, K > 0 ? b_use : nullptr, ldb_use, c_use, ldc_use,
                         stages, sync_mode, s, bt, cus, tm);
    if (rc == GEMM_OK && ps.c)
        rc = launch_pad_copy(c2, M, N8, N8, C, M, N, ldc, s);
    const int frc = temp_give(tm, ws, s);
    return rc != GEMM_OK ? rc : frc;
}

// Every GEMM entry point: validation, device, then the padded or the direct
// path.  noalloc: temporary memory comes from the device's scratch region
// (checked up front, so a call that does not fit enqueues nothing) instead
// of the pool.
int gemm_entry(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
               void* C, int64_t ldc, int stages, int sync_mode, void* stream, bool bt, bool noalloc)
{
    int rc = validate_shape(M, N, K, stages, sync_mode);
    if (rc != GEMM_OK)
        return rc;
    if (M == 0 || N == 0)
        return GEMM_OK;
    const bool reads = K > 0;
    if (!C || (reads && (!A || !B)))
        return GEMM_ERR_INVALID_VALUE;
    if (ldc < N || (reads && (lda < K || ldb < (bt ? K : N))))
        return GEMM_ERR_INVALID_VALUE;
    if (((uintptr_t)C & 1) != 0 || (reads && (((uintptr_t)A & 1) != 0 || ((uintptr_t)B & 1) != 0)))
        return GEMM_ERR_MISALIGNED;
    const int64_t c_bytes = span_bytes(M, N, ldc);
    if (reads && (overlaps(C, c_bytes, A, span_bytes(M, K, lda)) ||
                  overlaps(C, c_bytes, B, bt ? span_bytes(N, K, ldb) : span_bytes(K, N, ldb))))
        return GEMM_ERR_ALIAS;

    int cus = 0;
    TempMem tm;
    char* scratch_ptr = nullptr;
    rc = device_info(&cus, &tm.pool, &scratch_ptr, &tm.info);
    if (rc != GEMM_OK)
        return rc;
    hipStream_t s = (hipStream_t)stream;
    // The kernels load and store 16-byte row segments: every row must start on
    // a 16-byte boundary, and a row stride must fit the loads' offsets.
    // Anything else runs on zero-padded copies of the operands that need them.
    auto fits = [](const void* ptr, int64_t ld) { return ld % 8 == 0 && ld <= kMaxLd && ((uintptr_t)ptr & 15) == 0; };
    const PadSet ps = pad_set(N, K, !reads || fits(A, lda), !reads || fits(B, ldb), fits(C, ldc));
    const bool padded = ps.a || ps.b || ps.c;
    if (noalloc) {
        if (!scratch_ptr)
            return GEMM_ERR_DEVICE;
        tm.pool = nullptr;
        tm.fixed = scratch_ptr;
        tm.fixed_left = kScratchBytes;
        // Everything the call takes: the padded copies, then the split
        // workspace of the (padded) problem.
        int64_t need = padded ? align256(pad_bytes(M, N, K, ps)) : 0;
        if (reads) {
            gemm_bf16_plan_t pl;
            rc = fill_plan(M, N, K, bt, stages, sync_mode, cus, &pl);
            if (rc != GEMM_OK)
                return rc;
            need += align256(pl.workspace_bytes);
        }
        if (need > kScratchBytes)
            return GEMM_ERR_SCRATCH;
    }
    if (padded)
        return gemm_padded(M, N, K, A, lda, B, ldb, C, ldc, stages, sync_mode, s, bt, cus, tm, ps);
    return gemm_direct(M, N, K, A, lda, B, ldb, C, ldc, stages, sync_mode, s, bt, cus, tm);
}

// The fast path: N and K multiples of 8, operands addressable directly.
int gemm_direct(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb, void* C,
                int64_t ldc, int stages, int sync_mode, hipStream_t s, bool bt, int cus, TempMem& tm)
{
    int rc = GEMM_OK;
    const bool reads = K > 0;
    if (!reads) {
        const int64_t chunks = M * (N / 8);
        int64_t blocks = (chunks + 255) / 256;
        if (blocks > 65536)
            blocks = 65536;
        hipLaunchKernelGGL(k_zero_fill, dim3((unsigned)blocks), dim3(256), 0, s, (char*)C, M, N, ldc);
        return hipGetLastError() == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
    }
    gemm_bf16_plan_t pl;
    rc = fill_plan(M, N, K, bt, stages, sync_mode, cus, &pl);
    if (rc != GEMM_OK)
        return rc;
    Params p;
    p.A = (const char*)A;
    p.B = (const char*)B;
    p.C = (char*)C;
    p.M = M;
    p.N = N;
    p.K = K;
    p.lda = lda;
    p.ldb = ldb;
    p.ldc = ldc;
    p.tiles_m = (int32_t)((M + pl.bm - 1) / pl.bm);
    p.tiles_n = (int32_t)((N + pl.bn - 1) / pl.bn);
    p.tiles_mn = (int32_t)pl.tiles;
    p.splits = (int32_t)pl.k_splits;
    p.ksplit = K / pl.k_splits;
    p.span = (int32_t)(pl.tiles - pl.tail_tiles);
    p.tile_base = 0;
    p.tiles = p.span * p.splits;
    p.k_steps = (int32_t)pl.k_steps;
    p.group_m = 4;
    // The stepping load cursor addresses a whole operand from one resource
    // per tile, so it needs exact byte counts below kMaxRecords.
    p.small_span = span_bytes(M, K, lda) < (int64_t)kMaxRecords &&
                   (bt ? span_bytes(N, K, ldb) : span_bytes(K, N, ldb)) < (int64_t)kMaxRecords;
    p.partial = nullptr;
    p.spin_limit = g_spin_limit.load(std::memory_order_relaxed);
    p.clock_on = g_clock_on.load(std::memory_order_relaxed) ? 1u : 0u;
    const int64_t grid = pl.grid;
    if (p.splits == 1 && pl.tail_tiles == 0)
        return with_cfg(sync_mode, pl.stages, bt, [&]<class C>() { return launch<C>(p, grid, s); });

    // Split k range (all tiles, or the tail): fp32 partial tiles in
    // temporary memory taken for this call (pooled: stream-ordered memory
    // that lives for this call only, so calls on different streams never
    // share it).
    void* ws = nullptr;
    hipEvent_t ws_done = nullptr;   // the kept block's completion event (null: none to record)
    rc = temp_take(tm, pl.workspace_bytes, s, &ws, &ws_done);
    if (rc != GEMM_OK)
        return rc;
    Params q = p;   // the launch whose partial tiles are reduced
    if (pl.tail_tiles > 0) {
        rc = with_cfg(sync_mode, pl.stages, bt, [&]<class C>() { return launch<C>(p, grid, s); });
        q.splits = (int32_t)pl.tail_splits;
        q.ksplit = K / pl.tail_splits;
        q.span = (int32_t)pl.tail_tiles;
        q.tile_base = p.span;
        q.tiles = q.span * q.splits;
        q.k_steps = (int32_t)((q.ksplit + pl.bk - 1) / pl.bk);
    }
    q.partial = (float*)ws;
    if (rc == GEMM_OK) {
        const int64_t tail_grid = q.tiles < cus ? q.tiles : cus;
        rc = with_cfg(sync_mode, pl.stages, bt,
                      [&]<class C>() { return launch<C>(q, pl.tail_tiles > 0 ? tail_grid : grid, s); });
    }
    if (rc == GEMM_OK) {
        const int64_t units = (int64_t)q.span * pl.bm * pl.bn / 4;
        int64_t blocks = (units + 255) / 256;
        if (blocks > 65536)
            blocks = 65536;
        // The reduction is the workspace's last use: its completion records
        // the block's event.
        rc = with_cfg(sync_mode, pl.stages, bt, [&]<class C>() {
            hipExtLaunchKernelGGL(k_reduce_splits<C>, dim3((unsigned)blocks), dim3(256), 0, s, nullptr, ws_done, 0,
                                  q);
            return hipGetLastError() == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
        });
    }
    const int frc = temp_give(tm, ws, s, rc == GEMM_OK && ws_done != nullptr);
    return rc != GEMM_OK ? rc : frc;
}

}  // namespace

extern "C" {

int gemm_bf16(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
              void* C, int64_t ldc, int stages, int sync_mode, void* stream)
{
    return gemm_entry(M, N, K, A, lda, B, ldb, C, ldc, stages, sync_mode, stream, false, false);
}

int gemm_bf16_bt(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
                 void* C, int64_t ldc, int stages, int sync_mode, void* stream)
{
    return gemm_entry(M, N, K, A, lda, B, ldb, C, ldc, stages, sync_mode, stream, true, false);
}

int gemm_bf16_noalloc(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
                      void* C, int64_t ldc, int stages, int sync_mode, void* stream)
{
    return gemm_entry(M, N, K, A, lda, B, ldb, C, ldc, stages, sync_mode, stream, false, true);
}

int gemm_bf16_plan(int64_t M, int64_t N, int64_t K, int b_transposed, int stages, int sync_mode,
                   gemm_bf16_plan_t* out)
{
    if (!out)
        return GEMM_ERR_INVALID_VALUE;
    int rc = validate_shape(M, N, K, stages, sync_mode);
    if (rc != GEMM_OK)
        return rc;
    int cus = 0;
    rc = device_info(&cus);
    if (rc != GEMM_OK)
        return rc;
    return fill_plan(M, N, K, b_transposed, stages, sync_mode, cus, out);
}

int gemm_bf16_plan_cus(int64_t M, int64_t N, int64_t K, int b_transposed, int stages, int sync_mode,
                       int compute_units, gemm_bf16_plan_t* out)
{
    if (!out || compute_units < 1)
        return GEMM_ERR_INVALID_VALUE;
    const int rc = validate_shape(M, N, K, stages, sync_mode);
    if (rc != GEMM_OK)
        return rc;
    return fill_plan(M, N, K, b_transposed, stages, sync_mode, compute_units, out);
}

const char* gemm_bf16_strerror(int status)
{
    switch (status) {
    case GEMM_OK: return "success";
    case GEMM_ERR_INVALID_VALUE: return "invalid value (negative size, NULL pointer or leading dimension too small)";
    case GEMM_ERR_MISALIGNED: return "misaligned operand (bf16 pointers need 2-byte alignment)";
    case GEMM_ERR_UNSUPPORTED_SHAPE: return "unsupported shape (N and K at most 2^22, M below 2^31)";
    case GEMM_ERR_STAGES: return "stages must be 0 (default), 2, 3, 4, or 5 (split-window ring, barrier sync)";
    case GEMM_ERR_SYNC_MODE:
        return "sync_mode must be GEMM_SYNC_BARRIER, GEMM_SYNC_FLAGS, GEMM_SYNC_WAVESPEC or GEMM_SYNC_PINGPONG";
    case GEMM_ERR_DEVICE: return "no usable device (the current HIP device must be gfx950)";
    case GEMM_ERR_LAUNCH: return "kernel launch failed";
    case GEMM_ERR_ALIAS: return "C overlaps A or B";
    case GEMM_ERR_SCRATCH:
        return "the call needs more temporary memory than gemm_bf16_noalloc's scratch region "
               "(GEMM_NOALLOC_SCRATCH_BYTES) holds";
    default: return "unknown status";
    }
}

int64_t gemm_bf16_set_sync_spin_limit(int64_t polls)
{
    if (polls < 0 || polls > (int64_t)UINT32_MAX)
        return GEMM_ERR_INVALID_VALUE;
    return (int64_t)g_spin_limit.exchange(polls == 0 ? kSpinLimit : (uint32_t)polls);
}

int64_t gemm_bf16_sync_timeouts(int reset)
{
    int cus = 0;
    int rc = device_info(&cus);
    if (rc != GEMM_OK)
        return rc;
    if (hipDeviceSynchronize() != hipSuccess)
        return GEMM_ERR_DEVICE;
    unsigned long long v = 0;
    if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_sync_timeouts), sizeof v, 0, hipMemcpyDeviceToHost) != hipSuccess)
        return GEMM_ERR_DEVICE;
    if (reset) {
        const unsigned long long zero = 0;
        if (hipMemcpyToSymbol(HIP_SYMBOL(g_sync_timeouts), &zero, sizeof zero, 0, hipMemcpyHostToDevice) != hipSuccess)
            return GEMM_ERR_DEVICE;
    }
    return (int64_t)v;
}

int gemm_bf16_workspace_info(int64_t* blocks, int64_t* bytes, int64_t* busy)
{
    if (!blocks || !bytes || !busy)
        return GEMM_ERR_INVALID_VALUE;
    int cus = 0;
    DeviceInfo* info = nullptr;
    int rc = device_info(&cus, nullptr, nullptr, &info);
    if (rc != GEMM_OK)
        return rc;
    std::lock_guard<std::mutex> lock(g_dev_mutex);
    *blocks = (int64_t)info->blocks.size();
    *bytes = 0;
    *busy = 0;
    for (const WsBlock& b : info->blocks) {
        *bytes += b.bytes;
        *busy += b.busy ? 1 : 0;
    }
    return GEMM_OK;
}

int gemm_bf16_release_workspaces(void)
{
    int cus = 0;
    DeviceInfo* info = nullptr;
    int rc = device_info(&cus, nullptr, nullptr, &info);
    if (rc != GEMM_OK)
        return rc;
    // Under the lock no call can take a block; the device synchronisation
    // then finishes every use already enqueued, so the free blocks are idle.
    std::lock_guard<std::mutex> lock(g_dev_mutex);
    if (hipDeviceSynchronize() != hipSuccess) {
        (void)hipGetLastError();
        return GEMM_ERR_DEVICE;
    }
    int status = GEMM_OK;
    std::vector<WsBlock> keep;
    for (WsBlock& b : info->blocks) {
        // A block is busy only while a call on another thread enqueues its
        // work; that call still owns it.
        if (!b.busy && hipFreeAsync(b.ptr, nullptr) == hipSuccess) {
            (void)hipEventDestroy(b.done);
            continue;
        }
        if (!b.busy) {
            (void)hipGetLastError();
            status = GEMM_ERR_DEVICE;
        }
        keep.push_back(b);
    }
    info->blocks.swap(keep);
    if (hipStreamSynchronize(nullptr) != hipSuccess) {
        (void)hipGetLastError();
        status = GEMM_ERR_DEVICE;
    }
    if (info->pool && hipMemPoolTrimTo(info->pool, 0) != hipSuccess) {
        (void)hipGetLastError();
        status = GEMM_ERR_DEVICE;
    }
    return status;
}

int gemm_bf16_set_clock_sampling(int enable)
{
    return g_clock_on.exchange(enable != 0) ? 1 : 0;
}

int gemm_bf16_clock_samples(uint64_t* out, int reset)
{
    if (!out)
        return GEMM_ERR_INVALID_VALUE;
    int cus = 0;
    int rc = device_info(&cus);
    if (rc != GEMM_OK)
        return rc;
    int dev = 0, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0)
        return GEMM_ERR_DEVICE;
    if (hipDeviceSynchronize() != hipSuccess)
        return GEMM_ERR_DEVICE;
    static unsigned long long v[kClockSlots][16];   // guarded by g_dev_mutex
    std::lock_guard<std::mutex> lock(g_dev_mutex);
    if (hipMemcpyFromSymbol(v, HIP_SYMBOL(g_clock_sums), sizeof v, 0, hipMemcpyDeviceToHost) != hipSuccess)
        return GEMM_ERR_DEVICE;
    uint64_t sum[3] = {0, 0, 0};
    for (int i = 0; i < kClockSlots; ++i)
        for (int j = 0; j < 3; ++j)
            sum[j] += v[i][j];
    if (reset) {
        memset(v, 0, sizeof v);
        if (hipMemcpyToSymbol(HIP_SYMBOL(g_clock_sums), v, sizeof v, 0, hipMemcpyHostToDevice) != hipSuccess)
            return GEMM_ERR_DEVICE;
    }
    out[0] = sum[0];
    out[1] = sum[1];
    out[2] = sum[2];
    out[3] = (uint64_t)khz * 1000u;
    return GEMM_OK;
}

}  // extern "C"
