// Hardware-semantics probes for gfx950 (MI355X).
//
// The GEMM kernels rely on four instruction behaviours that the compiler
// builtins do not document in full.  Each probe runs one 64-lane wave on
// fixed-size buffers, records what the instruction produced, and returns it
// to the host, where a test compares it with the layout the kernels assume:
//   - global_load_lds_dwordx4: which LDS bytes each lane's 16-byte load lands
//     in, and that s_waitcnt vmcnt(0) covers the LDS write;
//   - v_mfma_f32_32x32x16_bf16 and v_mfma_f32_16x16x32_bf16: the operand and
//     accumulator lane layouts;
//   - ds_read_b64_tr_b16: which lane receives which 16-bit element;
//   - the fp32 -> bf16 conversion used by the epilogue (rounding mode);
//   - buffer range checking, with and without a scalar offset.
// Two more entry points are measurements rather than semantics probes: the
// matrix-core throughput the board sustains under its power limit on given
// operand data, with no global memory traffic (gemm_probe_mfma_ceiling), and
// the LDS read bandwidth of one compute unit in bytes per shader clock
// (gemm_probe_lds_read_bw).
// All accesses stay inside the buffers whose sizes are stated per entry
// point; the host wrapper checks pointer arguments before launching.
#include <hip/hip_runtime.h>
#include <stdint.h>

#define LDS_AS __attribute__((address_space(3)))

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) short i16x4_t;

namespace {

constexpr int kProbeLdsWords = 2048;   // 8 KiB of LDS per probe

// Each lane l fetches the 16-byte chunk src[perm[l]] and the hardware writes
// it into LDS at (lds_base_bytes + inst_offset + 16 * l) if the assumed layout
// holds.  Two loads are issued: one with the instruction offset 0 and one
// with 1024 bytes (which moves the global address by the same amount).  The whole 8 KiB window is then copied out.  src holds
// 128 chunks; perm holds 64 entries, taken modulo 64.
__global__ void __launch_bounds__(64) k_lds_dma(const uint4* __restrict__ src,
                                                const int* __restrict__ perm,
                                                int lds_base_bytes,
                                                uint32_t* __restrict__ dump)
{
    __shared__ __attribute__((aligned(16))) uint32_t lds[kProbeLdsWords];
    const int l = threadIdx.x;
    for (int i = l; i < kProbeLdsWords; i += 64)
        lds[i] = 0xDEADBEEFu;
    __syncthreads();
    char LDS_AS* base = (char LDS_AS*)lds + lds_base_bytes;
    const int p = perm[l] & 63;
    __builtin_amdgcn_global_load_lds(src + p, (void LDS_AS*)base, 16, 0, 0);
    // The instruction offset is added to the global address and to the LDS
    // address alike: this load reads chunk 64 + p and lands 1 KiB further on.
    __builtin_amdgcn_global_load_lds(src + p, (void LDS_AS*)base, 16, 1024, 0);
    // vmcnt(0) with expcnt and lgkmcnt left at their maxima: only the vector
    // memory counter is waited on before this single wave reads the LDS back.
    __builtin_amdgcn_s_waitcnt(0x0F70);
    for (int i = l; i < kProbeLdsWords; i += 64)
        dump[i] = lds[i];
}

// Buffer-resource loads into LDS and buffer stores, with hardware range
// checking.  The source resource covers src_nrec bytes and the destination
// resource dst_nrec bytes (raw buffers, stride 0).  Lane l loads 16 bytes at
// byte offset voff[l] into LDS at 16*l, the LDS window is copied to dump, and
// lane l then stores its 16 LDS bytes to dst at byte offset voff[l].  Offsets
// are taken modulo 64 KiB and rounded down to 16 bytes; the caller provides
// src and dst allocations of at least 64 KiB + 16 bytes, so every address
// the hardware could form lies inside them whether or not the range check
// suppresses it.
__global__ void __launch_bounds__(64) k_buffer_oob(const void* __restrict__ src, int src_nrec,
                                                   const uint32_t* __restrict__ voff,
                                                   uint32_t* __restrict__ dump,
                                                   void* __restrict__ dst, int dst_nrec)
{
    __shared__ __attribute__((aligned(16))) uint32_t lds[kProbeLdsWords];
    const int l = threadIdx.x;
    for (int i = l; i < kProbeLdsWords; i += 64)
        lds[i] = 0xDEADBEEFu;
    __syncthreads();
    const uint32_t off = voff[l] & 0xFFF0u;
    __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, src_nrec,
                                                                  0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (void LDS_AS*)lds, 16, off, 0, 0, 0);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    for (int i = l; i < kProbeLdsWords; i += 64)
        dump[i] = lds[i];
    typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;
    u32x4_t v = *(u32x4_t LDS_AS*)((char LDS_AS*)lds + 16 * l);
    __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(dst, (short)0, dst_nrec, 0x00020000);
    __builtin_amdgcn_raw_buffer_store_b128(v, rd, off, 0, 0);
}

// The same raw buffer load into LDS with a scalar offset: lane l loads 16
// bytes at byte offset (voff[l] mod 8 KiB, rounded down to 16) + soff into
// LDS at 16*l, against a resource of src_nrec bytes, and the LDS window is
// copied to dump.  Whether the hardware's range check counts the scalar
// offset decides which lanes read zeros.  soff is at most 4 KiB and the
// caller provides at least 12 KiB + 16 bytes of src, so every address the
// hardware could form lies inside it either way.
__global__ void __launch_bounds__(64) k_buffer_soffset(const void* __restrict__ src, int src_nrec,
                                                       const uint32_t* __restrict__ voff, uint32_t soff,
                                                       uint32_t* __restrict__ dump)
{
    __shared__ __attribute__((aligned(16))) uint32_t lds[kProbeLdsWords];
    const int l = threadIdx.x;
    for (int i = l; i < kProbeLdsWords; i += 64)
        lds[i] = 0xDEADBEEFu;
    __syncthreads();
    const uint32_t off = voff[l] & 0x1FF0u;
    __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, src_nrec,
                                                                  0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (void LDS_AS*)lds, 16, off, (int)soff, 0, 0);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    for (int i = l; i < kProbeLdsWords; i += 64)
        dump[i] = lds[i];
}

// One MFMA with zero accumulator: lane l supplies a[8l..8l+7] and
// b[8l..8l+7] as its operands and writes its 16 accumulator values to
// d[16l..16l+15].
__global__ void __launch_bounds__(64) k_mfma(const uint16_t* __restrict__ a,
                                             const uint16_t* __restrict__ b,
                                             float* __restrict__ d)
{
    const int l = threadIdx.x;
    bf16x8_t va, vb;
    __builtin_memcpy(&va, a + 8 * l, 16);
    __builtin_memcpy(&vb, b + 8 * l, 16);
    f32x16_t acc = {};
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, vb, acc, 0, 0, 0);
    for (int r = 0; r < 16; ++r)
        d[16 * l + r] = acc[r];
}

// The same for v_mfma_f32_16x16x32_bf16: lane l supplies a[8l..8l+7] and
// b[8l..8l+7] and writes its 4 accumulator values to d[4l..4l+3].
__global__ void __launch_bounds__(64) k_mfma16(const uint16_t* __restrict__ a,
                                               const uint16_t* __restrict__ b,
                                               float* __restrict__ d)
{
    const int l = threadIdx.x;
    bf16x8_t va, vb;
    __builtin_memcpy(&va, a + 8 * l, 16);
    __builtin_memcpy(&vb, b + 8 * l, 16);
    f32x4_t acc = {};
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, vb, acc, 0, 0, 0);
    for (int r = 0; r < 4; ++r)
        d[4 * l + r] = acc[r];
}

// LDS is filled with image[0..4095] (16-bit words); lane l then performs one
// ds_read_b64_tr_b16 at byte address addr[l] and writes its four 16-bit
// results to out[4l..4l+3].
__global__ void __launch_bounds__(64) k_ds_read_tr(const uint16_t* __restrict__ image,
                                                   const uint32_t* __restrict__ addr,
                                                   uint16_t* __restrict__ out)
{
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * kProbeLdsWords];
    const int l = threadIdx.x;
    for (int i = l; i < 2 * kProbeLdsWords; i += 64)
        lds[i] = image[i];
    __syncthreads();
    const uint32_t byte = addr[l] & (uint32_t)(4 * kProbeLdsWords - 8);   // in range, 8-byte aligned
    i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (i16x4_t LDS_AS*)((char LDS_AS*)lds + byte));
    for (int i = 0; i < 4; ++i)
        out[4 * l + i] = (uint16_t)v[i];
}

// fp32 -> bf16 with the conversion the GEMM epilogue uses (a pair at a time).
__global__ void __launch_bounds__(256) k_cvt(const float* __restrict__ in,
                                             uint16_t* __restrict__ out, int n_pairs)
{
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n_pairs)
        return;
    __bf16 lo = (__bf16)in[2 * i];
    __bf16 hi = (__bf16)in[2 * i + 1];
    uint16_t ulo, uhi;
    __builtin_memcpy(&ulo, &lo, 2);
    __builtin_memcpy(&uhi, &hi, 2);
    out[2 * i] = ulo;
    out[2 * i + 1] = uhi;
}

// Matrix-core ceiling.  Each workgroup has the shape of the GEMM kernels'
// MFMA waves: NW waves, each accumulating a 128 x (16 FN) fp32 tile as 8 x FN
// blocks of v_mfma_f32_16x16x32_bf16, so a 32-wide k-step is 8 FN MFMAs over
// 8 A and FN B fragments.  NW = 8, FN = 4 is the all-wave kernels' layout (two
// waves per SIMD, 128 x 64 per wave); NW = 4, FN = 8 gives one wave per SIMD a
// 128 x 128 tile (its 256 accumulator registers then need the accumulation
// register file).  The fragments come from `data` (bf16x8 vectors, taken
// modulo n_vec): two fragment sets alternate, so consecutive MFMAs see
// different operands, as in a GEMM.  FROM_LDS: 128 KiB of LDS are filled
// from `data` once, and every k-step re-reads its 8 + FN fragments per wave
// from LDS (1 KiB per read instruction, contiguous across lanes, at a base
// that moves every k-step within the first 64 KiB); otherwise
// the fragments stay in registers.  No global memory is touched after the
// start, and no synchronisation runs inside the loop.  Each thread writes one
// float of the accumulators to sink[blockIdx.x * 64 NW + threadIdx.x].
// A workgroup-iteration is NW * FN * 2^18 FLOP (2^23 for 8 x 4 and 4 x 8, 2^22
// for 4 x 4: the wave-specialised kernel's MFMA waves, one per SIMD).
constexpr int kCeilVecs = 8192;   // 128 KiB of 16-byte fragments

// NT threads per workgroup, of which the first NW waves run the loop.  The
// 4 x 4 shape is launched as the wave-specialised kernel is, 8 waves with 4
// of them doing MFMAs: the other 4 leave after the LDS fill, and the
// compiler gets the same budget of 256 registers per wave (given 512, it moves
// accumulators between register files inside the loop).
template <bool FROM_LDS, int NW, int FN, int NT>
__global__ void __launch_bounds__(NT) k_mfma_ceiling(const bf16x8_t* __restrict__ data, int n_vec, int iters,
                                                          float* __restrict__ sink, uint64_t* __restrict__ stamps)
{
    // Shader-clock and constant-rate timestamps at the start and the end of
    // the workgroup (s_memtime, s_memrealtime): their ratio over many
    // workgroups gives the clock the loop ran at, without a profiler.
    const uint64_t c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    static_assert((NW == 8 && FN == 4 && NT == 512) || (NW == 4 && FN == 8 && NT == 256) ||
                  (NW == 4 && FN == 4 && NT == 512), "wave shapes");
    constexpr int NF = 8 + FN;                 // fragments per k-step
    __shared__ bf16x8_t lds[kCeilVecs];
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    if constexpr (FROM_LDS) {
        for (int i = t; i < kCeilVecs; i += NT)
            lds[i] = data[(int)(((int64_t)blockIdx.x * 1031 + i) % n_vec)];
        __syncthreads();
    }
    if (w >= NW)
        return;
    bf16x8_t fa[2][8], fb[2][FN];
    const int64_t base = ((int64_t)blockIdx.x * NW * 64 + t) * 2 * NF;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            fa[s][i] = data[(int)((base + s * NF + i) % n_vec)];
#pragma unroll
        for (int j = 0; j < FN; ++j)
            fb[s][j] = data[(int)((base + s * NF + 8 + j) % n_vec)];
    }
    f32x4_t acc[8][FN];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
            acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if constexpr (FN == 8) {
        // 256 accumulator registers: placed in the accumulation register file
        // once, before the loop (a placement inside the loop makes the
        // compiler move them between register files every iteration).
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                asm volatile("" : "+a"(acc[i][j]));
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            if constexpr (FROM_LDS) {
                // The other set's fragments, for the next k-step.
                const int v0 = ((((it * 2 + s) * NF + w * 7) * 64) & (kCeilVecs / 2 - 1)) + lane;
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    fa[s ^ 1][i] = lds[v0 + i * 64];
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    fb[s ^ 1][j] = lds[v0 + (8 + j) * 64];
            }
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[s][j], fa[s][i], acc[i][j], 0, 0, 0);
        }
    }
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
            sum += acc[i][j][0] + acc[i][j][1] + acc[i][j][2] + acc[i][j][3];
    sink[(int64_t)blockIdx.x * NW * 64 + t] = sum;
    if (stamps && t == 0) {
        const uint64_t c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
        stamps[2 * blockIdx.x] = c1 - c0;
        stamps[2 * blockIdx.x + 1] = r1 - r0;
    }
}

// LDS read bandwidth: one workgroup of 1024 threads per compute unit (96 KiB
// of LDS each, so no two share a CU) fills 64 KiB of it, then each of its 16
// waves issues `iters` x 8 ds_read_b128 loads of 1 KiB each -- 64 lanes on
// 64 consecutive 16-byte slots, free of bank conflicts -- XOR-folding them
// into registers so that none can be dropped.  The next iteration's 8 loads
// are issued before the current ones are folded, so each wave keeps up to 16
// loads in flight.  The shader clock is stamped (s_memtime) after the fill
// and after a workgroup barrier at the end, so a stamp pair spans every
// wave's reads.  Bytes per clock of one CU = iters * 8 reads * 16 waves *
// 1024 bytes / elapsed ticks.
constexpr int kBwAlloc = 96 * 1024 / 16;      // 16-byte units allocated
constexpr int kBwThreads = 1024;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4v_t;

__global__ void __launch_bounds__(kBwThreads) k_lds_read_bw(int iters, uint32_t* __restrict__ sink,
                                                           uint64_t* __restrict__ stamps)
{
    __shared__ u32x4v_t lds[kBwAlloc];
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    for (int i = t; i < kBwAlloc; i += kBwThreads)
        lds[i] = u32x4v_t{(unsigned)i, (unsigned)i * 3u, (unsigned)i * 5u, (unsigned)i * 7u};
    __syncthreads();
    const uint64_t c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    // Iteration it of wave w reads the 8 KiB block (w + it) mod 8 of the 64
    // KiB at one address plus immediate offsets.
    auto block = [&](int it) { return lds + (((w + it) & 7) * 512 + lane); };
    u32x4v_t cur[8], nxt[8];
#pragma unroll
    for (int r = 0; r < 8; ++r)
        cur[r] = block(0)[r * 64];
    uint32_t acc0 = 0u, acc1 = 0u;
    for (int it = 1; it <= iters; ++it) {
        const u32x4v_t* src = block(it);
#pragma unroll
        for (int r = 0; r < 8; ++r)
            nxt[r] = src[r * 64];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            acc0 ^= cur[r].x ^ cur[r].y;
            acc1 ^= cur[r].z ^ cur[r].w;
            cur[r] = nxt[r];
        }
    }
    __syncthreads();
    const uint64_t c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
    sink[(int64_t)blockIdx.x * kBwThreads + t] = acc0 ^ acc1;
    if (stamps && t == 0) {
        stamps[2 * blockIdx.x] = c1 - c0;
        stamps[2 * blockIdx.x + 1] = r1 - r0;
    }
}

int launch_status()
{
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? 0 : -(int)e - 1000;
}

}  // namespace

extern "C" {

int gemm_probe_lds_dma(const void* src, const int* perm, int lds_base_bytes, uint32_t* dump,
                       void* stream)
{
    if (!src || !perm || !dump)
        return -1;
    if (lds_base_bytes < 0 || lds_base_bytes % 16 != 0 || lds_base_bytes + 2048 > 4 * kProbeLdsWords)
        return -1;
    hipLaunchKernelGGL(k_lds_dma, dim3(1), dim3(64), 0, (hipStream_t)stream,
                       (const uint4*)src, perm, lds_base_bytes, dump);
    return launch_status();
}

int gemm_probe_buffer_oob(const void* src, int src_nrec, const uint32_t* voff, uint32_t* dump,
                          void* dst, int dst_nrec, void* stream)
{
    if (!src || !voff || !dump || !dst || src_nrec < 0 || dst_nrec < 0)
        return -1;
    hipLaunchKernelGGL(k_buffer_oob, dim3(1), dim3(64), 0, (hipStream_t)stream, src, src_nrec,
                       voff, dump, dst, dst_nrec);
    return launch_status();
}

int gemm_probe_buffer_soffset(const void* src, int src_nrec, const uint32_t* voff, uint32_t soff, uint32_t* dump,
                              void* stream)
{
    if (!src || !voff || !dump || src_nrec < 0 || soff > 4096u || soff % 4u != 0)
        return -1;
    hipLaunchKernelGGL(k_buffer_soffset, dim3(1), dim3(64), 0, (hipStream_t)stream, src, src_nrec, voff, soff,
                       dump);
    return launch_status();
}

int gemm_probe_mfma(const uint16_t* a, const uint16_t* b, float* d, void* stream)
{
    if (!a || !b || !d)
        return -1;
    hipLaunchKernelGGL(k_mfma, dim3(1), dim3(64), 0, (hipStream_t)stream, a, b, d);
    return launch_status();
}

// a, b: 512 bf16 each; d: 256 floats.
int gemm_probe_mfma16(const uint16_t* a, const uint16_t* b, float* d, void* stream)
{
    if (!a || !b || !d)
        return -1;
    hipLaunchKernelGGL(k_mfma16, dim3(1), dim3(64), 0, (hipStream_t)stream, a, b, d);
    return launch_status();
}

int gemm_probe_ds_read_tr(const uint16_t* image, const uint32_t* addr, uint16_t* out, void* stream)
{
    if (!image || !addr || !out)
        return -1;
    hipLaunchKernelGGL(k_ds_read_tr, dim3(1), dim3(64), 0, (hipStream_t)stream, image, addr, out);
    return launch_status();
}

int gemm_probe_cvt_bf16(const float* in, uint16_t* out, int64_t n, void* stream)
{
    if (!in || !out || n < 0 || n % 2 != 0 || n > (int64_t)1 << 30)
        return -1;
    int pairs = (int)(n / 2);
    if (pairs == 0)
        return 0;
    hipLaunchKernelGGL(k_cvt, dim3((pairs + 255) / 256), dim3(256), 0, (hipStream_t)stream,
                       in, out, pairs);
    return launch_status();
}

// data: n_elems bf16 values (n_elems a positive multiple of 8, below 2^34);
// sink: blocks * 512 floats; stamps: null, or 2 * blocks 64-bit words that
// receive each workgroup's elapsed s_memtime and s_memrealtime ticks.
// Launches `blocks` workgroups, each running `iters` iterations of two
// 32-wide k-steps.  waves = 8: 8 waves of 128 x 64 (the all-wave kernels'
// layout, 2^23 FLOP per workgroup-iteration); waves = 4: 4 waves of 128 x 128
// (2^23); waves = -4: 4 waves of 128 x 64, one per SIMD, in a workgroup of 8
// whose other 4 waves exit at once (the wave-specialised kernel's MFMA waves,
// 2^22).
int gemm_probe_mfma_ceiling(const uint16_t* data, int64_t n_elems, int from_lds, int waves, int iters, int blocks,
                            float* sink, uint64_t* stamps, void* stream)
{
    if (!data || !sink || n_elems < 8 || n_elems % 8 != 0 || n_elems / 8 > ((int64_t)1 << 31) - 1 ||
        iters < 1 || iters > (1 << 20) || blocks < 1 || blocks > 65536 || (waves != 4 && waves != 8 && waves != -4))
        return -1;
    const int n_vec = (int)(n_elems / 8);
    const hipStream_t s = (hipStream_t)stream;
    const bf16x8_t* d = (const bf16x8_t*)data;
    if (waves == 8 && from_lds)
        hipLaunchKernelGGL(HIP_KERNEL_NAME(k_mfma_ceiling<true, 8, 4, 512>), dim3(blocks), dim3(512), 0, s, d, n_vec, iters, sink, stamps);
    else if (waves == 8)
        hipLaunchKernelGGL(HIP_KERNEL_NAME(k_mfma_ceiling<false, 8, 4, 512>), dim3(blocks), dim3(512), 0, s, d, n_vec, iters, sink, stamps);
    else if (waves == -4 && from_lds)
        hipLaunchKernelGGL(HIP_KERNEL_NAME(k_mfma_ceiling<true, 4, 4, 512>), dim3(blocks), dim3(512), 0, s, d, n_vec, iters, sink, stamps);
    else if (waves == -4)
        hipLaunchKernelGGL(HIP_KERNEL_NAME(k_mfma_ceiling<false, 4, 4, 512>), dim3(blocks), dim3(512), 0, s, d, n_vec, iters, sink, stamps);
    else if (from_lds)
        hipLaunchKernelGGL(HIP_KERNEL_NAME(k_mfma_ceiling<true, 4, 8, 256>), dim3(blocks), dim3(256), 0, s, d, n_vec, iters, sink, stamps);
    else
        hipLaunchKernelGGL(HIP_KERNEL_NAME(k_mfma_ceiling<false, 4, 8, 256>), dim3(blocks), dim3(256), 0, s, d, n_vec, iters, sink, stamps);
    return launch_status();
}

// sink: blocks * 1024 words; stamps: null, or 2 * blocks 64-bit words that
// receive each workgroup's elapsed s_memtime and s_memrealtime ticks over its
// reads.  Each workgroup reads (iters + 1) * 128 KiB.
int gemm_probe_lds_read_bw(int iters, int blocks, uint32_t* sink, uint64_t* stamps, void* stream)
{
    if (!sink || iters < 1 || iters > (1 << 20) || blocks < 1 || blocks > 65536)
        return -1;
    hipLaunchKernelGGL(k_lds_read_bw, dim3(blocks), dim3(kBwThreads), 0, (hipStream_t)stream, iters, sink, stamps);
    return launch_status();
}

// Tick rate of s_memrealtime on the current device, in Hz (0 on error).
int64_t gemm_probe_wall_clock_hz(void)
{
    int dev = 0, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess)
        return 0;
    return (int64_t)khz * 1000;
}

}  // extern "C"
