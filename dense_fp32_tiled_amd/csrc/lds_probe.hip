// lds_probe.hip -- timing of one LDS read pattern (see include/lds_probe.h).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lds_probe.h"

namespace {

struct Pattern {
    int32_t byte_addr[64];
};

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// 16 reads per asm block, then a wait for all of them, so the outputs are
// defined when the block ends (early-clobber keeps them off the address
// register).  Reusing four destinations is a write-after-write on loads that
// complete in order.
template <int WIDTH>
__device__ inline void read16(uint32_t addr, float& sink) {
    if constexpr (WIDTH == 1) {
        float r0, r1, r2, r3;
        asm volatile(
            "ds_read_b32 %0, %4\n ds_read_b32 %1, %4\n ds_read_b32 %2, %4\n ds_read_b32 %3, %4\n"
            "ds_read_b32 %0, %4\n ds_read_b32 %1, %4\n ds_read_b32 %2, %4\n ds_read_b32 %3, %4\n"
            "ds_read_b32 %0, %4\n ds_read_b32 %1, %4\n ds_read_b32 %2, %4\n ds_read_b32 %3, %4\n"
            "ds_read_b32 %0, %4\n ds_read_b32 %1, %4\n ds_read_b32 %2, %4\n ds_read_b32 %3, %4\n"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
            : "v"(addr)
            : "memory");
        sink += r0 + r1 + r2 + r3;
    } else if constexpr (WIDTH == 2) {
        f32x2 r0, r1, r2, r3;
        asm volatile(
            "ds_read_b64 %0, %4\n ds_read_b64 %1, %4\n ds_read_b64 %2, %4\n ds_read_b64 %3, %4\n"
            "ds_read_b64 %0, %4\n ds_read_b64 %1, %4\n ds_read_b64 %2, %4\n ds_read_b64 %3, %4\n"
            "ds_read_b64 %0, %4\n ds_read_b64 %1, %4\n ds_read_b64 %2, %4\n ds_read_b64 %3, %4\n"
            "ds_read_b64 %0, %4\n ds_read_b64 %1, %4\n ds_read_b64 %2, %4\n ds_read_b64 %3, %4\n"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
            : "v"(addr)
            : "memory");
        sink += r0[0] + r1[0] + r2[1] + r3[1];
    } else {
        f32x4 r0, r1, r2, r3;
        asm volatile(
            "ds_read_b128 %0, %4\n ds_read_b128 %1, %4\n ds_read_b128 %2, %4\n ds_read_b128 %3, %4\n"
            "ds_read_b128 %0, %4\n ds_read_b128 %1, %4\n ds_read_b128 %2, %4\n ds_read_b128 %3, %4\n"
            "ds_read_b128 %0, %4\n ds_read_b128 %1, %4\n ds_read_b128 %2, %4\n ds_read_b128 %3, %4\n"
            "ds_read_b128 %0, %4\n ds_read_b128 %1, %4\n ds_read_b128 %2, %4\n ds_read_b128 %3, %4\n"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
            : "v"(addr)
            : "memory");
        sink += r0[0] + r1[1] + r2[2] + r3[3];
    }
}

// Two-address reads: dwords at base and base + OFF1 (ds_read2_b32 offset1).
template <int OFF1>
__device__ inline void read2_16(uint32_t addr, float& sink) {
    f32x2 r0, r1, r2, r3;
    asm volatile(
        "ds_read2_b32 %0, %4 offset1:%5\n ds_read2_b32 %1, %4 offset1:%5\n"
        "ds_read2_b32 %2, %4 offset1:%5\n ds_read2_b32 %3, %4 offset1:%5\n"
        "ds_read2_b32 %0, %4 offset1:%5\n ds_read2_b32 %1, %4 offset1:%5\n"
        "ds_read2_b32 %2, %4 offset1:%5\n ds_read2_b32 %3, %4 offset1:%5\n"
        "ds_read2_b32 %0, %4 offset1:%5\n ds_read2_b32 %1, %4 offset1:%5\n"
        "ds_read2_b32 %2, %4 offset1:%5\n ds_read2_b32 %3, %4 offset1:%5\n"
        "ds_read2_b32 %0, %4 offset1:%5\n ds_read2_b32 %1, %4 offset1:%5\n"
        "ds_read2_b32 %2, %4 offset1:%5\n ds_read2_b32 %3, %4 offset1:%5\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
        : "v"(addr), "i"(OFF1)
        : "memory");
    sink += r0[0] + r1[1] + r2[0] + r3[1];
}

// 16 writes of WIDTH dwords at the lane's address, then a wait.  Every
// wavefront writes the same values to the same addresses; the LDS contents
// are never read back.
template <int WIDTH>
__device__ inline void write16(uint32_t addr, float v) {
    if constexpr (WIDTH == 1) {
        asm volatile(
            "ds_write_b32 %0, %1\n ds_write_b32 %0, %1\n ds_write_b32 %0, %1\n ds_write_b32 %0, %1\n"
            "ds_write_b32 %0, %1\n ds_write_b32 %0, %1\n ds_write_b32 %0, %1\n ds_write_b32 %0, %1\n"
            "ds_write_b32 %0, %1\n ds_write_b32 %0, %1\n ds_write_b32 %0, %1\n ds_write_b32 %0, %1\n"
            "ds_write_b32 %0, %1\n ds_write_b32 %0, %1\n ds_write_b32 %0, %1\n ds_write_b32 %0, %1\n"
            "s_waitcnt lgkmcnt(0)" ::"v"(addr), "v"(v) : "memory");
    } else if constexpr (WIDTH == 2) {
        const f32x2 d{v, v};
        asm volatile(
            "ds_write_b64 %0, %1\n ds_write_b64 %0, %1\n ds_write_b64 %0, %1\n ds_write_b64 %0, %1\n"
            "ds_write_b64 %0, %1\n ds_write_b64 %0, %1\n ds_write_b64 %0, %1\n ds_write_b64 %0, %1\n"
            "ds_write_b64 %0, %1\n ds_write_b64 %0, %1\n ds_write_b64 %0, %1\n ds_write_b64 %0, %1\n"
            "ds_write_b64 %0, %1\n ds_write_b64 %0, %1\n ds_write_b64 %0, %1\n ds_write_b64 %0, %1\n"
            "s_waitcnt lgkmcnt(0)" ::"v"(addr), "v"(d) : "memory");
    } else {
        const f32x4 d{v, v, v, v};
        asm volatile(
            "ds_write_b128 %0, %1\n ds_write_b128 %0, %1\n ds_write_b128 %0, %1\n ds_write_b128 %0, %1\n"
            "ds_write_b128 %0, %1\n ds_write_b128 %0, %1\n ds_write_b128 %0, %1\n ds_write_b128 %0, %1\n"
            "ds_write_b128 %0, %1\n ds_write_b128 %0, %1\n ds_write_b128 %0, %1\n ds_write_b128 %0, %1\n"
            "ds_write_b128 %0, %1\n ds_write_b128 %0, %1\n ds_write_b128 %0, %1\n ds_write_b128 %0, %1\n"
            "s_waitcnt lgkmcnt(0)" ::"v"(addr), "v"(d) : "memory");
    }
}

// MODE 1, 2, 4: ds_read_b32/b64/b128 of MODE dwords; MODE -16, -32:
// ds_read2_b32 with offset1 16 or 32 dwords; MODE 101, 102, 104:
// ds_write_b32/b64/b128.
template <int MODE>
__device__ inline void read_mode(uint32_t addr, float& sink) {
    if constexpr (MODE > 100)
        write16<MODE - 100>(addr, sink);
    else if constexpr (MODE > 0)
        read16<MODE>(addr, sink);
    else
        read2_16<-MODE>(addr, sink);
}

template <int WIDTH>
__global__ __launch_bounds__(1024) void lds_probe_kernel(Pattern p, int reps, uint64_t* cycles_out,
                                                          float* never_written) {
    __shared__ __attribute__((aligned(16))) float buf[LDS_PROBE_WORDS];
    for (int i = threadIdx.x; i < LDS_PROBE_WORDS; i += blockDim.x) buf[i] = (float)(i & 7);
    __syncthreads();
    const int lane = threadIdx.x % 64;
    // ds_read takes an LDS byte offset: cast buf to the LDS address space.
    typedef __attribute__((address_space(3))) float lds_float;
    const uint32_t addr = (uint32_t)(uintptr_t)((lds_float*)buf) + (uint32_t)p.byte_addr[lane];
    float sink = 0.0f;
    const uint64_t t0 = clock64();
    for (int r = 0; r < reps; ++r) read_mode<WIDTH>(addr, sink);
    const uint64_t t1 = clock64();
    if (lane == 0) cycles_out[threadIdx.x / 64] = t1 - t0;
    // keep the reads observable; sink is finite, so this store never happens
    if (sink < -1.0f && never_written) never_written[threadIdx.x] = sink;
}

// Throughput of the direct global->LDS copy: every wave of every workgroup
// issues reps x 16 copies of BYTES per lane (global_load_lds_dword or
// _dwordx4) into its own LDS piece, waiting for all of them after each 16,
// and reports the shader-clock cycles its loop took.  Lane l of wave w in
// workgroup b reads src + off0 + (b * waves + w) * wave_stride
// + (l / row_lanes) * ld_bytes + (l % row_lanes) * BYTES: a row-structured
// piece as in a GEMM tile copy (row_lanes lanes per row, rows ld_bytes
// apart).  The host checks that every byte read lies in the source buffer.
template <int BYTES>
__global__ __launch_bounds__(1024) void dma_probe_kernel(const char* src, uint32_t off0, uint32_t wave_stride,
                                                         uint32_t ld_bytes, int row_lanes, int reps,
                                                         uint64_t* cycles_out) {
    __shared__ __attribute__((aligned(16))) float buf[16 * 64 * 4];  // 16 waves x 64 lanes x 16 bytes
    const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
    typedef __attribute__((address_space(3))) float lds_float;
    const uint32_t lds = (uint32_t)__builtin_amdgcn_readfirstlane(
        (int)((uint32_t)(uintptr_t)((lds_float*)buf) + (uint32_t)(wave * 64 * BYTES)));
    const uint32_t off = off0 + (uint32_t)(blockIdx.x * (blockDim.x / 64) + wave) * wave_stride +
                         (uint32_t)(lane / row_lanes) * ld_bytes + (uint32_t)(lane % row_lanes) * BYTES;
    const uint64_t t0 = clock64();
    for (int r = 0; r < reps; ++r) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if constexpr (BYTES == 16)
                asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                             :
                             : "v"(off), "s"(src), "s"(lds)
                             : "memory", "m0");
            else
                asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
                             :
                             : "v"(off), "s"(src), "s"(lds)
                             : "memory", "m0");
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    }
    const uint64_t t1 = clock64();
    if (lane == 0) cycles_out[blockIdx.x * (blockDim.x / 64) + wave] = t1 - t0;
}

// Throughput of the vector ALU's fp32 FMA (v_fmac_f32, one product per lane,
// no packed forms): every lane runs reps x 64 FMAs over 8 independent
// accumulators, with no memory access in the loop, and each wave reports
// the shader-clock cycles its loop took.  The accumulators are stored only
// under a condition that the data never meets, so the FMAs stay live.
__global__ __launch_bounds__(1024) void valu_fma_probe_kernel(int reps, float x, float y, uint64_t* cycles_out,
                                                              float* never_written) {
    float a0 = (float)threadIdx.x, a1 = a0 + 1.0f, a2 = a0 + 2.0f, a3 = a0 + 3.0f;
    float a4 = a0 + 4.0f, a5 = a0 + 5.0f, a6 = a0 + 6.0f, a7 = a0 + 7.0f;
    const uint64_t t0 = clock64();
    for (int r = 0; r < reps; ++r) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            asm volatile(
                "v_fmac_f32 %0, %8, %9\n\tv_fmac_f32 %1, %8, %9\n\tv_fmac_f32 %2, %8, %9\n\t"
                "v_fmac_f32 %3, %8, %9\n\tv_fmac_f32 %4, %8, %9\n\tv_fmac_f32 %5, %8, %9\n\t"
                "v_fmac_f32 %6, %8, %9\n\tv_fmac_f32 %7, %8, %9"
                : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "+v"(a4), "+v"(a5), "+v"(a6), "+v"(a7)
                : "v"(x), "v"(y));
    }
    const uint64_t t1 = clock64();
    if (threadIdx.x % 64 == 0) cycles_out[blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64] = t1 - t0;
    const float sum = a0 + a1 + a2 + a3 + a4 + a5 + a6 + a7;
    if (sum != sum && never_written) never_written[blockIdx.x * blockDim.x + threadIdx.x] = sum;  // NaN only
}

// Matrix-pipe throughput of v_mfma_f32_32x32x2_f32 (4096 flops per wave
// instruction): every wave runs reps x 16 MFMAs round-robin over 4
// independent 32x32 accumulators, with no memory access in the loop, and
// reports the shader-clock cycles its loop took.  ACC_AGPR keeps the
// accumulators in AGPRs (inline asm with the "a" constraint, the register
// file the compiler uses for accumulators beyond 256 registers a lane);
// otherwise the compiler's builtin keeps them in VGPRs.  The results are
// stored only under a condition that the data never meets.
template <bool ACC_AGPR>
__global__ __launch_bounds__(1024) void mfma_probe_kernel(int reps, float x, float y, uint64_t* cycles_out,
                                                          float* never_written) {
    typedef float f32x16 __attribute__((ext_vector_type(16)));
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    const float a = x + (float)(threadIdx.x % 7), b = y;
    const uint64_t t0 = clock64();
    for (int r = 0; r < reps; ++r) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (ACC_AGPR) {
                asm volatile(
                    "v_mfma_f32_32x32x2_f32 %0, %4, %5, %0\n\t"
                    "v_mfma_f32_32x32x2_f32 %1, %4, %5, %1\n\t"
                    "v_mfma_f32_32x32x2_f32 %2, %4, %5, %2\n\t"
                    "v_mfma_f32_32x32x2_f32 %3, %4, %5, %3"
                    : "+a"(c0), "+a"(c1), "+a"(c2), "+a"(c3)
                    : "v"(a), "v"(b));
            } else {
                c0 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c0, 0, 0, 0);
                c1 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c1, 0, 0, 0);
                c2 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c2, 0, 0, 0);
                c3 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c3, 0, 0, 0);
            }
        }
    }
    const uint64_t t1 = clock64();
    if (threadIdx.x % 64 == 0) cycles_out[blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64] = t1 - t0;
    float sum = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) sum += c0[i] + c1[i] + c2[i] + c3[i];
    if (sum != sum && never_written) never_written[blockIdx.x * blockDim.x + threadIdx.x] = sum;  // NaN only
}

__global__ __launch_bounds__(256) void copy_f32_kernel(const f32x4* __restrict__ src, f32x4* __restrict__ dst,
                                                       int64_t n4) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x)
        dst[i] = src[i];
}

__global__ void xcc_id_kernel(int32_t* out) {
    int32_t x;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID, 0, 4)" : "=s"(x));
    if (threadIdx.x == 0) out[blockIdx.x] = x;
}

}  // namespace

extern "C" int probe_xcc_ids(int32_t* out, int32_t blocks, int32_t threads, void* stream) {
    if (out == nullptr || blocks < 1 || threads < 1 || threads > 1024) return -1;
    void* args[] = {&out};
    return hipLaunchKernel(reinterpret_cast<const void*>(xcc_id_kernel), dim3((unsigned)blocks),
                           dim3((unsigned)threads), args, 0, (hipStream_t)stream) == hipSuccess
               ? 0
               : -2;
}

extern "C" int probe_dma_throughput(const void* src, int64_t src_bytes, int32_t bytes_per_lane, int32_t blocks,
                                    int32_t waves, int32_t reps, int64_t off0, int64_t wave_stride, int64_t ld_bytes,
                                    int32_t row_lanes, uint64_t* cycles_out, void* stream) {
    if (src == nullptr || cycles_out == nullptr) return -1;
    if (bytes_per_lane != 4 && bytes_per_lane != 16) return -1;
    if (blocks < 1 || blocks > 4096 || waves < 1 || waves > 16 || reps < 1 || reps > 100000) return -1;
    if (row_lanes < 1 || row_lanes > 64 || 64 % row_lanes != 0) return -1;
    if (off0 < 0 || wave_stride < 0 || ld_bytes < 0) return -1;
    if ((((uintptr_t)src + (uint64_t)off0) % (uint64_t)bytes_per_lane) != 0 || wave_stride % bytes_per_lane != 0 ||
        ld_bytes % 4 != 0 || (bytes_per_lane == 16 && ld_bytes % 16 != 0))
        return -1;
    // the farthest byte any lane reads
    const int64_t last = off0 + (int64_t)(blocks * waves - 1) * wave_stride + (int64_t)(64 / row_lanes - 1) * ld_bytes +
                         (int64_t)row_lanes * bytes_per_lane;
    if (last > src_bytes || last > 0x7fffffff) return -1;
    const char* s = static_cast<const char*>(src);
    uint32_t o = (uint32_t)off0, ws = (uint32_t)wave_stride, ld = (uint32_t)ld_bytes;
    int rl = row_lanes, rp = reps;
    void* args[] = {&s, &o, &ws, &ld, &rl, &rp, &cycles_out};
    const void* kernel = bytes_per_lane == 16 ? reinterpret_cast<const void*>(dma_probe_kernel<16>)
                                              : reinterpret_cast<const void*>(dma_probe_kernel<4>);
    return hipLaunchKernel(kernel, dim3((unsigned)blocks), dim3((unsigned)(64 * waves)), args, 0,
                           (hipStream_t)stream) == hipSuccess
               ? 0
               : -2;
}

extern "C" int probe_valu_fma(int32_t blocks, int32_t waves, int32_t reps, uint64_t* cycles_out, void* stream) {
    if (cycles_out == nullptr || blocks < 1 || blocks > 4096 || waves < 1 || waves > 16 || reps < 1 ||
        reps > 1000000)
        return -1;
    int rp = reps;
    float x = 0.5f, y = 0.25f;  // finite accumulators: the store below never happens
    float* never_written = nullptr;
    void* args[] = {&rp, &x, &y, &cycles_out, &never_written};
    return hipLaunchKernel(reinterpret_cast<const void*>(valu_fma_probe_kernel), dim3((unsigned)blocks),
                           dim3((unsigned)(64 * waves)), args, 0, (hipStream_t)stream) == hipSuccess
               ? 0
               : -2;
}

extern "C" int probe_mfma_f32(int32_t blocks, int32_t waves, int32_t reps, int32_t acc_agpr, uint64_t* cycles_out,
                              void* stream) {
    if (cycles_out == nullptr || blocks < 1 || blocks > 4096 || waves < 1 || waves > 16 || reps < 1 ||
        reps > 1000000 || (acc_agpr != 0 && acc_agpr != 1))
        return -1;
    int rp = reps;
    float x = 0.5f, y = 0.25f;  // finite products: the store below never happens
    float* never_written = nullptr;
    void* args[] = {&rp, &x, &y, &cycles_out, &never_written};
    const void* kernel = acc_agpr ? reinterpret_cast<const void*>(mfma_probe_kernel<true>)
                                  : reinterpret_cast<const void*>(mfma_probe_kernel<false>);
    return hipLaunchKernel(kernel, dim3((unsigned)blocks), dim3((unsigned)(64 * waves)), args, 0,
                           (hipStream_t)stream) == hipSuccess
               ? 0
               : -2;
}

extern "C" int probe_copy_f32(const float* src, float* dst, int64_t n, void* stream) {
    if (n < 0 || n % 4 != 0) return -1;
    if (n == 0) return 0;
    if (src == nullptr || dst == nullptr) return -1;
    if ((((uintptr_t)src) & 15) != 0 || (((uintptr_t)dst) & 15) != 0) return -1;
    const uintptr_t s0 = (uintptr_t)src, d0 = (uintptr_t)dst, bytes = (uintptr_t)n * 4;
    if (s0 < d0 + bytes && d0 < s0 + bytes) return -1;
    int64_t n4 = n / 4;
    const f32x4* s4 = reinterpret_cast<const f32x4*>(src);
    f32x4* d4 = reinterpret_cast<f32x4*>(dst);
    int64_t blocks = (n4 + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    void* args[] = {&s4, &d4, &n4};
    return hipLaunchKernel(reinterpret_cast<const void*>(copy_f32_kernel), dim3((unsigned)blocks), dim3(256), args, 0,
                           (hipStream_t)stream) == hipSuccess
               ? 0
               : -2;
}

extern "C" int lds_probe_run(const int32_t* lane_words, int32_t width_words, int32_t waves, int32_t reps,
                             uint64_t* cycles_out, void* stream) {
    if (lane_words == nullptr || cycles_out == nullptr) return -1;
    const bool write = width_words > 100;
    const int32_t w0 = write ? width_words - 100 : width_words;
    if (w0 != 1 && w0 != 2 && w0 != 4 && w0 != -16 && w0 != -32) return -1;
    if (write && w0 < 0) return -1;
    if (waves < 1 || waves > 16 || reps < 1 || reps > 100000) return -1;
    // dwords one lane touches past its base, and the alignment the base needs
    const int32_t span = w0 > 0 ? w0 : -w0 + 1;
    const int32_t align = w0 > 0 ? w0 : 1;
    Pattern p;
    for (int l = 0; l < 64; ++l) {
        const int32_t w = lane_words[l];
        if (w < 0 || w % align != 0 || w + span > LDS_PROBE_WORDS) return -1;
        p.byte_addr[l] = w * 4;
    }
    float* never_written = nullptr;
    void* args[] = {&p, &reps, &cycles_out, &never_written};
    const void* kernel = width_words == 1     ? reinterpret_cast<const void*>(lds_probe_kernel<1>)
                         : width_words == 2   ? reinterpret_cast<const void*>(lds_probe_kernel<2>)
                         : width_words == 4   ? reinterpret_cast<const void*>(lds_probe_kernel<4>)
                         : width_words == -16 ? reinterpret_cast<const void*>(lds_probe_kernel<-16>)
                         : width_words == -32 ? reinterpret_cast<const void*>(lds_probe_kernel<-32>)
                         : width_words == 101 ? reinterpret_cast<const void*>(lds_probe_kernel<101>)
                         : width_words == 102 ? reinterpret_cast<const void*>(lds_probe_kernel<102>)
                                              : reinterpret_cast<const void*>(lds_probe_kernel<104>);
    return hipLaunchKernel(kernel, dim3(1), dim3(64 * waves), args, 0, (hipStream_t)stream) == hipSuccess ? 0 : -2;
}
