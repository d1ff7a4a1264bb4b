// launch.hpp -- launch plumbing shared by the library's translation units:
// the GEMM arguments, K slicing, and the launch of a tile kernel over the
// output tile grid.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_kernels.hpp"

namespace dft {

struct Args {
    int64_t M, N, K;
    const float* A;
    int64_t lda;
    const float* B;
    int64_t ldb;
    float* C;
    int64_t ldc;
};

// Rows of A (B) start 16-byte aligned: the operand may be loaded or copied
// 16 bytes per lane.  A tile's columns of B start at a multiple of the tile
// width, or at N - BN for an edge tile that the direct-copy kernels move back
// to end at N; so B also needs N % 4 == 0 for every copy to start on a
// 16-byte boundary.  (A's tiles start at whole rows and at multiples of BK
// along K, so lda alone decides for A.)
inline bool a_aligned(const Args& a) { return a.lda % 4 == 0 && ((uintptr_t)a.A & 15) == 0; }
inline bool b_aligned(const Args& a) { return a.ldb % 4 == 0 && a.N % 4 == 0 && ((uintptr_t)a.B & 15) == 0; }

// K slicing of one launch: `splits` slices of k_chunk (a multiple of BK)
// along gridDim.y, slice s writing C + s * c_split_stride.  A plain launch is
// one slice covering all of K.
struct Split {
    int64_t splits = 1, k_chunk = 0, c_split_stride = 0;
};

using LaunchFn = hipError_t (*)(const Args&, Split, hipStream_t);

// Launches go through hipLaunchKernel so that the returned status is this
// launch's own (hipGetLastError would also report errors left by earlier,
// unrelated runtime calls on the thread).
template <class Kernel>
hipError_t launch_tiles(Kernel kernel, int bm, int bn, int threads, const Args& a, Split sp, hipStream_t stream) {
    int64_t M = a.M, N = a.N, K = a.K, lda = a.lda, ldb = a.ldb, ldc = a.ldc;
    const float* A = a.A;
    const float* B = a.B;
    float* C = a.C;
    int64_t tiles_m = (M + bm - 1) / bm;
    int64_t tiles_n = (N + bn - 1) / bn;
    int64_t k_chunk = sp.splits > 1 ? sp.k_chunk : (K > 0 ? K : 1);
    int64_t c_split_stride = sp.c_split_stride;
    void* args[] = {&M, &N, &K, &A, &lda, &B, &ldb, &C, &ldc, &tiles_m, &tiles_n, &k_chunk, &c_split_stride};
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3((unsigned)(tiles_m * tiles_n), (unsigned)sp.splits),
                           dim3(threads), args, 0, stream);
}

template <class Cfg>
hipError_t launch_mfma(const Args& a, Split sp, hipStream_t stream) {
    return launch_tiles(gemm_mfma_kernel<Cfg>, Cfg::BM, Cfg::BN, Cfg::THREADS, a, sp, stream);
}

template <class Cfg>
hipError_t launch_ksplit(const Args& a, Split sp, hipStream_t stream) {
    return launch_tiles(gemm_mfma_ksplit_kernel<Cfg>, Cfg::BM, Cfg::BN, Cfg::THREADS, a, sp, stream);
}

template <class Cfg>
hipError_t launch_valu(const Args& a, Split sp, hipStream_t stream) {
    return launch_tiles(gemm_valu_kernel<Cfg>, Cfg::BM, Cfg::BN, Cfg::THREADS, a, sp, stream);
}

}  // namespace dft
