// default_config.hpp -- the default fp32 kernel: 256x256x32 workgroup tiles
// of 8 waves (128x64 each), direct global->LDS copies, the multiply
// software-pipelined across the K-tile barrier.
//
// Its 16-byte form (both operands' rows 16-byte aligned) is compiled in a
// translation unit of its own (gemm_default.hip).  The compiler's code for a
// kernel depends on what else its translation unit instantiates (inlining
// and scheduling decisions over shared helpers); in the one that holds every
// other variant, this kernel measured 2 % slower than alone, with 12 more
// instructions.  Compiled alone, its code no longer depends on the rest.
#pragma once

#include "launch.hpp"  // before the layouts: they name gemm_kernels.hpp's TileLayout
#include "generated/mfma_layouts.hpp"

namespace dft {

// VEC: floats per copy of A, VEC_B of B (4: 16-byte copies, 1: 4-byte); the
// uniform forms pass VEC_B as 0 (MfmaCfg's default), so they stay one type.
template <int VEC, int VEC_B = VEC>
using Mfma256x256Bk32Pipe = MfmaCfg<256, 256, 32, 128, 64, 2, 32, layouts::m32_256x256x32_pipe::A,
                                    layouts::m32_256x256x32_pipe::B, VEC, kXcdGroupedOrder, kLoadDirect, true,
                                    VEC_B == VEC ? 0 : VEC_B>;

// Launch of Mfma256x256Bk32Pipe<4> (defined in gemm_default.hip).
hipError_t launch_default_vec4(const Args& a, Split sp, hipStream_t stream);

}  // namespace dft
