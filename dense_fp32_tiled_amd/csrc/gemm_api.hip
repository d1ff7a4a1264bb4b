// gemm_api.hip -- the C ABI (include/dense_fp32_tiled.h): argument checks,
// variant dispatch and kernel launches for the gfx950 fp32 GEMM kernels.
#include <hip/hip_runtime.h>

#include <algorithm>

#include <mutex>
#include <stdint.h>
#include <string.h>

#include "dense_fp32_tiled.h"
#include "default_config.hpp"
#include "gemm_kernels.hpp"
#include "launch.hpp"
#include "mixed_kernels.hpp"
#include "generated/mfma_layouts.hpp"
#include "pad_choice.hpp"
#include <type_traits>

namespace dft {

// --------------------------------------------------------------------------
// Split-K reduction: C[i][j] = sum over s = 0, 1, ..., S-1 (in that order) of
// W[s][i][j], where W holds S packed M x N partial products.  The fixed order
// makes the result deterministic.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(int64_t M, int64_t N, int64_t S,
                                                            const float* __restrict__ W, float* __restrict__ C,
                                                            int64_t ldc) {
    const int64_t total = M * N;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        float acc = W[i];
        for (int64_t s = 1; s < S; ++s) acc += W[s * total + i];
        C[(i / N) * ldc + (i % N)] = acc;
    }
}

// --------------------------------------------------------------------------
// K == 0: C's M x N region is an empty sum.
__global__ void zero_fill_kernel(int64_t M, int64_t N, float* __restrict__ C, int64_t ldc) {
    const int64_t total = M * N;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x)
        C[(i / N) * ldc + (i % N)] = 0.0f;
}

}  // namespace dft

namespace {

using namespace dft;

// ---- tile configurations ------------------------------------------------------
// LDS layouts come from the host layout search (generated/mfma_layouts.hpp,
// one entry per shape in mfma_shapes.def and global load width).
template <class L, int STAGES, int VEC, int BM, int BN, int BK, int MB>
using MfmaAt = MfmaCfg<BM, BN, BK, 64, 64, STAGES, MB, typename L::A, typename L::B, VEC, kXcdGroupedOrder>;

template <int STAGES, int VEC>
using Mfma256 = MfmaAt<std::conditional_t<VEC == 4, layouts::m32_256x128x16_v4, layouts::m32_256x128x16_v1>,
                       STAGES, VEC, 256, 128, 16, 32>;
template <int VEC>
using Mfma256Plain = MfmaCfg<256, 128, 16, 64, 64, 2, 32, TileLayout<0>, TileLayout<0>, VEC, kXcdGroupedOrder>;
template <int VEC>
using Mfma16x256 = MfmaAt<std::conditional_t<VEC == 4, layouts::m16_256x128x16_v4, layouts::m16_256x128x16_v1>,
                          2, VEC, 256, 128, 16, 16>;
// Direct global->LDS copies for in-range tiles, 16 or 4 bytes per lane.
// The direct-copy variants that AUTO chooses from take a copy width per
// operand (VEC for A, VEC_B for B): an operand whose rows are 16-byte
// aligned keeps 16-byte copies when the other's are not.  VEC_B == VEC is
// passed as 0 (MfmaCfg's default), so the uniform forms stay one type.
template <int VEC, int VEC_B = VEC>
using Mfma256Direct = MfmaCfg<256, 128, 16, 64, 64, 2, 32, layouts::m32_256x128x16_direct::A,
                              layouts::m32_256x128x16_direct::B, VEC, kXcdGroupedOrder, kLoadDirect, false,
                              VEC_B == VEC ? 0 : VEC_B>;
template <int VEC, int VEC_B = VEC>
using Mfma128Direct = MfmaCfg<128, 128, 16, 64, 64, 2, 32, layouts::m32_128x128x16_direct::A,
                              layouts::m32_128x128x16_direct::B, VEC, kXcdGroupedOrder, kLoadDirect, false,
                              VEC_B == VEC ? 0 : VEC_B>;
// BK = 32 with 4-byte copies would need 32 staged floats per thread on edge
// tiles beside the accumulators; the forms with a 4-byte operand run BK = 16.
template <int VEC, int VEC_B = VEC>
using Mfma128Bk32Direct = std::conditional_t<
    VEC == 4 && VEC_B == 4,
    MfmaCfg<128, 128, 32, 64, 64, 2, 32, layouts::m32_128x128x32_direct::A, layouts::m32_128x128x32_direct::B, 4,
            kXcdGroupedOrder, kLoadDirect>,
    Mfma128Direct<VEC, VEC_B>>;
template <int VEC>
using Mfma256x256Direct = std::conditional_t<
    VEC == 4,
    MfmaCfg<256, 256, 16, 128, 64, 2, 32, layouts::m32_256x256x16_direct::A, layouts::m32_256x256x16_direct::B, 4,
            kXcdGroupedOrder, kLoadDirect>,
    Mfma256<2, 1>>;
template <int VEC>
using Mfma256x256W4Direct = std::conditional_t<
    VEC == 4,
    MfmaCfg<256, 256, 16, 128, 128, 2, 32, layouts::m32_256x256x16_w4_direct::A,
            layouts::m32_256x256x16_w4_direct::B, 4, kXcdGroupedOrder, kLoadDirect>,
    Mfma256<2, 1>>;
// The 256x256 tile with the chunked, cross-barrier pipelined multiply, at
// BK = 16 and BK = 32 (two 64 KiB stages: one workgroup per CU, as at BK = 16).
template <int VEC>
using Mfma256x256Pipe = std::conditional_t<
    VEC == 4,
    MfmaCfg<256, 256, 16, 128, 64, 2, 32, layouts::m32_256x256x16_pipe::A, layouts::m32_256x256x16_pipe::B, 4,
            kXcdGroupedOrder, kLoadDirect, true>,
    Mfma256<2, 1>>;
template <int VEC>
using Mfma16x256x256Direct = std::conditional_t<
    VEC == 4,
    MfmaCfg<256, 256, 16, 128, 64, 2, 16, layouts::m16_256x256x16_direct::A, layouts::m16_256x256x16_direct::B, 4,
            kXcdGroupedOrder, kLoadDirect>,
    Mfma256<2, 1>>;
template <int VEC>
using Mfma16x256x256W4Bk32Pipe = std::conditional_t<
    VEC == 4,
    MfmaCfg<256, 256, 32, 128, 128, 2, 16, layouts::m16_256x256x32_w4_pipe::A,
            layouts::m16_256x256x32_w4_pipe::B, 4, kXcdGroupedOrder, kLoadDirect, true>,
    Mfma256<2, 1>>;
// The 64x64 kernel copies directly at both widths: 16 bytes per lane for
// aligned operands, 4 bytes per lane (any row alignment) otherwise.
template <int VEC>
using Mfma64Direct = MfmaCfg<64, 64, 16, 32, 32, 2, 32, layouts::m32_64x64x16_direct::A,
                             layouts::m32_64x64x16_direct::B, VEC, kXcdGroupedOrder, kLoadDirect>;
// BK = 32 halves the barriers per k of the 64x64 tile (one per 16 MFMAs per
// wave instead of 8).  Its 4-byte form runs at 2 waves per SIMD (16 staged
// floats per thread on edge tiles).  The next tile's copies go out between
// the first 8 of its 16 MFMA steps (a wave's MFMAs form one dependent
// chain, which leaves it issue slots while each runs).  (The default
// 256x256 kernel keeps its copies before the first step: spread, they
// split its straight-line K tile for no measurable gain.)
template <int VEC, int VEC_B = VEC>
using Mfma64Bk32Direct = MfmaCfg<64, 64, 32, 32, 32, 2, 32, layouts::m32_64x64x32_direct::A,
                                 layouts::m32_64x64x32_direct::B, VEC, kXcdGroupedOrder, kLoadDirect, false,
                                 VEC_B == VEC ? 0 : VEC_B, 8>;
// The 64x64x32 tile with the pipelined multiply.
template <int VEC, int VEC_B = VEC>
using Mfma64Bk32Pipe = MfmaCfg<64, 64, 32, 32, 32, 2, 32, layouts::m32_64x64x32_direct::A,
                               layouts::m32_64x64x32_direct::B, VEC, kXcdGroupedOrder, kLoadDirect, true,
                               VEC_B == VEC ? 0 : VEC_B, 8>;
// Bases of the K-split variants (KsplitCfg): 32x64 and 32x32 tiles of
// 32x32-wave blocks, BK = 32.
template <int VEC, int VEC_B = VEC>
using Mfma32x64Direct = MfmaCfg<32, 64, 32, 32, 32, 2, 32, layouts::m32_32x64x32_direct::A,
                                layouts::m32_32x64x32_direct::B, VEC, kXcdGroupedOrder, kLoadDirect, false,
                                VEC_B == VEC ? 0 : VEC_B>;
template <int VEC, int VEC_B = VEC>
using Mfma32x32Direct = MfmaCfg<32, 32, 32, 32, 32, 2, 32, layouts::m32_32x32x32_direct::A,
                                layouts::m32_32x32x32_direct::B, VEC, kXcdGroupedOrder, kLoadDirect, false,
                                VEC_B == VEC ? 0 : VEC_B>;
// The K-split variants issue the next tile's copies between the first 8 of
// a tile's 16 MFMA steps (a wave's MFMAs form one dependent chain, which
// leaves it issue slots while each runs) instead of all before the first.
template <int VEC, int VEC_B = VEC>
using Mfma64Ks4 = KsplitCfg<Mfma64Bk32Direct<VEC, VEC_B>, 4, 8>;
template <int VEC, int VEC_B = VEC>
using Mfma32x64Ks4 = KsplitCfg<Mfma32x64Direct<VEC, VEC_B>, 4, 8>;
template <int VEC, int VEC_B = VEC>
using Mfma32x32Ks8 = KsplitCfg<Mfma32x32Direct<VEC, VEC_B>, 8, 8>;
template <int VEC, int VEC_B>
using Mfma64Ks2 = KsplitCfg<Mfma64Bk32Direct<VEC, VEC_B>, 2, 8>;
template <int VEC>
using Mfma128 = MfmaAt<std::conditional_t<VEC == 4, layouts::m32_128x128x16_v4, layouts::m32_128x128x16_v1>,
                       2, VEC, 128, 128, 16, 32>;
// BK = 32 with 4-byte loads needs 32 staged values and their addresses per
// thread, more registers than two waves per SIMD leave (it spilled); the
// 4-byte fallback of the BK = 32 variants therefore runs BK = 16.
template <int VEC>
using Mfma128Bk32 = std::conditional_t<VEC == 4, MfmaAt<layouts::m32_128x128x32_v4, 2, 4, 128, 128, 32, 32>,
                                       MfmaAt<layouts::m32_128x128x16_v1, 2, 1, 128, 128, 16, 32>>;

// LDS layouts of the vector-ALU kernel from the host layout search.
template <int VEC>
using ValuT = ValuCfg<128, 128, 16, 8, 8, 2, layouts::valu_128x128x16::A, layouts::valu_128x128x16::B, VEC>;

template <class Cfg>
void describe_common(gemm_tile_config& c, int variant, int vec) {
    c.variant = variant;
    c.bm = Cfg::BM; c.bn = Cfg::BN; c.bk = Cfg::BK;
    c.threads = Cfg::THREADS; c.wave_size = kWave;
    c.stages = Cfg::STAGES;
    c.barriers_per_tile = Cfg::STAGES == 2 ? 1 : 2;
    using TA = typename Cfg::TileA;
    using TB = typename Cfg::TileB;
    c.a_rows = TA::rows; c.a_cols = TA::cols; c.a_pad = TA::pad;
    c.a_row_stride = TA::row_stride; c.a_stage_elems = TA::stage_elems;
    c.b_rows = TB::rows; c.b_cols = TB::cols; c.b_pad = TB::pad;
    c.b_row_stride = TB::row_stride; c.b_stage_elems = TB::stage_elems;
    c.a_swz_unit = TA::swizzle.unit; c.a_swz_shift = TA::swizzle.shift; c.a_swz_mask = TA::swizzle.mask;
    c.b_swz_unit = TB::swizzle.unit; c.b_swz_shift = TB::swizzle.shift; c.b_swz_mask = TB::swizzle.mask;
    c.lds_bytes = Cfg::LDS_BYTES;
    c.vec_width = vec;
    c.lds_banks_b32 = kGfx950Lds.banks_b32; c.lds_lanes_b32 = kGfx950Lds.lanes_b32;
    c.lds_banks_b128 = kGfx950Lds.banks_b128; c.lds_lanes_b128 = kGfx950Lds.lanes_b128;
    c.xcd_tile_order = Cfg::ORDER == kXcdGroupedOrder ? 1 : 0;
    c.direct_to_lds = Cfg::LOAD == kLoadDirect ? 1 : 0;
    c.elem_bytes = 4;
    c.k_groups = 1;
}

template <class Cfg>
gemm_tile_config mfma_config(int variant, int vec) {
    gemm_tile_config c{};
    describe_common<Cfg>(c, variant, vec);
    c.tm = Cfg::WM; c.tn = Cfg::WN;
    c.a_transposed = 0;
    c.mfma_block = Cfg::Op::MB;
    c.k_groups = Cfg::KSPLIT;
    c.barriers_per_tile = Cfg::STAGES == 1 ? 2 : 1;  // per K tile (of a group, with the K split)
    if (Cfg::PIPE) c.direct_to_lds = 2;
    return c;
}

template <class Cfg>
gemm_tile_config valu_config(int variant, int vec) {
    gemm_tile_config c{};
    describe_common<Cfg>(c, variant, vec);
    c.tm = Cfg::TM; c.tn = Cfg::TN;
    c.a_transposed = 1;
    c.mfma_block = 0;
    return c;
}

struct Variant {
    LaunchFn vec4;    // 16-byte global loads (needs aligned A/B and ld % 4 == 0)
    LaunchFn scalar;  // 4-byte masked loads, any alignment
    LaunchFn a1b4;    // 4-byte loads of A, 16-byte of B (the scalar form where not built)
    LaunchFn a4b1;    // 16-byte loads of A, 4-byte of B
    gemm_tile_config (*config4)(int variant, int vec);
    gemm_tile_config (*config1)(int variant, int vec);
    int lds_bytes;
};

template <class C4, class C1, class C14 = C1, class C41 = C1>
Variant mfma_variant() {
    constexpr int lds = std::max({C4::LDS_BYTES, C1::LDS_BYTES, C14::LDS_BYTES, C41::LDS_BYTES});
    return Variant{launch_mfma<C4>, launch_mfma<C1>, launch_mfma<C14>, launch_mfma<C41>, mfma_config<C4>,
                   mfma_config<C1>, lds};
}
template <template <int, int> class V>
Variant mfma_variant_per_operand() {
    return mfma_variant<V<4, 4>, V<1, 1>, V<1, 4>, V<4, 1>>();
}
template <template <int, int> class V>
Variant ksplit_variant() {
    constexpr int lds = std::max({V<4, 4>::LDS_BYTES, V<1, 1>::LDS_BYTES, V<1, 4>::LDS_BYTES, V<4, 1>::LDS_BYTES});
    return Variant{launch_ksplit<V<4, 4>>, launch_ksplit<V<1, 1>>, launch_ksplit<V<1, 4>>, launch_ksplit<V<4, 1>>,
                   mfma_config<V<4, 4>>, mfma_config<V<1, 1>>, lds};
}
// The default kernel: its 16-byte form is launched from its own translation
// unit (gemm_default.hip), so this one never instantiates it.
Variant default_variant() {
    using P4 = Mfma256x256Bk32Pipe<4>;
    using P1 = Mfma256x256Bk32Pipe<1>;
    using P14 = Mfma256x256Bk32Pipe<1, 4>;
    using P41 = Mfma256x256Bk32Pipe<4, 1>;
    constexpr int lds = std::max({P4::LDS_BYTES, P1::LDS_BYTES, P14::LDS_BYTES, P41::LDS_BYTES});
    return Variant{launch_default_vec4, launch_mfma<P1>, launch_mfma<P14>, launch_mfma<P41>, mfma_config<P4>,
                   mfma_config<P1>, lds};
}

// Index = gemm_variant.  AUTO's entry is never launched (run() resolves AUTO
// to a concrete variant first); it describes the large-problem default.
const Variant kVariants[GEMM_VARIANT_COUNT] = {
    /* AUTO          */ default_variant(),
    /* MFMA          */ mfma_variant<Mfma256<2, 4>, Mfma256<2, 1>>(),
    /* VALU          */ {launch_valu<ValuT<4>>, launch_valu<ValuT<1>>, launch_valu<ValuT<1>>, launch_valu<ValuT<1>>,
                         valu_config<ValuT<4>>, valu_config<ValuT<1>>, ValuT<4>::LDS_BYTES},
    /* MFMA_STAGES1  */ mfma_variant<Mfma256<1, 4>, Mfma256<1, 1>>(),
    /* MFMA_NOPAD    */ mfma_variant<Mfma256Plain<4>, Mfma256Plain<1>>(),
    /* MFMA_SCALAR   */ mfma_variant<Mfma256<2, 1>, Mfma256<2, 1>>(),
    /* MFMA16        */ mfma_variant<Mfma16x256<4>, Mfma16x256<1>>(),
    /* MFMA_128      */ mfma_variant<Mfma128<4>, Mfma128<1>>(),
    /* MFMA_128_BK32 */ mfma_variant<Mfma128Bk32<4>, Mfma128Bk32<1>>(),
    /* MFMA_DIRECT   */ mfma_variant_per_operand<Mfma256Direct>(),
    /* MFMA_128_DIRECT      */ mfma_variant_per_operand<Mfma128Direct>(),
    /* MFMA_128_BK32_DIRECT */ mfma_variant_per_operand<Mfma128Bk32Direct>(),
    /* MFMA_64_DIRECT       */ mfma_variant<Mfma64Direct<4>, Mfma64Direct<1>>(),
    /* MFMA_256x256_DIRECT  */ mfma_variant<Mfma256x256Direct<4>, Mfma256x256Direct<1>>(),
    /* MFMA_256x256_W4_DIRECT */ mfma_variant<Mfma256x256W4Direct<4>, Mfma256x256W4Direct<1>>(),
    /* MFMA_256x256_PIPE      */ mfma_variant<Mfma256x256Pipe<4>, Mfma256x256Pipe<1>>(),
    /* MFMA_256x256_BK32_PIPE */ default_variant(),
    /* MFMA16_256x256_DIRECT  */ mfma_variant<Mfma16x256x256Direct<4>, Mfma16x256x256Direct<1>>(),
    /* MFMA16_256x256_W4_BK32_PIPE   */ mfma_variant<Mfma16x256x256W4Bk32Pipe<4>, Mfma16x256x256W4Bk32Pipe<1>>(),
    /* MFMA_64_BK32_DIRECT    */ mfma_variant_per_operand<Mfma64Bk32Direct>(),
    /* MFMA_64_KS4            */ ksplit_variant<Mfma64Ks4>(),
    /* MFMA_32x64_KS4         */ ksplit_variant<Mfma32x64Ks4>(),
    /* MFMA_32x32_KS8         */ ksplit_variant<Mfma32x32Ks8>(),
    /* MFMA_64_BK32_PIPE      */ mfma_variant_per_operand<Mfma64Bk32Pipe>(),
    /* MFMA_64_KS2            */ ksplit_variant<Mfma64Ks2>(),
};

// AUTO picks the direct-copy variant with the highest estimated rate: its
// measured full-chip rate at 4096^3-class sizes times the wave quantisation
// of its tile grid, tiles / (ceil(tiles / CUs) * CUs), the fraction of
// CU-rounds that have work.  The 256x128 and 128x128 kernels are built to
// run two workgroups per CU; with fewer tiles than two per CU they were
// measured about 12 % slower, which the estimate applies.  An edge tile
// moves back to end at M (N) when M >= BM (N >= BN) and then costs nothing
// extra; when M or N is smaller than the tile, the edge workgroups load
// through registers and are charged an extra round (rounds / (rounds + 1)).
// The full-chip rates depend on which operands have 16-byte aligned rows
// (a 4-byte operand costs each kernel differently: 4-byte copies of B are
// cheap for 256x128 tiles, those of A less so); they were measured per
// alignment class.  The 64x64 kernel's 4-wave workgroups reach its full
// rate only at three or more per CU.  When few output tiles meet a deep K,
// the K-split variants keep every CU's SIMDs busy with one workgroup.
int auto_variant(int64_t M, int64_t N, int64_t K, int num_cus, bool a_aligned = true, bool b_aligned = true) {
    struct Candidate {
        int variant, bm, bn, per_cu;
        double rate[4];   // TFLOP/s with every CU busy, by alignment: both, A only, B only, neither
        bool small_wg;    // 4-wave workgroups: below full rate at one or two per CU
        int64_t min_k;    // K-split variants: enough K tiles for every group (0: any K)
        int64_t min_k_one_round;  // the same when the grid has at most one tile per CU
    };
    const int cls = a_aligned ? (b_aligned ? 0 : 1) : (b_aligned ? 2 : 3);
    const int64_t t64 = ((M + 63) / 64) * ((N + 63) / 64);
    const Candidate candidates[] = {
        {GEMM_VARIANT_MFMA_256x256_BK32_PIPE, 256, 256, 1, {145.0, 134.0, 133.0, 130.0}, false, 0, 0},
        {GEMM_VARIANT_MFMA_DIRECT, 256, 128, 2, {144.0, 140.0, 130.0, 121.0}, false, 0, 0},
        {K >= 1024 ? GEMM_VARIANT_MFMA_128_BK32_DIRECT : GEMM_VARIANT_MFMA_128_DIRECT, 128, 128, 2,
         {144.0, 124.0, 130.0, 118.0}, false, 0, 0},
        // 64x64x32 with its copies between the MFMA steps: ahead of the
        // pipelined form on one-round grids and on multi-round grids with an
        // operand aligned; behind it (2047^3: 4 %) with neither aligned.
        {cls == 3 && t64 > num_cus ? GEMM_VARIANT_MFMA_64_BK32_PIPE : GEMM_VARIANT_MFMA_64_BK32_DIRECT, 64, 64, 1,
         {134.0, 120.0, 128.0, 110.0}, true, 0, 0},
        // K split inside the workgroup: 16 K tiles of 32 per group at
        // least; when the split's grid has at most one tile per CU, from
        // K = 1024 for 64x64 tiles, K = 256 for 32x32 and K = 128 (one K
        // tile per group) for 32x64, whose one-round grids leave the 64x64
        // kernel half the CUs or fewer (2176 x 192 x 448: 43 against 33;
        // with two rounds of 32x64 tiles the 64x64 kernel leads, 1536 x 384
        // x 320: 40 against 29).
        // 64x64 KS4 measured 5-7 % under the 64x64 kernel at K = 512 on
        // 1000^2 and 1024^2 grids, and any split up to 22 % under it on
        // grids of two or more rounds at K = 1024-2048.
        {GEMM_VARIANT_MFMA_64_KS4, 64, 64, 1, {117.0, K >= 4096 && t64 <= num_cus ? 126.0 : 108.0, 110.0, 103.0},
         false, 16 * 32 * 4, 1024},
        {GEMM_VARIANT_MFMA_32x64_KS4, 32, 64, 1, {101.0, 79.0, 95.0, 76.0}, false, 16 * 32 * 4, 128},
        // (32x32 KS8 from K = 256 on a one-round grid: at 256^3 5.3 TFLOP/s
        // against 3.7 for the 64x64 kernel.)
        {GEMM_VARIANT_MFMA_32x32_KS8, 32, 32, 1, {96.0, 66.0, 81.0, 63.0}, false, 16 * 32 * 8, 256},
        // Two groups: two waves per SIMD on a one-round 64x64 grid.  Measured
        // ahead of the 64x64x32 kernel with neither operand's rows aligned
        // (1000 x 999 x 513: 62 against 51) and, with only B's unaligned, on
        // one-round and multi-round grids alike (3000 x 2999 x 3000: 117
        // against 107; 2048 x 1023 x 2048: 105 against 92); behind it with
        // both aligned (1024^2 x 512: 78 against 83).  The four-group split
        // keeps the one-round grids of deep K (K >= 4096) with only B's
        // unaligned (1024 x 1023 x 4096: 102 against 101).
        {GEMM_VARIANT_MFMA_64_KS2, 64, 64, 1, {101.0, 124.0, 100.0, 99.0}, false, 16 * 32 * 2, 512},
    };
    int best = GEMM_VARIANT_MFMA_DIRECT;
    double best_rate = -1.0;
    for (const Candidate& c : candidates) {
        if (c.rate[cls] <= 0.0) continue;
        const int64_t tiles = ((M + c.bm - 1) / c.bm) * ((N + c.bn - 1) / c.bn);
        if (c.min_k > 0 && K < (tiles <= num_cus ? c.min_k_one_round : c.min_k)) continue;
        const int64_t rounds = tiles > 0 ? (tiles + num_cus - 1) / num_cus : 1;
        double rate = c.rate[cls] * (double)tiles / (double)(rounds * num_cus);
        if (tiles < (int64_t)c.per_cu * num_cus) rate *= c.per_cu > 1 ? 0.88 : 1.0;
        // One 4-wave workgroup per CU measured 78 % of the full rate, two 89 %.
        if (c.small_wg) rate *= tiles <= num_cus ? 0.78 : tiles <= 2 * (int64_t)num_cus ? 0.89 : 1.0;
        // Edge tiles move back to end at M (N) and run like interior ones
        // when M >= bm (N >= bn).  Otherwise the edge workgroups load every
        // tile through registers and take about twice as long; the last of
        // them adds about a round.
        const bool edge_m = M % c.bm && M < c.bm, edge_n = N % c.bn && N < c.bn;
        if (edge_m || edge_n) rate *= (double)rounds / (double)(rounds + 1);
        if (rate > best_rate * 1.02) {  // larger tiles win near-ties (listed first)
            best = c.variant;
            best_rate = rate;
        }
    }
    return best;
}

// ---- per-device properties (cached) ---------------------------------------------
struct DeviceInfo {
    int state;  // 0 unknown, 1 gfx950, -1 unsupported
    int max_lds;
    int num_cus;
};
constexpr int kMaxDevices = 64;
DeviceInfo g_devices[kMaxDevices];
std::mutex g_devices_mu;

int device_check(int* max_lds, int* num_cus) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return GEMM_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return GEMM_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_devices_mu);
    DeviceInfo& d = g_devices[dev];
    if (d.state == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return GEMM_ERR_HIP;
        d.state = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
        d.max_lds = (int)prop.sharedMemPerBlock;
        d.num_cus = prop.multiProcessorCount;
    }
    if (d.state != 1) return GEMM_ERR_UNSUPPORTED;
    *max_lds = d.max_lds;
    *num_cus = d.num_cus;
    return GEMM_OK;
}

bool overlaps(const void* p, int64_t p_bytes, const void* q, int64_t q_bytes) {
    const uintptr_t a0 = (uintptr_t)p, a1 = a0 + (uintptr_t)p_bytes;
    const uintptr_t b0 = (uintptr_t)q, b1 = b0 + (uintptr_t)q_bytes;
    return a0 < b1 && b0 < a1;
}

// Bytes spanned by a rows x cols row-major matrix with leading dimension ld.
int64_t span_bytes(int64_t rows, int64_t cols, int64_t ld, int64_t elem_bytes = 4) {
    if (rows == 0 || cols == 0) return 0;
    return ((rows - 1) * ld + cols) * elem_bytes;
}

int validate(const Args& a, int64_t ab_elem_bytes = 4) {
    if (a.M < 0 || a.N < 0 || a.K < 0) return GEMM_ERR_INVALID_DIM;
    const int64_t k1 = a.K > 1 ? a.K : 1, n1 = a.N > 1 ? a.N : 1;
    if (a.lda < k1 || a.ldb < n1 || a.ldc < n1) return GEMM_ERR_INVALID_LD;
    // Offsets up to M*ld must fit in int64 bytes with ample margin.
    const int64_t lim = (int64_t)1 << 60;
    if (a.M > lim / a.lda || a.K > lim / a.ldb || a.M > lim / a.ldc) return GEMM_ERR_TOO_LARGE;
    const bool c_used = a.M > 0 && a.N > 0;
    const bool ab_used = c_used && a.K > 0;
    if (c_used && a.C == nullptr) return GEMM_ERR_NULL;
    if (ab_used && (a.A == nullptr || a.B == nullptr)) return GEMM_ERR_NULL;
    if (ab_used) {
        const int64_t c_bytes = span_bytes(a.M, a.N, a.ldc);
        if (overlaps(a.C, c_bytes, a.A, span_bytes(a.M, a.K, a.lda, ab_elem_bytes)) ||
            overlaps(a.C, c_bytes, a.B, span_bytes(a.K, a.N, a.ldb, ab_elem_bytes)))
            return GEMM_ERR_ALIAS;
    }
    return GEMM_OK;
}

int launch_zero_fill(const Args& a, hipStream_t stream) {
    const int64_t total = a.M * a.N;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    int64_t M = a.M, N = a.N, ldc = a.ldc;
    float* C = a.C;
    void* args[] = {&M, &N, &C, &ldc};
    return hipLaunchKernel(reinterpret_cast<const void*>(zero_fill_kernel), dim3((unsigned)blocks), dim3(256), args,
                           0, stream) == hipSuccess
               ? GEMM_OK
               : GEMM_ERR_HIP;
}

// Checks shared by every entry point; on GEMM_OK with *done set, nothing is
// left to do (empty M or N, or K == 0 handled by a zero fill).  A and B hold
// ab_elem_bytes-byte elements (4, or 2 for 16-bit inputs).
int prologue(const Args& a, hipStream_t stream, int* max_lds, int* num_cus, bool* done, int64_t ab_elem_bytes = 4) {
    *done = false;
    int st = validate(a, ab_elem_bytes);
    if (st != GEMM_OK) return st;
    if (a.M == 0 || a.N == 0) {
        *done = true;
        return GEMM_OK;
    }
    st = device_check(max_lds, num_cus);
    if (st != GEMM_OK) return st;
    if (a.K == 0) {
        *done = true;
        return launch_zero_fill(a, stream);
    }
    return GEMM_OK;
}

int launch_variant(const Args& a, int variant, int max_lds, Split sp, hipStream_t stream) {
    const Variant& v = kVariants[variant];
    if (v.lds_bytes > max_lds) return GEMM_ERR_CONFIG;
    const gemm_tile_config cfg = v.config4(variant, 4);
    const int64_t tiles = ((a.M + cfg.bm - 1) / cfg.bm) * ((a.N + cfg.bn - 1) / cfg.bn);
    if (tiles > (int64_t)0x7fffffff / cfg.threads) return GEMM_ERR_TOO_LARGE;
    const bool a_al = a_aligned(a), b_al = b_aligned(a);
    const LaunchFn fn = a_al ? (b_al ? v.vec4 : v.a4b1) : (b_al ? v.a1b4 : v.scalar);
    return fn(a, sp, stream) == hipSuccess ? GEMM_OK : GEMM_ERR_HIP;
}

int run(const Args& a, hipStream_t stream, int variant) {
    if (variant < 0 || variant >= GEMM_VARIANT_COUNT) return GEMM_ERR_UNSUPPORTED;
    int max_lds = 0, num_cus = 0;
    bool done = false;
    const int st = prologue(a, stream, &max_lds, &num_cus, &done);
    if (st != GEMM_OK || done) return st;
    if (variant == GEMM_VARIANT_AUTO) variant = auto_variant(a.M, a.N, a.K, num_cus, a_aligned(a), b_aligned(a));
    return launch_variant(a, variant, max_lds, Split{}, stream);
}

// ---- split-K ------------------------------------------------------------------------
constexpr int kSplitKVariant = GEMM_VARIANT_MFMA_DIRECT;  // the slice kernel when none is named
constexpr int64_t kSplitKTileBm = 256, kSplitKTileBn = 128;  // its output tile
constexpr int64_t kSplitKTileBk = 16;  // K-tile depth the automatic split count is reckoned in
constexpr int kMaxSplits = 64;

// Slice length: whole K tiles of the slice kernel (depth bk), so slice
// boundaries fall on tile boundaries and keep 16-byte alignment.
int64_t splitk_chunk(int64_t K, int64_t splits, int64_t bk) {
    const int64_t tiles = (K + bk - 1) / bk;
    return ((tiles + splits - 1) / splits) * bk;
}

int64_t splitk_workspace_bytes(int64_t M, int64_t N, int64_t splits) { return splits * M * N * 4; }

int splitk_auto_splits(int64_t M, int64_t N, int64_t K, int num_cus) {
    // Enough slices to give every CU one workgroup of the 256x128 slice
    // kernel (measured best on 2048x256x16384 and 512x4096x4096: more slices
    // cost more in partial-product traffic than they gain in occupancy),
    // keeping at least eight 16-deep K tiles per slice.
    const int64_t tiles = ((M + kSplitKTileBm - 1) / kSplitKTileBm) * ((N + kSplitKTileBn - 1) / kSplitKTileBn);
    const int64_t ktiles = (K + kSplitKTileBk - 1) / kSplitKTileBk;
    int64_t s = ((int64_t)num_cus + tiles - 1) / tiles;
    if (s > ktiles / 8) s = ktiles / 8;
    if (s > kMaxSplits) s = kMaxSplits;
    return s < 1 ? 1 : (int)s;
}

int check_workspace(const Args& a, const void* workspace, int64_t workspace_bytes, int splits) {
    if (splits <= 1) return GEMM_OK;
    const int64_t need = splitk_workspace_bytes(a.M, a.N, splits);
    if (workspace == nullptr || workspace_bytes < need) return GEMM_ERR_WORKSPACE;
    if (overlaps(workspace, need, a.C, span_bytes(a.M, a.N, a.ldc)) ||
        overlaps(workspace, need, a.A, span_bytes(a.M, a.K, a.lda)) ||
        overlaps(workspace, need, a.B, span_bytes(a.K, a.N, a.ldb)))
        return GEMM_ERR_ALIAS;
    return GEMM_OK;
}

int run_splitk(const Args& a, void* workspace, int64_t workspace_bytes, int splits, hipStream_t stream,
               int variant) {
    if (variant < 0 || variant >= GEMM_VARIANT_COUNT) return GEMM_ERR_UNSUPPORTED;
    if (variant == GEMM_VARIANT_AUTO) variant = kSplitKVariant;
    if (splits < 0 || splits > kMaxSplits) return GEMM_ERR_INVALID_DIM;
    int st = validate(a);
    if (st != GEMM_OK) return st;
    // an explicit split count is checked against the workspace before any device call
    if (a.M > 0 && a.N > 0 && a.K > 0 && splits > 1) {
        st = check_workspace(a, workspace, workspace_bytes, splits);
        if (st != GEMM_OK) return st;
    }
    int max_lds = 0, num_cus = 0;
    bool done = false;
    st = prologue(a, stream, &max_lds, &num_cus, &done);
    if (st != GEMM_OK || done) return st;
    if (splits == 0) {
        splits = splitk_auto_splits(a.M, a.N, a.K, num_cus);
        st = check_workspace(a, workspace, workspace_bytes, splits);
        if (st != GEMM_OK) return st;
    }
    if (splits == 1) return launch_variant(a, variant, max_lds, Split{}, stream);
    // 1. every slice writes its partial product, packed M x N, into the workspace
    Args part = a;
    part.C = static_cast<float*>(workspace);
    part.ldc = a.N;
    const Split sp{splits, splitk_chunk(a.K, splits, kVariants[variant].config4(variant, 4).bk), a.M * a.N};
    st = launch_variant(part, variant, max_lds, sp, stream);
    if (st != GEMM_OK) return st;
    // 2. C = sum of the slices in ascending slice order
    int64_t M = a.M, N = a.N, S = splits, ldc = a.ldc;
    const float* W = static_cast<const float*>(workspace);
    float* C = a.C;
    int64_t blocks = (M * N + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    void* args[] = {&M, &N, &S, &W, &C, &ldc};
    return hipLaunchKernel(reinterpret_cast<const void*>(splitk_reduce_kernel), dim3((unsigned)blocks), dim3(256),
                           args, 0, stream) == hipSuccess
               ? GEMM_OK
               : GEMM_ERR_HIP;
}

// ---- split-K without allocation ----------------------------------------------------
// gemm_f32_splitk_noalloc keeps the slices' partial products in a file-scope
// device array instead of a caller's workspace: each GPU the library runs on
// holds its own copy until the process ends.  In host code `scratch` names a
// host-side stand-in, not device memory; the device address is looked up
// once per device (hipGetSymbolAddress, with that device current) and only
// that address is passed to kernels.  Every slice kernel stores its whole
// M x N partial product (an empty slice stores zeros), so nothing needs
// clearing between calls; calls that overlap on one GPU share the array and
// race.
constexpr int64_t kScratchBytes = (int64_t)64 << 20;
static __device__ __align__(256) float scratch[kScratchBytes / 4];

struct ScratchSlot {
    bool ready;
    void* ptr;
};
ScratchSlot g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

int scratch_address(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return GEMM_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return GEMM_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ScratchSlot& slot = g_scratch[dev];
    if (!slot.ready) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return GEMM_ERR_HIP;
        slot.ptr = p;
        slot.ready = true;
    }
    *out = slot.ptr;
    return GEMM_OK;
}

// splits == 0: the split count of gemm_f32_splitk, lowered until the
// partial products fit the array (down to 1, a plain launch).  An explicit
// split count whose partial products do not fit is an error.
int run_splitk_noalloc(const Args& a, int splits, hipStream_t stream) {
    if (splits < 0 || splits > kMaxSplits) return GEMM_ERR_INVALID_DIM;
    int st = validate(a);
    if (st != GEMM_OK) return st;
    const bool work = a.M > 0 && a.N > 0 && a.K > 0;
    if (work && splits > 1 && splitk_workspace_bytes(a.M, a.N, splits) > kScratchBytes) return GEMM_ERR_SCRATCH;
    int max_lds = 0, num_cus = 0;
    bool done = false;
    st = prologue(a, stream, &max_lds, &num_cus, &done);
    if (st != GEMM_OK || done) return st;
    if (splits == 0) {
        splits = splitk_auto_splits(a.M, a.N, a.K, num_cus);
        while (splits > 1 && splitk_workspace_bytes(a.M, a.N, splits) > kScratchBytes) --splits;
    }
    void* ws = nullptr;
    if (splits > 1) {
        st = scratch_address(&ws);
        if (st != GEMM_OK) return st;
    }
    return run_splitk(a, ws, splits > 1 ? kScratchBytes : 0, splits, stream, GEMM_VARIANT_AUTO);
}

// ---- 16-bit inputs, fp32 accumulation -----------------------------------------------
// Tile shapes of the mixed-precision kernels (layouts from the host search,
// mixed_shapes.def).  VEC 8: 16-byte direct copies; VEC 2: 4-byte direct
// copies; VEC 1: shifted 16-byte loads through registers, for rows only
// 2-byte aligned.
template <int TYPE, int VEC>
using Mixed256x128 = MixedCfg<TYPE, 256, 128, 32, 64, 64, 32, layouts::x32_256x128x32::A, layouts::x32_256x128x32::B,
                              VEC, 4, 2, kPipeNone>;
template <int TYPE, int VEC>
using Mixed256x256 = MixedCfg<TYPE, 256, 256, 32, 128, 64, 32, layouts::x32_256x256x32::A, layouts::x32_256x256x32::B,
                              VEC, 2>;
template <int TYPE, int VEC>
using Mixed256x128Bk64 = MixedCfg<TYPE, 256, 128, 64, 64, 64, 32, layouts::x32_256x128x64::A,
                                  layouts::x32_256x128x64::B, VEC, 2, 2, kPipeAcrossTiles>;
template <int TYPE, int VEC>
using Mixed256x256S3 = MixedCfg<TYPE, 256, 256, 32, 128, 64, 32, layouts::x32_256x256x32::A,
                                layouts::x32_256x256x32::B, VEC, 2, 3, kPipeAcrossTiles>;
template <int TYPE, int VEC>
using Mixed256x256Bk64 = MixedCfg<TYPE, 256, 256, 64, 128, 64, 32, layouts::x32_256x256x64::A,
                                  layouts::x32_256x256x64::B, VEC, 2, 2, kPipeAcrossTiles>;
template <int TYPE, int VEC>
using Mixed128x128Bk64 = MixedCfg<TYPE, 128, 128, 64, 64, 64, 32, layouts::x32_128x128x64::A,
                                  layouts::x32_128x128x64::B, VEC, 4, 2, kPipeAcrossTiles>;

// Small tiles and K split inside the workgroup, for grids of few output
// tiles (16-byte copies; the unaligned form is the shared 2-byte-load kernel).
template <int TYPE, int VEC>
using Mixed64 = MixedCfg<TYPE, 64, 64, 64, 32, 32, 32, layouts::x32_64x64x64::A, layouts::x32_64x64x64::B, VEC, 4, 2,
                         kPipeSteps>;
template <int TYPE, int VEC>
using Mixed32x64 = MixedCfg<TYPE, 32, 64, 64, 32, 32, 32, layouts::x32_32x64x64::A, layouts::x32_32x64x64::B, VEC,
                            4, 2, kPipeSteps>;
template <int TYPE, int VEC>
using Mixed64Ks2 = MixedKsplitCfg<Mixed64<TYPE, VEC>, 2>;
template <int TYPE, int VEC>
using Mixed64Ks4 = MixedKsplitCfg<Mixed64<TYPE, VEC>, 4>;
template <int TYPE, int VEC>
using Mixed32x64Ks4 = MixedKsplitCfg<Mixed32x64<TYPE, VEC>, 4>;

template <class Cfg>
hipError_t launch_mixed(const Args& a, hipStream_t stream) {
    int64_t M = a.M, N = a.N, K = a.K, lda = a.lda, ldb = a.ldb, ldc = a.ldc;
    const uint16_t* A = reinterpret_cast<const uint16_t*>(a.A);
    const uint16_t* B = reinterpret_cast<const uint16_t*>(a.B);
    float* C = a.C;
    int64_t tiles_m = (M + Cfg::BM - 1) / Cfg::BM;
    int64_t tiles_n = (N + Cfg::BN - 1) / Cfg::BN;
    void* args[] = {&M, &N, &K, &A, &lda, &B, &ldb, &C, &ldc, &tiles_m, &tiles_n};
    const void* kernel;
    if constexpr (Cfg::KSPLIT > 1)
        kernel = reinterpret_cast<const void*>(gemm_mixed_ksplit_kernel<Cfg>);
    else
        kernel = reinterpret_cast<const void*>(gemm_mixed_kernel<Cfg>);
    return hipLaunchKernel(kernel, dim3((unsigned)(tiles_m * tiles_n)), dim3(Cfg::THREADS), args, 0, stream);
}

template <class Cfg>
gemm_tile_config mixed_config(int variant, int vec) {
    gemm_tile_config c{};
    describe_common<Cfg>(c, variant, vec);
    c.tm = Cfg::WM; c.tn = Cfg::WN;
    c.a_transposed = 0;
    c.mfma_block = Cfg::Op::MB;
    c.elem_bytes = 2;
    c.k_groups = Cfg::KSPLIT;
    if (Cfg::KSPLIT > 1) c.barriers_per_tile = 1;  // per K tile of a group
    return c;
}

using MixedLaunchFn = hipError_t (*)(const Args&, hipStream_t);
struct MixedVariant {
    MixedLaunchFn vec8[2], vec2[2], scalar[2];  // by input type: 16-byte, 4-byte copies; registers
    gemm_tile_config (*config)(int variant, int vec);
    int lds_bytes;
};

// Operands whose rows are 4-byte aligned (even leading dimensions) run the
// variant's own kernel with 4-byte copies.  Rows only 2-byte aligned run
// `Unaligned` with VEC 1: raw 4-byte copies realigned in LDS where its
// tiles leave room for them (the 256x256x32 kernel for every 256x256
// variant: the three-stage and BK = 64 ones have none), else shifted 16-byte
// loads through registers; K-split variants use their base shape.
template <template <int, int> class Shape, template <int, int> class Unaligned = Shape>
MixedVariant mixed_variant() {
    return MixedVariant{{launch_mixed<Shape<kInputBf16, 8>>, launch_mixed<Shape<kInputF16, 8>>},
                        {launch_mixed<Shape<kInputBf16, 2>>, launch_mixed<Shape<kInputF16, 2>>},
                        {launch_mixed<Unaligned<kInputBf16, 1>>, launch_mixed<Unaligned<kInputF16, 1>>},
                        mixed_config<Shape<kInputBf16, 8>>,
                        Shape<kInputBf16, 8>::LDS_BYTES > Unaligned<kInputBf16, 1>::LDS_BYTES
                            ? Shape<kInputBf16, 8>::LDS_BYTES
                            : Unaligned<kInputBf16, 1>::LDS_BYTES};
}

// Index = gemm_mixed_variant; AUTO's entry describes the large-problem choice.
const MixedVariant kMixedVariants[GEMM_MIXED_COUNT] = {
    /* AUTO           */ mixed_variant<Mixed256x256Bk64, Mixed256x256>(),
    /* 256x128        */ mixed_variant<Mixed256x128>(),
    /* 256x256        */ mixed_variant<Mixed256x256>(),
    /* 256x128_BK64   */ mixed_variant<Mixed256x128Bk64>(),
    /* 128x128_BK64   */ mixed_variant<Mixed128x128Bk64>(),
    /* 256x256_S3     */ mixed_variant<Mixed256x256S3, Mixed256x256>(),
    /* 256x256_BK64   */ mixed_variant<Mixed256x256Bk64, Mixed256x256>(),
    /* 64x64          */ mixed_variant<Mixed64>(),
    /* 64x64_KS2      */ mixed_variant<Mixed64Ks2, Mixed64>(),
    /* 64x64_KS4      */ mixed_variant<Mixed64Ks4, Mixed64>(),
    /* 32x64_KS4      */ mixed_variant<Mixed32x64Ks4, Mixed32x64>(),
};

// AUTO for 16-bit inputs.  The 256x256 kernels run one workgroup per CU, the
// 128x128x64 kernel two; each is rated by the fraction of its CU-rounds that
// have work (rates 1200 and 1050 TFLOP/s), and 256x256 keeps a 10 % bias: a
// partial round of it was measured faster than the quantisation predicts (the
// idle CUs leave the busy ones more clock).  Between the two 256x256 kernels,
// BK = 64 wins when it divides K; otherwise its ragged last K tile goes
// through registers and the three-stage BK = 32 kernel was faster.
// When 256x256 tiles would fill less than half the CUs, the 64x64-tile
// kernels join: K split over 4 groups (64x64 at 420, 32x64 at 290 times
// their quantisation) when K >= 4096, over 2 groups (530 times
// min(1, 0.6 w)) when K >= 2048, and the plain 64x64 kernel (700 times
// min(1, 0.375 w)), w being 64x64 tiles per CU; listed first wins within
// 2 %.  On 24 measured bf16 shapes from 256^2 x 65536 to 8192^3 this picks
// the fastest variant or one within 4.6 % of it.
double round_fill(int64_t tiles, int64_t per_round) {
    return tiles > 0 ? (double)tiles / (double)(((tiles + per_round - 1) / per_round) * per_round) : 1.0;
}
int mixed_auto_variant(int64_t M, int64_t N, int64_t K, int num_cus) {
    const int64_t t256 = ((M + 255) / 256) * ((N + 255) / 256);
    const int64_t t128 = ((M + 127) / 128) * ((N + 127) / 128);
    const int64_t t64 = ((M + 63) / 64) * ((N + 63) / 64);
    const int64_t t32x64 = ((M + 31) / 32) * ((N + 63) / 64);
    const double e256 = round_fill(t256, num_cus), e128 = round_fill(t128, 2 * (int64_t)num_cus);
    const int big = K % 64 == 0 ? GEMM_MIXED_256x256_BK64 : GEMM_MIXED_256x256_S3;
    if (2 * t256 >= num_cus) return 1050.0 * e128 > 1.1 * 1200.0 * e256 ? GEMM_MIXED_128x128_BK64 : big;
    const double w64 = (double)t64 / (double)num_cus;
    struct Candidate {
        int variant;
        double rate;
    };
    Candidate candidates[6];
    int n = 0;
    // The K split over four groups from K = 4096, or when its grid has at
    // most one tile per CU from K = 1024 for 32x64 tiles and K = 2048 for
    // 64x64 (bf16 on one box: 32x64_KS4 11-25 % ahead of the previous pick
    // on 1-2k-row grids at K = 1024-3072; at 1024^3 64x64_KS4 ran 10 %
    // behind 64x64_KS2, four K tiles of 64 per group being too few).  Two
    // groups from K = 2048, or K = 1024 on a one-round grid.
    if (K >= 4096 || (K >= 2048 && t64 <= num_cus))
        candidates[n++] = {GEMM_MIXED_64x64_KS4, 420.0 * round_fill(t64, num_cus)};
    if (K >= 4096 || (K >= 1024 && t32x64 <= num_cus))
        candidates[n++] = {GEMM_MIXED_32x64_KS4, 290.0 * round_fill(t32x64, num_cus)};
    if (K >= 2048 || (K >= 1024 && t64 <= num_cus))
        candidates[n++] = {GEMM_MIXED_64x64_KS2, 530.0 * std::min(1.0, 0.6 * w64)};
    candidates[n++] = {GEMM_MIXED_64x64, 700.0 * std::min(1.0, 0.375 * w64)};
    candidates[n++] = {GEMM_MIXED_128x128_BK64, 1050.0 * e128};
    candidates[n++] = {big, 1.1 * 1200.0 * e256};
    int best = big;
    double best_rate = -1.0;
    for (int i = 0; i < n; ++i)
        if (candidates[i].rate > best_rate * 1.02) {
            best = candidates[i].variant;
            best_rate = candidates[i].rate;
        }
    return best;
}

int run_mixed(int input_type, const Args& a, hipStream_t stream, int variant) {
    if (input_type != GEMM_INPUT_BF16 && input_type != GEMM_INPUT_F16) return GEMM_ERR_UNSUPPORTED;
    if (variant < 0 || variant >= GEMM_MIXED_COUNT) return GEMM_ERR_UNSUPPORTED;
    int max_lds = 0, num_cus = 0;
    bool done = false;
    const int st = prologue(a, stream, &max_lds, &num_cus, &done, 2);
    if (st != GEMM_OK || done) return st;
    // 16-byte copies need rows 16-byte aligned (ld % 8 == 0, 16-byte bases);
    // 4-byte copies rows 4-byte aligned (even ld, 4-byte bases).  An edge
    // tile moved back to end at N starts its B columns at N - BN, so B's
    // copies also need N a multiple of the elements per copy.
    const bool rows16 = (a.lda % 8 == 0) && (a.ldb % 8 == 0) && (a.N % 8 == 0) && (((uintptr_t)a.A & 15) == 0) &&
                        (((uintptr_t)a.B & 15) == 0);
    const bool rows4 = (a.lda % 2 == 0) && (a.ldb % 2 == 0) && (a.N % 2 == 0) && (((uintptr_t)a.A & 3) == 0) &&
                       (((uintptr_t)a.B & 3) == 0);
    if (variant == GEMM_MIXED_AUTO) variant = mixed_auto_variant(a.M, a.N, a.K, num_cus);
    const MixedVariant& v = kMixedVariants[variant];
    if (v.lds_bytes > max_lds) return GEMM_ERR_CONFIG;
    const gemm_tile_config cfg = v.config(variant, 8);
    const int64_t tiles = ((a.M + cfg.bm - 1) / cfg.bm) * ((a.N + cfg.bn - 1) / cfg.bn);
    if (tiles > (int64_t)0x7fffffff / cfg.threads) return GEMM_ERR_TOO_LARGE;
    const MixedLaunchFn fn = rows16 ? v.vec8[input_type] : rows4 ? v.vec2[input_type] : v.scalar[input_type];
    return fn(a, stream) == hipSuccess ? GEMM_OK : GEMM_ERR_HIP;
}

}  // namespace

// ---- exported C ABI ---------------------------------------------------------------
extern "C" {

int gemm_f32(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda, const float* B, int64_t ldb,
             float* C, int64_t ldc, void* stream) {
    return run(Args{M, N, K, A, lda, B, ldb, C, ldc}, (hipStream_t)stream, GEMM_VARIANT_AUTO);
}

int gemm_f32_ex(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda, const float* B, int64_t ldb,
                float* C, int64_t ldc, void* stream, int variant) {
    return run(Args{M, N, K, A, lda, B, ldb, C, ldc}, (hipStream_t)stream, variant);
}

int gemm_f32_tile_config(int variant, gemm_tile_config* out) {
    if (out == nullptr) return GEMM_ERR_NULL;
    if (variant < 0 || variant >= GEMM_VARIANT_COUNT) return GEMM_ERR_UNSUPPORTED;
    *out = variant == GEMM_VARIANT_MFMA_SCALAR ? kVariants[variant].config1(variant, 1)
                                               : kVariants[variant].config4(variant, 4);
    return GEMM_OK;
}

int gemm_f32_auto_variant(int64_t M, int64_t N, int64_t K, int32_t num_cus) {
    if (M < 0 || N < 0 || K < 0 || num_cus < 1) return GEMM_ERR_INVALID_DIM;
    return auto_variant(M, N, K, num_cus);
}

int gemm_f32_auto_variant_ex(int64_t M, int64_t N, int64_t K, int32_t num_cus, int32_t a_rows_aligned,
                             int32_t b_rows_aligned) {
    if (M < 0 || N < 0 || K < 0 || num_cus < 1) return GEMM_ERR_INVALID_DIM;
    return auto_variant(M, N, K, num_cus, a_rows_aligned != 0, b_rows_aligned != 0);
}

int gemm_lds_choose_mfma_layout(int32_t bm, int32_t bn, int32_t bk, int32_t wm, int32_t wn, int32_t mb,
                                int32_t vec, int32_t direct, int32_t* out) {
    if (out == nullptr || (mb != 32 && mb != 16) || (vec != 1 && vec != 4)) return GEMM_ERR_INVALID_DIM;
    if (direct < 0 || direct > 2 || (direct && vec != 4)) return GEMM_ERR_INVALID_DIM;
    if (bm < 1 || bn < 1 || bk < 1 || wm < mb || wn < mb || bm % wm || bn % wn || wm % mb || wn % mb)
        return GEMM_ERR_INVALID_DIM;
    const int kb = 64 / mb, threads = (bm / wm) * (bn / wn) * kWaveLanes;
    if (bk % (4 * kb) || bk % vec || bn % vec || threads > 1024 || (bm * bk / vec) % threads ||
        (bk * bn / vec) % threads)
        return GEMM_ERR_INVALID_DIM;
    if (direct && ((bm * bk) % (threads * 4) || (bk * bn) % (threads * 4))) return GEMM_ERR_INVALID_DIM;
    if (direct == 2 && (bk / kb) % 8) return GEMM_ERR_INVALID_DIM;
    const MfmaShape shape{bm, bn, bk, wm, wn, threads, vec, mb, mb, kb, direct != 0, direct == 2};
    const LayoutChoice a = mfma_layout_a(shape, kGfx950Lds), b = mfma_layout_b(shape, kGfx950Lds);
    const int32_t v[8] = {a.pad, a.swz.unit, a.swz.shift, a.swz.mask, b.pad, b.swz.unit, b.swz.shift, b.swz.mask};
    for (int i = 0; i < 8; ++i) out[i] = v[i];
    return GEMM_OK;
}

int gemm_f32_splitk(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda, const float* B, int64_t ldb,
                    float* C, int64_t ldc, void* workspace, int64_t workspace_bytes, int splits, void* stream) {
    return run_splitk(Args{M, N, K, A, lda, B, ldb, C, ldc}, workspace, workspace_bytes, splits, (hipStream_t)stream,
                      GEMM_VARIANT_AUTO);
}

int gemm_f32_splitk_ex(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda, const float* B, int64_t ldb,
                       float* C, int64_t ldc, void* workspace, int64_t workspace_bytes, int splits, void* stream,
                       int variant) {
    return run_splitk(Args{M, N, K, A, lda, B, ldb, C, ldc}, workspace, workspace_bytes, splits, (hipStream_t)stream,
                      variant);
}

int gemm_f32_splitk_noalloc(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda, const float* B,
                            int64_t ldb, float* C, int64_t ldc, int splits, void* stream) {
    return run_splitk_noalloc(Args{M, N, K, A, lda, B, ldb, C, ldc}, splits, (hipStream_t)stream);
}

int gemm_f32_splitk_auto_variant(void) { return kSplitKVariant; }

int gemm_mixed_f32(int input_type, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                   int64_t ldb, float* C, int64_t ldc, void* stream, int variant) {
    // A and B travel in the fp32 argument block as untyped pointers; only
    // the mixed kernels read them, as 16-bit elements.
    return run_mixed(input_type,
                     Args{M, N, K, static_cast<const float*>(A), lda, static_cast<const float*>(B), ldb, C, ldc},
                     (hipStream_t)stream, variant);
}

int gemm_mixed_tile_config(int variant, gemm_tile_config* out) {
    if (out == nullptr) return GEMM_ERR_NULL;
    if (variant < 0 || variant >= GEMM_MIXED_COUNT) return GEMM_ERR_UNSUPPORTED;
    *out = kMixedVariants[variant].config(variant, 8);
    return GEMM_OK;
}

int gemm_mixed_auto_variant(int64_t M, int64_t N, int64_t K, int32_t num_cus) {
    if (M < 0 || N < 0 || K < 0 || num_cus < 1) return GEMM_ERR_INVALID_DIM;
    return mixed_auto_variant(M, N, K, num_cus);
}

int64_t gemm_f32_splitk_workspace_bytes(int64_t M, int64_t N, int64_t K, int splits, int32_t num_cus) {
    if (M < 0 || N < 0 || K < 0 || splits < 0 || splits > kMaxSplits || num_cus < 1) return GEMM_ERR_INVALID_DIM;
    if (splits == 0) splits = splitk_auto_splits(M, N, K, num_cus);
    return splits > 1 ? splitk_workspace_bytes(M, N, splits) : 0;
}

int gemm_f32_splitk_auto_splits(int64_t M, int64_t N, int64_t K, int32_t num_cus) {
    if (M < 0 || N < 0 || K < 0 || num_cus < 1) return GEMM_ERR_INVALID_DIM;
    return splitk_auto_splits(M, N, K, num_cus);
}

const char* gemm_f32_status_string(int status) {
    switch (status) {
        case GEMM_OK: return "success";
        case GEMM_ERR_INVALID_DIM: return "invalid dimension: M, N and K must be >= 0";
        case GEMM_ERR_INVALID_LD: return "invalid leading dimension: need lda >= max(1,K), ldb >= max(1,N), ldc >= max(1,N)";
        case GEMM_ERR_NULL: return "NULL pointer for an operand with non-zero extent";
        case GEMM_ERR_ALIAS: return "C overlaps A or B";
        case GEMM_ERR_UNSUPPORTED: return "unsupported: the current device is not gfx950, or the variant is unknown";
        case GEMM_ERR_CONFIG: return "tile configuration exceeds the device's LDS per workgroup";
        case GEMM_ERR_HIP: return "HIP runtime error or launch failure";
        case GEMM_ERR_TOO_LARGE: return "problem too large for the kernel's index range";
        case GEMM_ERR_WORKSPACE: return "split-K workspace missing or smaller than gemm_f32_splitk_workspace_bytes";
        case GEMM_ERR_SCRATCH:
            return "split-K partial products (splits * M * N * 4 bytes) exceed the library's 64 MiB static scratch "
                   "array";
        default: return "unknown status";
    }
}

int gemm_lds_layout(int32_t rows, int32_t cols, int32_t pad, int32_t stages, int32_t* row_stride,
                    int32_t* stage_elems, int32_t* total_elems, int32_t* bytes) {
    const LdsLayout l{rows, cols, pad, stages};
    if (!l.valid()) return GEMM_ERR_INVALID_DIM;
    if ((int64_t)rows * (cols + pad) * stages * 4 > 0x7fffffff) return GEMM_ERR_TOO_LARGE;
    if (row_stride) *row_stride = l.row_stride();
    if (stage_elems) *stage_elems = l.stage_elems();
    if (total_elems) *total_elems = l.total_elems();
    if (bytes) *bytes = l.bytes();
    return GEMM_OK;
}

int64_t gemm_lds_offset(int32_t rows, int32_t cols, int32_t pad, int32_t stages, int32_t stage, int32_t row,
                        int32_t col) {
    const LdsLayout l{rows, cols, pad, stages};
    if (!l.valid()) return -1;
    if (stage < 0 || stage >= stages || row < 0 || row >= rows || col < 0 || col >= cols) return -1;
    if ((int64_t)rows * (cols + pad) * stages > 0x7fffffff) return -1;
    return l.offset(stage, row, col);
}

int32_t gemm_lds_bank(int64_t word_offset, int32_t banks) {
    if (banks < 1 || word_offset < 0) return -1;
    return bank_of(word_offset, banks);
}

int32_t gemm_lds_conflict_degree(const int64_t* lane_words, int32_t lanes, int32_t width, int32_t banks,
                                 int32_t group) {
    if (lane_words == nullptr) return -1;
    return conflict_degree([=](int l) { return lane_words[l]; }, lanes, width, banks, group);
}

int32_t gemm_lds_access_cycles(const int64_t* lane_words, int32_t mode) {
    if (lane_words == nullptr) return -1;
    for (int l = 0; l < kWaveLanes; ++l)
        if (lane_words[l] < 0) return -1;
    auto at = [=](int l) { return lane_words[l]; };
    switch (mode) {
        case 1: case 2: case 4:
            return access_cycles(at, mode, false, kGfx950Lds);
        case 101: case 102: case 104:
            return access_cycles(at, mode - 100, true, kGfx950Lds);
        case -16: case -32: {  // ds_read2_b32: the second dword -mode words after the first
            const int off = -mode;
            return access_cycles(at, 1, false, kGfx950Lds) +
                   access_cycles([=](int l) { return lane_words[l] + off; }, 1, false, kGfx950Lds);
        }
        default:
            return -1;
    }
}

int32_t gemm_lds_page_pad(int32_t columns, int32_t simultaneous_rows, int32_t banks) {
    if (columns < 1 || simultaneous_rows < 0 || banks < 1) return -1;
    return page_pad(columns, simultaneous_rows, banks);
}

}  // extern "C"
