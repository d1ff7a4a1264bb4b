// gemm_kernels.hpp -- gfx950 kernels for C[M,N] = A[M,K] @ B[K,N], fp32.
//
// Structure common to every kernel (one workgroup per BM x BN output tile):
//   accumulators = 0
//   prologue: masked cooperative load of K tile 0 -> registers -> LDS stage 0, barrier
//   for t in [0, T):                                 T = ceil(K / BK)
//       issue the global loads of K tile t+1 into registers (if any)
//       inner product over LDS stage t & 1
//       write the registers into LDS stage (t+1) & 1, barrier
//   masked store of the accumulators
//
// The tiling, masks and zero fill are those of "My Triton From Scratch, Part
// 14: Shared-Memory Tiles" (sections "The canonical source pattern",
// "Cooperative copy mapping", "Zero-filled boundary tiles", "Synchronizing
// the block"); the padded, two-stage LDS layout and the single barrier per K
// tile are those of "Part 18: Shared Memory Optimization" (sections "A shared
// buffer needs a physical row stride", "One stage versus two stages", "What
// ping-pong changes about synchronization").  Unlike Part 18, the global loads
// of tile t+1 are in flight while tile t is multiplied.
//
// Why one barrier per tile is enough with two stages: the LDS writes of
// iteration t go to stage (t+1)&1, last read during iteration t-1, and every
// wave finished those reads before the barrier that ended iteration t-1.  The
// reads of iteration t hit stage t&1, whose writes (iteration t-1 or the
// prologue) all precede that same barrier.  The loop bounds are uniform across
// the workgroup, so every wave reaches every barrier.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "lds_layout.hpp"

// Debug build (DFT_LDS_POISON=1): every kernel fills its LDS with a NaN
// pattern before its first copy, so that a read of a word that no copy or
// store of the tile wrote puts a NaN into the result instead of stale data.
// Every consumed LDS word must hold a defined value ("My Triton From Scratch,
// Part 14: Shared-Memory Tiles", section "Zero-filled boundary tiles"); the
// parity tests run once against a library built this way.
#ifndef DFT_LDS_POISON
#define DFT_LDS_POISON 0
#endif

namespace dft {

// Fill `words` 4-byte LDS words from `lds` with a quiet NaN and wait for the
// whole workgroup (no-op unless DFT_LDS_POISON).
__device__ inline void poison_lds(void* lds, int words) {
    if constexpr (DFT_LDS_POISON) {
        uint32_t* w = static_cast<uint32_t*>(lds);
        // a NaN as fp32, and in both halves as bf16 or fp16
        for (int i = threadIdx.x; i < words; i += blockDim.x) w[i] = 0x7FC07FC0u;
        __syncthreads();
    }
}

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kWave = kWaveLanes;

// --------------------------------------------------------------------------
// A tile of a row-major global matrix: rows [row0, row0 + ROWS) and columns
// [col0, col0 + COLS), read under the mask (row < row_bound) & (col < col_bound)
// with zero fill.  Threads map to VEC-wide column groups in row-major order
// (consecutive threads take consecutive column groups of a row), so each
// wavefront reads whole row segments.
template <int ROWS, int COLS, int THREADS, int VEC>
struct TileLoader {
    static_assert(VEC == 1 || VEC == 4, "VEC must be 1 or 4");
    static_assert(COLS % VEC == 0, "tile width must be a multiple of VEC");
    static constexpr int VCOLS = COLS / VEC;
    static constexpr int SLOTS = ROWS * VCOLS;
    static_assert(SLOTS % THREADS == 0, "tile must split evenly over the threads");
    static constexpr int PER_THREAD = SLOTS / THREADS;

    float v[PER_THREAD][VEC];

    __device__ static int slot_row(int tid, int i) { return (tid + i * THREADS) / VCOLS; }
    __device__ static int slot_col(int tid, int i) { return ((tid + i * THREADS) % VCOLS) * VEC; }

    // `tile` points at element (row0, col0); rows_left = row_bound - row0 and
    // cols_left = col_bound - col0 (either may be <= 0: then all zero).  Both
    // are uniform over the workgroup, so the branch between the unmasked path
    // (the whole tile is in range) and the per-element masked path is a scalar
    // branch; only edge tiles take the masked path.
    __device__ void load(const float* __restrict__ tile, int64_t ld, int64_t rows_left,
                         int64_t cols_left, int tid) {
        if (rows_left >= ROWS && cols_left >= COLS) {
#pragma unroll
            for (int i = 0; i < PER_THREAD; ++i) {
                const float* p = tile + (int64_t)slot_row(tid, i) * ld + slot_col(tid, i);
                if constexpr (VEC == 4) {
                    const floatx4 x = *reinterpret_cast<const floatx4*>(p);
                    v[i][0] = x[0]; v[i][1] = x[1]; v[i][2] = x[2]; v[i][3] = x[3];
                } else {
                    v[i][0] = *p;
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < PER_THREAD; ++i) {
                const int r = slot_row(tid, i);
                const int c = slot_col(tid, i);
                const float* p = tile + (int64_t)r * ld + c;
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    v[i][e] = (r < rows_left && c + e < cols_left) ? p[e] : 0.0f;
            }
        }
    }

    // Row-major LDS destination: element (r, c) of the tile -> Tile::offset(stage, r, c).
    template <class Tile>
    __device__ void store(float* lds, int stage, int tid) const {
        static_assert(Tile::rows == ROWS && Tile::cols == COLS, "LDS tile shape mismatch");
#pragma unroll
        for (int i = 0; i < PER_THREAD; ++i) {
            float* q = lds + Tile::offset(stage, slot_row(tid, i), slot_col(tid, i));
            if constexpr (VEC == 4) {
                *reinterpret_cast<floatx4*>(q) = floatx4{v[i][0], v[i][1], v[i][2], v[i][3]};
            } else {
                *q = v[i][0];
            }
        }
    }

    // Masked load and LDS store of the whole tile, at most MAX_CH slots at a
    // time (the staging registers of those slots only), for kernels that
    // cannot hold all PER_THREAD slots beside their other live registers.
    template <class Tile, int MAX_CH>
    __device__ static void copy_in_chunks(const float* __restrict__ tile, int64_t ld, int64_t rows_left,
                                          int64_t cols_left, float* lds, int stage, int tid) {
        static_assert(Tile::rows == ROWS && Tile::cols == COLS, "LDS tile shape mismatch");
        constexpr int CH = MAX_CH < PER_THREAD ? MAX_CH : PER_THREAD;
        static_assert(PER_THREAD % CH == 0, "chunks must split the slots evenly");
        const bool full = rows_left >= ROWS && cols_left >= COLS;
#pragma unroll 1
        for (int i0 = 0; i0 < PER_THREAD; i0 += CH) {
            float v[CH][VEC];
#pragma unroll
            for (int i = 0; i < CH; ++i) {
                const int r = slot_row(tid, i0 + i), c = slot_col(tid, i0 + i);
                const float* p = tile + (int64_t)r * ld + c;
                if (full && VEC == 4) {
                    const floatx4 x = *reinterpret_cast<const floatx4*>(p);
#pragma unroll
                    for (int e = 0; e < VEC; ++e) v[i][e] = x[e];
                } else {
#pragma unroll
                    for (int e = 0; e < VEC; ++e) v[i][e] = (r < rows_left && c + e < cols_left) ? p[e] : 0.0f;
                }
            }
#pragma unroll
            for (int i = 0; i < CH; ++i) {
                float* q = lds + Tile::offset(stage, slot_row(tid, i0 + i), slot_col(tid, i0 + i));
                if constexpr (VEC == 4) {
                    *reinterpret_cast<floatx4*>(q) = floatx4{v[i][0], v[i][1], v[i][2], v[i][3]};
                } else {
                    *q = v[i][0];
                }
            }
        }
    }

    // Transposed LDS destination: element (r, c) -> Tile::offset(stage, c, r).
    template <class Tile>
    __device__ void store_transposed(float* lds, int stage, int tid) const {
        static_assert(Tile::rows == COLS && Tile::cols == ROWS, "LDS tile shape mismatch");
#pragma unroll
        for (int i = 0; i < PER_THREAD; ++i) {
            const int r = slot_row(tid, i), c = slot_col(tid, i);
#pragma unroll
            for (int e = 0; e < VEC; ++e) lds[Tile::offset(stage, c + e, r)] = v[i][e];
        }
    }
};

// Workgroup -> output tile.
struct TileCoord {
    int64_t m0, n0;
};

// Plain row-major order over the tile grid.
__device__ inline TileCoord tile_row_major(int64_t b, int64_t tiles_n, int bm, int bn) {
    return TileCoord{(b / tiles_n) * bm, (b % tiles_n) * bn};
}

// XCD-aware order.  The dispatcher hands workgroup b to XCD b % 8, and each
// XCD has its own L2.  Workgroups are first renumbered so that every XCD's
// share is one contiguous range of tile indices, then tile indices walk the
// grid GROUP_M tile rows at a time, column-major inside a group, so an XCD's
// tiles form a compact block that shares A rows and B columns in its L2.
template <int GROUP_M>
__device__ inline TileCoord tile_xcd_grouped(int64_t b, int64_t tiles_m, int64_t tiles_n, int bm, int bn) {
    constexpr int64_t kXcds = 8;
    const int64_t tiles = tiles_m * tiles_n;
    const int64_t q = tiles / kXcds, rem = tiles % kXcds;
    const int64_t x = b % kXcds, j = b / kXcds;
    const int64_t t = x < rem ? x * (q + 1) + j : rem * (q + 1) + (x - rem) * q + j;
    const int64_t per_group = GROUP_M * tiles_n;
    const int64_t first = (t / per_group) * GROUP_M;
    const int64_t rows = tiles_m - first < GROUP_M ? tiles_m - first : GROUP_M;
    const int64_t in = t % per_group;
    return TileCoord{(first + in % rows) * bm, (in / rows) * bn};
}

// --------------------------------------------------------------------------
// Matrix-core variant.  Wavefronts tile the workgroup's BM x BN block as
// WAVES_M x WAVES_N; each owns a WM x WN sub-tile of MB x NB MFMA blocks.
//
// fp32 MFMA operand layouts (lane l, g = l / MB, r = l % MB):
//   A operand: A[row r][k g],  B operand: B[k g][col r]  (KB = 64 / MB k-groups)
//   v_mfma_f32_32x32x2_f32: result register v (0..15) is D[8*(v/4) + 4*g + v%4][r]
//   v_mfma_f32_16x16x4_f32: result register v (0..3)  is D[4*g + v][r]
// Within a BK tile, k-group g reduces k in [g*KG, (g+1)*KG), KG = BK / KB:
// MFMA step j consumes k = g*KG + j for group g.  Every k of the tile is used
// exactly once per output element (a permutation of the summation order), and
// each lane's A values for one tile are KG consecutive floats of one LDS row,
// read with 16-byte loads.
template <int MB, int KB>
struct MfmaOp;

template <>
struct MfmaOp<32, 2> {
    static constexpr int MB = 32, NB = 32, KB = 2, ACC = 16;
    using acc_t = floatx16;
    __device__ static acc_t mma(float a, float b, acc_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
    __device__ static int out_row(int lane, int v) { return 8 * (v / 4) + 4 * (lane / 32) + (v % 4); }
};

template <>
struct MfmaOp<16, 4> {
    static constexpr int MB = 16, NB = 16, KB = 4, ACC = 4;
    using acc_t = floatx4;
    __device__ static acc_t mma(float a, float b, acc_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
    __device__ static int out_row(int lane, int v) { return 4 * (lane / 16) + v; }
};

// LDS layout of one operand tile: row pad, or XOR swizzle (see LdsTile).
template <int Pad, int Unit = 0, int Shift = 0, int Mask = 0>
struct TileLayout {
    static constexpr int pad = Pad, unit = Unit, shift = Shift, mask = Mask;
};

enum TileOrder { kRowMajorOrder = 0, kXcdGroupedOrder = 1 };

// How K tiles reach LDS: through registers (global load, then LDS store), or
// by the direct global->LDS copy for in-range tiles (DirectCopy).
enum LoadPath { kLoadRegisters = 0, kLoadDirect = 1 };

// PIPE (direct copies only): the multiply of a K tile runs in chunks of four
// k per lane group, the LDS fragments of chunk q+1 being read while chunk q
// multiplies, and the last chunk of tile t multiplies after the barrier,
// while the first fragments of tile t+1 are read; the matrix pipe then idles
// only for the barrier itself, not for the LDS latency behind it.
// COPY_STEPS (direct copies only): the next tile's copies are issued between
// the first COPY_STEPS MFMA steps of the current one (0: all before the
// first step).
template <int BM_, int BN_, int BK_, int WM_, int WN_, int STAGES_, int MB_, class LayA, class LayB, int VEC_,
          int ORDER_ = kRowMajorOrder, int LOAD_ = kLoadRegisters, bool PIPE_ = false, int VEC_B_ = 0,
          int COPY_STEPS_ = 0>
struct MfmaCfg {
    using Op = MfmaOp<MB_, 64 / MB_>;
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
    // VEC: floats per global load or direct copy of A; VEC_B: the same for B
    // (defaults to VEC).  4 needs 16-byte aligned rows, 1 takes any.
    static constexpr int STAGES = STAGES_, VEC = VEC_, ORDER = ORDER_, LOAD = LOAD_;
    static constexpr int VEC_B = VEC_B_ ? VEC_B_ : VEC_;
    static constexpr bool PIPE = PIPE_;
    static constexpr int COPY_STEPS = COPY_STEPS_;
    static constexpr int KSPLIT = 1;  // wave groups splitting K inside the workgroup (KsplitCfg)
    static constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN;
    static constexpr int THREADS = WAVES_M * WAVES_N * kWave;
    static constexpr int MI = WM / Op::MB, NI = WN / Op::NB;
    static constexpr int KG = BK / Op::KB;  // k values per lane group per tile
    // Register budget (waves per SIMD the compiler must fit): 4 (<= 128
    // VGPRs) when the tile reaches LDS by direct copies (16-byte, or 4-byte
    // with 32x32 wave tiles), or through registers with at most 12 staged
    // floats per thread; 3 for more staged floats (128x128 tiles through
    // registers: 16 or 32, which spill at 4); 2 for 4-byte loads through
    // registers (four times the load registers) and for 4-byte copies with
    // 64x64 wave tiles or more than 8 staged floats per thread, whose edge
    // tiles load 4 bytes at a time.
    // 1 for 128x128 wave tiles (256 accumulators: the whole register file
    // at one wave per SIMD).
    static constexpr int STAGED = (BM * BK + BK * BN) / THREADS;
    // Direct-copy kernels with this few staged floats per thread give edge
    // workgroups a loop of their own: the operand in range is still copied
    // directly, the other is prefetched through registers across the multiply.
    static constexpr bool EDGE_PREFETCH = STAGED <= 8;
    static constexpr int MIN_WAVES = WM * WN >= 128 * 128 ? 1
                                     : WM * WN > 64 * 64 ||
                                               ((VEC != 4 || VEC_B != 4) &&
                                                (LOAD == kLoadRegisters || WM * WN >= 64 * 64 || STAGED > 8))
                                           ? 2
                                     : (LOAD == kLoadDirect || STAGED <= 12) ? 4
                                                                             : 3;
    using TileA = LdsTile<BM, BK, LayA::pad, STAGES, LayA::unit, LayA::shift, LayA::mask>;
    using TileB = LdsTile<BK, BN, LayB::pad, STAGES, LayB::unit, LayB::shift, LayB::mask>;
    static constexpr int LDS_BYTES = TileA::bytes + TileB::bytes;
    static_assert(BM % WM == 0 && BN % WN == 0 && WM % Op::MB == 0 && WN % Op::NB == 0, "wave tiling");
    static_assert(KG % 4 == 0 && TileA::row_stride % 4 == 0, "A fragments are read 16 bytes at a time");
    static_assert(TileB::row_stride % VEC_B == 0 && TileA::row_stride % VEC == 0, "aligned LDS stores");
    static_assert(STAGES == 1 || STAGES == 2, "one or two stages");
    static_assert(LOAD == kLoadRegisters || (STAGES == 2 && LayA::pad == 0 && LayB::pad == 0),
                  "direct copies need two stages and unpadded rows");
    static_assert(!PIPE || (LOAD == kLoadDirect && KG % 8 == 0),
                  "the pipeline runs on direct copies, with an even number of 4-k chunks per tile");

    // Pipelined fragment addressing: A block row i of chunk q at
    // a_base(q) + i * MB rows; B step kk of block column n at
    // b_base(n % PB) + kk rows + (n / PB) * PB * NB words.  Holds when the
    // swizzle term of an address does not change along those strides.
    static constexpr int Q = KG / 4, PB = NI < 2 ? NI : 2;
    static constexpr bool pipelined_addressing() {
        for (int w = 0; w < WAVES_M * WAVES_N; ++w)
            for (int l = 0; l < kWave; ++l) {
                const int g = l / Op::MB, r = l % Op::MB;
                const int wm0 = (w / WAVES_N) * WM, wn0 = (w % WAVES_N) * WN;
                for (int q = 0; q < Q; ++q)
                    for (int i = 0; i < MI; ++i)
                        if (TileA::offset(0, wm0 + i * Op::MB + r, g * KG + 4 * q) !=
                            TileA::offset(0, wm0 + r, g * KG + 4 * q) + i * Op::MB * TileA::row_stride)
                            return false;
                for (int n = 0; n < NI; ++n)
                    for (int kk = 0; kk < KG; ++kk)
                        if (TileB::offset(0, g * KG + kk, wn0 + n * Op::NB + r) !=
                            TileB::offset(0, g * KG, wn0 + (n % PB) * Op::NB + r) + kk * TileB::row_stride +
                                (n / PB) * PB * Op::NB)
                            return false;
            }
        return true;
    }
    static_assert(!PIPE || pipelined_addressing(), "layout does not admit pipelined fragment addressing");
};

// One direct global->LDS copy instruction (gfx950 global_load_lds_dwordx4):
// each lane reads 16 bytes at its own global address, and the wavefront
// writes them to LDS at byte address lds_base + 16 * lane; lds_base must be
// wave-uniform and is taken from M0 (one wait state is required between
// writing M0 and the copy).  M0 is declared clobbered, so the compiler keeps
// nothing of its own there across the statement.  Written as an asm
// statement because the compiler's own form of this copy makes it wait for
// every outstanding copy before any later LDS read, which would serialise
// the copy of the next K tile with the multiply of the current one; as asm
// the copy is invisible to the compiler's wait-count tracking, so completion
// is waited for explicitly (wait_vector_memory) before the barrier that
// publishes the stage.  The "memory" clobber keeps LDS accesses from being
// moved across it.
//
// The address is a wave-uniform 64-bit base in scalar registers plus a
// 32-bit byte offset per lane (no 64-bit address arithmetic per lane and
// copy).  The base and LDS address are wave-uniform by construction; where
// the compiler cannot prove it (a scalar operand must be), READ_FIRST takes
// them from the first lane.  That costs registers elsewhere in some kernels,
// so it is used only where needed.
__device__ inline const void* first_lane(const void* p) {
    const uint64_t b = (uint64_t)(uintptr_t)p;
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
    return (const void*)(uintptr_t)(lo | (hi << 32));
}
__device__ inline uint32_t first_lane(uint32_t v) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)v); }

template <bool READ_FIRST = false>
__device__ inline void copy16_to_lds(const void* uniform_base, uint32_t byte_offset, uint32_t lds_base) {
    const void* base = READ_FIRST ? first_lane(uniform_base) : uniform_base;
    const uint32_t lds = READ_FIRST ? first_lane(lds_base) : lds_base;
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %1"
        :
        : "v"(byte_offset), "s"(base), "s"(lds)
        : "memory", "m0");
}

// The same copy moving 4 bytes per lane (global_load_lds_dword): LDS byte
// address lds_base + 4 * lane; the global address needs only 4-byte
// alignment, so it serves operands whose rows are not 16-byte aligned.
// The base and LDS address are always read from the first lane: in some of
// the kernels that use this form the compiler cannot prove them uniform.
__device__ inline void copy4_to_lds(const void* uniform_base, uint32_t byte_offset, uint32_t lds_base) {
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %0, %1"
        :
        : "v"(byte_offset), "s"(first_lane(uniform_base)), "s"(first_lane(lds_base))
        : "memory", "m0");
}

// Direct global->LDS copy of one operand tile.  A stage of an unpadded tile
// is cut into pieces of 64 lanes x BYTES (16: 1 KiB, or 4: 256 bytes),
// piece i * WAVES + w being written by wavefront w's i-th copy instruction,
// and the lane that writes LDS word p fetches the elements the tile layout
// keeps there: row p / cols, word column swizzle(row, p % cols) (the XOR
// swizzle is its own inverse, and moves groups of 4 words, so a lane's
// BYTES stay contiguous).  The tile is laid out in 4-byte words; an element
// of type T is 4 / sizeof(T) per word (1 for fp32, 2 for 16-bit inputs).
// The fetch offsets do not depend on the K tile, so they are computed once.
template <class Tile, int THREADS, class T = float, int BYTES = 16, bool READ_FIRST = false>
struct DirectCopy {
    static_assert(sizeof(T) == 4 || sizeof(T) == 2, "4- or 2-byte elements");
    static_assert(BYTES == 16 || BYTES == 4, "16- or 4-byte copies");
    static constexpr int PER_WORD = 4 / (int)sizeof(T);
    static constexpr int LANE_WORDS = BYTES / 4;  // LDS words one lane writes per copy
    static_assert(Tile::pad == 0, "direct copies write whole rows contiguously");
    static constexpr int WAVES = THREADS / kWave;
    static constexpr int PIECE = kWave * LANE_WORDS;  // fp32 words per instruction per wavefront
    static_assert(Tile::stage_elems % (PIECE * WAVES) == 0, "tile must split evenly over the wavefronts");
    static constexpr int PER_WAVE = Tile::stage_elems / (PIECE * WAVES);

    // Logical (row, col) of the element(s) stored at LDS word `word` of a stage.
    static constexpr void source(int word, int& row, int& col) {
        row = word / Tile::cols;
        col = Swizzle{Tile::swizzle.unit, Tile::swizzle.shift, Tile::swizzle.mask}.apply(row, word % Tile::cols);
    }
    // Every lane's group of LANE_WORDS words of a stage is fetched from the
    // elements the tile layout (which the fragment reads use) places there.
    static constexpr bool matches_layout() {
        for (int word = 0; word < Tile::stage_elems; word += LANE_WORDS) {
            int row = 0, col = 0;
            source(word, row, col);
            if (row >= Tile::rows || col % LANE_WORDS != 0 || col >= Tile::cols || Tile::offset(0, row, col) != word)
                return false;
        }
        return true;
    }
    static_assert(matches_layout(), "direct copies must fill the LDS tile in its own layout");

    // Copy i of a lane fetches from row row_0 + i * ROUND_ROWS.  When a round
    // of pieces (one per wavefront) covers whole rows and a whole number of
    // swizzle periods, the
    // column is the same for every i, so one offset per lane and a uniform
    // row stride describe all copies (fewer registers); otherwise each copy
    // keeps its own offset.
    static constexpr int SWIZZLE_ROWS = Tile::swizzle.unit ? (Tile::swizzle.mask + 1) << Tile::swizzle.shift : 1;
    static constexpr bool STRIDED =
        (WAVES * PIECE) % Tile::cols == 0 && ((WAVES * PIECE / Tile::cols) % SWIZZLE_ROWS) == 0;
    static constexpr int ROUND_ROWS = STRIDED ? WAVES * PIECE / Tile::cols : 0;
    static constexpr bool strided_matches() {
        if (!STRIDED) return true;
        for (int w = 0; w < WAVES; ++w)
            for (int lane = 0; lane < kWave; ++lane) {
                int r0 = 0, c0 = 0;
                source(w * PIECE + LANE_WORDS * lane, r0, c0);
                for (int i = 1; i < PER_WAVE; ++i) {
                    int r = 0, c = 0;
                    source((i * WAVES + w) * PIECE + LANE_WORDS * lane, r, c);
                    if (r != r0 + i * ROUND_ROWS || c != c0) return false;
                }
            }
        return true;
    }
    static_assert(strided_matches(), "strided copies must fetch what the per-copy offsets would");

    // Byte offsets from the tile origin must fit 31 bits: they are below
    // Tile::rows * ld elements.  A kernel copies directly only when
    // fits(ld, origin) holds (a uniform condition) and loads through
    // registers otherwise.  4-byte copies also need the operand 4-byte
    // aligned (16-byte copies are only launched on 16-byte aligned operands).
    __host__ __device__ static constexpr bool fits(int64_t ld) {
        return ld <= (((int64_t)1 << 31) - 1) / ((int64_t)Tile::rows * (int64_t)sizeof(T));
    }
    __device__ static bool fits(int64_t ld, const T* operand) {
        return fits(ld) && (BYTES == 16 || ((uintptr_t)operand & 3) == 0);
    }

    uint32_t off[STRIDED ? 1 : PER_WAVE];  // byte offset(s) of this lane's bytes from the tile origin
    int64_t round_stride;                  // elements between copy i and i+1 (strided form)
    uint32_t lds_piece;                    // byte offset of this wavefront's first piece in a stage (uniform)

    __device__ DirectCopy(int64_t ld, int wave_uniform, int lane)
        : round_stride((int64_t)ROUND_ROWS * ld), lds_piece(wave_uniform * PIECE * 4) {
#pragma unroll
        for (int i = 0; i < (STRIDED ? 1 : PER_WAVE); ++i) {
            int row = 0, col = 0;
            source((i * WAVES + wave_uniform) * PIECE + LANE_WORDS * lane, row, col);
            off[i] = (uint32_t)(((int64_t)row * ld + (int64_t)col * PER_WORD) * (int64_t)sizeof(T));
        }
    }

    // Issue the copies of the tile at `origin` into `stage` of the LDS tile
    // at `lds`; they complete asynchronously (vector memory counter).
    // Requires fits(ld).
    template <class W>
    __device__ void issue(const T* origin, W* lds, int stage) const {
#pragma unroll
        for (int i = 0; i < PER_WAVE; ++i) issue_one(origin, lds, stage, i);
    }
    // Copy i (0 <= i < PER_WAVE, a constant after unrolling) of those.
    template <class W>
    __device__ void issue_one(const T* origin, W* lds, int stage, int i) const {
        static_assert(sizeof(W) == 4, "LDS tiles are addressed in 4-byte words");
        typedef __attribute__((address_space(3))) W lds_word;
        const uint32_t base = (uint32_t)(uintptr_t)(lds_word*)lds + lds_piece + stage * (Tile::stage_elems * 4);
        const T* row_base = STRIDED ? origin + i * round_stride : origin;
        if constexpr (BYTES == 16)
            copy16_to_lds<READ_FIRST>(row_base, STRIDED ? off[0] : off[i], base + i * (WAVES * PIECE * 4));
        else
            copy4_to_lds(row_base, STRIDED ? off[0] : off[i], base + i * (WAVES * PIECE * 4));
    }
};

// Wait until this wavefront's outstanding vector memory operations, direct
// LDS copies included, have completed (s_waitcnt vmcnt(0); the expcnt and
// lgkmcnt fields of the immediate are left at their no-wait maxima).
__device__ inline void wait_vector_memory() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Wait until at most N of this wavefront's vector memory operations are
// outstanding (s_waitcnt vmcnt(N): N's low 4 bits in bits 3:0 of the
// immediate, its high 2 bits in bits 15:14).  They complete in issue order,
// so this waits for all but the N most recently issued.
template <int N>
__device__ inline void wait_vector_memory_at_most() {
    static_assert(N >= 0 && N <= 63, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Store of a wavefront's MFMA accumulators.  The accumulators hold the
// BM x BN block whose first row and column are (ma, na); the workgroup owns
// rows [m0, M) and columns [n0, N) of it (m0 >= ma and n0 >= na: a tile moved
// back to end at M or N leaves the rows or columns before m0 or n0 to the
// workgroup that owns them).  Unmasked when the block is the workgroup's own
// and wholly in range (a uniform branch), else under the mask.  For a fixed
// result register, the MB lanes of a k-group write consecutive floats of one
// row.
// f(std::integral_constant<int, I>{}) for I = 0, 1, ..., N - 1, in order.
template <class F, int... I>
__device__ inline void static_for_each(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ inline void static_for(F&& f) {
    static_for_each(f, std::make_integer_sequence<int, N>{});
}

template <class Op, int BM, int BN, int MI, int NI>
__device__ inline void store_accumulators(float* __restrict__ C, int64_t ldc, int64_t M, int64_t N, int64_t ma,
                                          int64_t na, int64_t m0, int64_t n0, int wm0, int wn0, int lane,
                                          const typename Op::acc_t (&acc)[MI][NI], int j_lo = 0,
                                          int j_hi = MI * NI * Op::ACC) {
    const int r = lane % Op::MB;
    const bool full = ma == m0 && na == n0 && m0 + BM <= M && n0 + BN <= N;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int n = 0; n < NI; ++n) {
            const int64_t gn = na + wn0 + n * Op::NB + r;
            const int64_t gm0 = ma + wm0 + i * Op::MB;
            float* cp = C + gm0 * ldc + gn;
#pragma unroll
            for (int v = 0; v < Op::ACC; ++v) {
                const int j = (i * NI + n) * Op::ACC + v;  // flat index of the value
                if (j < j_lo || j >= j_hi) continue;
                const int dr = Op::out_row(lane, v);
                if (full || (gm0 + dr >= m0 && gm0 + dr < M && gn >= n0 && gn < N)) cp[dr * ldc] = acc[i][n][v];
            }
        }
}

// Whether a kernel moves its overhanging edge tiles back inside C (below):
// the direct-copy kernels, and any configuration that says so.
template <class Cfg, class = void>
struct moves_edge_tiles : std::bool_constant<Cfg::LOAD == kLoadDirect> {};
template <class Cfg>
struct moves_edge_tiles<Cfg, std::void_t<decltype(Cfg::MOVE_EDGE_TILES)>>
    : std::bool_constant<Cfg::LOAD == kLoadDirect || Cfg::MOVE_EDGE_TILES> {};

// Origin of the operand tiles of a workgroup whose output tile starts at
// (m0, n0).  Direct-copy kernels (and the register kernels for 16-bit rows
// that are only 2-byte aligned) move a tile that overhangs M (N) back so
// that it ends at M (N), when M >= BM (N >= BN): an A row beyond M feeds only
// outputs beyond M, and a B column beyond N only outputs beyond N, so the
// moved tile's rows are all in range and need no zero fill (its copies run
// like an interior tile's), and its outputs are the same sums; the rows and
// columns that it recomputes before m0 and n0 are not stored.  Only the K
// direction needs zero fill.
template <class Cfg>
__device__ inline TileCoord operand_origin(TileCoord own, int64_t M, int64_t N) {
    if constexpr (!moves_edge_tiles<Cfg>::value) return own;
    const int64_t ma = own.m0 + Cfg::BM > M && M >= Cfg::BM ? M - Cfg::BM : own.m0;
    const int64_t na = own.n0 + Cfg::BN > N && N >= Cfg::BN ? N - Cfg::BN : own.n0;
    return TileCoord{ma, na};
}

template <class Cfg>
__device__ inline TileCoord tile_of_block(int64_t tiles_m, int64_t tiles_n) {
    if constexpr (Cfg::ORDER == kXcdGroupedOrder)
        return tile_xcd_grouped<8>(blockIdx.x, tiles_m, tiles_n, Cfg::BM, Cfg::BN);
    else
        return tile_row_major(blockIdx.x, tiles_n, Cfg::BM, Cfg::BN);
}

// Slice of the K range a workgroup reduces: blockIdx.y selects k in
// [y * k_chunk, min(K, (y + 1) * k_chunk)) and output C + y * c_split_stride
// (split-K); a plain launch has gridDim.y == 1 and k_chunk >= K.  k_chunk is a
// multiple of BK, so 16-byte alignment of the operand tiles is preserved.
struct KSlice {
    const float* A;
    const float* B;
    float* C;
    int64_t K;  // length of this slice (may be <= 0: an empty sum)
};
__device__ inline KSlice k_slice(const float* A, const float* B, float* C, int64_t K, int64_t ldb, int64_t k_chunk,
                                 int64_t c_split_stride) {
    const int64_t y = blockIdx.y;
    const int64_t kb = y * k_chunk;
    const int64_t len = K - kb < k_chunk ? K - kb : k_chunk;
    return KSlice{A + kb, B + kb * ldb, C + y * c_split_stride, len};
}

template <class Cfg>
__global__ __launch_bounds__(Cfg::THREADS, Cfg::MIN_WAVES) void gemm_mfma_kernel(
    int64_t M, int64_t N, int64_t K_total, const float* __restrict__ A_in, int64_t lda,
    const float* __restrict__ B_in, int64_t ldb, float* __restrict__ C_out, int64_t ldc, int64_t tiles_m,
    int64_t tiles_n, int64_t k_chunk, int64_t c_split_stride) {
    const KSlice ks = k_slice(A_in, B_in, C_out, K_total, ldb, k_chunk, c_split_stride);
    const float* __restrict__ A = ks.A;
    const float* __restrict__ B = ks.B;
    float* __restrict__ C = ks.C;
    const int64_t K = ks.K;
    using Op = typename Cfg::Op;
    using TileA = typename Cfg::TileA;
    using TileB = typename Cfg::TileB;
    using acc_t = typename Op::acc_t;
    constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, KG = Cfg::KG;
    constexpr int MI = Cfg::MI, NI = Cfg::NI, THREADS = Cfg::THREADS;

    __shared__ __attribute__((aligned(16))) float lds_a[TileA::total_elems];
    __shared__ __attribute__((aligned(16))) float lds_b[TileB::total_elems];
    poison_lds(lds_a, TileA::total_elems);
    poison_lds(lds_b, TileB::total_elems);

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = tid / kWave;
    const int wm0 = (wave / Cfg::WAVES_N) * Cfg::WM;
    const int wn0 = (wave % Cfg::WAVES_N) * Cfg::WN;
    const int g = lane / Op::MB, r = lane % Op::MB;

    const TileCoord own = tile_of_block<Cfg>(tiles_m, tiles_n);
    const TileCoord tc = operand_origin<Cfg>(own, M, N);
    const int64_t m0 = tc.m0, n0 = tc.n0;

    acc_t acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
            for (int v = 0; v < Op::ACC; ++v) acc[i][j][v] = 0.0f;

    TileLoader<BM, BK, THREADS, Cfg::VEC> ldr_a;
    TileLoader<BK, BN, THREADS, Cfg::VEC_B> ldr_b;
    const float* a_tile = A + m0 * lda;  // advances by BK columns per K tile
    const float* b_tile = B + n0;        // advances by BK rows per K tile
    const int64_t T = K > 0 ? (K + BK - 1) / BK : 0;

    auto load_tile = [&](int64_t t) {
        const int64_t k0 = t * BK;
        ldr_a.load(a_tile + k0, lda, M - m0, K - k0, tid);
        ldr_b.load(b_tile + k0 * ldb, ldb, K - k0, N - n0, tid);
    };
    auto multiply = [&](int stage) {
        floatx4 af[MI][KG / 4];
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int q = 0; q < KG / 4; ++q)
                af[i][q] = *reinterpret_cast<const floatx4*>(
                    lds_a + TileA::offset(stage, wm0 + i * Op::MB + r, g * KG + 4 * q));
#pragma unroll
        for (int j = 0; j < KG; ++j) {
            float bf[NI];
#pragma unroll
            for (int n = 0; n < NI; ++n) bf[n] = lds_b[TileB::offset(stage, g * KG + j, wn0 + n * Op::NB + r)];
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int n = 0; n < NI; ++n) acc[i][n] = Op::mma(af[i][j / 4][j % 4], bf[n], acc[i][n]);
        }
    };

    // Two stages through registers: the global loads of tile t+1 are issued
    // before the multiply of tile t and written to LDS after it.
    auto two_stage_registers = [&]() {
        if (T > 0) {
            load_tile(0);
            ldr_a.template store<TileA>(lds_a, 0, tid);
            ldr_b.template store<TileB>(lds_b, 0, tid);
        }
        __syncthreads();
        for (int64_t t = 0; t < T; ++t) {
            const int s = (int)(t & 1);
            const bool more = t + 1 < T;
            if (more) load_tile(t + 1);
            multiply(s);
            if (more) {
                ldr_a.template store<TileA>(lds_a, s ^ 1, tid);
                ldr_b.template store<TileB>(lds_b, s ^ 1, tid);
            }
            __syncthreads();
        }
    };

    if constexpr (Cfg::LOAD == kLoadDirect) {
        // Two stages filled by direct copies: the copies of tile t+1 are in
        // flight during the multiply of tile t, and each wave waits for its
        // own copies before the barrier, after which the whole stage is in
        // LDS.  A tile not wholly in range needs zero fill: the last K tile
        // when BK does not divide K, and every tile of a workgroup whose
        // tile cannot move back inside C (M < BM or N < BN) or whose
        // operand is too wide for the copies' offsets.  It is loaded
        // through registers with masks after the multiply, so that no
        // staging registers are live across it.  Both choices are uniform.
        // Kernels with different copy widths for A and B lose the compiler's
        // proof that the 16-byte copies' bases are uniform.
        constexpr bool READ_FIRST = Cfg::VEC != Cfg::VEC_B;
        using DA = DirectCopy<TileA, THREADS, float, 4 * Cfg::VEC, READ_FIRST>;
        using DB = DirectCopy<TileB, THREADS, float, 4 * Cfg::VEC_B, READ_FIRST>;
        const DA dma_a(lda, __builtin_amdgcn_readfirstlane(wave), lane);
        const DB dma_b(ldb, __builtin_amdgcn_readfirstlane(wave), lane);
        // Pieces [CS_lo, CS_hi) of the next tile's copies, issued after MFMA
        // step kk when COPY_STEPS > 0 (A's copies first, then B's).
        constexpr int COPY_STEPS = Cfg::COPY_STEPS;
        constexpr int PC = DA::PER_WAVE + DB::PER_WAVE;
        auto issue_after_step = [&](int kk, int64_t t_next, int nstage) {
            if constexpr (COPY_STEPS > 0) {
                if (kk < COPY_STEPS) {
#pragma unroll
                    for (int p = kk * PC / COPY_STEPS; p < (kk + 1) * PC / COPY_STEPS; ++p) {
                        if (p < DA::PER_WAVE)
                            dma_a.issue_one(a_tile + t_next * BK, lds_a, nstage, p);
                        else
                            dma_b.issue_one(b_tile + t_next * BK * ldb, lds_b, nstage, p - DA::PER_WAVE);
                    }
                }
            }
        };
        // The multiply with those copies between its steps; B of step j + 1
        // is read before step j's copies (the copies are ordered with every
        // memory access), so it lands during step j.
        auto multiply_spread = [&](int stage, int64_t t_next, int nstage, bool copy) {
            floatx4 af[MI][KG / 4];
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int q = 0; q < KG / 4; ++q)
                    af[i][q] = *reinterpret_cast<const floatx4*>(
                        lds_a + TileA::offset(stage, wm0 + i * Op::MB + r, g * KG + 4 * q));
            float bf[2][NI];
#pragma unroll
            for (int n = 0; n < NI; ++n) bf[0][n] = lds_b[TileB::offset(stage, g * KG, wn0 + n * Op::NB + r)];
#pragma unroll
            for (int j = 0; j < KG; ++j) {
                if (j + 1 < KG) {
#pragma unroll
                    for (int n = 0; n < NI; ++n)
                        bf[(j + 1) % 2][n] = lds_b[TileB::offset(stage, g * KG + j + 1, wn0 + n * Op::NB + r)];
                }
#pragma unroll
                for (int i = 0; i < MI; ++i)
#pragma unroll
                    for (int n = 0; n < NI; ++n)
                        acc[i][n] = Op::mma(af[i][j / 4][j % 4], bf[j % 2][n], acc[i][n]);
                if (copy) issue_after_step(j, t_next, nstage);
            }
        };
        // A's tiles are wholly in range when the workgroup's rows are (but for
        // a ragged last K tile), B's when its columns are.
        const bool rows_in = M - m0 >= BM && DA::fits(lda, A);
        const bool cols_in = N - n0 >= BN && DB::fits(ldb, B);
        const bool interior = rows_in && cols_in;
        auto fill = [&](int64_t t, int stage) {
            const int64_t k0 = t * BK;
            const bool k_in = K - k0 >= BK;
            if (rows_in && k_in) {
                dma_a.issue(a_tile + k0, lds_a, stage);
            } else {
                ldr_a.load(a_tile + k0, lda, M - m0, K - k0, tid);
                ldr_a.template store<TileA>(lds_a, stage, tid);
            }
            if (cols_in && k_in) {
                dma_b.issue(b_tile + k0 * ldb, lds_b, stage);
            } else {
                ldr_b.load(b_tile + k0 * ldb, ldb, K - k0, N - n0, tid);
                ldr_b.template store<TileB>(lds_b, stage, tid);
            }
        };
        if (T > 0) fill(0, 0);
        wait_vector_memory();
        __syncthreads();
        if constexpr (Cfg::PIPE) {
            // Iteration t copies tile t+1 directly iff the workgroup is
            // interior and tile t+1 is wholly in range (t + 1 < K / BK).
            // (Copying the in-range operand of an edge workgroup directly
            // and only the other through registers measured 4% slower on
            // interior workgroups too: the two conditions cost registers
            // and scheduling freedom in the loop.)
            const int64_t t_direct = interior ? K / BK - 1 : 0;
            // Software pipeline over the MFMA steps of a K tile (step kk
            // consumes k = g * KG + kk for lane group g).  The B fragments of
            // step kk+1 are read while step kk multiplies; the A fragments
            // come in chunks of four steps (one 16-byte read per row block),
            // chunk q+1 being read at the start of chunk q.  Steps and chunks
            // alternate between two register buffers (KG and KG / 4 are
            // even, so step 0 and chunk 0 of every tile use buffer 0).  The
            // last step of tile t multiplies after the barrier, while the
            // first fragments of tile t+1 are read, so the matrix pipe idles
            // only for the barrier itself.  Every read of stage s completes
            // before that barrier (it waits for them, and the last step's
            // registers are needed after it anyway), so the copies issued
            // after it may overwrite stage s.
            constexpr int Q = Cfg::Q, PB = Cfg::PB;
            int a_base[Q], b_base[PB];
#pragma unroll
            for (int q = 0; q < Q; ++q) a_base[q] = TileA::offset(0, wm0 + r, g * KG + 4 * q);
#pragma unroll
            for (int p = 0; p < PB; ++p) b_base[p] = TileB::offset(0, g * KG, wn0 + p * Op::NB + r);
            floatx4 fa[2][MI];
            float fb[2][NI];
            auto read_a = [&](int buf, int stage, int q) {
                const float* base = lds_a + stage * TileA::stage_elems + a_base[q];
#pragma unroll
                for (int i = 0; i < MI; ++i)
                    fa[buf][i] = *reinterpret_cast<const floatx4*>(base + i * Op::MB * TileA::row_stride);
            };
            auto read_b = [&](int buf, int stage, int kk) {
#pragma unroll
                for (int n = 0; n < NI; ++n)
                    fb[buf][n] = lds_b[stage * TileB::stage_elems + b_base[n % PB] + kk * TileB::row_stride +
                                       (n / PB) * PB * Op::NB];
            };
            auto mma_step = [&](int abuf, int j, int bbuf) {
#pragma unroll
                for (int i = 0; i < MI; ++i)
#pragma unroll
                    for (int n = 0; n < NI; ++n) acc[i][n] = Op::mma(fa[abuf][i][j], fb[bbuf][n], acc[i][n]);
            };
            if (T > 0) {
                read_a(0, 0, 0);
                read_b(0, 0, 0);
            }
            for (int64_t t = 0; t < T; ++t) {
                const int s = (int)(t & 1);
                const bool more = t + 1 < T;
                const bool direct = t < t_direct;
                if (direct && COPY_STEPS == 0) {
                    dma_a.issue(a_tile + (t + 1) * BK, lds_a, s ^ 1);
                    dma_b.issue(b_tile + (t + 1) * BK * ldb, lds_b, s ^ 1);
                }
#pragma unroll
                for (int kk = 0; kk + 1 < KG; ++kk) {
                    const int q = kk / 4, j = kk % 4;
                    if (j == 0 && q + 1 < Q) read_a((q + 1) & 1, s, q + 1);
                    read_b((kk + 1) & 1, s, kk + 1);
                    __builtin_amdgcn_sched_barrier(0);
                    mma_step(q & 1, j, kk & 1);
                    __builtin_amdgcn_sched_barrier(0);
                    if (direct) issue_after_step(kk, t + 1, s ^ 1);
                }
                if (more && !direct) {
                    // Next tile through registers (zero fill), a few slots at
                    // a time: the staging registers of whole tiles would not
                    // fit beside the live fragment buffers.
                    using LoaderA = TileLoader<BM, BK, THREADS, Cfg::VEC>;
                    using LoaderB = TileLoader<BK, BN, THREADS, Cfg::VEC_B>;
                    const int64_t k0 = (t + 1) * BK;
                    LoaderA::template copy_in_chunks<TileA, Cfg::VEC == 4 ? 4 : 2>(a_tile + k0, lda, M - m0, K - k0,
                                                                                    lds_a, s ^ 1, tid);
                    LoaderB::template copy_in_chunks<TileB, Cfg::VEC_B == 4 ? 4 : 2>(b_tile + k0 * ldb, ldb, K - k0,
                                                                                      N - n0, lds_b, s ^ 1, tid);
                }
                wait_vector_memory();
                __syncthreads();
                if (more) {
                    read_a(0, s ^ 1, 0);
                    read_b(0, s ^ 1, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
                mma_step(1, 3, 1);
                __builtin_amdgcn_sched_barrier(0);
            }
        } else if (interior || !Cfg::EDGE_PREFETCH) {
            // Interior workgroups, and every workgroup of kernels without
            // EDGE_PREFETCH (the edge loop below would not fit their register
            // budget beside this one).  Both operands copied directly when the
            // workgroup is interior, else through registers; a ragged last K tile (K % BK)
            // goes through registers after the multiply.  (Prefetching it
            // across the multiply, as the edge loop below does, measured
            // slower here: it costs every iteration a branch and registers.)
            const int64_t t_direct = interior ? K / BK - 1 : 0;
            for (int64_t t = 0; t < T; ++t) {
                const int s = (int)(t & 1);
                const bool more = t + 1 < T;
                const bool direct = t < t_direct;
                if constexpr (COPY_STEPS > 0) {
                    multiply_spread(s, t + 1, s ^ 1, direct);
                } else {
                    if (direct) {
                        dma_a.issue(a_tile + (t + 1) * BK, lds_a, s ^ 1);
                        dma_b.issue(b_tile + (t + 1) * BK * ldb, lds_b, s ^ 1);
                    }
                    multiply(s);
                }
                if (more && !direct) {
                    load_tile(t + 1);
                    ldr_a.template store<TileA>(lds_a, s ^ 1, tid);
                    ldr_b.template store<TileB>(lds_b, s ^ 1, tid);
                }
                wait_vector_memory();
                __syncthreads();
            }
        } else if constexpr (Cfg::EDGE_PREFETCH) {
            // Edge workgroup, per operand: a direct copy when that operand's
            // next tile is in range, else a masked load through registers,
            // issued before the multiply and stored after it (as in the
            // register path; the staging registers are few).
            const int64_t t_direct_a = rows_in ? K / BK - 1 : 0;
            const int64_t t_direct_b = cols_in ? K / BK - 1 : 0;
            for (int64_t t = 0; t < T; ++t) {
                const int s = (int)(t & 1);
                const bool more = t + 1 < T;
                const bool direct_a = t < t_direct_a, direct_b = t < t_direct_b;
                const int64_t k1 = (t + 1) * BK;
                if (direct_a) dma_a.issue(a_tile + k1, lds_a, s ^ 1);
                if (direct_b) dma_b.issue(b_tile + k1 * ldb, lds_b, s ^ 1);
                if (more && !direct_a) ldr_a.load(a_tile + k1, lda, M - m0, K - k1, tid);
                if (more && !direct_b) ldr_b.load(b_tile + k1 * ldb, ldb, K - k1, N - n0, tid);
                multiply(s);
                if (more && !direct_a) ldr_a.template store<TileA>(lds_a, s ^ 1, tid);
                if (more && !direct_b) ldr_b.template store<TileB>(lds_b, s ^ 1, tid);
                wait_vector_memory();
                __syncthreads();
            }
        }
    } else if constexpr (Cfg::STAGES == 2) {
        two_stage_registers();
    } else {
        // One stage: write, barrier, read, barrier (the two-barrier protocol).
        for (int64_t t = 0; t < T; ++t) {
            load_tile(t);
            ldr_a.template store<TileA>(lds_a, 0, tid);
            ldr_b.template store<TileB>(lds_b, 0, tid);
            __syncthreads();
            multiply(0);
            __syncthreads();
        }
    }

    store_accumulators<Op, BM, BN, MI, NI>(C, ldc, M, N, m0, n0, own.m0, own.n0, wm0, wn0, lane, acc);
}

// --------------------------------------------------------------------------
// K split inside the workgroup.  KSPLIT groups of waves share one output
// tile: group q reduces the K tiles t = q, q + KSPLIT, q + 2 KSPLIT, ... in a
// pair of LDS stages of its own, with Base's wave tiling, direct copies and
// two-stage loop (the copy of its next tile in flight during the multiply of
// the current one).  A grid of few output tiles (deep K, small M and N) then
// still runs several waves per SIMD, without a workspace.  Every group runs
// ceil(T / KSPLIT) iterations (a group past its last tile skips the
// multiply), so all waves reach every barrier.  A ragged last K tile goes
// through registers, stored to LDS after the multiply of the group's
// previous tile (its global loads issued before that multiply where the
// registers allow), and its multiply runs only the MFMA steps that hold
// in-range columns.  At the end wave w of
// every group holds the same outputs in the same lanes and registers; group
// q owns the q-th of KSPLIT equal slices of those values.  Each group leaves
// the other groups' slices in LDS, in lane order, and after a barrier adds
// the others' partial sums for its own slice in group order (a fixed order:
// the result is deterministic) and stores that slice of C.
template <class Base, int KSPLIT_, int COPY_STEPS_ = 0>
struct KsplitCfg {
    static_assert(Base::LOAD == kLoadDirect && Base::STAGES == 2 && !Base::PIPE,
                  "groups run Base's two-stage direct-copy loop");
    static_assert(KSPLIT_ >= 2, "at least two groups");
    using Op = typename Base::Op;
    static constexpr int KSPLIT = KSPLIT_;
    static constexpr int BM = Base::BM, BN = Base::BN, BK = Base::BK, WM = Base::WM, WN = Base::WN;
    static constexpr int VEC = Base::VEC, VEC_B = Base::VEC_B, ORDER = Base::ORDER, LOAD = kLoadDirect;
    static constexpr bool PIPE = false;
    static constexpr int WAVES_N = Base::WAVES_N, MI = Base::MI, NI = Base::NI, KG = Base::KG;
    static constexpr int GROUP_THREADS = Base::THREADS, GROUP_WAVES = GROUP_THREADS / kWave;
    static constexpr int THREADS = GROUP_THREADS * KSPLIT;
    static constexpr int COPY_STEPS = COPY_STEPS_;
    static constexpr int STAGES = 2 * KSPLIT;  // stages 2q, 2q+1 belong to group q
    static constexpr int MIN_WAVES = Base::MIN_WAVES > THREADS / 256 ? Base::MIN_WAVES : THREADS / 256;
    using TileA = LdsTile<BM, BK, 0, STAGES, Base::TileA::swizzle.unit, Base::TileA::swizzle.shift,
                          Base::TileA::swizzle.mask>;
    using TileB = LdsTile<BK, BN, 0, STAGES, Base::TileB::swizzle.unit, Base::TileB::swizzle.shift,
                          Base::TileB::swizzle.mask>;
    static constexpr int LDS_BYTES = TileA::bytes + TileB::bytes;
    // Exchanged partial sums, over the stages' LDS: slice p of group q's
    // values (q != p) for every wave, KSPLIT x KSPLIT regions in all.
    static constexpr int PARTIAL_VALUES = MI * NI * Op::ACC;  // per lane
    static constexpr int SLICE_VALUES = PARTIAL_VALUES / KSPLIT;
    static_assert(PARTIAL_VALUES % KSPLIT == 0, "the groups' slices are equal");
    static_assert(KSPLIT * KSPLIT * GROUP_WAVES * SLICE_VALUES * kWave <= TileA::total_elems + TileB::total_elems,
                  "the partial sums fit in the stages");
};

template <class Cfg>
__global__ __launch_bounds__(Cfg::THREADS, Cfg::MIN_WAVES) void gemm_mfma_ksplit_kernel(
    int64_t M, int64_t N, int64_t K_total, const float* __restrict__ A_in, int64_t lda,
    const float* __restrict__ B_in, int64_t ldb, float* __restrict__ C_out, int64_t ldc, int64_t tiles_m,
    int64_t tiles_n, int64_t k_chunk, int64_t c_split_stride) {
    const KSlice ks = k_slice(A_in, B_in, C_out, K_total, ldb, k_chunk, c_split_stride);
    const float* __restrict__ A = ks.A;
    const float* __restrict__ B = ks.B;
    float* __restrict__ C = ks.C;
    const int64_t K = ks.K;
    using Op = typename Cfg::Op;
    using TileA = typename Cfg::TileA;
    using TileB = typename Cfg::TileB;
    using acc_t = typename Op::acc_t;
    constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, KG = Cfg::KG, KS = Cfg::KSPLIT;
    constexpr int MI = Cfg::MI, NI = Cfg::NI, GT = Cfg::GROUP_THREADS;

    // One array: A's stages, then B's; the partial sums reuse all of it.
    __shared__ __attribute__((aligned(16))) float lds[TileA::total_elems + TileB::total_elems];
    poison_lds(lds, TileA::total_elems + TileB::total_elems);
    float* const lds_a = lds;
    float* const lds_b = lds + TileA::total_elems;

    const int tid = threadIdx.x;
    const int group = __builtin_amdgcn_readfirstlane(tid / GT);  // whole waves belong to one group
    const int gtid = tid % GT;                                     // thread within the group
    const int lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(gtid / kWave);  // wave within the group
    const int wm0 = (wave / Cfg::WAVES_N) * Cfg::WM;
    const int wn0 = (wave % Cfg::WAVES_N) * Cfg::WN;
    const int g = lane / Op::MB, r = lane % Op::MB;

    const TileCoord own = tile_of_block<Cfg>(tiles_m, tiles_n);
    const TileCoord tc = operand_origin<Cfg>(own, M, N);
    const int64_t m0 = tc.m0, n0 = tc.n0;

    acc_t acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
            for (int v = 0; v < Op::ACC; ++v) acc[i][j][v] = 0.0f;

    TileLoader<BM, BK, GT, Cfg::VEC> ldr_a;
    TileLoader<BK, BN, GT, Cfg::VEC_B> ldr_b;
    const float* a_tile = A + m0 * lda;
    const float* b_tile = B + n0;
    const int64_t T = K > 0 ? (K + BK - 1) / BK : 0;  // K tiles
    const int64_t TF = K / BK;                        // K tiles wholly in range
    const int64_t ITERS = (TF + KS - 1) / KS;         // per group, over whole tiles

    constexpr bool READ_FIRST = Cfg::VEC != Cfg::VEC_B;
    using DA = DirectCopy<TileA, GT, float, 4 * Cfg::VEC, READ_FIRST>;
    using DB = DirectCopy<TileB, GT, float, 4 * Cfg::VEC_B, READ_FIRST>;
    const DA dma_a(lda, wave, lane);
    const DB dma_b(ldb, wave, lane);
    const bool interior = M - m0 >= BM && N - n0 >= BN && DA::fits(lda, A) && DB::fits(ldb, B);

    // Tile t of this group into stage `stage`: directly when in range, else
    // through registers with zero fill (by the group's threads).
    auto copy_direct = [&](int64_t t, int stage) {
        dma_a.issue(a_tile + t * BK, lds_a, stage);
        dma_b.issue(b_tile + t * BK * ldb, lds_b, stage);
    };
    auto load_registers = [&](int64_t t) {
        const int64_t k0 = t * BK;
        ldr_a.load(a_tile + k0, lda, M - m0, K - k0, gtid);
        ldr_b.load(b_tile + k0 * ldb, ldb, K - k0, N - n0, gtid);
    };
    auto store_registers = [&](int stage) {
        ldr_a.template store<TileA>(lds_a, stage, gtid);
        ldr_b.template store<TileB>(lds_b, stage, gtid);
    };
    // MFMA step j takes k = j + KG g in lane group g, so a tile with only
    // `steps` columns in range needs steps j < min(steps, KG).
    auto multiply = [&](int stage, int steps) {
        floatx4 af[MI][KG / 4];
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int q = 0; q < KG / 4; ++q)
                af[i][q] = *reinterpret_cast<const floatx4*>(
                    lds_a + TileA::offset(stage, wm0 + i * Op::MB + r, g * KG + 4 * q));
#pragma unroll
        for (int j = 0; j < KG; ++j) {
            if (j < steps) {  // uniform; constant true for whole tiles
                float bf[NI];
#pragma unroll
                for (int n = 0; n < NI; ++n) bf[n] = lds_b[TileB::offset(stage, g * KG + j, wn0 + n * Op::NB + r)];
#pragma unroll
                for (int i = 0; i < MI; ++i)
#pragma unroll
                    for (int n = 0; n < NI; ++n) acc[i][n] = Op::mma(af[i][j / 4][j % 4], bf[n], acc[i][n]);
            }
        }
    };
    // The next tile's direct copies issued between the MFMA steps of the
    // current one, within the first COPY_STEPS steps (0: all before the
    // multiply).
    constexpr int COPY_STEPS = Cfg::COPY_STEPS;
    constexpr int PC = DA::PER_WAVE + DB::PER_WAVE;
    auto multiply_copy = [&](int stage, int64_t tn, int nstage, bool copy) {
        const float* a_src = a_tile + tn * BK;
        const float* b_src = b_tile + tn * BK * ldb;
        floatx4 af[MI][KG / 4];
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int q = 0; q < KG / 4; ++q)
                af[i][q] = *reinterpret_cast<const floatx4*>(
                    lds_a + TileA::offset(stage, wm0 + i * Op::MB + r, g * KG + 4 * q));
        // B of step j + 1 is read before step j's copies (the copies are
        // ordered with every memory access), so it lands during step j.
        float bf[2][NI];
#pragma unroll
        for (int n = 0; n < NI; ++n) bf[0][n] = lds_b[TileB::offset(stage, g * KG, wn0 + n * Op::NB + r)];
#pragma unroll
        for (int j = 0; j < KG; ++j) {
            if (j + 1 < KG) {
#pragma unroll
                for (int n = 0; n < NI; ++n)
                    bf[(j + 1) % 2][n] = lds_b[TileB::offset(stage, g * KG + j + 1, wn0 + n * Op::NB + r)];
            }
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int n = 0; n < NI; ++n) acc[i][n] = Op::mma(af[i][j / 4][j % 4], bf[j % 2][n], acc[i][n]);
            if (j < COPY_STEPS && copy) {
#pragma unroll
                for (int p = j * PC / (COPY_STEPS > 0 ? COPY_STEPS : 1);
                     p < (j + 1) * PC / (COPY_STEPS > 0 ? COPY_STEPS : 1); ++p) {
                    if (p < DA::PER_WAVE)
                        dma_a.issue_one(a_src, lds_a, nstage, p);
                    else
                        dma_b.issue_one(b_src, lds_b, nstage, p - DA::PER_WAVE);
                }
            }
        }
    };
    const int tail_steps = (int)(K - TF * BK) < KG ? (int)(K - TF * BK) : KG;  // the ragged tile's steps
    // Registers to hold a staged tile across the multiply: 512 threads (a
    // 256-register budget) and at most 16 values per thread per tile.
    constexpr bool HOIST = Cfg::THREADS <= 512 && GT >= 256;

    const int stage0 = 2 * group;
    if (group < T) {
        if (interior && group < TF) {
            copy_direct(group, stage0);
        } else {
            load_registers(group);
            store_registers(stage0);
        }
    }
    wait_vector_memory();
    __syncthreads();
    for (int64_t it = 0; it < ITERS; ++it) {
        const int s = stage0 + (int)(it & 1), ns = stage0 + (int)((it & 1) ^ 1);
        const int64_t t = it * KS + group, tn = t + KS;
        const bool direct = interior && tn < TF;
        const bool staged = tn < T && !direct;  // tile tn through registers, around the multiply
        if constexpr (COPY_STEPS > 0) {
            if (HOIST && staged) load_registers(tn);
            if (t < TF) multiply_copy(s, tn, ns, direct);  // direct implies t < TF
        } else {
            if (direct) copy_direct(tn, ns);
            if (HOIST && staged) load_registers(tn);
            if (t < TF) multiply(s, KG);
        }
        if (staged) {
            if (!HOIST) load_registers(tn);
            store_registers(ns);
        }
        wait_vector_memory();
        __syncthreads();
    }
    // The ragged last tile TF belongs to group TF % KS, which stored it into
    // the stage after its last whole tile's (its first stage if it has none)
    // and has not written that stage since.
    if (T > TF) {
        if (group == (int)(TF % KS)) multiply(stage0 + (int)(((TF - group) / KS) & 1), tail_steps);
        __syncthreads();
    }

    // Every LDS read of the loop and of the ragged tile completed before the
    // last barrier.  Region (p, q): group q's partial sums of group p's
    // slice, one float per lane per value.  Each group runs its own copy of
    // the exchange (P = its index), so every register and LDS offset in it
    // is a constant.
    constexpr int SV = Cfg::SLICE_VALUES, GW = Cfg::GROUP_WAVES;
    float* const exch = lds + wave * SV * kWave + lane;
    auto region = [&](int p, int q) { return exch + (p * KS + q) * GW * SV * kWave; };
    auto for_each_group = [&](auto&& body) {
        static_for<KS>([&](auto P_) {
            if (group == decltype(P_)::value) body(P_);
        });
    };
    for_each_group([&](auto P_) {
        constexpr int P = decltype(P_)::value;
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int n = 0; n < NI; ++n)
#pragma unroll
                for (int v = 0; v < Op::ACC; ++v) {
                    const int j = (i * NI + n) * Op::ACC + v;
                    if (j / SV != P) region(j / SV, P)[(j % SV) * kWave] = acc[i][n][v];
                }
    });
    __syncthreads();
    for_each_group([&](auto P_) {
        constexpr int P = decltype(P_)::value;
#pragma unroll
        for (int q = 0; q < KS; ++q) {
            if (q == P) continue;
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int n = 0; n < NI; ++n)
#pragma unroll
                    for (int v = 0; v < Op::ACC; ++v) {
                        const int j = (i * NI + n) * Op::ACC + v;
                        if (j / SV == P) acc[i][n][v] += region(P, q)[(j % SV) * kWave];
                    }
        }
        store_accumulators<Op, BM, BN, MI, NI>(C, ldc, M, N, m0, n0, own.m0, own.n0, wm0, wn0, lane, acc, P * SV,
                                               P * SV + SV);
    });
}

// --------------------------------------------------------------------------
// Vector-ALU variant.  THREADS = (BM/TM) x (BN/TN) threads; thread (ty, tx)
// owns a TM x TN register tile made of two TM/2-row halves (rows ty*TM/2 and
// BM/2 + ty*TM/2) and two TN/2-column halves, so that neighbouring threads
// read neighbouring 16-byte LDS words.  A is stored k-major in LDS (At[k][m]),
// B row-major (B[k][n]); per k each thread reads TM + TN values with 16-byte
// loads and issues TM * TN FMAs.
template <int BM_, int BN_, int BK_, int TM_, int TN_, int STAGES_, class LayA, class LayB, int VEC_>
struct ValuCfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, TM = TM_, TN = TN_;
    static constexpr int STAGES = STAGES_, VEC = VEC_;
    static constexpr int THREADS_M = BM / TM, THREADS_N = BN / TN;
    static constexpr int THREADS = THREADS_M * THREADS_N;
    static constexpr int MIN_WAVES = 2;
    static constexpr int ORDER = kRowMajorOrder;
    static constexpr int LOAD = kLoadRegisters;
    using TileA = LdsTile<BK, BM, LayA::pad, STAGES, LayA::unit, LayA::shift, LayA::mask>;  // k-major
    using TileB = LdsTile<BK, BN, LayB::pad, STAGES, LayB::unit, LayB::shift, LayB::mask>;
    static constexpr int LDS_BYTES = TileA::bytes + TileB::bytes;
    static_assert(TM == 8 && TN == 8, "register tile is two 4-wide halves per axis");
    static_assert(TileA::row_stride % 4 == 0 && TileB::row_stride % 4 == 0, "16-byte LDS reads");
};

template <class Cfg>
__global__ __launch_bounds__(Cfg::THREADS, Cfg::MIN_WAVES) void gemm_valu_kernel(
    int64_t M, int64_t N, int64_t K_total, const float* __restrict__ A_in, int64_t lda,
    const float* __restrict__ B_in, int64_t ldb, float* __restrict__ C_out, int64_t ldc, int64_t tiles_m,
    int64_t tiles_n, int64_t k_chunk, int64_t c_split_stride) {
    const KSlice ks = k_slice(A_in, B_in, C_out, K_total, ldb, k_chunk, c_split_stride);
    const float* __restrict__ A = ks.A;
    const float* __restrict__ B = ks.B;
    float* __restrict__ C = ks.C;
    const int64_t K = ks.K;
    using TileA = typename Cfg::TileA;
    using TileB = typename Cfg::TileB;
    constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, THREADS = Cfg::THREADS;

    __shared__ __attribute__((aligned(16))) float lds_a[TileA::total_elems];
    __shared__ __attribute__((aligned(16))) float lds_b[TileB::total_elems];
    poison_lds(lds_a, TileA::total_elems);
    poison_lds(lds_b, TileB::total_elems);

    const int tid = threadIdx.x;
    const int ty = tid / Cfg::THREADS_N, tx = tid % Cfg::THREADS_N;
    const TileCoord tc = tile_of_block<Cfg>(tiles_m, tiles_n);
    const int64_t m0 = tc.m0, n0 = tc.n0;

    float acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = 0.0f;

    TileLoader<BM, BK, THREADS, Cfg::VEC> ldr_a;
    TileLoader<BK, BN, THREADS, Cfg::VEC> ldr_b;
    const float* a_tile = A + m0 * lda;
    const float* b_tile = B + n0;
    const int64_t T = K > 0 ? (K + BK - 1) / BK : 0;
    const int am = ty * 4, bn = tx * 4;

    auto load_tile = [&](int64_t t) {
        const int64_t k0 = t * BK;
        ldr_a.load(a_tile + k0, lda, M - m0, K - k0, tid);
        ldr_b.load(b_tile + k0 * ldb, ldb, K - k0, N - n0, tid);
    };
    // Per k: four 16-byte LDS reads (TM values of A, TN values of B) and
    // TM * TN FMAs.  The reads for k+1 are issued before the FMAs of k.  After
    // each k an empty asm statement that takes every accumulator as an operand
    // and clobbers memory pins the FMAs of k before the reads of k+2: without
    // it the compiler hoists all BK steps' reads (BK * 16 registers) and spills.
    auto multiply = [&](int stage) {
        floatx4 cur[4], nxt[4];
        auto read_k = [&](int k, floatx4* x) {
            x[0] = *reinterpret_cast<const floatx4*>(lds_a + TileA::offset(stage, k, am));
            x[1] = *reinterpret_cast<const floatx4*>(lds_a + TileA::offset(stage, k, BM / 2 + am));
            x[2] = *reinterpret_cast<const floatx4*>(lds_b + TileB::offset(stage, k, bn));
            x[3] = *reinterpret_cast<const floatx4*>(lds_b + TileB::offset(stage, k, BN / 2 + bn));
        };
        read_k(0, cur);
#pragma unroll
        for (int k = 0; k < BK; ++k) {
            if (k + 1 < BK) read_k(k + 1, nxt);
            const float a[8] = {cur[0][0], cur[0][1], cur[0][2], cur[0][3], cur[1][0], cur[1][1], cur[1][2], cur[1][3]};
            const float b[8] = {cur[2][0], cur[2][1], cur[2][2], cur[2][3], cur[3][0], cur[3][1], cur[3][2], cur[3][3]};
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                asm volatile("" : "+v"(acc[i][0]), "+v"(acc[i][1]), "+v"(acc[i][2]), "+v"(acc[i][3]),
                             "+v"(acc[i][4]), "+v"(acc[i][5]), "+v"(acc[i][6]), "+v"(acc[i][7])::"memory");
#pragma unroll
            for (int q = 0; q < 4; ++q) cur[q] = nxt[q];
        }
    };

    if constexpr (Cfg::STAGES == 2) {
        if (T > 0) {
            load_tile(0);
            ldr_a.template store_transposed<TileA>(lds_a, 0, tid);
            ldr_b.template store<TileB>(lds_b, 0, tid);
        }
        __syncthreads();
        for (int64_t t = 0; t < T; ++t) {
            const int s = (int)(t & 1);
            const bool more = t + 1 < T;
            if (more) load_tile(t + 1);
            multiply(s);
            if (more) {
                ldr_a.template store_transposed<TileA>(lds_a, s ^ 1, tid);
                ldr_b.template store<TileB>(lds_b, s ^ 1, tid);
            }
            __syncthreads();
        }
    } else {
        for (int64_t t = 0; t < T; ++t) {
            load_tile(t);
            ldr_a.template store_transposed<TileA>(lds_a, 0, tid);
            ldr_b.template store<TileB>(lds_b, 0, tid);
            __syncthreads();
            multiply(0);
            __syncthreads();
        }
    }

    // Masked store; 16-byte stores where the four columns are in range and aligned.
    const bool vec_ok = (ldc % 4 == 0) && ((reinterpret_cast<uintptr_t>(C) & 15) == 0);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t gm = m0 + (i < 4 ? am + i : BM / 2 + am + i - 4);
        if (gm >= M) continue;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int64_t gn = n0 + (half == 0 ? bn : BN / 2 + bn);
            float* p = C + gm * ldc + gn;
            if (vec_ok && gn + 4 <= N) {
                *reinterpret_cast<floatx4*>(p) =
                    floatx4{acc[i][4 * half], acc[i][4 * half + 1], acc[i][4 * half + 2], acc[i][4 * half + 3]};
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (gn + e < N) p[e] = acc[i][4 * half + e];
            }
        }
    }
}

}  // namespace dft
