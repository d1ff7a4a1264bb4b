// mixed_kernels.hpp -- gfx950 kernel for C[M,N] = A[M,K] @ B[K,N] with 16-bit
// inputs (bf16 or fp16, row-major, given as bit patterns) and fp32
// accumulation and output.
//
// This is the mixed-precision step that "My Triton From Scratch, Part 18:
// Shared Memory Optimization" announces as the next part: the same masked,
// zero-filled tiling and two-stage LDS pipeline as the fp32 kernels
// (gemm_kernels.hpp), with 16-bit operand tiles and the 16-bit matrix-core
// instructions.  Products of two bf16 (or fp16) values are exact in fp32, so
// the result differs from the exact sum only by the fp32 accumulation.
//
// Per wavefront and MFMA step (KB elements of k):
//   A fragment: lane l of k-group g = l / MB holds A[row l % MB][8g .. 8g+7],
//               16 consecutive bytes of an LDS row (one 16-byte read);
//   B fragment: lane l holds B[8g .. 8g+7][column l % MB], a column segment
//               of the row-major B tile, delivered by two transposing reads
//               (ds_read_b64_tr_b16): in each group of 16 lanes, lane j gives
//               the address of 4 consecutive elements of row j / 4 of a 4 x 16
//               block, and lane i receives element i of each of the 4 rows.
// Both layouts were checked on the device against a host model of the
// instruction.  Tiles are filled by direct global->LDS copies (DirectCopy)
// when in range, else through registers with zero fill.
#pragma once

#include <type_traits>

#include "gemm_kernels.hpp"

namespace dft {

enum InputType { kInputBf16 = 0, kInputF16 = 1 };

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int TYPE, int MB>
struct Mfma16Op;

template <int TYPE>
struct Mfma16Op<TYPE, 32> {
    static constexpr int MB = 32, NB = 32, KB = 16, ACC = 16;
    using acc_t = floatx16;
    __device__ static acc_t mma(u32x4 a, u32x4 b, acc_t c) {
        if constexpr (TYPE == kInputBf16)
            return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                           c, 0, 0, 0);
        else
            return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                          0, 0, 0);
    }
    __device__ static int out_row(int lane, int v) { return MfmaOp<32, 2>::out_row(lane, v); }
    // k-group of a lane and first column of its 16-lane group within the block
    __host__ __device__ static constexpr int kgroup(int lane) { return lane / 32; }
    __host__ __device__ static constexpr int col_base(int lane) { return 16 * ((lane / 16) % 2); }
};

template <int TYPE>
struct Mfma16Op<TYPE, 16> {
    static constexpr int MB = 16, NB = 16, KB = 32, ACC = 4;
    using acc_t = floatx4;
    __device__ static acc_t mma(u32x4 a, u32x4 b, acc_t c) {
        if constexpr (TYPE == kInputBf16)
            return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                           c, 0, 0, 0);
        else
            return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                          0, 0, 0);
    }
    __device__ static int out_row(int lane, int v) { return MfmaOp<16, 4>::out_row(lane, v); }
    __host__ __device__ static constexpr int kgroup(int lane) { return lane / 16; }
    __host__ __device__ static constexpr int col_base(int) { return 0; }
};

// Orders the scheduling region that ends here as N pairs of one MFMA then
// one LDS read, and closes it.  Placed after a step's fragment reads for
// the next step and its MFMAs, it spreads those reads over the MFMAs, so
// they issue while the matrix pipe works instead of in one burst ahead of
// it (groups left without a read stay empty).
template <int N>
__device__ __forceinline__ void alternate_mfma_and_lds_reads() {
#pragma unroll
    for (int q = 0; q < N; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
    }
    __builtin_amdgcn_sched_barrier(0);
}

// A tile of a row-major 16-bit matrix, rows [row0, row0 + ROWS) and columns
// [col0, col0 + COLS), read under the mask (row < row_bound) & (col <
// col_bound) with zero fill, through registers; VEC = 8 (16-byte loads, when
// aligned) or 1.  Threads map to VEC-wide column groups in row-major order.
// Used for tiles the direct copy cannot take (edges) and for unaligned
// operands.
template <int ROWS, int COLS, int THREADS, int VEC>
struct TileLoader16 {
    static_assert(VEC == 1 || VEC == 8, "VEC must be 1 or 8");
    static_assert(COLS % 8 == 0, "tile width must be a multiple of 8 elements");
    static constexpr int VCOLS = COLS / VEC;
    static constexpr int SLOTS = ROWS * VCOLS;
    static_assert(SLOTS % THREADS == 0, "tile must split evenly over the threads");
    static constexpr int PER_THREAD = SLOTS / THREADS;

    uint16_t v[PER_THREAD][VEC];

    __device__ static int slot_row(int tid, int i) { return (tid + i * THREADS) / VCOLS; }
    __device__ static int slot_col(int tid, int i) { return ((tid + i * THREADS) % VCOLS) * VEC; }

    __device__ void load(const uint16_t* __restrict__ tile, int64_t ld, int64_t rows_left, int64_t cols_left,
                         int tid) {
        if (rows_left >= ROWS && cols_left >= COLS) {
#pragma unroll
            for (int i = 0; i < PER_THREAD; ++i) {
                const uint16_t* p = tile + (int64_t)slot_row(tid, i) * ld + slot_col(tid, i);
                if constexpr (VEC == 8) {
                    const u32x4 x = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        v[i][2 * e] = (uint16_t)(x[e] & 0xffffu);
                        v[i][2 * e + 1] = (uint16_t)(x[e] >> 16);
                    }
                } else {
                    v[i][0] = *p;
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < PER_THREAD; ++i) {
                const int r = slot_row(tid, i);
                const int c = slot_col(tid, i);
                const uint16_t* p = tile + (int64_t)r * ld + c;
#pragma unroll
                for (int e = 0; e < VEC; ++e) v[i][e] = (r < rows_left && c + e < cols_left) ? p[e] : (uint16_t)0;
            }
        }
    }

    // Masked load and LDS store of the whole tile, at most MAX_CH slots at a
    // time (the staging registers of those slots only), for kernels that
    // cannot hold all PER_THREAD slots beside their other live registers.
    template <class Tile, int MAX_CH>
    __device__ static void copy_in_chunks(const uint16_t* __restrict__ tile, int64_t ld, int64_t rows_left,
                                          int64_t cols_left, uint32_t* lds, int stage, int tid) {
        static_assert(Tile::rows == ROWS && 2 * Tile::cols == COLS, "LDS tile shape mismatch");
        constexpr int CH = MAX_CH < PER_THREAD ? MAX_CH : PER_THREAD;
        static_assert(PER_THREAD % CH == 0, "chunks must split the slots evenly");
        const bool full = rows_left >= ROWS && cols_left >= COLS;
#pragma unroll 1
        for (int i0 = 0; i0 < PER_THREAD; i0 += CH) {
            uint32_t w[CH][VEC == 8 ? 4 : 1];
            uint16_t h[CH];
#pragma unroll
            for (int i = 0; i < CH; ++i) {
                const int r = slot_row(tid, i0 + i), c = slot_col(tid, i0 + i);
                const uint16_t* p = tile + (int64_t)r * ld + c;
                if constexpr (VEC == 8) {
                    if (full) {
                        const u32x4 x = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
                        for (int e = 0; e < 4; ++e) w[i][e] = x[e];
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const uint32_t lo = (r < rows_left && c + 2 * e < cols_left) ? p[2 * e] : 0u;
                            const uint32_t hi = (r < rows_left && c + 2 * e + 1 < cols_left) ? p[2 * e + 1] : 0u;
                            w[i][e] = lo | (hi << 16);
                        }
                    }
                } else {
                    h[i] = (r < rows_left && c < cols_left) ? *p : (uint16_t)0;
                }
            }
#pragma unroll
            for (int i = 0; i < CH; ++i) {
                const int r = slot_row(tid, i0 + i), c = slot_col(tid, i0 + i);
                if constexpr (VEC == 8) {
                    *reinterpret_cast<u32x4*>(lds + Tile::offset(stage, r, c / 2)) =
                        u32x4{w[i][0], w[i][1], w[i][2], w[i][3]};
                } else {
                    reinterpret_cast<uint16_t*>(lds + Tile::offset(stage, r, c / 2))[c % 2] = h[i];
                }
            }
        }
    }

    // Element (r, c) -> 16-bit half (c % 2) of word Tile::offset(stage, r, c / 2).
    template <class Tile>
    __device__ void store(uint32_t* lds, int stage, int tid) const {
        static_assert(Tile::rows == ROWS && 2 * Tile::cols == COLS, "LDS tile shape mismatch");
#pragma unroll
        for (int i = 0; i < PER_THREAD; ++i) {
            const int r = slot_row(tid, i), c = slot_col(tid, i);
            if constexpr (VEC == 8) {
                u32x4 x;
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = (uint32_t)v[i][2 * e] | ((uint32_t)v[i][2 * e + 1] << 16);
                *reinterpret_cast<u32x4*>(lds + Tile::offset(stage, r, c / 2)) = x;
            } else {
                reinterpret_cast<uint16_t*>(lds + Tile::offset(stage, r, c / 2))[c % 2] = v[i][0];
            }
        }
    }
};

// A tile of a row-major 16-bit matrix whose rows are only 2-byte aligned
// (an odd leading dimension or base), read 16 bytes per slot through
// registers.  A slot's 8 elements are fetched as the five 4-byte-aligned
// words that hold them (a 16-byte load from the word holding the first
// element, and a 4-byte load of the word after those four), then moved down
// by 0 or 2 bytes (v_alignbyte) as they are stored to LDS, so the loads can
// be issued well before the store.  Every word read holds an element of the
// slot (when the slot starts word-aligned the fifth load repeats the fourth
// word), so no read leaves the pages of the operand.  In a tile that
// overhangs the matrix (the last K tile when BK does not divide K; edge
// tiles move back inside C) the slots not wholly in range take masked
// 2-byte loads with zero fill.
template <int ROWS, int COLS, int THREADS>
struct TileLoaderShifted16 {
    static constexpr int VCOLS = COLS / 8;
    static constexpr int SLOTS = ROWS * VCOLS;
    static_assert(COLS % 8 == 0 && SLOTS % THREADS == 0, "tile must split evenly over the threads");
    static constexpr int PER_THREAD = SLOTS / THREADS;

    static_assert(PER_THREAD <= 32, "one shift bit per slot");
    uint32_t w[PER_THREAD][5];
    uint32_t shifted;  // bit i: slot i's elements start 2 bytes into its first word

    __device__ static int slot_row(int tid, int i) { return (tid + i * THREADS) / VCOLS; }
    __device__ static int slot_col(int tid, int i) { return ((tid + i * THREADS) % VCOLS) * 8; }

    // The 8 elements of the slot at (r, c) of a tile whose rows_left x
    // cols_left corner is in range, from p (2-byte aligned) at that slot:
    // the five words, and whether they start 2 bytes early.  A slot not
    // wholly in range is read element by element with zero fill (shift 0).
    __device__ static void fetch_whole(const uint16_t* p, uint32_t (&w)[5], uint32_t& s) {
        s = (uint32_t)(uintptr_t)p & 2u;
        // pointer arithmetic (not an integer round trip) keeps the loads in
        // the global address space
        const uint32_t* q = reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(p) - s);
        u32x4 x;
        __builtin_memcpy(&x, q, sizeof(x));
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = x[e];
        w[4] = q[s ? 4 : 3];
    }
    __device__ static void fetch(const uint16_t* p, int r, int c, int64_t rows_left, int64_t cols_left,
                                 uint32_t (&w)[5], uint32_t& s) {
        if (r < rows_left && c + 8 <= cols_left) {
            fetch_whole(p, w, s);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t lo = (r < rows_left && c + 2 * e < cols_left) ? p[2 * e] : 0u;
                const uint32_t hi = (r < rows_left && c + 2 * e + 1 < cols_left) ? p[2 * e + 1] : 0u;
                w[e] = lo | (hi << 16);
            }
            w[4] = 0;
            s = 0;
        }
    }
    __device__ static u32x4 shifted_words(const uint32_t (&w)[5], uint32_t s) {
        return u32x4{__builtin_amdgcn_alignbyte(w[1], w[0], s), __builtin_amdgcn_alignbyte(w[2], w[1], s),
                     __builtin_amdgcn_alignbyte(w[3], w[2], s), __builtin_amdgcn_alignbyte(w[4], w[3], s)};
    }

    __device__ void load(const uint16_t* __restrict__ tile, int64_t ld, int64_t rows_left, int64_t cols_left,
                         int tid) {
        shifted = 0;
        if (rows_left >= ROWS && cols_left >= COLS) {  // whole tile in range: no per-slot test
#pragma unroll
            for (int i = 0; i < PER_THREAD; ++i) {
                uint32_t s = 0;
                fetch_whole(tile + (int64_t)slot_row(tid, i) * ld + slot_col(tid, i), w[i], s);
                shifted |= (s >> 1) << i;
            }
        } else {
#pragma unroll
            for (int i = 0; i < PER_THREAD; ++i) {
                const int r = slot_row(tid, i), c = slot_col(tid, i);
                uint32_t s = 0;
                fetch(tile + (int64_t)r * ld + c, r, c, rows_left, cols_left, w[i], s);
                shifted |= (s >> 1) << i;
            }
        }
    }

    // Masked load and LDS store of the whole tile, CH slots at a time (the
    // staging registers of those slots only), for a tile loaded while the
    // multiply's registers are live.
    template <class Tile, int CH>
    __device__ static void copy_in_chunks(const uint16_t* __restrict__ tile, int64_t ld, int64_t rows_left,
                                          int64_t cols_left, uint32_t* lds, int stage, int tid) {
        static_assert(Tile::rows == ROWS && 2 * Tile::cols == COLS, "LDS tile shape mismatch");
        static_assert(PER_THREAD % CH == 0, "chunks must split the slots evenly");
#pragma unroll 1
        for (int i0 = 0; i0 < PER_THREAD; i0 += CH) {
            uint32_t w[CH][5], s[CH];
#pragma unroll
            for (int i = 0; i < CH; ++i) {
                const int r = slot_row(tid, i0 + i), c = slot_col(tid, i0 + i);
                fetch(tile + (int64_t)r * ld + c, r, c, rows_left, cols_left, w[i], s[i]);
            }
#pragma unroll
            for (int i = 0; i < CH; ++i) {
                const int r = slot_row(tid, i0 + i), c = slot_col(tid, i0 + i);
                *reinterpret_cast<u32x4*>(lds + Tile::offset(stage, r, c / 2)) = shifted_words(w[i], s[i]);
            }
        }
    }

    // Element (r, c) -> 16-bit half (c % 2) of word Tile::offset(stage, r, c / 2).
    template <class Tile>
    __device__ void store(uint32_t* lds, int stage, int tid) const {
        static_assert(Tile::rows == ROWS && 2 * Tile::cols == COLS, "LDS tile shape mismatch");
#pragma unroll
        for (int i = 0; i < PER_THREAD; ++i) {
            const int r = slot_row(tid, i), c = slot_col(tid, i);
            *reinterpret_cast<u32x4*>(lds + Tile::offset(stage, r, c / 2)) =
                shifted_words(w[i], ((shifted >> i) & 1u) * 2u);
        }
    }
};

// Direct 4-byte copies of a tile of a row-major 16-bit matrix whose rows are
// only 2-byte aligned (ROWS rows of COLS elements).  A row whose first
// element is the upper half of a 4-byte word (shift 2) has its elements in
// COLS / 2 + 1 words.  The main copies fetch, for every row, the COLS / 2
// words from the one holding its first element into a plain row-major main
// area.  The word after those is, for a tile of A followed by another whole
// K tile, the first main word of the same row in that tile, which the
// realignment reads from that tile's main area; otherwise (B, whose tile
// rows are K indices, and A's last whole tile) the extra copies fetch it
// into an extra area (one word per row, 64 rows per copy instruction; for a
// row that starts word-aligned, a second copy of its last word, so that no
// read leaves the row's own words).  realign() then
// moves each row down by its shift, 4 words at a time, into the kernel's LDS
// tile layout: output word c of a row is bytes shift .. shift+3 of raw
// words c, c+1.  A round of main copies covers an even number of whole rows,
// so the shift of the row a lane fetches, and its column, are the same in
// every round: one offset per lane and a uniform row stride describe all
// main copies.  Tile origins advance by whole words along K, so the shifts
// and offsets hold for every K tile.
template <int ROWS, int COLS, int THREADS>
struct RawCopy16 {
    static constexpr int WAVES = THREADS / kWave;
    static constexpr int RW = COLS / 2;  // main words per row
    static constexpr int MAIN = ROWS * RW;
    static constexpr int ROUND = WAVES * kWave;  // words per round of main copies
    static constexpr int ROUND_ROWS = RW > 0 && ROUND % RW == 0 ? ROUND / RW : 0;
    static constexpr int PER_WAVE = MAIN / ROUND;
    static constexpr int EXTRA_COPIES = (ROWS + kWave - 1) / kWave;
    static constexpr int EXTRA_WORDS = EXTRA_COPIES * kWave;
    static constexpr int GROUPS = MAIN / 4;  // realign groups of 4 words
    // Every thread realigns (REALIGNERS: measured no faster when only one
    // of the two waves on each SIMD did, the other multiplying meanwhile).
    static constexpr int REALIGNERS = THREADS;
    static constexpr int REALIGN_GROUPS = GROUPS / REALIGNERS;
    static constexpr bool OK = COLS % 8 == 0 && ROUND_ROWS > 0 && ROUND_ROWS % 2 == 0 && MAIN % ROUND == 0 &&
                               EXTRA_COPIES <= WAVES && GROUPS % REALIGNERS == 0 && REALIGN_GROUPS <= 32;

    // Byte offsets from the tile origin fit 31 bits.
    __host__ __device__ static constexpr bool fits(int64_t ld) {
        return ld <= (((int64_t)1 << 31) - 4 * RW - 8) / (2 * (int64_t)ROWS);
    }
    // Shift (bytes) of row `row` of a tile whose origin is `lead` bytes past a word boundary.
    __device__ static uint32_t row_shift(uint32_t lead, int64_t row, int64_t ld) {
        return (lead + 2u * ((uint32_t)(row * ld) & 1u)) & 2u;
    }
    // Byte offset of the word holding row `row`'s first element from the word holding the origin.
    __device__ static uint32_t row_start(uint32_t lead, int64_t row, int64_t ld) {
        return (uint32_t)(lead + 2 * row * ld) - row_shift(lead, row, ld);
    }

    uint32_t main_off;    // this lane's main copy in round 0
    uint32_t extra_off;   // this lane's extra copy (the wave that makes one)
    uint32_t lead;        // origin & 2
    int64_t round_bytes;  // ROUND_ROWS rows
    int wave;             // wave-uniform
    uint32_t shifted;     // bit i: realign group i of this thread has shift 2

    __device__ RawCopy16(int64_t ld, uint32_t lead_, int wave_uniform, int lane, int tid)
        : lead(lead_), round_bytes((int64_t)ROUND_ROWS * ld * 2), wave(wave_uniform) {
        const int word = wave * kWave + lane;
        main_off = row_start(lead, word / RW, ld) + 4u * (uint32_t)(word % RW);
        const int64_t row = wave * kWave + lane < ROWS ? wave * kWave + lane : ROWS - 1;
        extra_off = row_start(lead, row, ld) + 4u * (uint32_t)(row_shift(lead, row, ld) ? RW : RW - 1);
        shifted = 0;
#pragma unroll
        for (int i = 0; i < REALIGN_GROUPS; ++i)
            shifted |= (row_shift(lead, (tid + i * REALIGNERS) / (RW / 4), ld) >> 1) << i;
    }

    // Issue the main copies of the tile at `origin` into `main` (MAIN
    // words); they complete asynchronously (vector memory counter).
    __device__ void issue_main(const uint16_t* origin, uint32_t* main) const {
        static_assert(OK, "tile shape unsuited to raw copies");
        typedef __attribute__((address_space(3))) uint32_t lds_word;
        const char* base = reinterpret_cast<const char*>(origin) - lead;
        const uint32_t lds = (uint32_t)(uintptr_t)(lds_word*)main;
#pragma unroll
        for (int i = 0; i < PER_WAVE; ++i)
            copy4_to_lds(base + i * round_bytes, main_off, lds + 4u * (uint32_t)((i * WAVES + wave) * kWave));
    }
    // The extra copies (waves below EXTRA_COPIES) into `extra` (EXTRA_WORDS words).
    __device__ void issue_extra(const uint16_t* origin, uint32_t* extra) const {
        typedef __attribute__((address_space(3))) uint32_t lds_word;
        if (wave < EXTRA_COPIES)
            copy4_to_lds(reinterpret_cast<const char*>(origin) - lead, extra_off,
                         (uint32_t)(uintptr_t)(lds_word*)extra + 4u * (uint32_t)(wave * kWave));
    }

    // Rows of the landed tile at `main`, shifted into place, to `stage` of
    // the LDS tile at `lds` (threads below REALIGNERS).  The word after row
    // r's main words is after[r * after_stride]: in the next K tile's main
    // area (stride RW) or in an extra area (stride 1).
    template <class Tile>
    __device__ void realign(const uint32_t* main, const uint32_t* after, int after_stride, uint32_t* lds, int stage,
                            int tid) const {
        static_assert(Tile::rows == ROWS && Tile::cols == RW, "LDS tile shape mismatch");
#pragma unroll
        for (int i = 0; i < REALIGN_GROUPS; ++i) {
            const int g = tid + i * REALIGNERS;
            const int row = g / (RW / 4), j = g % (RW / 4);
            const u32x4 x = *reinterpret_cast<const u32x4*>(main + row * RW + 4 * j);
            const uint32_t next = j + 1 < RW / 4 ? main[row * RW + 4 * j + 4] : after[row * after_stride];
            const uint32_t sh = ((shifted >> i) & 1u) * 2u;
            const u32x4 y{__builtin_amdgcn_alignbyte(x[1], x[0], sh), __builtin_amdgcn_alignbyte(x[2], x[1], sh),
                          __builtin_amdgcn_alignbyte(x[3], x[2], sh), __builtin_amdgcn_alignbyte(next, x[3], sh)};
            *reinterpret_cast<u32x4*>(lds + Tile::offset(stage, row, 4 * j)) = y;
            // two groups at a time: bounds the registers live beside the
            // multiply's accumulators and fragments
            if (i % 2 == 1) __builtin_amdgcn_sched_barrier(0);
        }
    }
};

// PIPELINE: 0, fragments read next to their MFMAs; 1, the fragments of MFMA
// step st+1 read during the MFMAs of step st (twice the fragment
// registers); 2, as 1 and across K tiles too: the last step of tile t
// multiplies after the barrier, while the first fragments of tile t+1 are
// read (direct-copy path; it shortens the time the copies of tile t+1 have
// before the barrier waits for them, so it pays with four steps per tile or
// three stages).
enum PipelineLevel { kPipeNone = 0, kPipeSteps = 1, kPipeAcrossTiles = 2 };

template <int TYPE_, int BM_, int BN_, int BK_, int WM_, int WN_, int MB_, class LayA, class LayB, int VEC_,
          int MIN_WAVES_, int STAGES_ = 2, int PIPELINE_ = kPipeSteps>
struct MixedCfg {
    using Op = Mfma16Op<TYPE_, MB_>;
    static constexpr int TYPE = TYPE_;
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
    static constexpr int VEC = VEC_;
    static constexpr int MIN_WAVES = VEC != 8 && MIN_WAVES_ > 2 ? 2 : MIN_WAVES_;
    static constexpr int ORDER = kXcdGroupedOrder;
    // VEC 8: 16-byte direct copies; 2: 4-byte direct copies (two elements,
    // rows 4-byte aligned); 1: 2-byte loads through registers.
    static_assert(VEC == 8 || VEC == 2 || VEC == 1, "16-byte, 4-byte or 2-byte operand access");
    static constexpr int LOAD = VEC == 1 ? kLoadRegisters : kLoadDirect;
    static constexpr int LOADER_VEC = VEC == 8 ? 8 : 1;  // register-path loads (edge and ragged tiles)
    // The register kernels (VEC 1) also move edge tiles back inside C, so
    // that only the K direction takes masked loads.
    static constexpr bool MOVE_EDGE_TILES = true;
    static constexpr int STAGES = STAGES_;  // LDS stages of the direct-copy pipeline (register paths use two)
    static constexpr int PIPELINE = PIPELINE_;
    static constexpr int KSPLIT = 1;  // wave groups splitting K inside the workgroup (MixedKsplitCfg)
    static_assert(STAGES >= 2 && STAGES <= 4, "two to four stages");
    static constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN;
    static constexpr int THREADS = WAVES_M * WAVES_N * kWave;
    static constexpr int MI = WM / Op::MB, NI = WN / Op::NB;
    static constexpr int STEPS = BK / Op::KB;
    using TileA = LdsTile<BM, BK / 2, LayA::pad, STAGES, LayA::unit, LayA::shift, LayA::mask>;  // 4-byte words
    using TileB = LdsTile<BK, BN / 2, LayB::pad, STAGES, LayB::unit, LayB::shift, LayB::mask>;
    // VEC 1: raw 4-byte copies of both operands (RawCopy16) realigned in
    // LDS, when the shape suits them and they fit beside the tiles; shifted
    // loads through registers otherwise (and for tiles that cannot move
    // inside C).
    // A's main copies in three stages (a tile's realignment reads the next
    // tile's), one A extra area (A's last whole K tile), B's main copies in
    // two stages and B's extra copies in three (issued a tile ahead of B's
    // main copies, since each fetches words of 64 different rows).
    using RawA = RawCopy16<BM, BK, THREADS>;
    using RawB = RawCopy16<BK, BN, THREADS>;
    static constexpr int RAW_A_OFF = 0, RAW_AX_OFF = 3 * RawA::MAIN, RAW_B_OFF = RAW_AX_OFF + RawA::EXTRA_WORDS,
                         RAW_BX_OFF = RAW_B_OFF + 2 * RawB::MAIN;
    static constexpr int RAW_WORDS = RAW_BX_OFF + 3 * RawB::EXTRA_WORDS;
    // (Eight-wave kernels only: the raw stages would cost the smaller
    // kernels their second workgroup per CU, measured slower.)
    static constexpr bool RAW = VEC == 1 && RawA::OK && RawB::OK && STAGES == 2 && THREADS >= 512 &&
                                TileA::bytes + TileB::bytes + RAW_WORDS * 4 <= 160 * 1024;
    static constexpr int LDS_BYTES = TileA::bytes + TileB::bytes + (RAW ? RAW_WORDS * 4 : 0);
    static_assert(BM % WM == 0 && BN % WN == 0 && WM % Op::MB == 0 && WN % Op::NB == 0, "wave tiling");
    static_assert(BK % Op::KB == 0, "whole MFMA steps per K tile");
    static_assert(LayA::pad == 0 && LayB::pad == 0, "direct copies need unpadded rows");
    static_assert(PIPELINE != kPipeAcrossTiles || STEPS % 2 == 0,
                  "across tiles, steps alternate between two fragment buffers");

    // Fragment addresses as per-lane bases plus compile-time offsets: A block
    // row i of step st at a_base(st) + i * MB rows, B block column n at
    // b_base(n) + (st * KB + 4 rr) rows for its two transposing reads rr.
    static constexpr bool based_addressing() {
        for (int w = 0; w < WAVES_M * WAVES_N; ++w)
            for (int l = 0; l < kWave; ++l) {
                const int g = l / Op::MB, r = l % Op::MB;
                const int wm0 = (w / WAVES_N) * WM, wn0 = (w % WAVES_N) * WN;
                const int tr_row = 8 * Op::kgroup(l) + (l % 16) / 4, tr_col = Op::col_base(l) + 4 * (l % 4);
                for (int st = 0; st < STEPS; ++st) {
                    const int col = st * (Op::KB / 2) + 4 * g;
                    for (int i = 0; i < MI; ++i)
                        if (TileA::offset(0, wm0 + i * Op::MB + r, col) !=
                            TileA::offset(0, wm0 + r, col) + i * Op::MB * TileA::row_stride)
                            return false;
                }
                for (int n = 0; n < NI; ++n) {
                    const int col = (wn0 + n * Op::NB + tr_col) / 2;
                    for (int st = 0; st < STEPS; ++st)
                        for (int rr = 0; rr < 2; ++rr)
                            if (TileB::offset(0, st * Op::KB + tr_row + 4 * rr, col) !=
                                TileB::offset(0, tr_row, col) + (st * Op::KB + 4 * rr) * TileB::row_stride)
                                return false;
                }
            }
        return true;
    }
    static_assert(based_addressing(), "layout does not admit base-plus-offset fragment addressing");
};

template <class Cfg>
__global__ __launch_bounds__(Cfg::THREADS, Cfg::MIN_WAVES) void gemm_mixed_kernel(
    int64_t M, int64_t N, int64_t K, const uint16_t* __restrict__ A, int64_t lda, const uint16_t* __restrict__ B,
    int64_t ldb, float* __restrict__ C, int64_t ldc, int64_t tiles_m, int64_t tiles_n) {
    using Op = typename Cfg::Op;
    using TileA = typename Cfg::TileA;
    using TileB = typename Cfg::TileB;
    using acc_t = typename Op::acc_t;
    constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK;
    constexpr int MI = Cfg::MI, NI = Cfg::NI, THREADS = Cfg::THREADS;

    __shared__ __attribute__((aligned(16))) uint32_t lds_a[TileA::total_elems];
    __shared__ __attribute__((aligned(16))) uint32_t lds_b[TileB::total_elems];
    __shared__ __attribute__((aligned(16))) uint32_t lds_raw[Cfg::RAW ? Cfg::RAW_WORDS : 4];
    poison_lds(lds_a, TileA::total_elems);
    poison_lds(lds_b, TileB::total_elems);
    if constexpr (Cfg::RAW) poison_lds(lds_raw, Cfg::RAW_WORDS);

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = tid / kWave;
    const int wm0 = (wave / Cfg::WAVES_N) * Cfg::WM;
    const int wn0 = (wave % Cfg::WAVES_N) * Cfg::WN;
    const int g = lane / Op::MB, r = lane % Op::MB;
    // transposing B reads: this lane's address within its 16-lane group
    const int tr_row = 8 * Op::kgroup(lane) + (lane % 16) / 4;
    const int tr_col = Op::col_base(lane) + 4 * (lane % 4);  // elements

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

    // Rows only 2-byte aligned (VEC 1): shifted 16-byte loads.
    std::conditional_t<Cfg::VEC == 1, TileLoaderShifted16<BM, BK, THREADS>,
                       TileLoader16<BM, BK, THREADS, Cfg::LOADER_VEC>> ldr_a;
    std::conditional_t<Cfg::VEC == 1, TileLoaderShifted16<BK, BN, THREADS>,
                       TileLoader16<BK, BN, THREADS, Cfg::LOADER_VEC>> ldr_b;
    const uint16_t* a_tile = A + m0 * lda;
    const uint16_t* b_tile = B + n0;
    const int64_t T = K > 0 ? (K + BK - 1) / BK : 0;

    auto load_tile = [&](int64_t t) {
        const int64_t k0 = t * BK;
        ldr_a.load(a_tile + k0, lda, M - m0, K - k0, tid);
        ldr_b.load(b_tile + k0 * ldb, ldb, K - k0, N - n0, tid);
    };
    auto store_tile = [&](int stage) {
        ldr_a.template store<TileA>(lds_a, stage, tid);
        ldr_b.template store<TileB>(lds_b, stage, tid);
    };
    typedef __attribute__((address_space(3))) uint32_t lds_word;
    typedef __attribute__((address_space(3))) shortx4 lds_short4;
    // Fragments of one MFMA step: A with 16-byte reads, B with two transposing
    // 8-byte reads per block column.
    int a_base[Cfg::STEPS], b_base[NI];
#pragma unroll
    for (int st = 0; st < Cfg::STEPS; ++st) a_base[st] = TileA::offset(0, wm0 + r, st * (Op::KB / 2) + 4 * g);
#pragma unroll
    for (int n = 0; n < NI; ++n) b_base[n] = TileB::offset(0, tr_row, (wn0 + n * Op::NB + tr_col) / 2);
    auto read_fragments = [&](int stage, int st, u32x4 (&af)[MI], u32x4 (&bf)[NI]) {
        const uint32_t* a = lds_a + stage * TileA::stage_elems + a_base[st];
#pragma unroll
        for (int i = 0; i < MI; ++i) af[i] = *reinterpret_cast<const u32x4*>(a + i * Op::MB * TileA::row_stride);
#pragma unroll
        for (int n = 0; n < NI; ++n) {
            shortx4 half[2];
#pragma unroll
            for (int rr = 0; rr < 2; ++rr) {
                const int word = stage * TileB::stage_elems + b_base[n] + (st * Op::KB + 4 * rr) * TileB::row_stride;
                half[rr] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)((lds_word*)lds_b + word));
            }
            const u32x2 lo = __builtin_bit_cast(u32x2, half[0]), hi = __builtin_bit_cast(u32x2, half[1]);
            bf[n] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        }
    };
    // Software-pipelined over the MFMA steps of a tile: the fragments of step
    // st+1 are read while the MFMAs of step st run, so the LDS latency is
    // hidden inside the wavefront instead of stalling the matrix pipe.  The
    // scheduling barriers keep the compiler from sinking the reads back next
    // to their MFMAs (which it does to save registers).
    // `early` runs before the MFMAs of step 0 and `mid` after those of the
    // first half of the steps: the kernels for 2-byte-aligned rows move the
    // next tile into LDS there, while the matrix pipe works through MFMAs
    // already issued.
    constexpr int MID_STEP = Cfg::STEPS / 2 - 1;
    auto multiply_with = [&](int stage, auto&& early, auto&& mid) {
        if constexpr (Cfg::PIPELINE != kPipeNone) {
            u32x4 af[2][MI], bf[2][NI];
            read_fragments(stage, 0, af[0], bf[0]);
            __builtin_amdgcn_sched_barrier(0);
            early();
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int st = 0; st < Cfg::STEPS; ++st) {
                if (st + 1 < Cfg::STEPS) read_fragments(stage, st + 1, af[(st + 1) & 1], bf[(st + 1) & 1]);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < MI; ++i)
#pragma unroll
                    for (int n = 0; n < NI; ++n) acc[i][n] = Op::mma(af[st & 1][i], bf[st & 1][n], acc[i][n]);
                __builtin_amdgcn_sched_barrier(0);
                if (st == MID_STEP) {
                    mid();
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        } else {
            early();
#pragma unroll
            for (int st = 0; st < Cfg::STEPS; ++st) {
                u32x4 af[MI], bf[NI];
                read_fragments(stage, st, af, bf);
#pragma unroll
                for (int i = 0; i < MI; ++i)
#pragma unroll
                    for (int n = 0; n < NI; ++n) acc[i][n] = Op::mma(af[i], bf[n], acc[i][n]);
                if (st == MID_STEP) mid();
            }
        }
    };
    auto multiply = [&](int stage) { multiply_with(stage, [] {}, [] {}); };

    // Tile t into `stage` through registers, with zero fill, for kernels
    // with 4-byte copies: 2 bytes per element (their rows need not be
    // 16-byte aligned), a few slots at a time, since a whole tile's
    // elements and addresses would not fit beside the accumulators.
    auto fill_in_chunks = [&](int64_t t, int stage) {
        const int64_t k0 = t * BK;
        TileLoader16<BM, BK, THREADS, 1>::template copy_in_chunks<TileA, 2>(a_tile + k0, lda, M - m0, K - k0, lds_a,
                                                                           stage, tid);
        TileLoader16<BK, BN, THREADS, 1>::template copy_in_chunks<TileB, 2>(b_tile + k0 * ldb, ldb, K - k0, N - n0,
                                                                           lds_b, stage, tid);
    };
    // Two stages through registers, each refill issued after the multiply
    // (workgroups whose tile cannot move back inside C, and unaligned
    // operands below).
    auto two_stage_registers = [&]() {
        if (T > 0) {
            if constexpr (Cfg::VEC == 2) {
                fill_in_chunks(0, 0);
            } else {
                load_tile(0);
                store_tile(0);
            }
        }
        __syncthreads();
        for (int64_t t = 0; t < T; ++t) {
            const int s = (int)(t & 1);
            multiply(s);
            if (t + 1 < T) {
                if constexpr (Cfg::VEC == 2) {
                    fill_in_chunks(t + 1, s ^ 1);
                } else {
                    load_tile(t + 1);
                    store_tile(s ^ 1);
                }
            }
            __syncthreads();
        }
    };

    if constexpr (Cfg::LOAD == kLoadDirect) {
        using DA = DirectCopy<TileA, THREADS, uint16_t, Cfg::VEC == 8 ? 16 : 4>;
        using DB = DirectCopy<TileB, THREADS, uint16_t, Cfg::VEC == 8 ? 16 : 4>;
        const bool interior = M - m0 >= BM && N - n0 >= BN && DA::fits(lda) && DB::fits(ldb);
        if (interior) {
            // S-stage pipeline of direct copies: during the multiply of tile t
            // the copies of tiles t+1 .. t+S-1 are in flight, tile t+S-1 going
            // into the stage tile t-1 used (every wave finished reading it
            // before the barrier that ended iteration t-1).  Before the barrier
            // that ends iteration t each wave waits until its copies of tile
            // t+1 have landed, i.e. until at most the copies of tiles
            // t+2 .. t+S-1 are outstanding.  A ragged last K tile (K % BK != 0)
            // needs zero fill: it is loaded through registers instead, which
            // makes that iteration wait for everything.
            constexpr int S = Cfg::STAGES;
            constexpr int COPIES = DA::PER_WAVE + DB::PER_WAVE;  // per wavefront and K tile
            const DA dma_a(lda, __builtin_amdgcn_readfirstlane(wave), lane);
            const DB dma_b(ldb, __builtin_amdgcn_readfirstlane(wave), lane);
            const int64_t TF = K / BK;  // K tiles wholly in range
            for (int p = 0; p < S - 1 && p < T; ++p) {
                if (p < TF) {
                    dma_a.issue(a_tile + p * BK, lds_a, p);
                    dma_b.issue(b_tile + p * BK * ldb, lds_b, p);
                } else {
                    if constexpr (Cfg::VEC == 2) {
                        fill_in_chunks(p, p);
                    } else {
                        load_tile(p);
                        store_tile(p);
                    }
                }
            }
            wait_vector_memory();
            __syncthreads();
            int s = 0;  // stage of tile t
            if constexpr (Cfg::PIPELINE == kPipeAcrossTiles) {
                // The last step of tile t multiplies after the barrier that
                // ends iteration t, from registers read before it, while the
                // fragments of step 0 of tile t+1 are read.  A ragged last
                // K tile goes through registers a few slots at a time, the
                // last step's fragments being live.
                u32x4 af[2][MI], bf[2][NI];
                auto mma_step = [&](const u32x4 (&a)[MI], const u32x4 (&b)[NI]) {
#pragma unroll
                    for (int i = 0; i < MI; ++i)
#pragma unroll
                        for (int n = 0; n < NI; ++n) acc[i][n] = Op::mma(a[i], b[n], acc[i][n]);
                };
                if (T > 0) read_fragments(0, 0, af[0], bf[0]);
                for (int64_t t = 0; t < T; ++t) {
                    const int ps = s == 0 ? S - 1 : s - 1;  // stage of tile t + S - 1
                    const int ns = s + 1 == S ? 0 : s + 1;  // stage of tile t + 1
                    const int64_t nt = t + S - 1;
                    const bool direct = nt < TF;
                    if (direct) {
                        dma_a.issue(a_tile + nt * BK, lds_a, ps);
                        dma_b.issue(b_tile + nt * BK * ldb, lds_b, ps);
                    }
#pragma unroll
                    for (int st = 0; st + 1 < Cfg::STEPS; ++st) {
                        read_fragments(s, st + 1, af[(st + 1) & 1], bf[(st + 1) & 1]);
                        mma_step(af[st & 1], bf[st & 1]);
                        alternate_mfma_and_lds_reads<MI * NI>();
                    }
                    if (nt < T && !direct) {
                        // ragged last K tile through registers, a few slots at a time
                        using LoaderA = TileLoader16<BM, BK, THREADS, Cfg::LOADER_VEC>;
                        using LoaderB = TileLoader16<BK, BN, THREADS, Cfg::LOADER_VEC>;
                        const int64_t k0 = nt * BK;
                        LoaderA::template copy_in_chunks<TileA, 2>(a_tile + k0, lda, M - m0, K - k0, lds_a, ps, tid);
                        LoaderB::template copy_in_chunks<TileB, 2>(b_tile + k0 * ldb, ldb, K - k0, N - n0, lds_b, ps, tid);
                    }
                    if (direct)
                        wait_vector_memory_at_most<(S - 2) * COPIES>();
                    else
                        wait_vector_memory();
                    __syncthreads();
                    // (read on the last tile too, from a stage whose values go
                    // unused, so that the reads share one block with the MFMAs
                    // and alternate with them)
                    read_fragments(ns, 0, af[0], bf[0]);
                    mma_step(af[1], bf[1]);
                    alternate_mfma_and_lds_reads<MI * NI>();
                    s = ns;
                }
            } else {
                for (int64_t t = 0; t < T; ++t) {
                    const int ps = s == 0 ? S - 1 : s - 1;  // stage of tile t + S - 1
                    const int64_t nt = t + S - 1;
                    const bool direct = nt < TF;
                    if (direct) {
                        dma_a.issue(a_tile + nt * BK, lds_a, ps);
                        dma_b.issue(b_tile + nt * BK * ldb, lds_b, ps);
                    }
                    multiply(s);
                    if (nt < T && !direct) {
                        if constexpr (Cfg::VEC == 2) {
                            fill_in_chunks(nt, ps);
                        } else {
                            load_tile(nt);
                            store_tile(ps);
                        }
                    }
                    if (direct)
                        wait_vector_memory_at_most<(S - 2) * COPIES>();
                    else
                        wait_vector_memory();
                    __syncthreads();
                    s = s + 1 == S ? 0 : s + 1;
                }
            }
        } else {
            two_stage_registers();
        }
    } else {
        // Rows only 2-byte aligned.
        bool raw_done = false;
        if constexpr (Cfg::RAW) {
            using RA = typename Cfg::RawA;
            using RB = typename Cfg::RawB;
            if (M - m0 >= BM && N - n0 >= BN && RA::fits(lda) && RB::fits(ldb)) {
                // Tile u (each K tile wholly in range) is realigned halfway
                // through the multiply of tile u-1, into the tile stage that
                // multiply does not read (every wave finished reading it
                // before the barrier that ended iteration u-2).  It reads A's
                // main copies of tiles u and u+1 (A's extra copies for the
                // last whole tile) and B's main and extra copies of tile u;
                // iteration t issues A's main and B's extra copies of tile
                // t+3 and B's main copies of tile t+2, so each has landed
                // (waited for before the barrier that ends iteration t) an
                // iteration or more before it is read, and goes into a stage
                // whose previous tile was realigned before that barrier; A's
                // extra copies (of the last whole tile) are issued first.  A
                // ragged last K tile goes through registers.
                const int wv = __builtin_amdgcn_readfirstlane(wave);
                const RA raw_a(lda, (uint32_t)(uintptr_t)a_tile & 2u, wv, lane, tid);
                const RB raw_b(ldb, (uint32_t)(uintptr_t)b_tile & 2u, wv, lane, tid);
                const int64_t TF = K / BK;  // K tiles wholly in range
                static_assert(RA::REALIGNERS == RB::REALIGNERS, "one set of realigning waves");
                const bool realigner = wv < RA::REALIGNERS / kWave;
                uint32_t* const a_main = lds_raw + Cfg::RAW_A_OFF;
                uint32_t* const a_extra = lds_raw + Cfg::RAW_AX_OFF;
                uint32_t* const b_main = lds_raw + Cfg::RAW_B_OFF;
                uint32_t* const b_extra = lds_raw + Cfg::RAW_BX_OFF;
                auto issue3 = [&](int64_t u, int r3) {  // A main, B extra of tile u into ring slot r3
                    raw_a.issue_main(a_tile + u * BK, a_main + r3 * RA::MAIN);
                    raw_b.issue_extra(b_tile + u * BK * ldb, b_extra + r3 * RB::EXTRA_WORDS);
                };
                auto issue2 = [&](int64_t u, int r2) { raw_b.issue_main(b_tile + u * BK * ldb, b_main + r2 * RB::MAIN); };
                auto fill_tile = [&](int64_t u, int stage, int r3, int r2) {
                    if (u < TF) {
                        if (!realigner) return;
                        const bool last = u + 1 == TF;
                        const uint32_t* a_after = last ? a_extra : a_main + (r3 == 2 ? 0 : r3 + 1) * RA::MAIN;
                        raw_a.template realign<TileA>(a_main + r3 * RA::MAIN, a_after, last ? 1 : RA::RW, lds_a,
                                                      stage, tid);
                        raw_b.template realign<TileB>(b_main + r2 * RB::MAIN, b_extra + r3 * RB::EXTRA_WORDS, 1,
                                                      lds_b, stage, tid);
                    } else {
                        fill_in_chunks(u, stage);
                    }
                };
                if (TF > 0) raw_a.issue_extra(a_tile + (TF - 1) * BK, a_extra);  // for the last whole tile
                for (int p = 0; p < 3 && p < TF; ++p) issue3(p, p);
                for (int p = 0; p < 2 && p < TF; ++p) issue2(p, p);
                wait_vector_memory();
                __syncthreads();
                if (T > 0) fill_tile(0, 0, 0, 0);
                __syncthreads();
                int r3 = 0, r2 = 0;  // ring slots of tile t
                for (int64_t t = 0; t < T; ++t) {
                    const int s = (int)(t & 1);
                    const int n3 = r3 == 2 ? 0 : r3 + 1, n2 = r2 ^ 1;  // slots of tile t+1
                    if (t + 3 < TF) issue3(t + 3, r3);
                    if (t + 2 < TF) issue2(t + 2, r2);
                    multiply_with(s, [] {}, [&] {
                        if (t + 1 < T) fill_tile(t + 1, s ^ 1, n3, n2);
                    });
                    wait_vector_memory();
                    __syncthreads();
                    r3 = n3;
                    r2 = n2;
                }
                raw_done = true;
            }
        }
        if (!raw_done) {
            // Two LDS stages filled through registers.  Halfway through the
            // multiply of tile t (stage s) each thread stores tile t+1,
            // loaded during the iteration before, to the other stage (every
            // wave finished reading it before the barrier that ended
            // iteration t-1), then issues the loads of tile t+2 into the
            // registers just freed: a load has a whole iteration to land,
            // and the stores run beside MFMAs already issued.
            if (T > 0) {
                load_tile(0);
                store_tile(0);
            }
            if (T > 1) load_tile(1);
            __syncthreads();
            for (int64_t t = 0; t < T; ++t) {
                const int s = (int)(t & 1);
                multiply_with(s, [] {}, [&] {
                    if (t + 1 < T) store_tile(s ^ 1);
                    if (t + 2 < T) load_tile(t + 2);
                });
                __syncthreads();
            }
        }
    }

    store_accumulators<Op, BM, BN, MI, NI>(C, ldc, M, N, m0, n0, own.m0, own.n0, wm0, wn0, lane, acc);
}

// --------------------------------------------------------------------------
// K split inside the workgroup for 16-bit inputs (the fp32 KsplitCfg's
// scheme): KSPLIT groups of waves share one output tile, group q taking K
// tiles q, q + KSPLIT, ... through its own pair of LDS stages with Base's
// wave tiling, direct copies and step-pipelined multiply; group p then adds
// the others' partial sums of its slice of the outputs in LDS, in group
// order, and stores that slice.  Copies of 16 bytes (VEC 8) or 4 bytes
// (VEC 2), as the base's.
template <class Base, int KSPLIT_>
struct MixedKsplitCfg {
    static_assert(Base::LOAD == kLoadDirect && Base::STAGES == 2, "groups run Base's two-stage direct-copy loop");
    static_assert(KSPLIT_ >= 2, "at least two groups");
    using Op = typename Base::Op;
    static constexpr int TYPE = Base::TYPE, KSPLIT = KSPLIT_;
    static constexpr int BM = Base::BM, BN = Base::BN, BK = Base::BK, WM = Base::WM, WN = Base::WN;
    static constexpr int VEC = Base::VEC, ORDER = Base::ORDER, LOAD = kLoadDirect, PIPELINE = kPipeSteps;
    static constexpr int LOADER_VEC = Base::LOADER_VEC;
    static constexpr int WAVES_N = Base::WAVES_N, MI = Base::MI, NI = Base::NI, STEPS = Base::STEPS;
    static constexpr int GROUP_THREADS = Base::THREADS, GROUP_WAVES = GROUP_THREADS / kWave;
    static constexpr int THREADS = GROUP_THREADS * KSPLIT;
    static constexpr int STAGES = 2 * KSPLIT;  // stages 2q, 2q+1 belong to group q
    static constexpr int MIN_WAVES = Base::MIN_WAVES > THREADS / 256 ? Base::MIN_WAVES : THREADS / 256;
    using TileA = LdsTile<BM, BK / 2, 0, STAGES, Base::TileA::swizzle.unit, Base::TileA::swizzle.shift,
                          Base::TileA::swizzle.mask>;
    using TileB = LdsTile<BK, BN / 2, 0, STAGES, Base::TileB::swizzle.unit, Base::TileB::swizzle.shift,
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
__global__ __launch_bounds__(Cfg::THREADS, Cfg::MIN_WAVES) void gemm_mixed_ksplit_kernel(
    int64_t M, int64_t N, int64_t K, const uint16_t* __restrict__ A, int64_t lda, const uint16_t* __restrict__ B,
    int64_t ldb, float* __restrict__ C, int64_t ldc, int64_t tiles_m, int64_t tiles_n) {
    using Op = typename Cfg::Op;
    using TileA = typename Cfg::TileA;
    using TileB = typename Cfg::TileB;
    using acc_t = typename Op::acc_t;
    constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, KS = Cfg::KSPLIT;
    constexpr int MI = Cfg::MI, NI = Cfg::NI, GT = Cfg::GROUP_THREADS;

    // One array: A's stages, then B's; the partial sums reuse all of it.
    __shared__ __attribute__((aligned(16))) uint32_t lds[TileA::total_elems + TileB::total_elems];
    poison_lds(lds, TileA::total_elems + TileB::total_elems);
    uint32_t* const lds_a = lds;
    uint32_t* const lds_b = lds + TileA::total_elems;

    const int tid = threadIdx.x;
    const int group = __builtin_amdgcn_readfirstlane(tid / GT);
    const int gtid = tid % GT;
    const int lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(gtid / kWave);
    const int wm0 = (wave / Cfg::WAVES_N) * Cfg::WM;
    const int wn0 = (wave % Cfg::WAVES_N) * Cfg::WN;
    const int g = lane / Op::MB, r = lane % Op::MB;
    const int tr_row = 8 * Op::kgroup(lane) + (lane % 16) / 4;
    const int tr_col = Op::col_base(lane) + 4 * (lane % 4);

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

    TileLoader16<BM, BK, GT, Cfg::LOADER_VEC> ldr_a;
    TileLoader16<BK, BN, GT, Cfg::LOADER_VEC> ldr_b;
    const uint16_t* a_tile = A + m0 * lda;
    const uint16_t* b_tile = B + n0;
    const int64_t T = K > 0 ? (K + BK - 1) / BK : 0;
    const int64_t TF = K / BK;
    const int64_t ITERS = (T + KS - 1) / KS;

    using DA = DirectCopy<TileA, GT, uint16_t, Cfg::VEC == 8 ? 16 : 4>;
    using DB = DirectCopy<TileB, GT, uint16_t, Cfg::VEC == 8 ? 16 : 4>;
    const DA dma_a(lda, wave, lane);
    const DB dma_b(ldb, wave, lane);
    const bool interior = M - m0 >= BM && N - n0 >= BN && DA::fits(lda) && DB::fits(ldb);

    auto copy_direct = [&](int64_t t, int stage) {
        dma_a.issue(a_tile + t * BK, lds_a, stage);
        dma_b.issue(b_tile + t * BK * ldb, lds_b, stage);
    };
    auto copy_registers = [&](int64_t t, int stage) {
        const int64_t k0 = t * BK;
        if constexpr (Cfg::VEC == 2) {  // 2-byte loads, a few slots at a time
            TileLoader16<BM, BK, GT, 1>::template copy_in_chunks<TileA, 2>(a_tile + k0, lda, M - m0, K - k0, lds_a,
                                                                          stage, gtid);
            TileLoader16<BK, BN, GT, 1>::template copy_in_chunks<TileB, 2>(b_tile + k0 * ldb, ldb, K - k0, N - n0,
                                                                          lds_b, stage, gtid);
        } else {
            ldr_a.load(a_tile + k0, lda, M - m0, K - k0, gtid);
            ldr_b.load(b_tile + k0 * ldb, ldb, K - k0, N - n0, gtid);
            ldr_a.template store<TileA>(lds_a, stage, gtid);
            ldr_b.template store<TileB>(lds_b, stage, gtid);
        }
    };
    typedef __attribute__((address_space(3))) uint32_t lds_word;
    typedef __attribute__((address_space(3))) shortx4 lds_short4;
    int a_base[Cfg::STEPS], b_base[NI];
#pragma unroll
    for (int st = 0; st < Cfg::STEPS; ++st) a_base[st] = TileA::offset(0, wm0 + r, st * (Op::KB / 2) + 4 * g);
#pragma unroll
    for (int n = 0; n < NI; ++n) b_base[n] = TileB::offset(0, tr_row, (wn0 + n * Op::NB + tr_col) / 2);
    auto read_fragments = [&](int stage, int st, u32x4 (&af)[MI], u32x4 (&bf)[NI]) {
        const uint32_t* a = lds_a + stage * TileA::stage_elems + a_base[st];
#pragma unroll
        for (int i = 0; i < MI; ++i) af[i] = *reinterpret_cast<const u32x4*>(a + i * Op::MB * TileA::row_stride);
#pragma unroll
        for (int n = 0; n < NI; ++n) {
            shortx4 half[2];
#pragma unroll
            for (int rr = 0; rr < 2; ++rr) {
                const int word = stage * TileB::stage_elems + b_base[n] + (st * Op::KB + 4 * rr) * TileB::row_stride;
                half[rr] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)((lds_word*)lds_b + word));
            }
            const u32x2 lo = __builtin_bit_cast(u32x2, half[0]), hi = __builtin_bit_cast(u32x2, half[1]);
            bf[n] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        }
    };
    auto multiply = [&](int stage) {
        u32x4 af[2][MI], bf[2][NI];
        read_fragments(stage, 0, af[0], bf[0]);
#pragma unroll
        for (int st = 0; st < Cfg::STEPS; ++st) {
            if (st + 1 < Cfg::STEPS) read_fragments(stage, st + 1, af[(st + 1) & 1], bf[(st + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int n = 0; n < NI; ++n) acc[i][n] = Op::mma(af[st & 1][i], bf[st & 1][n], acc[i][n]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    const int stage0 = 2 * group;
    if (group < T) {
        if (interior && group < TF)
            copy_direct(group, stage0);
        else
            copy_registers(group, stage0);
    }
    wait_vector_memory();
    __syncthreads();
    for (int64_t it = 0; it < ITERS; ++it) {
        const int s = stage0 + (int)(it & 1), ns = stage0 + (int)((it & 1) ^ 1);
        const int64_t t = it * KS + group, tn = t + KS;
        const bool direct = interior && tn < TF;
        if (direct) copy_direct(tn, ns);
        if (t < T) multiply(s);
        if (tn < T && !direct) copy_registers(tn, ns);
        wait_vector_memory();
        __syncthreads();
    }

    // Every LDS read of the loop completed before its last barrier.  Region
    // (p, q): group q's partial sums of group p's slice, one float per lane
    // per value.  Each group runs its own copy of the exchange (P = its
    // index), so every register and LDS offset in it is a constant.
    constexpr int SV = Cfg::SLICE_VALUES, GW = Cfg::GROUP_WAVES;
    float* const exch = reinterpret_cast<float*>(lds) + wave * SV * kWave + lane;
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

}  // namespace dft
