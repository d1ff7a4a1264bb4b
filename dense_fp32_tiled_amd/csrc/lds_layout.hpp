// lds_layout.hpp -- LDS tile layout and bank model (host and device, constexpr).
//
// A tile staged in LDS has a logical shape (rows x cols), a physical row
// stride (cols + pad) and a number of stages.  Producers (the cooperative
// global->LDS copy) and consumers (the inner product) both address it through
// LdsTile::offset, so a change of padding or staging cannot desynchronise them
// ("My Triton From Scratch, Part 18: Shared Memory Optimization", sections "A
// shared buffer needs a physical row stride" and "Every producer and consumer
// must use the new stride").
//
// The bank model generalises the pages' one-warp rule (32 banks,
// bank = word % 32, section "Why shared-memory banks matter"): the bank count
// and the number of lanes the LDS services together per access width are
// parameters, and the conflict degree of an instruction is computed from the
// actual lane -> address pattern, for reads and writes alike.
#pragma once

#include <stdint.h>

namespace dft {

constexpr int kWaveLanes = 64;  // lanes per wavefront on gfx950

// --------------------------------------------------------------------------
// Physical layout of one staged tile.
struct LdsLayout {
    int rows, cols, pad, stages;

    constexpr bool valid() const { return rows > 0 && cols > 0 && pad >= 0 && stages > 0; }
    constexpr int row_stride() const { return cols + pad; }
    constexpr int stage_elems() const { return rows * row_stride(); }
    constexpr int total_elems() const { return stages * stage_elems(); }
    constexpr int bytes() const { return total_elems() * 4; }
    constexpr int offset(int stage, int row, int col) const {
        return stage * stage_elems() + row * row_stride() + col;
    }
};

// Optional XOR swizzle of columns by row: physical column =
// col ^ (unit * ((row >> shift) & mask)).  unit is a multiple of 4 words, so
// 16-byte groups of four columns stay contiguous and aligned; the XOR only
// permutes columns within aligned blocks of unit * (mask + 1) words.
struct Swizzle {
    int unit, shift, mask;  // unit == 0: no swizzle
    constexpr int apply(int row, int col) const { return unit ? (col ^ (unit * ((row >> shift) & mask))) : col; }
};
constexpr Swizzle kNoSwizzle{0, 0, 0};

template <int Rows, int Cols, int Pad, int Stages, int SwzUnit = 0, int SwzShift = 0, int SwzMask = 0>
struct LdsTile {
    static_assert(Rows > 0 && Cols > 0 && Pad >= 0 && Stages > 0, "invalid LDS tile");
    static_assert(SwzUnit == 0 || (SwzUnit % 4 == 0 && (SwzMask & (SwzMask + 1)) == 0 &&
                                   Cols % (SwzUnit * (SwzMask + 1)) == 0),
                  "swizzle must permute 16-byte groups within aligned blocks of the row");
    static constexpr int rows = Rows, cols = Cols, pad = Pad, stages = Stages;
    static constexpr int row_stride = Cols + Pad;
    static constexpr int stage_elems = Rows * row_stride;
    static constexpr int total_elems = Stages * stage_elems;
    static constexpr int bytes = total_elems * 4;
    static constexpr Swizzle swizzle{SwzUnit, SwzShift, SwzMask};
    static constexpr LdsLayout layout() { return LdsLayout{Rows, Cols, Pad, Stages}; }

    // constexpr functions are callable from both host and device code in HIP
    static constexpr int offset(int stage, int row, int col) {
        return stage * stage_elems + row * row_stride + Swizzle{SwzUnit, SwzShift, SwzMask}.apply(row, col);
    }
};

// --------------------------------------------------------------------------
// Bank model.  For each access width the LDS services a group of lanes per
// pass over a number of 4-byte banks (reads and stores differ); a pass costs
// its conflict degree (the worst number of distinct dwords one bank must
// deliver in it) in cycles, and an instruction the sum over its passes.
struct LdsGeometry {
    int banks_b32, lanes_b32;    // 4-byte reads
    int banks_b64, lanes_b64;    // 8-byte reads
    int banks_b128, lanes_b128;  // 16-byte reads
    int st_banks_b32, st_lanes_b32;    // 4-byte stores
    int st_banks_b64, st_lanes_b64;    // 8-byte stores
    int st_banks_b128, st_lanes_b128;  // 16-byte stores
    bool b128_parity_passes;  // 16-byte reads: the lanes of a pass as in access_cycles

    constexpr int banks_for_width(int width_words, bool store = false) const {
        if (store) return width_words == 1 ? st_banks_b32 : width_words == 2 ? st_banks_b64 : st_banks_b128;
        return width_words == 1 ? banks_b32 : width_words == 2 ? banks_b64 : banks_b128;
    }
    constexpr int group_for_width(int width_words, bool store = false) const {
        if (store) return width_words == 1 ? st_lanes_b32 : width_words == 2 ? st_lanes_b64 : st_lanes_b128;
        return width_words == 1 ? lanes_b32 : width_words == 2 ? lanes_b64 : lanes_b128;
    }
};

// gfx950 (MI355X), measured with the LDS probe (timed single-instruction
// patterns, 4 wavefronts): 4-byte reads behave as 32 banks serviced 32 lanes
// per pass (a stride of 64 dwords costs no more than a stride of 32); 8-byte
// reads as 64 banks, 32 lanes per pass; 16-byte reads as 64 banks, 16 lanes
// per pass (256 bytes per pass; a stride of 64 dwords is 16-way, 32 is
// 8-way), the 16 lanes of a pass chosen as access_cycles states.  4-byte
// stores behave as 32 banks x 32 lanes, 8-byte stores as 32 banks x 16
// lanes, 16-byte stores as 32 banks x 8 lanes (a stride of 8 dwords is
// 2-way, 32 is 8-way).  The pages' figure (32 banks per 32-lane warp) is
// NVIDIA's and matches only the 4-byte case.
constexpr LdsGeometry kGfx950Lds{32, 32, 64, 32, 64, 16, 32, 32, 32, 16, 32, 8, true};

constexpr int bank_of(int64_t word, int banks) { return (int)(((word % banks) + banks) % banks); }

constexpr int gcd_int(int a, int b) { return b == 0 ? a : gcd_int(b, a % b); }

// The pages' rule: a stride of `columns` words reaches banks/gcd(columns,banks)
// distinct banks before repeating; pad one word when more rows are read at once.
constexpr int page_pad(int columns, int simultaneous_rows, int banks) {
    return simultaneous_rows > banks / gcd_int(columns, banks) ? 1 : 0;
}

// Conflict degree of one access pattern (see gemm_lds_conflict_degree in the
// public header for the definition).  `addr(l, e)` gives the dword that lane
// l touches as its element e (e < width); for a plain access these are
// consecutive, for a two-address access (ds_read2) they are not.
// Limits: group * width <= 256 dwords, banks <= 128; returns -1 beyond them.
template <class Addr>
constexpr int conflict_degree2(Addr addr, int lanes, int width, int banks, int group) {
    if (lanes < 1 || width < 1 || banks < 1 || banks > 128 || group < 1 || group * width > 256) return -1;
    int worst = 1;
    for (int g0 = 0; g0 < lanes; g0 += group) {
        const int g1 = g0 + group < lanes ? g0 + group : lanes;
        // distinct dwords per bank, as per-bank linked lists
        int head[128] = {};
        int count[128] = {};
        int64_t word_of[257] = {};
        int next_of[257] = {};
        int n = 1;  // entry 0 is the list terminator
        for (int l = g0; l < g1; ++l) {
            for (int e = 0; e < width; ++e) {
                const int64_t word = addr(l, e);
                const int b = bank_of(word, banks);
                bool seen = false;
                for (int i = head[b]; i != 0; i = next_of[i])
                    if (word_of[i] == word) { seen = true; break; }
                if (seen) continue;
                word_of[n] = word;
                next_of[n] = head[b];
                head[b] = n++;
                if (++count[b] > worst) worst = count[b];
            }
        }
    }
    return worst;
}

template <class Addr>
constexpr int conflict_degree(Addr addr, int lanes, int width, int banks, int group) {
    return conflict_degree2([=](int l, int e) { return addr(l) + e; }, lanes, width, banks, group);
}

// Pass of lane l of a 16-byte read: its half-wave (l / 32) and the bit
// parity of its 4-lane group's index within the half ((l / 4) % 8), so that
// each pass takes two 4-lane groups of each parity class from one half.
// Of the lane partitions into four passes of 16 given by two bit-parity
// functions of l, only this one and three that also fold in bits 0 and 1
// reproduce every 16-byte read the probe timed (the 16x16x4 MFMA's
// A-fragment read conflict-free among them); 16 consecutive lanes per pass
// does not.
constexpr int b128_pass_of(int l) {
    const int q = (l >> 2) & 7;
    return ((l >> 5) << 1) | ((q ^ (q >> 1) ^ (q >> 2)) & 1);
}

// Cycles one wavefront-wide access of `width` consecutive dwords per lane
// (lane l from dword addr(l)) costs under geometry g: the sum over its
// passes of each pass's conflict degree.  A pass is `group` consecutive
// lanes, except for 16-byte reads under g.b128_parity_passes
// (b128_pass_of).
template <class Addr>
constexpr int access_cycles(Addr addr, int width, bool store, LdsGeometry g) {
    const int banks = g.banks_for_width(width, store), group = g.group_for_width(width, store);
    if (width < 1 || banks < 1 || banks > 128 || group < 1 || group * width > 256 || kWaveLanes % group) return -1;
    int total = 0;
    if (!store && width == 4 && g.b128_parity_passes && group == 16) {
        for (int pass = 0; pass < kWaveLanes / 16; ++pass) {
            int lanes[16] = {};
            int n = 0;
            for (int l = 0; l < kWaveLanes; ++l)
                if (b128_pass_of(l) == pass) lanes[n++] = l;
            total += conflict_degree2([=](int i, int e) { return addr(lanes[i]) + e; }, n, width, banks, n);
        }
        return total;
    }
    for (int g0 = 0; g0 < kWaveLanes; g0 += group)
        total += conflict_degree2([=](int l, int e) { return addr(g0 + l) + e; }, group, width, banks, group);
    return total;
}

}  // namespace dft
