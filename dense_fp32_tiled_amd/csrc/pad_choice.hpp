// pad_choice.hpp -- LDS layout (row padding or XOR swizzle) for each kernel,
// derived at compile time from the bank model and the kernel's own lane ->
// address patterns.
//
// For every LDS access a kernel issues on a tile (fragment reads by every
// wavefront, cooperative stores by every thread) the conflict degree is
// computed from the exact addresses the lanes touch; a layout's cost is the
// sum over those accesses of their LDS cycles (access_cycles: per pass, its
// conflict degree), per K tile.  Candidates are row
// pads that keep 16-byte alignment and XOR swizzles of 16-byte column groups
// (no pad); the cheapest wins, ties going to no change, then to a pad, then to
// a swizzle.  This replaces the pages' one-pattern rule ("My Triton From
// Scratch, Part 18: Shared Memory Optimization", section "Choosing padding
// instead of hard-coding it"), which models a single one-warp read of A.
#pragma once

#include "lds_layout.hpp"

namespace dft {

constexpr int kMaxPad = 32;

struct LayoutChoice {
    int pad;
    Swizzle swz;
};

constexpr int64_t layout_word(LayoutChoice c, int cols, int row, int col) {
    return (int64_t)row * (cols + c.pad) + c.swz.apply(row, col);
}

// Cost (LDS cycles, access_cycles) of one wavefront-wide access: lane l
// touches (row(l), col(l)) .. +width; `store` selects the store geometry.
template <class RowCol>
constexpr int pattern_cost(LayoutChoice c, int cols, int width, LdsGeometry g, RowCol rc, bool store = false) {
    return access_cycles(
        [=](int l) {
            int row = 0, col = 0;
            rc(l, row, col);
            return layout_word(c, cols, row, col);
        },
        width, store, g);
}

// Cost of a two-address access (ds_read2_b32): lane l touches (row(l, e),
// col(l, e)) for e = 0, 1.  Measured on gfx950 (LDS probe), the LDS serves it
// as two 4-byte accesses, one per address, each with the 4-byte geometry.
template <class RowCol2>
constexpr int pattern_cost_pair(LayoutChoice c, int cols, LdsGeometry g, RowCol2 rc) {
    int total = 0;
    for (int e = 0; e < 2; ++e)
        total += pattern_cost(c, cols, 1, g, [=](int l, int& row, int& col) { rc(l, e, row, col); });
    return total;
}

struct AcceptAll {
    constexpr bool operator()(LayoutChoice) const { return true; }
};

// Search pads 0, 4, ..., kMaxPad (only 0 unless allow_pad), then swizzles;
// `cost(choice)` sums a tile's access costs; only layouts `accept` admits
// are candidates (the plain layout always is).
template <class Cost, class Accept = AcceptAll>
constexpr LayoutChoice choose_layout(Cost cost, int cols, bool allow_pad = true, Accept accept = {}) {
    LayoutChoice best{0, kNoSwizzle};
    int best_cost = cost(best);
    for (int pad = 4; allow_pad && pad <= kMaxPad; pad += 4) {
        const LayoutChoice c{pad, kNoSwizzle};
        if (!accept(c)) continue;
        const int v = cost(c);
        if (v < best_cost) { best = c; best_cost = v; }
    }
    for (int unit = 4; unit <= 32; unit *= 2)
        for (int mask = 1; mask <= 7; mask = 2 * mask + 1)
            for (int shift = 0; shift <= 4; ++shift) {
                if (cols % (unit * (mask + 1)) != 0) continue;
                const LayoutChoice c{0, Swizzle{unit, shift, mask}};
                if (!accept(c)) continue;
                const int v = cost(c);
                if (v < best_cost) { best = c; best_cost = v; }
            }
    return best;
}

// ---- matrix-core kernel ---------------------------------------------------------
// A row-major [BM][BK], B row-major [BK][BN]; MFMA block MB x NB x KB; lane l
// belongs to k-group l / MB and reduces k in [group * KG, (group + 1) * KG),
// KG = BK / KB, one k per MFMA step.  `direct`: tiles reach LDS by direct
// global->LDS copies, whose writes fill 1 KiB of consecutive words per
// wavefront instruction (no bank conflicts whatever the layout, and no room
// for row padding), so only the fragment reads are costed and only unpadded
// layouts are candidates.
//
// `pipelined` (direct copies only): the kernel addresses its fragments as a
// per-lane base plus compile-time offsets, so that the addresses of a whole
// K tile cost a few registers: A block row i of chunk q at
// base_a(q) + i * MB rows, B step kk of block column n at
// base_b(n % PB) + kk rows + (n / PB) * PB * NB words, PB = min(2, WN / NB).
// Only layouts whose swizzle keeps that form are candidates
// (pipelined_a_ok, pipelined_b_ok).
struct MfmaShape {
    int bm, bn, bk, wm, wn, threads, vec, mb, nb, kb;
    bool direct = false;
    bool pipelined = false;
    constexpr int kg() const { return bk / kb; }
    constexpr int waves() const { return threads / kWaveLanes; }
    constexpr int waves_n() const { return bn / wn; }
    constexpr int pb() const { return wn / nb < 2 ? wn / nb : 2; }
};

constexpr bool pipelined_a_ok(MfmaShape s, LayoutChoice c) {
    const int stride = s.bk + c.pad;
    for (int w = 0; w < s.waves(); ++w)
        for (int l = 0; l < kWaveLanes; ++l) {
            const int row0 = (w / s.waves_n()) * s.wm + l % s.mb;
            for (int q = 0; q < s.kg() / 4; ++q) {
                const int col = (l / s.mb) * s.kg() + 4 * q;
                const int64_t base = layout_word(c, s.bk, row0, col);
                for (int i = 1; i < s.wm / s.mb; ++i)
                    if (layout_word(c, s.bk, row0 + i * s.mb, col) != base + (int64_t)i * s.mb * stride) return false;
            }
        }
    return true;
}

constexpr bool pipelined_b_ok(MfmaShape s, LayoutChoice c) {
    const int stride = s.bn + c.pad, pb = s.pb();
    for (int w = 0; w < s.waves(); ++w)
        for (int l = 0; l < kWaveLanes; ++l) {
            const int row0 = (l / s.nb) * s.kg(), col0 = (w % s.waves_n()) * s.wn + l % s.nb;
            for (int n = 0; n < s.wn / s.nb; ++n) {
                const int64_t base = layout_word(c, s.bn, row0, col0 + (n % pb) * s.nb);
                for (int kk = 0; kk < s.kg(); ++kk)
                    if (layout_word(c, s.bn, row0 + kk, col0 + n * s.nb) !=
                        base + (int64_t)kk * stride + (int64_t)(n / pb) * pb * s.nb)
                        return false;
            }
        }
    return true;
}

// Every A access of one K tile: fragment reads (16-byte, KG/4 per block row
// of every wavefront) and the cooperative stores (vec-wide).
constexpr int mfma_a_cost(MfmaShape s, LayoutChoice c, LdsGeometry g) {
    int total = 0;
    for (int w = 0; w < s.waves(); ++w) {
        const int wm0 = (w / s.waves_n()) * s.wm;
        for (int mi = 0; mi < s.wm / s.mb; ++mi)
            for (int q = 0; q < s.kg() / 4; ++q)
                total += pattern_cost(c, s.bk, 4, g, [=](int l, int& row, int& col) {
                    row = wm0 + mi * s.mb + l % s.mb;
                    col = (l / s.mb) * s.kg() + 4 * q;
                });
        const int vcols = s.bk / s.vec;
        for (int i = 0; !s.direct && i < (s.bm * vcols) / s.threads; ++i)
            total += pattern_cost(
                c, s.bk, s.vec, g,
                [=](int l, int& row, int& col) {
                    const int idx = w * kWaveLanes + l + i * s.threads;
                    row = idx / vcols;
                    col = (idx % vcols) * s.vec;
                },
                true);
    }
    return total;
}

// Every B access of one K tile: the 4-byte fragment reads (KG per block
// column of every wavefront) and the cooperative stores.  The compiler merges
// the reads of block columns 2p and 2p+1 (same row, NB words apart) into one
// two-address ds_read2_b32, costed as such a pair.
constexpr int mfma_b_cost(MfmaShape s, LayoutChoice c, LdsGeometry g) {
    int total = 0;
    const int ni_count = s.wn / s.nb;
    for (int w = 0; w < s.waves(); ++w) {
        const int wn0 = (w % s.waves_n()) * s.wn;
        for (int j = 0; j < s.kg(); ++j) {
            for (int ni = 0; ni + 1 < ni_count; ni += 2)
                total += pattern_cost_pair(c, s.bn, g, [=](int l, int e, int& row, int& col) {
                    row = (l / s.nb) * s.kg() + j;
                    col = wn0 + (ni + e) * s.nb + l % s.nb;
                });
            if (ni_count % 2)
                total += pattern_cost(c, s.bn, 1, g, [=](int l, int& row, int& col) {
                    row = (l / s.nb) * s.kg() + j;
                    col = wn0 + (ni_count - 1) * s.nb + l % s.nb;
                });
        }
        const int vcols = s.bn / s.vec;
        for (int i = 0; !s.direct && i < (s.bk * vcols) / s.threads; ++i)
            total += pattern_cost(
                c, s.bn, s.vec, g,
                [=](int l, int& row, int& col) {
                    const int idx = w * kWaveLanes + l + i * s.threads;
                    row = idx / vcols;
                    col = (idx % vcols) * s.vec;
                },
                true);
    }
    return total;
}

constexpr LayoutChoice mfma_layout_a(MfmaShape s, LdsGeometry g) {
    return choose_layout([=](LayoutChoice c) { return mfma_a_cost(s, c, g); }, s.bk, !s.direct,
                         [=](LayoutChoice c) { return !s.pipelined || pipelined_a_ok(s, c); });
}
constexpr LayoutChoice mfma_layout_b(MfmaShape s, LdsGeometry g) {
    return choose_layout([=](LayoutChoice c) { return mfma_b_cost(s, c, g); }, s.bn, !s.direct,
                         [=](LayoutChoice c) { return !s.pipelined || pipelined_b_ok(s, c); });
}

// ---- matrix-core kernel with 16-bit inputs (bf16 / fp16) ------------------------
// Tiles hold two elements per 4-byte word: A [BM][BK/2 words], B [BK][BN/2
// words], both filled by direct copies (no LDS store instructions, no pad).
// One MFMA step consumes KB elements of k: lane l of k-group g = l / MB reads
// 8 consecutive k of A row l % MB (one 16-byte read at word column
// step * KB/2 + 4g) and receives 8 consecutive k of B column l % MB through
// two transposing 8-byte reads (ds_read_b64_tr_b16).  Measured lane mapping
// of that read: in each group of 16 lanes, lane j supplies the address of
// row (j / 4), columns 4 (j % 4) .. 4 (j % 4) + 3 of a 4 x 16 block, and lane
// i receives column i of the block's four rows.  So for B, lane j of group
// G = l / 16 addresses row step*KB + 8 kg + 4 rr + j / 4 (read rr = 0, 1) and
// element column n_base(G) + 4 (j % 4), with kg = l / 32, n_base = 16 (G % 2)
// for 32 x 32 blocks, and kg = G, n_base = 0 for 16 x 16 blocks.
struct Mixed16Shape {
    int bm, bn, bk, wm, wn, threads, mb;
    constexpr int kb() const { return mb == 32 ? 16 : 32; }
    constexpr int steps() const { return bk / kb(); }
    constexpr int waves() const { return threads / kWaveLanes; }
    constexpr int waves_n() const { return bn / wn; }
};

constexpr int mixed_a_cost(Mixed16Shape s, LayoutChoice c, LdsGeometry g) {
    int total = 0;
    const int cols = s.bk / 2;
    for (int w = 0; w < s.waves(); ++w) {
        const int wm0 = (w / s.waves_n()) * s.wm;
        for (int st = 0; st < s.steps(); ++st)
            for (int mi = 0; mi < s.wm / s.mb; ++mi)
                total += pattern_cost(c, cols, 4, g, [=](int l, int& row, int& col) {
                    row = wm0 + mi * s.mb + l % s.mb;
                    col = st * (s.kb() / 2) + 4 * (l / s.mb);
                });
    }
    return total;
}

constexpr int mixed_b_cost(Mixed16Shape s, LayoutChoice c, LdsGeometry g) {
    int total = 0;
    const int cols = s.bn / 2;
    for (int w = 0; w < s.waves(); ++w) {
        const int wn0 = (w % s.waves_n()) * s.wn;
        for (int st = 0; st < s.steps(); ++st)
            for (int ni = 0; ni < s.wn / s.mb; ++ni)
                for (int rr = 0; rr < 2; ++rr)
                    total += pattern_cost(c, cols, 2, g, [=](int l, int& row, int& col) {
                        const int grp = l / 16, j = l % 16;
                        const int kg = s.mb == 32 ? l / 32 : grp;
                        const int nb = s.mb == 32 ? 16 * (grp % 2) : 0;
                        row = st * s.kb() + 8 * kg + 4 * rr + j / 4;
                        col = (wn0 + ni * s.mb + nb + 4 * (j % 4)) / 2;
                    });
    }
    return total;
}

constexpr LayoutChoice mixed_layout_a(Mixed16Shape s, LdsGeometry g) {
    return choose_layout([=](LayoutChoice c) { return mixed_a_cost(s, c, g); }, s.bk / 2, false);
}
constexpr LayoutChoice mixed_layout_b(Mixed16Shape s, LdsGeometry g) {
    return choose_layout([=](LayoutChoice c) { return mixed_b_cost(s, c, g); }, s.bn / 2, false);
}

// ---- vector-ALU kernel: A k-major [BK][BM], B row-major [BK][BN] ----
// Thread t (of `threads`) owns rows (t / threads_n) * 4 (+ BM / 2) and columns
// (t % threads_n) * 4 (+ BN / 2) of the output tile.  Per k it reads 4 + 4
// consecutive words of row k of At and of B (16-byte reads); the tiles are
// stored by the cooperative copy: B row-major with `vec`-wide stores, A
// transposed with one 4-byte store per element.  Every wavefront's accesses
// are costed (the swizzle makes them differ by wavefront).
struct ValuShape {
    int bm, bn, bk, threads_n, threads, vec;
    constexpr int waves() const { return threads / kWaveLanes; }
};

constexpr int valu_a_cost(ValuShape s, LayoutChoice c, LdsGeometry g) {
    int total = 0;
    const int vcols = s.bk / s.vec;
    for (int w = 0; w < s.waves(); ++w) {
        for (int k = 0; k < s.bk; ++k)
            for (int half = 0; half < 2; ++half)
                total += pattern_cost(c, s.bm, 4, g, [=](int l, int& row, int& col) {
                    row = k;
                    col = half * (s.bm / 2) + ((w * kWaveLanes + l) / s.threads_n) * 4;
                });
        for (int i = 0; i < s.bm * vcols / s.threads; ++i)
            for (int e = 0; e < s.vec; ++e)
                total += pattern_cost(
                    c, s.bm, 1, g,
                    [=](int l, int& row, int& col) {
                        const int slot = w * kWaveLanes + l + i * s.threads;
                        row = s.vec * (slot % vcols) + e;
                        col = slot / vcols;
                    },
                    true);
    }
    return total;
}
constexpr int valu_b_cost(ValuShape s, LayoutChoice c, LdsGeometry g) {
    int total = 0;
    const int vcols = s.bn / s.vec;
    for (int w = 0; w < s.waves(); ++w) {
        for (int k = 0; k < s.bk; ++k)
            for (int half = 0; half < 2; ++half)
                total += pattern_cost(c, s.bn, 4, g, [=](int l, int& row, int& col) {
                    row = k;
                    col = half * (s.bn / 2) + ((w * kWaveLanes + l) % s.threads_n) * 4;
                });
        for (int i = 0; i < s.bk * vcols / s.threads; ++i)
            total += pattern_cost(
                c, s.bn, s.vec, g,
                [=](int l, int& row, int& col) {
                    const int slot = w * kWaveLanes + l + i * s.threads;
                    row = slot / vcols;
                    col = s.vec * (slot % vcols);
                },
                true);
    }
    return total;
}
constexpr LayoutChoice valu_layout_a(ValuShape s, LdsGeometry g) {
    return choose_layout([=](LayoutChoice c) { return valu_a_cost(s, c, g); }, s.bm);
}
constexpr LayoutChoice valu_layout_b(ValuShape s, LdsGeometry g) {
    return choose_layout([=](LayoutChoice c) { return valu_b_cost(s, c, g); }, s.bn);
}

}  // namespace dft
