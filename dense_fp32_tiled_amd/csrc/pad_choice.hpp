// pad_choice.hpp -- LDS row padding for each kernel, derived at compile time
// from the bank model and the kernel's own lane -> address patterns.
//
// For every LDS access a kernel issues on a tile (fragment reads, cooperative
// stores) the conflict degree is computed from the exact addresses the lanes
// of one wavefront touch; the pad minimises the sum of degree x instructions
// per K tile over those accesses, among pads that keep 16-byte alignment.
// This replaces the pages' one-pattern rule ("My Triton From Scratch, Part
// 18: Shared Memory Optimization", section "Choosing padding instead of
// hard-coding it"), which models a single one-warp read of A.
#pragma once

#include "lds_layout.hpp"

namespace dft {

constexpr int kMaxPad = 32;

// ---- matrix-core kernel: A row-major [BM][BK+pad], B row-major [BK][BN+pad] --
struct MfmaShape {
    int bm, bn, bk, wm, wn, threads, vec;
    constexpr int kh() const { return bk / 2; }
};

// A fragment read (16-byte): lane l reads row l%32 at column (l/32)*BK/2.
constexpr int mfma_a_read_degree(MfmaShape s, int pad, LdsGeometry g) {
    const int stride = s.bk + pad;
    return conflict_degree([=](int l) { return (int64_t)(l % 32) * stride + (l / 32) * s.kh(); },
                           kWaveLanes, 4, g.banks_for_width(4), g.group_for_width(4));
}
// Cooperative store of A (vec-wide): slot l -> row l/(BK/vec), column vec*(l%(BK/vec)).
constexpr int mfma_a_write_degree(MfmaShape s, int pad, LdsGeometry g) {
    const int stride = s.bk + pad, vcols = s.bk / s.vec;
    return conflict_degree([=](int l) { return (int64_t)(l / vcols) * stride + s.vec * (l % vcols); },
                           kWaveLanes, s.vec, g.banks_for_width(s.vec), g.group_for_width(s.vec));
}
// B fragment read (4-byte): lane l reads row (l/32)*BK/2 + j at column l%32.
constexpr int mfma_b_read_degree(MfmaShape s, int pad, LdsGeometry g) {
    const int stride = s.bn + pad;
    return conflict_degree([=](int l) { return (int64_t)((l / 32) * s.kh()) * stride + (l % 32); },
                           kWaveLanes, 1, g.banks_for_width(1), g.group_for_width(1));
}
constexpr int mfma_b_write_degree(MfmaShape s, int pad, LdsGeometry g) {
    const int stride = s.bn + pad, vcols = s.bn / s.vec;
    return conflict_degree([=](int l) { return (int64_t)(l / vcols) * stride + s.vec * (l % vcols); },
                           kWaveLanes, s.vec, g.banks_for_width(s.vec), g.group_for_width(s.vec));
}

// LDS passes one access of `width_words` costs at conflict degree `degree`.
constexpr int access_cost(int degree, int width_words, LdsGeometry g) {
    return degree * (kWaveLanes / g.group_for_width(width_words));
}

// Cost per wavefront per K tile: instructions x passes x degree.
constexpr int mfma_a_cost(MfmaShape s, int pad, LdsGeometry g) {
    const int reads = (s.wm / 32) * (s.kh() / 4);
    const int writes = (s.bm * s.bk) / (s.vec * s.threads);
    return reads * access_cost(mfma_a_read_degree(s, pad, g), 4, g) +
           writes * access_cost(mfma_a_write_degree(s, pad, g), s.vec, g);
}
constexpr int mfma_b_cost(MfmaShape s, int pad, LdsGeometry g) {
    const int reads = (s.wn / 32) * s.kh();
    const int writes = (s.bk * s.bn) / (s.vec * s.threads);
    return reads * access_cost(mfma_b_read_degree(s, pad, g), 1, g) +
           writes * access_cost(mfma_b_write_degree(s, pad, g), s.vec, g);
}

template <class Cost>
constexpr int argmin_pad(Cost cost) {
    int best_pad = 0, best = cost(0);
    for (int pad = 4; pad <= kMaxPad; pad += 4) {
        const int c = cost(pad);
        if (c < best) { best = c; best_pad = pad; }
    }
    return best_pad;
}

constexpr int mfma_pad_a(MfmaShape s, LdsGeometry g) {
    return argmin_pad([=](int pad) { return mfma_a_cost(s, pad, g); });
}
constexpr int mfma_pad_b(MfmaShape s, LdsGeometry g) {
    return argmin_pad([=](int pad) { return mfma_b_cost(s, pad, g); });
}

// ---- vector-ALU kernel: A k-major [BK][BM+pad], B row-major [BK][BN+pad] ----
struct ValuShape {
    int bm, bn, bk, threads_n, threads, vec;
};

// At read (16-byte): lane l of wave 0 reads At[k][(l/threads_n)*4].
constexpr int valu_a_read_degree(ValuShape s, int pad, LdsGeometry g) {
    (void)pad;
    return conflict_degree([=](int l) { return (int64_t)(l / s.threads_n) * 4; }, kWaveLanes, 4,
                           g.banks_for_width(4), g.group_for_width(4));
}
// Transposed store of A: slot l holds A[l/(BK/vec)][vec*(l%(BK/vec)) + e]; element e goes to
// At[vec*(l%(BK/vec)) + e][l/(BK/vec)] with a 4-byte store.
constexpr int valu_a_write_degree(ValuShape s, int pad, LdsGeometry g) {
    const int stride = s.bm + pad, vcols = s.bk / s.vec;
    return conflict_degree([=](int l) { return (int64_t)(s.vec * (l % vcols)) * stride + l / vcols; },
                           kWaveLanes, 1, g.banks_for_width(1), g.group_for_width(1));
}
constexpr int valu_b_read_degree(ValuShape s, int pad, LdsGeometry g) {
    (void)pad;
    return conflict_degree([=](int l) { return (int64_t)(l % s.threads_n) * 4; }, kWaveLanes, 4,
                           g.banks_for_width(4), g.group_for_width(4));
}
constexpr int valu_b_write_degree(ValuShape s, int pad, LdsGeometry g) {
    const int stride = s.bn + pad, vcols = s.bn / s.vec;
    return conflict_degree([=](int l) { return (int64_t)(l / vcols) * stride + s.vec * (l % vcols); },
                           kWaveLanes, s.vec, g.banks_for_width(s.vec), g.group_for_width(s.vec));
}
constexpr int valu_pad_a(ValuShape s, LdsGeometry g) {
    return argmin_pad([=](int pad) {
        return 2 * s.bk * access_cost(valu_a_read_degree(s, pad, g), 4, g) +
               (s.bm * s.bk / s.threads) * access_cost(valu_a_write_degree(s, pad, g), 1, g);
    });
}
constexpr int valu_pad_b(ValuShape s, LdsGeometry g) {
    return argmin_pad([=](int pad) {
        return 2 * s.bk * access_cost(valu_b_read_degree(s, pad, g), 4, g) +
               (s.bk * s.bn / (s.vec * s.threads)) * access_cost(valu_b_write_degree(s, pad, g), s.vec, g);
    });
}

}  // namespace dft
