/*
 * dense_fp32_tiled.h -- C ABI of the MI355X (gfx950) masked, LDS-tiled fp32
 * matrix multiply  C[M,N] = A[M,K] @ B[K,N].
 *
 * The operation is the one built up in "My Triton From Scratch, Part 14:
 * Shared-Memory Tiles": dot(block<BMxBK>, block<BKxBN>) -> block<BMxBN>
 * (opening section), per output tile and accumulated over a runtime K loop
 * (section "Staging inside a runtime K loop").  Operand tiles are read with
 * the masks (rows < M) & (cols < K) for A and (rows < K) & (cols < N) for B,
 * and out-of-range elements are zero-filled (sections "The canonical source
 * pattern", "Matching the safety mask", "Zero-filled boundary tiles"); the
 * output is stored under the mask (rows < M) & (cols < N) (section
 * "Preserving shared dependencies").  Zero fill makes the tiled result equal
 * to the plain sum over k in [0, K) for every in-range element.
 *
 * Conventions for every entry point below
 *   - Matrices are row-major.  Element (i, k) of A is A[i*lda + k]; likewise
 *     B with ldb and C with ldc.  Leading dimensions are in elements and may
 *     exceed the logical width; elements in the gap are never read or written.
 *   - A, B and C are DEVICE pointers owned by the caller.  The library keeps no
 *     pointer after the call returns, allocates no device memory and holds no
 *     per-call state; it caches only per-device properties.
 *   - C = A @ B overwrites C (no alpha/beta).  C must not overlap A or B.
 *   - M == 0 or N == 0: nothing is launched.  K == 0: the M x N region of C is
 *     set to zero (an empty sum).
 *   - Arguments are validated on the host before anything is launched, so an
 *     error status means nothing was enqueued.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *     null stream of the current device).  Device-side faults surface at the
 *     caller's next synchronisation, not in the returned status.
 *   - The current HIP device must be a gfx950 (MI355X).
 *   - Entry points are reentrant; calls on different streams may overlap.
 */
#ifndef DENSE_FP32_TILED_H
#define DENSE_FP32_TILED_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point (0 = success). */
typedef enum {
    GEMM_OK = 0,
    GEMM_ERR_INVALID_DIM = -1,  /* M, N or K negative */
    GEMM_ERR_INVALID_LD = -2,   /* lda < max(1,K), ldb < max(1,N) or ldc < max(1,N) */
    GEMM_ERR_NULL = -3,         /* a NULL pointer for an operand with non-zero extent */
    GEMM_ERR_ALIAS = -4,        /* the address range of C overlaps that of A or B */
    GEMM_ERR_UNSUPPORTED = -5,  /* no gfx950 device current, or unknown variant */
    GEMM_ERR_CONFIG = -6,       /* variant's LDS footprint exceeds the device limit */
    GEMM_ERR_HIP = -7,          /* a HIP runtime call or the launch failed */
    GEMM_ERR_TOO_LARGE = -8     /* a size overflows the kernel's index range */
} gemm_status;

/* Kernel variants.  Every variant computes the same operation; they differ in
 * how (see gemm_f32_tile_config for each one's tile geometry). */
typedef enum {
    GEMM_VARIANT_AUTO = 0,          /* the default: currently GEMM_VARIANT_MFMA */
    GEMM_VARIANT_MFMA = 1,          /* fp32 matrix-core (v_mfma_f32_32x32x2_f32) inner product */
    GEMM_VARIANT_VALU = 2,          /* register-tiled vector-ALU fp32 FMA inner product */
    GEMM_VARIANT_MFMA_STAGES1 = 3,  /* ablation: one LDS stage, two barriers per K tile, no prefetch */
    GEMM_VARIANT_MFMA_NOPAD = 4,    /* ablation: LDS rows without padding */
    GEMM_VARIANT_MFMA_SCALAR = 5,   /* ablation: 4-byte global loads even when 16-byte loads are legal */
    GEMM_VARIANT_COUNT = 6
} gemm_variant;

/* Tile geometry of one variant.  The LDS tiles follow the layout of
 * "My Triton From Scratch, Part 18: Shared Memory Optimization", section
 * "A shared buffer needs a physical row stride": row_stride = cols + pad,
 * stage_elems = rows * row_stride, and element (stage, row, col) lives at
 * stage * stage_elems + row * row_stride + col (in fp32 words). */
typedef struct {
    int32_t variant;
    int32_t bm, bn, bk;          /* output tile BM x BN, reduction tile BK */
    int32_t threads, wave_size;  /* threads per workgroup, lanes per wavefront */
    int32_t tm, tn;              /* outputs per thread (VALU) or per wave (MFMA) along M and N */
    int32_t stages;              /* LDS stages (1 or 2) */
    int32_t barriers_per_tile;   /* workgroup barriers per K tile */
    int32_t a_rows, a_cols, a_pad, a_row_stride, a_stage_elems; /* LDS tile of A */
    int32_t b_rows, b_cols, b_pad, b_row_stride, b_stage_elems; /* LDS tile of B */
    int32_t lds_bytes;           /* stages * (a_stage_elems + b_stage_elems) * 4 */
    int32_t vec_width;           /* fp32 elements per global load when aligned (1 or 4) */
    int32_t lds_banks_b32;       /* LDS geometry the padding was derived for: banks and */
    int32_t lds_lanes_b32;       /*   lanes serviced per pass for 4-byte accesses ... */
    int32_t lds_banks_b128;      /*   ... and for 16-byte accesses */
    int32_t lds_lanes_b128;
    int32_t a_transposed;        /* 1 if A is stored k-major in LDS (a_rows = BK) */
} gemm_tile_config;

/* C = A @ B with the default variant.  M, N, K >= 0; lda >= max(1,K),
 * ldb >= max(1,N), ldc >= max(1,N).  Returns a gemm_status. */
int gemm_f32(int64_t M, int64_t N, int64_t K,
             const float *A, int64_t lda,
             const float *B, int64_t ldb,
             float *C, int64_t ldc,
             void *stream);

/* As gemm_f32 with an explicit gemm_variant.  When lda or ldb is not a
 * multiple of 4, or A or B is not 16-byte aligned, the variant's 16-byte
 * loads are illegal and the call runs the same variant with 4-byte masked
 * loads (a fallback, not an error; results are identical). */
int gemm_f32_ex(int64_t M, int64_t N, int64_t K,
                const float *A, int64_t lda,
                const float *B, int64_t ldb,
                float *C, int64_t ldc,
                void *stream, int variant);

/* Fills *out with the tile geometry of `variant`.  Pure host call (touches no
 * device).  Returns GEMM_OK, GEMM_ERR_NULL or GEMM_ERR_UNSUPPORTED. */
int gemm_f32_tile_config(int variant, gemm_tile_config *out);

/* Static, NUL-terminated description of a status code (never NULL). */
const char *gemm_f32_status_string(int status);

/* ---- Host-side layout model -------------------------------------------------
 * The LDS layout and bank model the kernels are compiled from, exported so
 * that tests can check them against the values the pages print.  Pure host
 * calls; they touch no device. */

/* Physical LDS layout of a rows x cols fp32 tile with `pad` words of row
 * padding and `stages` copies ("My Triton From Scratch, Part 18", section "A
 * shared buffer needs a physical row stride").  Writes row_stride,
 * stage_elems, total_elems and bytes (any output pointer may be NULL).
 * Returns GEMM_OK, or GEMM_ERR_INVALID_DIM for rows/cols < 1, pad < 0 or
 * stages < 1. */
int gemm_lds_layout(int32_t rows, int32_t cols, int32_t pad, int32_t stages,
                    int32_t *row_stride, int32_t *stage_elems,
                    int32_t *total_elems, int32_t *bytes);

/* Word offset of (stage, row, col) in that layout, or -1 when a coordinate
 * is outside [0,stages) x [0,rows) x [0,cols) or the layout is invalid. */
int64_t gemm_lds_offset(int32_t rows, int32_t cols, int32_t pad, int32_t stages,
                        int32_t stage, int32_t row, int32_t col);

/* Bank of a 4-byte LDS word: word_offset mod banks ("My Triton From
 * Scratch, Part 18", section "Why shared-memory banks matter").  -1 if
 * banks < 1 or word_offset < 0. */
int32_t gemm_lds_bank(int64_t word_offset, int32_t banks);

/* Bank-conflict degree of one LDS instruction: lanes are serviced in
 * consecutive groups of `group` lanes; within a group, the cost is the
 * largest number of DISTINCT dword addresses that fall in one bank (the same
 * address read by several lanes is a broadcast and costs one).  Lane l
 * accesses `width` consecutive dwords starting at lane_words[l].  Returns the
 * maximum over groups (1 = conflict-free), or -1 on bad arguments. */
int32_t gemm_lds_conflict_degree(const int64_t *lane_words, int32_t lanes,
                                 int32_t width, int32_t banks, int32_t group);

/* The pages' padding rule for the A-tile column read ("My Triton From
 * Scratch, Part 18", section "Choosing padding instead of hard-coding it"):
 * distinct = banks / gcd(columns, banks); pad = simultaneous_rows > distinct.
 * Returns -1 on bad arguments. */
int32_t gemm_lds_page_pad(int32_t columns, int32_t simultaneous_rows, int32_t banks);

#ifdef __cplusplus
}
#endif

#endif /* DENSE_FP32_TILED_H */
