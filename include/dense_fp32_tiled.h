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
 * gemm_mixed_f32 (end of this header) computes the same product from bf16 or
 * fp16 A and B with fp32 accumulation; the conventions below apply to it with
 * 2-byte A and B elements.
 *
 * Conventions for every entry point below
 *   - Matrices are row-major.  Element (i, k) of A is A[i*lda + k]; likewise
 *     B with ldb and C with ldc.  Leading dimensions are in elements and may
 *     exceed the logical width; elements in the gap are never read or written.
 *   - A, B and C are DEVICE pointers owned by the caller.  The library keeps no
 *     pointer after the call returns, allocates no device memory and holds no
 *     per-call state; it caches only per-device properties.
 *   - C = A @ B overwrites C (no alpha/beta).  C must not overlap A or B (nor a
 *     split-K workspace any operand).
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
    GEMM_ERR_UNSUPPORTED = -5,  /* no gfx950 device current, or unknown variant or input type */
    GEMM_ERR_CONFIG = -6,       /* variant's LDS footprint (both operands' tiles, every stage and
                                   its padding) exceeds the device's LDS per workgroup: the budget
                                   check of "My Triton From Scratch, Part 18", section "Shared-memory
                                   budget checks include stages and padding", and of Part 14, section
                                   "Tracking the shared-memory budget"; as there, the check runs for
                                   the operand pair before anything is launched, so a failure leaves
                                   nothing half done */
    GEMM_ERR_HIP = -7,          /* a HIP runtime call or the launch failed */
    GEMM_ERR_TOO_LARGE = -8,    /* a size overflows the kernel's index range */
    GEMM_ERR_WORKSPACE = -9,    /* split-K workspace missing or too small */
    GEMM_ERR_SCRATCH = -10      /* gemm_f32_splitk_noalloc: partial products exceed its static array */
} gemm_status;

/* Kernel variants.  Every variant computes the same operation; they differ in
 * how (see gemm_f32_tile_config for each one's tile geometry). */
typedef enum {
    GEMM_VARIANT_AUTO = 0,          /* picks a direct-copy MFMA variant from M, N, K (gemm_f32_auto_variant) */
    GEMM_VARIANT_MFMA = 1,          /* v_mfma_f32_32x32x2_f32, 256x128x16 workgroup tile, 8 waves of 64x64 */
    GEMM_VARIANT_VALU = 2,          /* register-tiled vector-ALU fp32 FMA, 128x128x16, 8x8 per thread */
    GEMM_VARIANT_MFMA_STAGES1 = 3,  /* ablation of MFMA: one LDS stage, two barriers per K tile, no prefetch */
    GEMM_VARIANT_MFMA_NOPAD = 4,    /* ablation of MFMA: plain LDS rows (no padding, no swizzle) */
    GEMM_VARIANT_MFMA_SCALAR = 5,   /* ablation of MFMA: 4-byte global loads even when 16-byte loads are legal */
    GEMM_VARIANT_MFMA16 = 6,        /* as MFMA with v_mfma_f32_16x16x4_f32 */
    GEMM_VARIANT_MFMA_128 = 7,      /* as MFMA with a 128x128x16 workgroup tile (4 waves) */
    GEMM_VARIANT_MFMA_128_BK32 = 8, /* as MFMA_128 with BK = 32 (its 4-byte-load fallback uses BK = 16) */
    GEMM_VARIANT_MFMA_DIRECT = 9,   /* as MFMA with in-range tiles copied global->LDS directly (no registers) */
    GEMM_VARIANT_MFMA_128_DIRECT = 10,      /* as MFMA_128 with direct global->LDS copies */
    GEMM_VARIANT_MFMA_128_BK32_DIRECT = 11, /* as MFMA_128_BK32 with direct global->LDS copies */
    GEMM_VARIANT_MFMA_64_DIRECT = 12,       /* 64x64x16 tile, 4 waves of 32x32, direct copies (few output tiles) */
    GEMM_VARIANT_MFMA_256x256_DIRECT = 13,  /* 256x256x16 tile, 8 waves of 128x64 (2 per SIMD), direct copies */
    GEMM_VARIANT_MFMA_256x256_W4_DIRECT = 14, /* 256x256x16 tile, 4 waves of 128x128 (1 per SIMD), direct copies */
    GEMM_VARIANT_MFMA_256x256_PIPE = 15,      /* as MFMA_256x256_DIRECT, multiply software-pipelined (fragments one
                                                 MFMA step ahead, the last step after the K-tile barrier) */
    GEMM_VARIANT_MFMA_256x256_BK32_PIPE = 16, /* as MFMA_256x256_PIPE with BK = 32 (128 KiB of LDS): AUTO's choice
                                                 for large problems */
    GEMM_VARIANT_MFMA16_256x256_DIRECT = 17,  /* as MFMA_256x256_DIRECT with v_mfma_f32_16x16x4_f32 */
    GEMM_VARIANT_MFMA16_256x256_W4_BK32_PIPE = 18, /* 16x16x4, 256x256x32 tile, 4 waves of 128x128, pipelined */
    GEMM_VARIANT_MFMA_64_BK32_DIRECT = 19,    /* as MFMA_64_DIRECT with BK = 32 (half the barriers): AUTO's choice
                                                 for few output tiles */
    GEMM_VARIANT_MFMA_64_KS4 = 20,    /* 64x64x32 tile, K split over 4 groups of 4 waves inside the workgroup
                                         (partial sums added in LDS, in group order): deep K, few tiles */
    GEMM_VARIANT_MFMA_32x64_KS4 = 21, /* 32x64x32 tile, 4 groups of 2 waves */
    GEMM_VARIANT_MFMA_32x32_KS8 = 22, /* 32x32x32 tile, 8 groups of 1 wave */
    GEMM_VARIANT_MFMA_64_BK32_PIPE = 23, /* as MFMA_64_BK32_DIRECT with the pipelined multiply */
    GEMM_VARIANT_MFMA_64_KS2 = 24,    /* 64x64x32 tile, K split over 2 groups of 4 waves (two waves per SIMD) */
    GEMM_VARIANT_COUNT = 25
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
    int32_t lds_banks_b32;       /* LDS geometry the layout was derived for: banks and */
    int32_t lds_lanes_b32;       /*   lanes serviced per pass for 4-byte accesses ... */
    int32_t lds_banks_b128;      /*   ... and for 16-byte accesses */
    int32_t lds_lanes_b128;
    int32_t a_transposed;        /* 1 if A is stored k-major in LDS (a_rows = BK) */
    int32_t a_swz_unit, a_swz_shift, a_swz_mask; /* XOR swizzle of A's LDS columns (unit 0 = none): */
    int32_t b_swz_unit, b_swz_shift, b_swz_mask; /*   col ^ (unit * ((row >> shift) & mask)) */
    int32_t mfma_block;          /* MFMA block size (32 or 16), 0 for the VALU variant */
    int32_t xcd_tile_order;      /* 1 if workgroups are mapped to tiles in the XCD-grouped order */
    int32_t direct_to_lds;       /* 1 if in-range tiles are copied global->LDS without registers (16 bytes
                                    per lane, LDS rows unpadded); edge tiles, and launches whose tile byte
                                    span exceeds 31 bits (a very wide lda or ldb), still go through
                                    registers; 2 if, in addition, the multiply is software-pipelined
                                    across the K-tile barrier (fragments read one MFMA step ahead) */
    int32_t elem_bytes;          /* bytes per A / B element: 4 (fp32), 2 (bf16 / fp16, gemm_mixed_f32);
                                    LDS tile fields count 4-byte words, so a row of a 16-bit tile holds
                                    2 * cols elements */
    int32_t k_groups;            /* groups of waves that split K inside the workgroup (1: none); each
                                    group has 2 of the `stages`, `threads` counts all groups, tm x tn
                                    is one wave's tile within a group */
} gemm_tile_config;

/* C = A @ B with the default variant.  M, N, K >= 0; lda >= max(1,K),
 * ldb >= max(1,N), ldc >= max(1,N).  Returns a gemm_status.
 * One workgroup per BM x BN output tile, reducing over K tiles with masked,
 * zero-filled operand tiles and a masked store: the program of "My Triton
 * From Scratch, Part 14: Shared-Memory Tiles", section "The canonical source
 * pattern", staged through LDS as in its sections "Cooperative copy mapping"
 * and "Staging inside a runtime K loop". */
int gemm_f32(int64_t M, int64_t N, int64_t K,
             const float *A, int64_t lda,
             const float *B, int64_t ldb,
             float *C, int64_t ldc,
             void *stream);

/* As gemm_f32 with an explicit gemm_variant.  When lda (ldb) is not a
 * multiple of 4, or A (B) is not 16-byte aligned (for B also: N not a
 * multiple of 4, since an edge tile moved back to end at N starts its
 * columns at N - BN), that operand cannot be loaded or copied 16 bytes per
 * lane, and the call runs the variant's kernel that moves it 4 bytes per
 * lane instead: a fallback, not an error, with the same result up to the
 * order of the fp32 additions.  This is the rule of "My Triton From Scratch,
 * Part 18", section "Why a conservative matcher matters": a specialised
 * lowering applies only where its preconditions hold, and otherwise the
 * existing correct form runs.  The variants AUTO chooses
 * from (MFMA_256x256_BK32_PIPE, MFMA_DIRECT, MFMA_128_DIRECT,
 * MFMA_128_BK32_DIRECT, MFMA_64_BK32_DIRECT) decide per operand and keep
 * 16-byte copies for an aligned one; the others move both operands 4 bytes
 * at a time.  The fallback kernel has the variant's tile, except 128x128x16
 * for the 128x128x32 variants and 256x128x16 through registers for
 * MFMA_256x256_DIRECT, MFMA_256x256_W4_DIRECT, MFMA_256x256_PIPE and the
 * MFMA16_256x256 variants, whose 4-byte versions would not fit their
 * registers. */
int gemm_f32_ex(int64_t M, int64_t N, int64_t K,
                const float *A, int64_t lda,
                const float *B, int64_t ldb,
                float *C, int64_t ldc,
                void *stream, int variant);

/* Split-K: C = A @ B with the K range cut into `splits` slices of whole K
 * tiles, each reduced by its own workgroups (the kernel of
 * gemm_f32_splitk_auto_variant), so that problems with few 128x128 output
 * tiles still occupy every CU.
 * Slice s writes its partial product, packed M x N, to workspace + s*M*N
 * floats; a second kernel then sets C = sum of the slices in ascending slice
 * order, so the result is deterministic for a given `splits`.
 *   workspace: DEVICE buffer owned by the caller, at least
 *              gemm_f32_splitk_workspace_bytes(M, N, K, splits, num_cus) bytes
 *              (may be NULL when that is 0); its contents on entry are ignored
 *              and on return unspecified.  It must not overlap A, B or C.
 *   splits: 1..64, or 0 for gemm_f32_splitk_auto_splits on the current
 *           device.  splits == 1 is a plain launch and needs no workspace.
 * Other arguments and conventions as gemm_f32.  Returns a gemm_status;
 * GEMM_ERR_WORKSPACE if the workspace is missing or too small. */
int gemm_f32_splitk(int64_t M, int64_t N, int64_t K,
                    const float *A, int64_t lda,
                    const float *B, int64_t ldb,
                    float *C, int64_t ldc,
                    void *workspace, int64_t workspace_bytes, int splits, void *stream);

/* As gemm_f32_splitk with the slices computed by the kernel of `variant`
 * (GEMM_VARIANT_AUTO: that of gemm_f32_splitk_auto_variant); slices are
 * whole K tiles of that kernel.  The workspace and split count rules are
 * gemm_f32_splitk's.  Returns GEMM_ERR_UNSUPPORTED for an unknown variant. */
int gemm_f32_splitk_ex(int64_t M, int64_t N, int64_t K,
                       const float *A, int64_t lda,
                       const float *B, int64_t ldb,
                       float *C, int64_t ldc,
                       void *workspace, int64_t workspace_bytes, int splits, void *stream, int variant);

/* Split-K for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): as
 * gemm_f32_splitk, with the partial products kept in a 64 MiB array that the
 * library holds in device memory, one per GPU it runs on, until the process
 * ends, instead of a caller's workspace.  Allocates nothing and calls no
 * allocating routine; the array's device address is looked up on the first
 * call on each device.
 *   splits: 2..64 need splits * M * N * 4 <= 64 MiB, else GEMM_ERR_SCRATCH
 *           (before anything is enqueued); 1 is a plain launch; 0 takes
 *           gemm_f32_splitk_auto_splits, lowered until the partial products
 *           fit (down to 1; on a 256-CU device the automatic count always
 *           fits, its partial products stay near 32 MiB or below).
 * The array keeps the last call's contents; nothing in it needs clearing
 * (every slice writes its whole partial product).  Calls that overlap on one
 * GPU (e.g. on two streams) share the array and race: serialise them.
 * Other arguments, conventions and the result are gemm_f32_splitk's for the
 * same split count. */
int gemm_f32_splitk_noalloc(int64_t M, int64_t N, int64_t K,
                            const float *A, int64_t lda,
                            const float *B, int64_t ldb,
                            float *C, int64_t ldc,
                            int splits, void *stream);

/* The variant gemm_f32_splitk runs the slices with.  Pure host call. */
int gemm_f32_splitk_auto_variant(void);

/* Workspace bytes gemm_f32_splitk needs (splits * M * N * 4, or 0 when the
 * resolved split count is 1); splits == 0 resolves with num_cus compute
 * units.  Pure host call.  Returns GEMM_ERR_INVALID_DIM on bad arguments. */
int64_t gemm_f32_splitk_workspace_bytes(int64_t M, int64_t N, int64_t K, int splits, int32_t num_cus);

/* The split count gemm_f32_splitk uses for splits == 0: enough slices for
 * one workgroup per CU over the 256x128 output tiles, at most 64, and at
 * least eight 16-deep K tiles per slice.  Pure host call. */
int gemm_f32_splitk_auto_splits(int64_t M, int64_t N, int64_t K, int32_t num_cus);

/* Fills *out with the tile geometry of `variant`: its BM x BN x BK tiles
 * ("My Triton From Scratch, Part 14", section "A global tile description")
 * and each operand's LDS tile with its row stride, stages and byte footprint
 * (Part 18, sections "A shared buffer needs a physical row stride" and
 * "Shared-memory budget checks include stages and padding").  Pure host call
 * (touches no device).  Returns GEMM_OK, GEMM_ERR_NULL or
 * GEMM_ERR_UNSUPPORTED. */
int gemm_f32_tile_config(int variant, gemm_tile_config *out);

/* Static, NUL-terminated description of a status code (never NULL).  Every
 * failure is reported before anything is enqueued (argument and budget
 * checks run first, as the LDS budget check of "My Triton From Scratch,
 * Part 14", section "Tracking the shared-memory budget", makes a failure
 * atomic), except GEMM_ERR_HIP for a launch the runtime refused.  Unknown
 * codes give "unknown status". */
const char *gemm_f32_status_string(int status);

/* The variant GEMM_VARIANT_AUTO runs for an M x N x K problem on a device with
 * `num_cus` compute units, both operands' rows 16-byte aligned: the
 * candidate with the highest rate estimate.  Candidates and full-chip rates:
 * MFMA_256x256_BK32_PIPE 145 TFLOP/s, MFMA_DIRECT (256x128) 144, the 128x128
 * direct variant (BK 32 when K >= 1024, else 16) 144, the 64x64x32 kernel
 * 134 (MFMA_64_BK32_DIRECT; MFMA_64_BK32_PIPE when neither operand's rows
 * are aligned and its grid has more than num_cus tiles); when K >= 2048 also MFMA_64_KS4 117 and MFMA_32x64_KS4 101, and when
 * K >= 4096 MFMA_32x32_KS8 96 (K split inside the workgroup; when the
 * split's grid has at most num_cus tiles, already from K >= 1024 for
 * MFMA_64_KS4, K >= 128 for MFMA_32x64_KS4 and K >= 256 for
 * MFMA_32x32_KS8).  Estimate:
 * the rate times the wave quantisation of the tile grid,
 * tiles / (ceil(tiles / num_cus) * num_cus); times 0.88 for the 256x128 and
 * 128x128 kernels with fewer tiles than two per CU (they are built for two
 * workgroups per CU); for the 64x64 kernel times 0.78 with at most one tile
 * per CU and 0.89 with at most two (its 4-wave workgroups need several per
 * CU); and times rounds / (rounds + 1) when M or N is smaller than, and not
 * a multiple of, the tile (its edge workgroups then load through
 * registers; when M >= BM and N >= BN an edge tile is moved back to end at
 * M or N and runs as an interior one).  A candidate listed earlier wins
 * within 2 %.  Pure host call.  Returns a gemm_variant, or
 * GEMM_ERR_INVALID_DIM for negative sizes or num_cus < 1. */
int gemm_f32_auto_variant(int64_t M, int64_t N, int64_t K, int32_t num_cus);

/* As gemm_f32_auto_variant for operands whose rows may not be 16-byte
 * aligned: a_rows_aligned (b_rows_aligned) nonzero when lda (ldb) is a
 * multiple of 4 and A (B) is 16-byte aligned, the condition under which
 * that operand is copied 16 bytes per lane; otherwise 4 bytes per lane.
 * The rates (TFLOP/s with every CU busy, for 256x256 pipelined, 256x128,
 * 128x128 and 64x64x32) are, for both aligned, 145, 144, 144, 134; only A
 * aligned 134, 140, 124, 120; only B aligned 133, 130, 130, 128; neither
 * 130, 121, 118, 110; for MFMA_64_KS4, MFMA_32x64_KS4 and MFMA_32x32_KS8
 * (both aligned 117, 101, 96 as above) only A aligned 108 (126 on a
 * one-round grid with K >= 4096), 79, 66; only B
 * aligned 110, 95, 81; neither 103, 76, 63; MFMA_64_KS2 (from K >= 1024, or
 * K >= 512 when its grid has at most num_cus tiles) 101, 124, 100, 99: it
 * wins with neither operand aligned in one round of tiles (1000 x 999 x
 * 513), and with only A aligned on 64x64 grids of any size (3000 x 2999 x
 * 3000).  With neither aligned and more 64x64 tiles than CUs the 64x64x32
 * candidate is MFMA_64_BK32_PIPE, else MFMA_64_BK32_DIRECT.
 * GEMM_VARIANT_AUTO in gemm_f32 / gemm_f32_ex applies this with
 * the operands' actual alignment.  gemm_f32_auto_variant is this
 * with both flags set.  Pure host call. */
int gemm_f32_auto_variant_ex(int64_t M, int64_t N, int64_t K, int32_t num_cus, int32_t a_rows_aligned,
                             int32_t b_rows_aligned);

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

/* LDS cycles one 64-lane instruction costs under the measured gfx950 bank
 * model the layout search uses (the cost behind "My Triton From Scratch,
 * Part 18", section "Choosing padding instead of hard-coding it"): per pass
 * of the access width's lane group, that pass's conflict degree, summed.
 * A pass is that many consecutive lanes, except for 16-byte reads, where the
 * four passes of 16 lanes are the lanes of one half-wave (l / 32) whose
 * 4-lane group index ((l / 4) mod 8) has even, or odd, bit parity.
 * lane_words: 64 dword offsets (host array, not retained), lane l's access
 * starting at lane_words[l].  mode: 1, 2, 4 = 4-, 8-, 16-byte reads;
 * 101, 102, 104 = 4-, 8-, 16-byte stores; -16 or -32 = a two-address 4-byte
 * read (ds_read2_b32) whose second dword is 16 or 32 words after the first.
 * Geometry: reads 32 banks x 32 lanes (4-byte), 64 x 32 (8-byte), 64 x 16
 * (16-byte); stores 32 x 32 (4-byte), 32 x 16 (8-byte), 32 x 8 (16-byte).
 * Excludes the issue time a conflict-free instruction takes anyway
 * (measured about 3.4 cycles for 4- and 8-byte reads, 4 for 16-byte and
 * two-address reads and 4-byte stores, 7.2 for 8-byte stores, 13 for
 * 16-byte stores).  Returns -1
 * for a null array, a negative offset or an unknown mode. */
int32_t gemm_lds_access_cycles(const int64_t *lane_words, int32_t mode);

/* The LDS layout search the MFMA kernels are built with, for a workgroup tile
 * bm x bn x bk of (bm/wm) x (bn/wn) wavefronts, MFMA blocks mb x mb (32 or
 * 16) and global loads of `vec` floats (1 or 4) through registers, or, with
 * direct = 1 (vec must be 4), direct global->LDS copies: their LDS writes are
 * contiguous and cannot be padded, so only the fragment reads are costed and
 * only unpadded layouts are candidates.  direct = 2 is the pipelined kernels'
 * search (bk / (64 / mb) a multiple of 8): as 1, and only layouts whose
 * fragment addresses are a per-lane base plus compile-time offsets (A block
 * row i at base + i * mb rows, B step k at base + k rows) are candidates.  Writes {pad, swz_unit, swz_shift,
 * swz_mask} of A to out[0..3] and of B to out[4..7].  Returns GEMM_OK or
 * GEMM_ERR_INVALID_DIM. */
int gemm_lds_choose_mfma_layout(int32_t bm, int32_t bn, int32_t bk, int32_t wm, int32_t wn, int32_t mb,
                                int32_t vec, int32_t direct, int32_t *out);

/* The pages' padding rule for the A-tile column read ("My Triton From
 * Scratch, Part 18", section "Choosing padding instead of hard-coding it"):
 * distinct = banks / gcd(columns, banks); pad = simultaneous_rows > distinct.
 * Returns -1 on bad arguments. */
int32_t gemm_lds_page_pad(int32_t columns, int32_t simultaneous_rows, int32_t banks);

/* ---- 16-bit inputs, fp32 accumulation ---------------------------------------
 * The mixed-precision step that "My Triton From Scratch, Part 18: Shared
 * Memory Optimization" announces as its next part: C (fp32) = A @ B with A
 * and B in bf16 or fp16, products accumulated in fp32 on the matrix cores
 * (v_mfma_f32_32x32x16_bf16 / _f16).  A product of two 16-bit values is
 * exact in fp32, so C differs from the exact sum of products only by the fp32
 * accumulation.  Same tiling, masking and zero fill as the fp32 kernels. */
typedef enum {
    GEMM_INPUT_BF16 = 0,  /* bfloat16 bit patterns (8-bit exponent, 7-bit fraction) */
    GEMM_INPUT_F16 = 1    /* IEEE binary16 bit patterns */
} gemm_input_type;

typedef enum {
    GEMM_MIXED_AUTO = 0,          /* picks one of the below from M, N (gemm_mixed_auto_variant) */
    GEMM_MIXED_256x128 = 1,       /* 256x128x32 tile, 8 waves of 64x64, 4 waves per SIMD */
    GEMM_MIXED_256x256 = 2,       /* 256x256x32 tile, 8 waves of 128x64, 2 waves per SIMD */
    GEMM_MIXED_256x128_BK64 = 3,  /* 256x128x64 tile, 8 waves of 64x64 */
    GEMM_MIXED_128x128_BK64 = 4,  /* 128x128x64 tile, 4 waves of 64x64 */
    GEMM_MIXED_256x256_S3 = 5,    /* as 256x256 with three LDS stages (copies two tiles ahead) */
    GEMM_MIXED_256x256_BK64 = 6,  /* 256x256x64 tile, 8 waves of 128x64, two stages */
    GEMM_MIXED_64x64 = 7,         /* 64x64x64 tile, 4 waves of 32x32 (few output tiles) */
    GEMM_MIXED_64x64_KS2 = 8,     /* 64x64x64 tile, K split over 2 groups of 4 waves inside the workgroup */
    GEMM_MIXED_64x64_KS4 = 9,     /* 64x64x64 tile, K split over 4 groups of 4 waves */
    GEMM_MIXED_32x64_KS4 = 10,    /* 32x64x64 tile, K split over 4 groups of 2 waves */
    GEMM_MIXED_COUNT = 11
} gemm_mixed_variant;

/* C = A @ B, A and B of `input_type` (gemm_input_type), C fp32.  A, B, C are
 * DEVICE pointers owned by the caller; M, N, K >= 0; lda >= max(1,K),
 * ldb >= max(1,N), ldc >= max(1,N), in elements.  16-byte direct copies
 * need lda and ldb multiples of 8 and A, B 16-byte aligned; otherwise, with
 * lda and ldb even and A, B 4-byte aligned, the variant's kernel runs with
 * 4-byte copies (two elements per lane); otherwise the 256x128x32 kernel
 * runs with 2-byte loads through registers (the same result up to the order
 * of the fp32 additions).  Validation and
 * asynchrony as gemm_f32.  Returns a gemm_status; GEMM_ERR_UNSUPPORTED for an
 * unknown input type or variant. */
int gemm_mixed_f32(int input_type, int64_t M, int64_t N, int64_t K,
                   const void *A, int64_t lda,
                   const void *B, int64_t ldb,
                   float *C, int64_t ldc,
                   void *stream, int variant);

/* Tile geometry of a gemm_mixed_variant (elem_bytes = 2).  Pure host call. */
int gemm_mixed_tile_config(int variant, gemm_tile_config *out);

/* The variant GEMM_MIXED_AUTO runs.  e is the fraction of CU-rounds with
 * work for a tile, tiles / (ceil(tiles / per_round) * per_round), with
 * per_round = num_cus for 256x256, 64x64 and 32x64 tiles and 2 * num_cus
 * for 128x128; "big" is 256x256_BK64 when K is a multiple of 64, else
 * 256x256_S3 (with 16- or 4-byte copies alike).  When 256x256 tiles number at least num_cus / 2: 128x128_BK64
 * if 1050 * e128 > 1.1 * 1200 * e256, else big.  Otherwise the highest of
 * these estimates (listed first wins within 2 %): 64x64_KS4 420 * e64 and
 * 32x64_KS4 290 * e32x64, each when K >= 4096, or when its grid has at most
 * num_cus tiles and K >= 2048 (64x64) or K >= 1024 (32x64); 64x64_KS2
 * 530 * min(1, 0.6 w) when K >= 2048, or K >= 1024 with at most num_cus
 * 64x64 tiles; 64x64 700 * min(1, 0.375 w); 128x128_BK64 1050 * e128;
 * big 1.1 * 1200 * e256 (w: 64x64 tiles per CU).  Pure host call;
 * GEMM_ERR_INVALID_DIM for negative sizes or num_cus < 1. */
int gemm_mixed_auto_variant(int64_t M, int64_t N, int64_t K, int32_t num_cus);

#ifdef __cplusplus
}
#endif

#endif /* DENSE_FP32_TILED_H */
