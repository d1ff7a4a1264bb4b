/*
 * lds_probe.h -- microbenchmark of the gfx950 LDS bank geometry.
 *
 * The pages model shared memory as 32 four-byte banks serviced one warp at a
 * time ("My Triton From Scratch, Part 18: Shared Memory Optimization",
 * section "Why shared-memory banks matter"), which is NVIDIA's geometry.  The
 * LDS padding of the GEMM kernels is derived from a bank count and from how
 * many lanes the LDS services together per access width; this probe measures
 * those on the device by timing one access pattern: every lane of `waves`
 * wavefronts (one workgroup) issues `reps` x 16 LDS reads of `width_words`
 * dwords at its own dword address, with no other work, and the time per
 * instruction is returned.  Conflicting patterns take proportionally longer.
 */
#ifndef LDS_PROBE_H
#define LDS_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Largest dword address + width a pattern may touch (a 64 KiB LDS buffer). */
#define LDS_PROBE_WORDS 16384

/*
 * lane_words: HOST array of 64 dword addresses, one per lane (the same
 *             pattern is used by every wavefront).
 * width_words: 1, 2 or 4 (ds_read_b32 / b64 / b128; every address must be a
 *             multiple of width_words and address + width_words <=
 *             LDS_PROBE_WORDS), or -16 / -32: ds_read2_b32 reading the dwords
 *             at address and address + 16 (or 32); address + 17 (or 33) <=
 *             LDS_PROBE_WORDS; or 101, 102, 104: ds_write_b32 / b64 / b128 of
 *             1, 2 or 4 dwords, with the alignment and bound of the read of
 *             the same width.
 * waves: 1..16 wavefronts in the workgroup.  reps: 1..100000.
 * cycles_out: DEVICE buffer of `waves` uint64 values, owned by the caller;
 *             wave w writes the shader-clock cycles its read loop took.
 * stream: hipStream_t (NULL = null stream).
 * Returns 0, -1 for invalid arguments (nothing is launched), -2 if the
 * launch failed.  Asynchronous: read cycles_out after synchronising.
 */
int lds_probe_run(const int32_t *lane_words, int32_t width_words, int32_t waves, int32_t reps,
                  uint64_t *cycles_out, void *stream);

/*
 * XCD (accelerator complex die) each workgroup of a 1-D launch runs on:
 * launches `blocks` workgroups of `threads` threads; workgroup b writes its
 * XCC_ID hardware register to out[b].  out: DEVICE buffer of `blocks` int32,
 * owned by the caller.  Returns 0, -1 for invalid arguments, -2 if the launch
 * failed.
 */
int probe_xcc_ids(int32_t *out, int32_t blocks, int32_t threads, void *stream);

/*
 * Throughput of the direct global->LDS copy (global_load_lds_dword for
 * bytes_per_lane 4, _dwordx4 for 16), as the GEMM kernels use it to fill
 * their LDS tiles: `blocks` workgroups of `waves` wavefronts; every wave
 * issues reps x 16 copies into an LDS piece of its own, waiting for them
 * after each 16, and writes the shader-clock cycles its loop took to
 * cycles_out[block * waves + wave] (DEVICE buffer of blocks * waves uint64,
 * owned by the caller).  Lane l of wave w of workgroup b reads
 * src + off0 + (b * waves + w) * wave_stride + (l / row_lanes) * ld_bytes
 * + (l % row_lanes) * bytes_per_lane: row_lanes lanes per row, rows ld_bytes
 * apart, like the copy of one piece of a tile of a matrix with that pitch.
 * src: DEVICE buffer of src_bytes bytes, owned by the caller; every byte read
 * must lie inside it (checked), src + off0 aligned to bytes_per_lane,
 * wave_stride a multiple of it, ld_bytes a multiple of 4 (16 for 16-byte
 * copies).  blocks 1..4096, waves 1..16, reps 1..100000, row_lanes a
 * divisor of 64.  Returns 0, -1 for invalid arguments (nothing is
 * launched), -2 if the launch failed.  Asynchronous.
 */
int probe_dma_throughput(const void *src, int64_t src_bytes, int32_t bytes_per_lane, int32_t blocks,
                         int32_t waves, int32_t reps, int64_t off0, int64_t wave_stride, int64_t ld_bytes,
                         int32_t row_lanes, uint64_t *cycles_out, void *stream);

/*
 * Throughput of the vector ALU's fp32 fused multiply-add in its one-product
 * form (v_fmac_f32; the library is built without packed fp32): `blocks`
 * workgroups of `waves` wavefronts; every lane runs reps x 64 FMAs over 8
 * independent accumulators with no memory access, and each wave writes the
 * shader-clock cycles of its loop to cycles_out[block * waves + wave]
 * (DEVICE buffer of blocks * waves uint64, owned by the caller).  blocks
 * 1..4096, waves 1..16, reps 1..1000000.  Returns 0, -1 for invalid
 * arguments (nothing is launched), -2 if the launch failed.  Asynchronous.
 */
int probe_valu_fma(int32_t blocks, int32_t waves, int32_t reps, uint64_t *cycles_out, void *stream);

/*
 * Throughput of the matrix pipe on v_mfma_f32_32x32x2_f32 (2*32*32*2 = 4096
 * flops per wave instruction) with register operands: `blocks` workgroups of
 * `waves` wavefronts; every wave runs reps x 16 MFMAs over 4 independent
 * accumulators with no memory access, and writes the shader-clock cycles of
 * its loop to cycles_out[block * waves + wave] (DEVICE buffer of
 * blocks * waves uint64, owned by the caller).  acc_agpr = 1 keeps the
 * accumulators in AGPRs, 0 in VGPRs.  blocks 1..4096, waves 1..16, reps
 * 1..1000000.  Returns 0, -1 for invalid arguments (nothing is launched),
 * -2 if the launch failed.  Asynchronous.
 */
int probe_mfma_f32(int32_t blocks, int32_t waves, int32_t reps, int32_t acc_agpr, uint64_t *cycles_out,
                   void *stream);

/*
 * Reference kernel for calibrating the HBM traffic counters: dst[i] = src[i]
 * for i < n, 16-byte loads and stores, grid-stride.  It reads and writes
 * exactly 4*n bytes.  src and dst are DEVICE pointers owned by the caller,
 * 16-byte aligned and not overlapping; n >= 0 and a multiple of 4.  Returns
 * 0, -1 for invalid arguments (nothing is launched), -2 if the launch failed.
 */
int probe_copy_f32(const float *src, float *dst, int64_t n, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LDS_PROBE_H */
