/*
 * libskipln_tune -- the kernels of libskipln with their tuning, introspection
 * and bandwidth-probe entry points, for tests, sweeps and benchmarks.
 *
 * It is built from the same kernel objects as the operator library
 * (skipln.h); every result it computes is the same operator.  What it adds:
 * forcing a kernel family or a row-tile geometry, an explicit launch
 * configuration (tiling, tiles per block, output store policy), the kernel the
 * automatic choice takes for a call, the argument checks of every operation,
 * and two streaming kernels that measure the attainable HBM rates.  Memory,
 * ownership, streams and status codes as in skipln.h.
 */
#ifndef SKIPLN_TUNE_H
#define SKIPLN_TUNE_H

#include "skipln.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Kernel families, for skipln_tune_forward / skipln_tune_select.  The automatic
 * choice: row tiles up to 2048 chunks of 16 bytes per row, the LDS-staged
 * kernel for longer rows of the reducing operations, the register-resident
 * kernel for BiasSoftmax rows beyond it, then -- for calls that bring a
 * workspace (skipln_forward_ws) -- the split-row kernels, except for calls of
 * at least as many rows as the device has compute units (256 on MI355X) of
 * RMS, or of float32 layer norm up to 65536 values, which the generic kernel
 * runs faster without a workspace; rows that are not
 * whole chunks, or tensors not 16-byte aligned, take element-wise row tiles
 * up to 16384 values, and the generic kernel anything else. */
enum {
    SKIPLN_VARIANT_AUTO = 0,      /* what the operator library picks */
    SKIPLN_VARIANT_GENERIC = 1,   /* one workgroup per row, any hidden size and
                                     alignment: aligned rows of whole 16-byte
                                     chunks read twice with 16-byte accesses,
                                     others in three element-wise passes */
    SKIPLN_VARIANT_ROWTILE = 2,   /* row held in registers, 16-byte accesses:
                                     needs hidden*sizeof(T) % 16 == 0, 16-byte
                                     aligned pointers, hidden <= 4096*16/sizeof(T) */
    SKIPLN_VARIANT_MULTIWAVE = 3, /* ROWTILE with at least two wavefronts per
                                     row (exercises the cross-wave combine) */
    SKIPLN_VARIANT_LDSROW = 4,    /* long rows: one 1024-lane block per row, the
                                     row's binary32 values staged in LDS; layer
                                     norm, simplified and BiasSoftmax, 16-byte
                                     chunks, aligned pointers,
                                     hidden * 4 <= 163584 bytes */
    SKIPLN_VARIANT_SPLITROW = 5,  /* rows cut into slices of 16 KiB per tensor,
                                     one workgroup per slice, two kernels
                                     (partial results, then merge and
                                     normalize) through a workspace: layer norm,
                                     simplified and BiasSoftmax, 16-byte chunks,
                                     aligned pointers, at most 64 slices
                                     (262144 float32 / 524288 float16 values);
                                     with a workspace only; the residual may
                                     not alias input or skip (the automatic
                                     choice then takes the generic kernel) */
    SKIPLN_VARIANT_ELEMENT = 6,   /* row held in registers, one element per
                                     access: any hidden size up to 16384,
                                     tensors aligned to their element size
                                     (what the automatic choice takes for rows
                                     that are not whole 16-byte chunks) */
    SKIPLN_VARIANT_REGROW = 7,    /* long rows of BiasSoftmax: one 1024-lane
                                     block per row, the row's raw data in
                                     registers (up to 20 chunks per lane:
                                     163840 float16 / 81920 float32 values),
                                     z = data + bias formed again in each of
                                     two passes from the bias rows re-read
                                     through the caches; 16-byte chunks,
                                     aligned pointers; no workspace */
    SKIPLN_VARIANT_SPAN = 8,      /* span row tiles: a row of any length read
                                     as the aligned 16-byte chunks its bytes
                                     touch, elements of neighbouring rows
                                     masked; every tensor 16-byte aligned at
                                     its base; rows spanning up to 2048
                                     chunks (what the automatic choice takes
                                     for rows that are not whole 16-byte
                                     chunks) */
    SKIPLN_VARIANT_GEOMETRY = 64, /* + g: ROWTILE with row-tile geometry g,
                                     0 <= g < skipln_tune_rowtile_geometries(), for
                                     tests and tuning */
    SKIPLN_VARIANT_ELEMENT_GEOMETRY = 128, /* + g: ELEMENT with geometry g,
                                     0 <= g < skipln_tune_element_geometries() */
    SKIPLN_VARIANT_SPAN_GEOMETRY = 192 /* + g: SPAN with geometry g,
                                     0 <= g < skipln_tune_span_geometries() */
};

/* How the row-tile kernel distributes row tiles over workgroups (see
 * skipln_tune_forward_config). */
enum {
    SKIPLN_TILE_CONTIGUOUS = 0,     /* block b: tiles b*T .. b*T + T - 1 */
    SKIPLN_TILE_STRIDED = 1,        /* block b: tiles b, b + grid, b + 2*grid, ... */
    SKIPLN_TILE_SKIP_STATIONARY = 2 /* broadcast skip: block b keeps its skip rows
                                       in registers and walks T batches;
                                       otherwise as SKIPLN_TILE_STRIDED */
};

/* Output store policy of the row-tile and register-resident kernels:
 * automatic (system-scope for launches writing 512 MiB or more, measured
 * faster there), non-temporal, or non-temporal with system-scope coherence. */
enum { SKIPLN_STORE_AUTO = -1, SKIPLN_STORE_STREAM = 0, SKIPLN_STORE_THROUGH = 1 };

/* Operation `op` with the kernel family forced (SKIPLN_VARIANT_*;
 * SKIPLN_VARIANT_AUTO is the operator library's choice), with or without a
 * workspace (NULL / 0: none).  The arguments and the operation's rules are
 * those of skipln_forward_ws.  Returns SKIPLN_ERR_UNSUPPORTED when the family
 * cannot run the shape or alignment, SKIPLN_ERR_VARIANT for an unknown one. */
SKIPLN_API int skipln_tune_forward(int op, const void* input, const void* skip, int skip_mode, int64_t skip_rows,
                                   const void* gamma, const void* beta, const void* bias,
                                   void* out, void* residual_out, int64_t rows, int64_t hidden,
                                   float eps, int dtype, int variant, void* workspace, int64_t workspace_bytes,
                                   skipln_stream_t stream);

/* Operation `op` on the row tiles with an explicit launch configuration; the
 * result is the same operator.  geometry: row-tile geometry
 * (0 <= geometry < skipln_tune_rowtile_geometries()), -1 for the automatic
 * choice, or SKIPLN_VARIANT_ELEMENT_GEOMETRY + g for element-wise geometry g.
 * tiles_per_block (T) > 0: row tiles (batches, for
 * SKIPLN_TILE_SKIP_STATIONARY) per block; 0: the launcher's choice -- three
 * batches per block for SKIPLN_TILE_SKIP_STATIONARY, otherwise a grid of the
 * blocks the device holds at once (SKIPLN_TILE_CONTIGUOUS then behaves as
 * SKIPLN_TILE_STRIDED).  tiling: SKIPLN_TILE_*.  store: SKIPLN_STORE_*.
 * Returns SKIPLN_ERR_UNSUPPORTED when the geometry cannot hold the row or the
 * tensors are not 16-byte aligned, SKIPLN_ERR_SHAPE for tiles_per_block < 0,
 * SKIPLN_ERR_VARIANT for an unknown geometry, tiling or store policy. */
SKIPLN_API int skipln_tune_forward_config(int op, const void* input, const void* skip, int skip_mode,
                                          int64_t skip_rows, const void* gamma, const void* beta, const void* bias,
                                          void* out, void* residual_out, int64_t rows, int64_t hidden,
                                          float eps, int dtype, int geometry, int64_t tiles_per_block, int tiling,
                                          int store, skipln_stream_t stream);

/* Operation `op` on the row tiles, one row tile per block, in one of the two
 * kernel forms such launches can take: form 0 holds gamma, beta and bias in
 * registers from the start (the form whose blocks may walk several tiles);
 * form 1 loads gamma and beta only once the tile's sum is formed and has no
 * next-tile prefetch, so it needs far fewer registers, and a compute unit
 * holds at most `blocks_per_cu` of its blocks (0: as many as its registers
 * allow; -1: the operator library's table; the limit is set through the
 * launch's LDS).  geometry: row-tile geometry, or -1 for the automatic
 * choice.  store: SKIPLN_STORE_*.  The result is the same operator.
 * Returns SKIPLN_ERR_UNSUPPORTED when the geometry cannot hold the row or the
 * tensors are not 16-byte aligned, SKIPLN_ERR_VARIANT for an unknown
 * geometry, form, store policy, or blocks_per_cu < -1. */
SKIPLN_API int skipln_tune_forward_form(int op, const void* input, const void* skip, int skip_mode,
                                        int64_t skip_rows, const void* gamma, const void* beta, const void* bias,
                                        void* out, void* residual_out, int64_t rows, int64_t hidden,
                                        float eps, int dtype, int geometry, int form, int blocks_per_cu, int store,
                                        skipln_stream_t stream);

/* Blocks of row-tile geometry `geometry` (0 <= geometry <
 * skipln_tune_rowtile_geometries()) a compute unit of the current device holds
 * at once for operation `op` and `dtype`, in kernel form `form` (0 or 1, as
 * in skipln_tune_forward_form) with form 1 held to `blocks_per_cu` (0: no
 * limit; -1: the operator library's table) exactly as
 * skipln_tune_forward_form launches it: a count >= 1, or a negative status
 * code (SKIPLN_ERR_OP, SKIPLN_ERR_DTYPE, SKIPLN_ERR_VARIANT for an unknown
 * geometry or form or blocks_per_cu < -1, checked before any HIP call). */
SKIPLN_API int skipln_tune_blocks_per_cu(int op, int dtype, int geometry, int form, int blocks_per_cu);

/* Workspace bytes skipln_tune_forward needs for this variant (0: none), or a
 * negative status code.  Host code only. */
SKIPLN_API int64_t skipln_tune_workspace_bytes(int op, int64_t rows, int64_t hidden, int dtype, int skip_mode,
                                               int64_t skip_rows, int variant);

/* Kernel that skipln_tune_forward (variant) would launch for a call of
 * `rows` rows (< 0: fewer than the device's compute units) of `hidden`
 * values, with or without a workspace, on a device of `cus` compute units
 * (<= 0: the current device's, a HIP call; otherwise host code only): a
 * kernel id >= 0 (name via skipln_tune_kernel_name) or a negative status
 * code.  `aligned16` says whether every tensor pointer is 16-byte aligned. */
SKIPLN_API int skipln_tune_select(int op, int64_t rows, int64_t hidden, int dtype, int skip_mode, int aligned16,
                                  int variant, int with_workspace, int cus);

/* Stable name of a kernel id ("generic_f32", "rowtile_f16_g256_c4",
 * "rms_rowtile_f32_g192_c1_b192", "biasadd_generic_f16",
 * "softmax_rowtile_f16_g8_c1", ...); "unknown" for an invalid id. */
SKIPLN_API const char* skipln_tune_kernel_name(int kernel_id);

/* Number of row-tile geometries (SKIPLN_VARIANT_GEOMETRY + g), of
 * element-wise ones (SKIPLN_VARIANT_ELEMENT_GEOMETRY + g) and of span ones
 * (SKIPLN_VARIANT_SPAN_GEOMETRY + g). */
SKIPLN_API int skipln_tune_rowtile_geometries(void);
SKIPLN_API int skipln_tune_element_geometries(void);
SKIPLN_API int skipln_tune_span_geometries(void);

/* The argument checks of operation `op` (the rules of skipln_forward_ws):
 * host code only, no HIP call, no pointer dereferenced. */
SKIPLN_API int skipln_tune_validate(int op, const void* input, const void* skip, int skip_mode, int64_t skip_rows,
                                    const void* gamma, const void* beta, const void* bias,
                                    const void* out, const void* residual_out, int64_t rows, int64_t hidden,
                                    float eps, int dtype);

/* Streaming copy of `bytes` bytes from src to dst (device memory, 16-byte
 * aligned, bytes % 16 == 0, no overlap), with the access pattern of the
 * row-tile kernel's streamed input and outputs (16-byte non-temporal loads
 * and stores, persistent grid).
 * It is the reference for the bandwidth one kernel can reach on the device
 * and for calibrating hardware byte counters against a known byte count.
 * Returns SKIPLN_OK, SKIPLN_ERR_NULL, SKIPLN_ERR_SHAPE (bytes < 0 or not a
 * multiple of 16, misaligned pointers), SKIPLN_ERR_ALIAS or SKIPLN_ERR_LAUNCH. */
SKIPLN_API int skipln_tune_copy(void* dst, const void* src, int64_t bytes, skipln_stream_t stream);

/* Streaming probe with the access pattern of the row kernels (16-byte
 * non-temporal accesses, one tile of `block` lanes x `chunks_per_lane`
 * chunks per stream and workgroup; block 64, 256 or 1024, chunks_per_lane 1
 * or 4): reads 0-2 input streams (src0, then src1; NULL = not read) and
 * writes 0-2 output streams (dst0, then dst1) of `bytes` bytes each.  It
 * measures the HBM rate a kernel of that pattern attains for each mix of
 * reads and writes, the ceiling the row kernels are compared with.
 * xcd_granule (1 .. 65536): tiles in address order (1), or each XCD handed
 * xcd_granule consecutive tiles per round of 8 x xcd_granule (the dispatcher
 * deals workgroup b to XCD b mod 8): the address granularity at which the
 * eight XCDs share the streams, which for a row kernel is one row.
 * store_through: 0 = non-temporal stores; 1 = non-temporal stores with
 * system-scope coherence (the policy the row-tile kernels use for launches
 * that write 512 MiB or more, and the register-resident softmax for such
 * launches whose rows are whole 16 KiB slabs).
 * Outputs: dst0 = src0 XOR src1 (a chunk's index when nothing is read),
 * dst1 = dst0 + 1 per 32-bit word, whatever the tile order.  Device memory,
 * 16-byte aligned, bytes % 16 == 0, outputs overlapping nothing.  Returns
 * SKIPLN_OK, SKIPLN_ERR_NULL (no stream, or src1/dst1 without src0/dst0),
 * SKIPLN_ERR_SHAPE, SKIPLN_ERR_ALIAS, SKIPLN_ERR_VARIANT (tile shape or
 * granule) or SKIPLN_ERR_LAUNCH. */
SKIPLN_API int skipln_tune_stream(const void* src0, const void* src1, void* dst0, void* dst1, int64_t bytes, int block,
                  int chunks_per_lane, int64_t xcd_granule, int store_through, skipln_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SKIPLN_TUNE_H */
