// C ABI of libskipln: argument checks, kernel choice and launch.
//
// The checks follow the contracts of the com.microsoft SkipLayerNormalization
// WebGPU manifest (`derive`): epsilon must be non-negative (`epsilonOk`), the
// hidden size positive and gamma/beta/bias of length H (`rank2CoreContract`,
// `betaContract`), all tensors of one element type (`f32MainDtypes`,
// `f16MainDtypes`), a broadcast skip (S, H) read cyclically by the (N*S) rows
// (`broadcastSkipShapeOk`, `Params.skipRows`).  Aliasing rules are this
// library's own: an output may only coincide exactly with a tensor that is
// read row by row by the lane group that later writes the same row.
#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include <cmath>

#include "../../include/skipln.h"
#include "skipln_internal.h"

static_assert(SKIPLN_TILE_CONTIGUOUS == skipln::kTileContiguous && SKIPLN_TILE_STRIDED == skipln::kTileStrided &&
                  SKIPLN_TILE_SKIP_STATIONARY == skipln::kTileSkipStationary,
              "tiling modes of the ABI and the kernels agree");

namespace {

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
    bool empty() const { return hi <= lo; }
};

Range span(const void* p, int64_t bytes) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return Range{a, a + static_cast<uintptr_t>(bytes)};
}

bool overlap(const Range& a, const Range& b) {
    return !a.empty() && !b.empty() && a.lo < b.hi && b.lo < a.hi;
}

bool same(const Range& a, const Range& b) { return a.lo == b.lo && a.hi == b.hi; }

int elem_size(int dtype) { return dtype == SKIPLN_F32 ? 4 : 2; }

int validate(const void* input, const void* skip, int skip_mode, int64_t skip_rows, const void* gamma,
             const void* beta, const void* bias, const void* out, const void* residual_out, int64_t rows,
             int64_t hidden, float eps, int dtype) {
    if (dtype != SKIPLN_F32 && dtype != SKIPLN_F16) return SKIPLN_ERR_DTYPE;
    if (skip_mode != SKIPLN_SKIP_EXACT && skip_mode != SKIPLN_SKIP_BROADCAST) return SKIPLN_ERR_MODE;
    if (!(eps >= 0.0f)) return SKIPLN_ERR_EPS;  // also rejects NaN
    if (rows < 0 || hidden <= 0 || hidden > INT32_MAX) return SKIPLN_ERR_SHAPE;
    const int64_t sz = elem_size(dtype);
    if (rows > INT64_MAX / hidden / sz) return SKIPLN_ERR_SHAPE;
    if (skip_mode == SKIPLN_SKIP_BROADCAST) {
        if (skip_rows <= 0 || rows % skip_rows != 0) return SKIPLN_ERR_SHAPE;
    }
    if (rows == 0) return SKIPLN_OK;
    if (!input || !skip || !gamma || !out) return SKIPLN_ERR_NULL;

    const bool bcast = skip_mode == SKIPLN_SKIP_BROADCAST;
    const int64_t row_bytes = hidden * sz;
    const Range r_in = span(input, rows * row_bytes);
    const Range r_skip = span(skip, (bcast ? skip_rows : rows) * row_bytes);
    const Range r_gamma = span(gamma, row_bytes);
    const Range r_beta = span(beta, beta ? row_bytes : 0);
    const Range r_bias = span(bias, bias ? row_bytes : 0);
    const Range r_out = span(out, rows * row_bytes);
    const Range r_res = span(residual_out, residual_out ? rows * row_bytes : 0);

    for (const Range& o : {r_out, r_res}) {
        if (o.empty()) continue;
        if (overlap(o, r_in) && !same(o, r_in)) return SKIPLN_ERR_ALIAS;
        if (overlap(o, r_skip) && (bcast || !same(o, r_skip))) return SKIPLN_ERR_ALIAS;
        if (overlap(o, r_gamma) || overlap(o, r_beta) || overlap(o, r_bias)) return SKIPLN_ERR_ALIAS;
    }
    if (overlap(r_out, r_res)) return SKIPLN_ERR_ALIAS;
    return SKIPLN_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Kernel id (>= 0) for this variant, or -status.
int select(int64_t hidden, int dtype, bool broadcast, bool vec_ok, int variant) {
    const int base = dtype * skipln::kIdsPerType;
    const int v = dtype == SKIPLN_F32 ? 4 : 8;  // elements per 16-byte chunk
    const bool chunked = vec_ok && hidden % v == 0;
    if (variant == SKIPLN_VARIANT_GENERIC) return base + skipln::kGenericIndex;
    if (variant == SKIPLN_VARIANT_AUTO || variant == SKIPLN_VARIANT_ROWTILE ||
        variant == SKIPLN_VARIANT_MULTIWAVE) {
        const int g =
            chunked ? skipln::rowtile_pick(hidden, dtype, broadcast, variant == SKIPLN_VARIANT_MULTIWAVE) : -1;
        if (g >= 0) return base + skipln::kRowtileFirst + g;
        if (variant == SKIPLN_VARIANT_AUTO) return base + skipln::kGenericIndex;
        return -SKIPLN_ERR_UNSUPPORTED;
    }
    if (variant >= SKIPLN_VARIANT_GEOMETRY && variant < SKIPLN_VARIANT_GEOMETRY + skipln::rowtile_count()) {
        const int g = variant - SKIPLN_VARIANT_GEOMETRY;
        // The geometry must hold the whole row.
        if (!chunked || !skipln::rowtile_holds(g, hidden, dtype)) return -SKIPLN_ERR_UNSUPPORTED;
        return base + skipln::kRowtileFirst + g;
    }
    return -SKIPLN_ERR_VARIANT;
}

bool all_aligned16(const void* input, const void* skip, const void* gamma, const void* beta, const void* bias,
                   const void* out, const void* residual_out) {
    return aligned16(input) && aligned16(skip) && aligned16(gamma) && aligned16(beta) && aligned16(bias) &&
           aligned16(out) && aligned16(residual_out);
}

// Tiling of the automatic launch.  Streaming rows (exact skip): one tile per
// block, so blocks are dispatched in address order and the set of rows in
// flight stays compact; this reached the 2-read/2-write streaming rate on
// MI355X.  A broadcast skip is shared by every batch: each block keeps its
// skip rows (and gamma/beta) in registers and walks the batches.
skipln::Tiling auto_tiling(bool broadcast) {
    skipln::Tiling t;
    t.tiles_per_block = broadcast ? 0 : 1;
    t.mode = broadcast ? skipln::kTileSkipStationary : skipln::kTileStrided;
    return t;
}

skipln::Args make_args(const void* input, const void* skip, int skip_mode, int64_t skip_rows, const void* gamma,
                       const void* beta, const void* bias, void* out, void* residual_out, int64_t rows,
                       int64_t hidden, float eps) {
    skipln::Args a;
    a.input = input;
    a.skip = skip;
    a.gamma = gamma;
    a.beta = beta;
    a.bias = bias;
    a.out = out;
    a.residual = residual_out;
    a.rows = rows;
    a.skip_rows = skip_mode == SKIPLN_SKIP_BROADCAST ? skip_rows : 0;
    a.hidden = static_cast<int32_t>(hidden);
    a.eps = eps;
    a.tiles_per_block = 1;
    a.tiling = skipln::kTileStrided;
    return a;
}

int status_of(hipError_t e) {
    if (e == hipSuccess) return SKIPLN_OK;
    if (e == hipErrorInvalidDevice || e == hipErrorNoDevice) return SKIPLN_ERR_DEVICE;
    return SKIPLN_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int skipln_validate(const void* input, const void* skip, int skip_mode, int64_t skip_rows, const void* gamma,
                    const void* beta, const void* bias, const void* out, const void* residual_out, int64_t rows,
                    int64_t hidden, float eps, int dtype) {
    return validate(input, skip, skip_mode, skip_rows, gamma, beta, bias, out, residual_out, rows, hidden, eps,
                    dtype);
}

int skipln_select(int64_t hidden, int dtype, int skip_mode, int aligned, int variant) {
    if (dtype != SKIPLN_F32 && dtype != SKIPLN_F16) return -SKIPLN_ERR_DTYPE;
    if (skip_mode != SKIPLN_SKIP_EXACT && skip_mode != SKIPLN_SKIP_BROADCAST) return -SKIPLN_ERR_MODE;
    if (hidden <= 0 || hidden > INT32_MAX) return -SKIPLN_ERR_SHAPE;
    return select(hidden, dtype, skip_mode == SKIPLN_SKIP_BROADCAST, aligned != 0, variant);
}

int skipln_forward_variant(const void* input, const void* skip, int skip_mode, int64_t skip_rows,
                           const void* gamma, const void* beta, const void* bias, void* out, void* residual_out,
                           int64_t rows, int64_t hidden, float eps, int dtype, int variant,
                           skipln_stream_t stream) {
    int st = validate(input, skip, skip_mode, skip_rows, gamma, beta, bias, out, residual_out, rows, hidden, eps,
                      dtype);
    if (st != SKIPLN_OK) return st;
    const bool vec_ok = all_aligned16(input, skip, gamma, beta, bias, out, residual_out);
    const int id = skipln_select(hidden, dtype, skip_mode, vec_ok ? 1 : 0, variant);
    if (id < 0) return -id;
    if (rows == 0) return SKIPLN_OK;

    const skipln::Args a = make_args(input, skip, skip_mode, skip_rows, gamma, beta, bias, out, residual_out, rows,
                                     hidden, eps);
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const int index = id % skipln::kIdsPerType;
    if (index == skipln::kGenericIndex) return status_of(skipln::launch_generic(a, dtype, s));
    return status_of(skipln::launch_rowtile(a, dtype, index - skipln::kRowtileFirst,
                                            auto_tiling(skip_mode == SKIPLN_SKIP_BROADCAST), s));
}

int skipln_forward_config(const void* input, const void* skip, int skip_mode, int64_t skip_rows,
                          const void* gamma, const void* beta, const void* bias, void* out, void* residual_out,
                          int64_t rows, int64_t hidden, float eps, int dtype, int geometry, int64_t tiles_per_block,
                          int tiling, skipln_stream_t stream) {
    int st = validate(input, skip, skip_mode, skip_rows, gamma, beta, bias, out, residual_out, rows, hidden, eps,
                      dtype);
    if (st != SKIPLN_OK) return st;
    if (tiles_per_block < 0) return SKIPLN_ERR_SHAPE;
    if (tiling != SKIPLN_TILE_CONTIGUOUS && tiling != SKIPLN_TILE_STRIDED && tiling != SKIPLN_TILE_SKIP_STATIONARY)
        return SKIPLN_ERR_VARIANT;
    const bool vec_ok = all_aligned16(input, skip, gamma, beta, bias, out, residual_out);
    if (geometry < -1 || geometry >= skipln::rowtile_count()) return SKIPLN_ERR_VARIANT;
    const int variant = geometry < 0 ? SKIPLN_VARIANT_ROWTILE : SKIPLN_VARIANT_GEOMETRY + geometry;
    const int id = skipln_select(hidden, dtype, skip_mode, vec_ok ? 1 : 0, variant);
    if (id < 0) return -id;
    if (rows == 0) return SKIPLN_OK;
    const skipln::Args a = make_args(input, skip, skip_mode, skip_rows, gamma, beta, bias, out, residual_out, rows,
                                     hidden, eps);
    skipln::Tiling t;
    t.tiles_per_block = tiles_per_block;
    t.mode = tiling;
    return status_of(skipln::launch_rowtile(a, dtype, id % skipln::kIdsPerType - skipln::kRowtileFirst, t,
                                            reinterpret_cast<hipStream_t>(stream)));
}

int skipln_forward(const void* input, const void* skip, int skip_mode, int64_t skip_rows, const void* gamma,
                   const void* beta, const void* bias, void* out, void* residual_out, int64_t rows, int64_t hidden,
                   float eps, int dtype, skipln_stream_t stream) {
    return skipln_forward_variant(input, skip, skip_mode, skip_rows, gamma, beta, bias, out, residual_out, rows,
                                  hidden, eps, dtype, SKIPLN_VARIANT_AUTO, stream);
}

int skipln_copy(void* dst, const void* src, int64_t bytes, skipln_stream_t stream) {
    if (bytes < 0 || bytes % 16 != 0) return SKIPLN_ERR_SHAPE;
    if (bytes == 0) return SKIPLN_OK;
    if (!dst || !src) return SKIPLN_ERR_NULL;
    if (!aligned16(dst) || !aligned16(src)) return SKIPLN_ERR_SHAPE;
    if (overlap(span(dst, bytes), span(src, bytes))) return SKIPLN_ERR_ALIAS;
    return status_of(skipln::launch_copy(dst, src, bytes / 16, reinterpret_cast<hipStream_t>(stream)));
}

int skipln_rowtile_geometries(void) { return skipln::rowtile_count(); }

const char* skipln_kernel_name(int kernel_id) { return skipln::kernel_name(kernel_id); }

const char* skipln_status_string(int status) {
    switch (status) {
        case SKIPLN_OK: return "ok";
        case SKIPLN_ERR_NULL: return "a required pointer is NULL";
        case SKIPLN_ERR_SHAPE: return "invalid shape (rows, hidden or skip_rows)";
        case SKIPLN_ERR_DTYPE: return "unsupported element type";
        case SKIPLN_ERR_MODE: return "unknown skip mode";
        case SKIPLN_ERR_EPS: return "epsilon must be a non-negative number";
        case SKIPLN_ERR_ALIAS: return "an output overlaps an input or the other output";
        case SKIPLN_ERR_UNSUPPORTED: return "the forced kernel family cannot run this shape or alignment";
        case SKIPLN_ERR_LAUNCH: return "kernel launch failed";
        case SKIPLN_ERR_DEVICE: return "no usable HIP device";
        case SKIPLN_ERR_VARIANT: return "unknown variant";
        default: return "unknown status";
    }
}

int skipln_version(void) { return 1; }

}  // extern "C"
