// C ABI of the tuning library (include/skipln_tune.h): the operator's kernels
// with a forced kernel family or launch configuration, the kernel choice and
// kernel names, every operation's argument checks, and the bandwidth probes.
// Built from the same kernel objects and host logic as the operator library.
#include "../../include/skipln_tune.h"
#include "skipln_core.h"

static_assert(SKIPLN_TILE_CONTIGUOUS == skipln::kTileContiguous && SKIPLN_TILE_STRIDED == skipln::kTileStrided &&
                  SKIPLN_TILE_SKIP_STATIONARY == skipln::kTileSkipStationary,
              "tiling modes of the ABI and the kernels agree");
static_assert(SKIPLN_VARIANT_AUTO == skipln::core::kVariantAuto &&
                  SKIPLN_VARIANT_GENERIC == skipln::core::kVariantGeneric &&
                  SKIPLN_VARIANT_ROWTILE == skipln::core::kVariantRowtile &&
                  SKIPLN_VARIANT_MULTIWAVE == skipln::core::kVariantMultiwave &&
                  SKIPLN_VARIANT_LDSROW == skipln::core::kVariantLdsRow &&
                  SKIPLN_VARIANT_SPLITROW == skipln::core::kVariantSplitRow &&
                  SKIPLN_VARIANT_ELEMENT == skipln::core::kVariantElement &&
                  SKIPLN_VARIANT_REGROW == skipln::core::kVariantRegRow &&
                  SKIPLN_VARIANT_SPAN == skipln::core::kVariantSpan &&
                  SKIPLN_VARIANT_SPAN_GEOMETRY == skipln::core::kVariantSpanGeometry &&
                  SKIPLN_VARIANT_GEOMETRY == skipln::core::kVariantGeometry &&
                  SKIPLN_VARIANT_ELEMENT_GEOMETRY == skipln::core::kVariantElementGeometry,
              "kernel families of the ABI and the host logic agree");
static_assert(SKIPLN_STORE_AUTO == skipln::core::kStoreAuto && SKIPLN_STORE_STREAM == skipln::core::kStoreStream &&
                  SKIPLN_STORE_THROUGH == skipln::core::kStoreThrough,
              "store policies of the ABI and the host logic agree");

using skipln::core::make_call;
using skipln::core::run;
using skipln::core::status_of;
using skipln::core::Workspace;

namespace {

struct Range {
    uintptr_t lo, hi;
};

Range span(const void* p, int64_t bytes) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return Range{a, a + static_cast<uintptr_t>(bytes)};
}

bool overlap(const Range& a, const Range& b) { return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi; }

}  // namespace

extern "C" {

SKIPLN_API int skipln_tune_forward(int op, const void* input, const void* skip, int skip_mode, int64_t skip_rows,
                                   const void* gamma, const void* beta, const void* bias, void* out,
                                   void* residual_out, int64_t rows, int64_t hidden, float eps, int dtype, int variant,
                                   void* workspace, int64_t workspace_bytes, skipln_stream_t stream) {
    if (workspace_bytes < 0) return SKIPLN_ERR_WORKSPACE;
    const auto c = make_call(op, input, skip, skip_mode, skip_rows, gamma, beta, bias, out, residual_out, rows, hidden,
                             eps, dtype);
    if (workspace == nullptr) return run(c, variant, nullptr, stream);
    const Workspace ws{workspace, workspace_bytes};
    return run(c, variant, nullptr, stream, &ws);
}

SKIPLN_API int skipln_tune_forward_config(int op, const void* input, const void* skip, int skip_mode,
                                          int64_t skip_rows, const void* gamma, const void* beta, const void* bias,
                                          void* out, void* residual_out, int64_t rows, int64_t hidden, float eps,
                                          int dtype, int geometry, int64_t tiles_per_block, int tiling, int store,
                                          skipln_stream_t stream) {
    if (tiles_per_block < 0) return SKIPLN_ERR_SHAPE;
    if (tiling != SKIPLN_TILE_CONTIGUOUS && tiling != SKIPLN_TILE_STRIDED && tiling != SKIPLN_TILE_SKIP_STATIONARY)
        return SKIPLN_ERR_VARIANT;
    if (store != SKIPLN_STORE_AUTO && store != SKIPLN_STORE_STREAM && store != SKIPLN_STORE_THROUGH)
        return SKIPLN_ERR_VARIANT;
    const bool elem = geometry >= SKIPLN_VARIANT_ELEMENT_GEOMETRY;
    if (elem ? geometry >= SKIPLN_VARIANT_ELEMENT_GEOMETRY + skipln::elem_count()
             : (geometry < -1 || geometry >= skipln::rowtile_count()))
        return SKIPLN_ERR_VARIANT;
    skipln::Tiling t;
    t.tiles_per_block = tiles_per_block;
    t.mode = tiling;
    const int variant = elem ? geometry : geometry < 0 ? SKIPLN_VARIANT_ROWTILE : SKIPLN_VARIANT_GEOMETRY + geometry;
    return run(make_call(op, input, skip, skip_mode, skip_rows, gamma, beta, bias, out, residual_out, rows, hidden, eps,
                         dtype),
               variant, &t, stream, nullptr, store);
}

SKIPLN_API int skipln_tune_forward_form(int op, const void* input, const void* skip, int skip_mode, int64_t skip_rows,
                                        const void* gamma, const void* beta, const void* bias, void* out,
                                        void* residual_out, int64_t rows, int64_t hidden, float eps, int dtype,
                                        int geometry, int form, int blocks_per_cu, int store, skipln_stream_t stream) {
    if (form != skipln::kFormWalk && form != skipln::kFormOneTile) return SKIPLN_ERR_VARIANT;
    if (blocks_per_cu < skipln::kBlocksAuto) return SKIPLN_ERR_VARIANT;
    if (store != SKIPLN_STORE_AUTO && store != SKIPLN_STORE_STREAM && store != SKIPLN_STORE_THROUGH)
        return SKIPLN_ERR_VARIANT;
    if (geometry < -1 || geometry >= skipln::rowtile_count()) return SKIPLN_ERR_VARIANT;
    skipln::Tiling t;
    t.tiles_per_block = 1;
    t.mode = skipln::kTileStrided;
    t.form = form;
    t.blocks_per_cu = blocks_per_cu;
    const int variant = geometry < 0 ? SKIPLN_VARIANT_ROWTILE : SKIPLN_VARIANT_GEOMETRY + geometry;
    return run(make_call(op, input, skip, skip_mode, skip_rows, gamma, beta, bias, out, residual_out, rows, hidden, eps,
                         dtype),
               variant, &t, stream, nullptr, store);
}

SKIPLN_API int skipln_tune_blocks_per_cu(int op, int dtype, int geometry, int form, int blocks_per_cu) {
    if (!skipln::core::known_op(op)) return -SKIPLN_ERR_OP;
    if (dtype != SKIPLN_F32 && dtype != SKIPLN_F16) return -SKIPLN_ERR_DTYPE;
    if (geometry < 0 || geometry >= skipln::rowtile_count()) return -SKIPLN_ERR_VARIANT;
    if (form != skipln::kFormWalk && form != skipln::kFormOneTile) return -SKIPLN_ERR_VARIANT;
    if (blocks_per_cu < skipln::kBlocksAuto) return -SKIPLN_ERR_VARIANT;
    int occ = 0;
    const hipError_t e = skipln::rowtile_occupancy(op, dtype, geometry, form, blocks_per_cu, &occ);
    if (e != hipSuccess) return -status_of(e);
    return occ;
}

SKIPLN_API int64_t skipln_tune_workspace_bytes(int op, int64_t rows, int64_t hidden, int dtype, int skip_mode,
                                               int64_t skip_rows, int variant) {
    if (variant == SKIPLN_VARIANT_AUTO)
        return skipln::core::auto_workspace_bytes(op, rows, hidden, dtype, skip_mode, skip_rows);
    if (!skipln::core::known_op(op)) return -SKIPLN_ERR_OP;
    if (dtype != SKIPLN_F32 && dtype != SKIPLN_F16) return -SKIPLN_ERR_DTYPE;
    if (!skipln::core::mode_ok(op, skip_mode)) return -SKIPLN_ERR_MODE;
    if (rows < 0 || hidden <= 0 || hidden > INT32_MAX) return -SKIPLN_ERR_SHAPE;
    if (skip_mode != SKIPLN_SKIP_EXACT && (skip_rows <= 0 || rows % skip_rows != 0)) return -SKIPLN_ERR_SHAPE;
    const int id = skipln::core::select(op, hidden, dtype, skip_mode != SKIPLN_SKIP_EXACT, true, true, variant, true,
                                        -1, 0);
    if (id < 0) return id;
    if (rows == 0) return 0;
    const auto c = make_call(op, nullptr, nullptr, skip_mode, skip_rows, nullptr, nullptr, nullptr, nullptr, nullptr,
                             rows, hidden, 0.0f, dtype);
    return skipln::core::workspace_needed(c, id % skipln::kIdsPerType);
}

SKIPLN_API int skipln_tune_select(int op, int64_t rows, int64_t hidden, int dtype, int skip_mode, int aligned,
                                  int variant, int with_workspace, int cus) {
    if (!skipln::core::known_op(op)) return -SKIPLN_ERR_OP;
    if (dtype != SKIPLN_F32 && dtype != SKIPLN_F16) return -SKIPLN_ERR_DTYPE;
    if (!skipln::core::mode_ok(op, skip_mode)) return -SKIPLN_ERR_MODE;
    if (hidden <= 0 || hidden > INT32_MAX) return -SKIPLN_ERR_SHAPE;
    if (cus <= 0) {
        const hipError_t e = skipln::core::device_cus(&cus);
        if (e != hipSuccess) return -status_of(e);
    }
    return skipln::core::select(op, hidden, dtype, skip_mode != SKIPLN_SKIP_EXACT, aligned != 0, true, variant,
                                with_workspace != 0, rows, cus);
}

SKIPLN_API const char* skipln_tune_kernel_name(int kernel_id) { return skipln::kernel_name(kernel_id); }

SKIPLN_API int skipln_tune_rowtile_geometries(void) { return skipln::rowtile_count(); }

SKIPLN_API int skipln_tune_element_geometries(void) { return skipln::elem_count(); }

SKIPLN_API int skipln_tune_span_geometries(void) { return skipln::span_count(); }

SKIPLN_API int skipln_tune_validate(int op, const void* input, const void* skip, int skip_mode, int64_t skip_rows,
                                    const void* gamma, const void* beta, const void* bias, const void* out,
                                    const void* residual_out, int64_t rows, int64_t hidden, float eps, int dtype) {
    return skipln::core::validate(
        make_call(op, input, skip, skip_mode, skip_rows, gamma, beta, bias, out, residual_out, rows, hidden, eps, dtype));
}

SKIPLN_API int skipln_tune_copy(void* dst, const void* src, int64_t bytes, skipln_stream_t stream) {
    if (bytes < 0 || bytes % 16 != 0) return SKIPLN_ERR_SHAPE;
    if (bytes == 0) return SKIPLN_OK;
    if (!dst || !src) return SKIPLN_ERR_NULL;
    if (!skipln::core::aligned16(dst) || !skipln::core::aligned16(src)) return SKIPLN_ERR_SHAPE;
    if (overlap(span(dst, bytes), span(src, bytes))) return SKIPLN_ERR_ALIAS;
    return status_of(skipln::launch_copy(dst, src, bytes / 16, reinterpret_cast<hipStream_t>(stream)));
}

SKIPLN_API int skipln_tune_stream(const void* src0, const void* src1, void* dst0, void* dst1, int64_t bytes,
                                  int block, int chunks_per_lane, int64_t xcd_granule, int store_through,
                                  skipln_stream_t stream) {
    if (!skipln::stream_shape_ok(block, chunks_per_lane)) return SKIPLN_ERR_VARIANT;
    if (xcd_granule < 1 || xcd_granule > skipln::kMaxStreamGranule) return SKIPLN_ERR_VARIANT;
    if (bytes < 0 || bytes % 16 != 0) return SKIPLN_ERR_SHAPE;
    if (src1 && !src0) return SKIPLN_ERR_NULL;  // inputs fill src0 first
    if (dst1 && !dst0) return SKIPLN_ERR_NULL;  // outputs fill dst0 first
    const int reads = (src0 != nullptr) + (src1 != nullptr);
    const int writes = (dst0 != nullptr) + (dst1 != nullptr);
    if (reads + writes == 0) return SKIPLN_ERR_NULL;
    if (bytes == 0) return SKIPLN_OK;
    for (const void* p : {src0, src1, static_cast<const void*>(dst0), static_cast<const void*>(dst1)})
        if (p && !skipln::core::aligned16(p)) return SKIPLN_ERR_SHAPE;
    const Range r[4] = {span(src0, src0 ? bytes : 0), span(src1, src1 ? bytes : 0), span(dst0, dst0 ? bytes : 0),
                        span(dst1, dst1 ? bytes : 0)};
    for (int o = 2; o < 4; ++o)
        for (int i = 0; i < 4; ++i)
            if (i != o && overlap(r[o], r[i])) return SKIPLN_ERR_ALIAS;
    return status_of(skipln::launch_stream(reads, writes, block, chunks_per_lane, xcd_granule, store_through != 0, src0,
                                           src1, dst0, dst1, bytes / 16, reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"
