// Internal interface between the C-ABI layer (skipln_api.cpp) and the HIP
// kernels (skipln_kernels.hip).  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace skipln {

// Arguments of one SkipLayerNormalization launch, already validated.
struct Args {
    const void* input;
    const void* skip;
    const void* gamma;
    const void* beta;  // nullptr: no shift
    const void* bias;  // nullptr: no bias
    void* out;
    void* residual;    // nullptr: residual not written
    int64_t rows;
    int64_t skip_rows; // > 0: row r reads skip row r % skip_rows (cyclic)
    int64_t skip_group;// > 0: row r reads skip row r / skip_group (grouped);
                       // both 0: exact skip (row r reads skip row r)
    int32_t hidden;
    float eps;
    // Row-tile kernels: tiles (RPB rows each) per block and how a block
    // walks them (kTile*).  Set by the launcher.
    int64_t tiles_per_block;
    int32_t tiling;
    // Row-tile and register-resident kernels: write outputs with the
    // system-scope store policy (set for launches writing at least
    // kStoreThroughBytes of rows of whole 128-byte lines, where it was
    // measured faster).
    int32_t store_through;
};

constexpr int64_t kStoreThroughBytes = int64_t(512) << 20;

// Tiling modes of the row-tile kernel (values of Args::tiling and of the
// C ABI's tiling argument).
constexpr int kTileContiguous = 0;      // block b: tiles b*T .. b*T + T - 1
constexpr int kTileStrided = 1;         // block b: tiles b, b + grid, ...
constexpr int kTileSkipStationary = 2;  // broadcast skip: fixed skip rows per block

// Kernel forms of the row tiles: blocks that may walk several tiles (the
// next tile's loads issued while the current one finishes; parameters held
// in registers throughout), blocks of exactly one tile (no prefetch, gamma
// and beta loaded once the sum is formed: far fewer registers), and the
// latter with a streamed first skip tile (small launches).
constexpr int kFormAuto = -1;
constexpr int kFormWalk = 0;
constexpr int kFormOneTile = 1;
constexpr int kFormStreamSkip = 2;
// Blocks per compute unit of a single-tile launch: the launcher's table.
constexpr int kBlocksAuto = -1;

// Launches that favour the single-tile form (the row-tile launcher's table)
// and, for the longest rows, 1024-lane row tiles in that form: the input
// (and so skip and output) spans at least kLargeLaunchStreamBytes (2 GiB
// moved with the residual, eight times the 256 MiB last-level cache) and
// every row is whole 128-byte cache lines.  Rows that end inside a line
// share it with the next row, which another block writes; there the
// single-tile form measured 4-20 % slower than the walking form or the
// LDS-staged kernel (2 GiB launches: float16 rows of 2056 values 555 against
// 502 us, float32 rows of 1028 values 531 against 511, float16 rows of 22600
// values 560 against 467 on the LDS kernel).
constexpr int64_t kLargeLaunchStreamBytes = int64_t(512) << 20;
inline bool single_tile_launch(int64_t rows, int64_t hidden, int elem_bytes) {
    if (rows <= 0 || hidden <= 0) return false;
    const int64_t row_bytes = hidden * elem_bytes;
    return row_bytes % 128 == 0 && rows >= (kLargeLaunchStreamBytes + row_bytes - 1) / row_bytes;
}

// How a row-tile launch distributes tiles over blocks.
struct Tiling {
    int64_t tiles_per_block;  // 0: the launcher's choice (skip-stationary:
                              // 3 batches per block; otherwise a grid of the
                              // blocks the device holds at once)
    int mode;                 // kTile*
    // Launches of one tile per block (not skip-stationary): the kernel form
    // (kFormAuto: the launcher's table) and, for kFormOneTile, the blocks a
    // compute unit may hold (kBlocksAuto: the table's; 0: as many as the
    // kernel's registers allow).
    int form = kFormAuto;
    int blocks_per_cu = kBlocksAuto;
};

// Operations sharing the row kernels.
constexpr int kOpLayerNorm = 0;   // SkipLayerNormalization
constexpr int kOpSimplified = 1;  // its root-mean-square ("simplified") form
constexpr int kOpBiasAdd = 2;     // BiasAdd: (x + bias) + skip, no normalization
constexpr int kOpBiasSoftmax = 3; // BiasSoftmax: softmax over the row of x + skip
constexpr int kNumOps = 4;

// Kernel ids: (op * 2 + dtype) * kIdsPerType + index, index 0 = generic,
// kRowtileFirst.. = row tiles of 16-byte chunks, kElemFirst.. = row tiles of
// single elements, kRegRowIndex = the register-resident long-row softmax,
// kSplitRowIndex = the split-row kernel pair, kLdsRowIndex = the LDS-staged
// long-row kernel, kSpanFirst.. = span row tiles (rows that are not whole
// chunks, read as aligned 16-byte chunks).
constexpr int kIdsPerType = 128;
constexpr int kGenericIndex = 0;
constexpr int kRowtileFirst = 1;
constexpr int kElemFirst = 64;
constexpr int kSpanFirst = 96;
constexpr int kRegRowIndex = 125;
constexpr int kSplitRowIndex = 126;
constexpr int kLdsRowIndex = 127;

// LDS a block may use on gfx950 (160 KiB), less room for the reduction
// scratch: the long-row kernel holds hidden * 4 bytes.
constexpr int64_t kLdsRowBytes = 163840 - 256;
// Row-tile geometries hold at most this many 16-byte chunks efficiently;
// longer rows go to the long-row kernel (1024-lane row tiles spill).
constexpr int64_t kRowtileMaxAutoChunks = 2048;

// Number of row-tile geometries and the one chosen for operation `op`,
// `hidden` (elements) and the skip form, or -1 when none holds the row.
// multiwave_only: the smallest geometry whose row group spans two or more
// wavefronts.  rows: the launch's row count (< 0: not known), which decides
// where launches of the single-tile form take other geometries.
int rowtile_count();
int rowtile_pick(int op, int64_t hidden, int dtype, bool broadcast, bool multiwave_only, int64_t rows = -1);
// Whether geometry g holds a row of `hidden` elements (16-byte chunks).
bool rowtile_holds(int geometry, int64_t hidden, int dtype);
// The same for the element-wise row tiles (rows of any length, tensors
// aligned to their element size only): number of geometries, the automatic
// choice (or -1: none holds the row), and whether geometry g holds it.
int elem_count();
int elem_pick(int op, int64_t hidden);
bool elem_holds(int geometry, int64_t hidden);
// Tiling of an automatic element-wise launch with geometry g.
Tiling elem_tiling(int geometry);
const char* kernel_name(int kernel_id);

// Enqueue one kernel; return 0 or a hipError_t value.
hipError_t launch_generic(const Args& a, int op, int dtype, hipStream_t stream);
hipError_t launch_ldsrow(const Args& a, int op, int dtype, hipStream_t stream);
// Whether the long-row kernel runs this operation and row (16-byte chunks,
// row of binary32 values within kLdsRowBytes).
bool ldsrow_holds(int op, int64_t hidden, int dtype);
// Register-resident long rows (BiasSoftmax): whether the kernel holds the row
// (16-byte chunks, at most 16 per lane of a 1024-lane block), and the launch.
bool regrow_holds(int op, int64_t hidden, int dtype);
hipError_t launch_regrow(const Args& a, int op, int dtype, hipStream_t stream);
hipError_t launch_rowtile(const Args& a, int op, int dtype, int geometry, Tiling tiling, hipStream_t stream);
hipError_t launch_elem(const Args& a, int op, int dtype, int geometry, Tiling tiling, hipStream_t stream);
// One operation's row tiles (chunks / elements), instantiated per operation
// in its own translation unit.
template <int OP>
hipError_t launch_rowtile_for(const Args& a, int dtype, int geometry, Tiling tiling, hipStream_t stream);
template <int OP>
hipError_t launch_elem_for(const Args& a, int dtype, int geometry, Tiling tiling, hipStream_t stream);
// Blocks of row-tile geometry g's kernel a compute unit holds at once, in
// kernel form kFormWalk or kFormOneTile (held to blocks_per_cu as a launch of
// that form is; kBlocksAuto: the launcher's table).
hipError_t rowtile_occupancy(int op, int dtype, int geometry, int form, int blocks_per_cu, int* out);
template <int OP>
hipError_t rowtile_occupancy_for(int dtype, int geometry, int form, int blocks_per_cu, int* out);
// Split-row kernels (rows cut into slices of 1024 chunks, one workgroup per
// slice, partials through a caller-provided workspace): whether they run
// this operation and row (16-byte chunks, at most 64 slices), the workspace
// bytes a launch needs, and the launch (workspace 16-byte aligned).
bool split_holds(int op, int64_t hidden, int dtype);
int64_t split_workspace_bytes(const Args& a, int dtype);
hipError_t launch_split(const Args& a, int op, int dtype, void* workspace, hipStream_t stream);
// Register-resident long rows of the normalizations (layer norm and its
// root-mean-square form): whether the kernel holds this row, and its launch.
bool regnorm_holds(int op, int64_t hidden, int dtype);
hipError_t launch_regnorm(const Args& a, int op, int dtype, hipStream_t stream);
// Span row tiles (rows of any length, every tensor 16-byte aligned): the
// number of geometries, geometry g's group, chunks per lane and block,
// whether it holds a row of `hidden` values, the geometry a forced span
// launch takes for the operation (the first in its order that holds the row,
// or -1), the automatic choice (or -1: another family), and the launch (one
// row per group, one tile of rows per block).
int span_count();
bool span_geometry(int geometry, int* g, int* ch, int* block);
bool span_holds(int geometry, int64_t hidden, int dtype);
int span_fit(int op, int64_t hidden, int dtype);
int span_pick(int op, int64_t hidden, int dtype, bool broadcast);
hipError_t launch_span(const Args& a, int op, int dtype, int geometry, hipStream_t stream);
hipError_t launch_copy(void* dst, const void* src, int64_t chunks, hipStream_t stream);
// Streaming probe: `reads` (0-2) input streams s0, s1 to `writes` (0-2)
// output streams d0, d1 of `chunks` 16-byte chunks each, in tiles of `block`
// lanes x `per_lane` chunks (shapes stream_shape_ok accepts), `granule`
// consecutive tiles per XCD (1 = address order), stores with the
// system-scope policy when `through` is set.
bool stream_shape_ok(int block, int per_lane);
constexpr int64_t kMaxStreamGranule = 1 << 16;
hipError_t launch_stream(int reads, int writes, int block, int per_lane, int64_t granule, int through,
                         const void* s0, const void* s1, void* d0, void* d1, int64_t chunks, hipStream_t stream);

}  // namespace skipln
