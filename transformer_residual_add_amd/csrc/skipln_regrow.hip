// Register-resident long rows for BiasSoftmax (com.microsoft BiasSoftmax
// manifest: `description`, the softmax over each row of data + bias; the
// long-row variants for blocks too large for one workgroup's shared memory).
//
// One 1024-lane block per row at a time, persistent over rows.  Lane t keeps
// the row's raw data chunks t, t + 1024, ..., t + 19 * 1024 in VGPRs (80
// VGPRs: rows of up to 163840 float16 or 81920 float32 values; 126 VGPRs in
// all, no spills), so the data
// crosses HBM once, and forms z = fl32(data + bias) afresh in each of the two
// passes, re-reading the bias row -- from LDS when one bias row serves every
// data row (a vocabulary's logit bias), else through the caches:
//   pass 1: per lane, a running maximum m and the sum s of 2^((z - m) log2 e),
//           rescaled whenever m grows (the single-pass softmax statistics of
//           Milakov and Gimelshein, "Online normalizer calculation for
//           softmax", 2018); merged across the wavefront and across the 16
//           wavefronts through LDS into the row maximum M and sum S;
//   pass 2: out = 2^((z - M) log2 e) / S; once the whole row is stored, the
//           next row's data loads are issued into the freed registers.
// Special values follow the definition: a NaN or +inf anywhere, or a row of
// -inf only, makes the whole row NaN; -inf terms of other rows give 0.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "skipln_device.h"
#include "skipln_internal.h"
#include "skipln_rowtile.h"

namespace skipln {
namespace {
using namespace device;

constexpr int kRegRowBlock = 1024;
constexpr int kRegRowChunks = 20;  // chunks of data per lane
constexpr int kBiasAhead = 2;      // bias chunks loaded ahead of use
constexpr int kLdsSlabs = 9;       // bias slabs a block parks in LDS (144 KiB)

// Rows are addressed through buffer resources (base and byte size of one
// row, in scalar registers).  Chunk k of lane t is at lane offset t * 16 (a
// vector register) plus slab offset k * 16 KiB (a scalar register).  A lane
// whose chunk lies past the row's end gets a lane offset beyond any row, so
// the hardware range check masks the access -- a load returns zeros without
// touching memory, a store is dropped -- whether or not the check counts the
// scalar offset.  No branch surrounds the memory accesses, so the compiler
// can wait for each load on its own (loads complete in issue order) rather
// than for all of them.
constexpr int kNonTemporal = 2;         // cache policy of the data loads
constexpr int kSlabBytes = kRegRowBlock * 16;
constexpr int kPastRow = 0x40000000;    // lane offset beyond every row

__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* row_base, int row_bytes) {
    return buffer_rsrc(row_base, row_bytes);
}

// CH: slabs of the row (chunks per lane); the launch picks the smallest
// instantiated count that covers the row.  SB (shared bias): every row reads
// bias row 0 (one bias row, as a vocabulary's logit bias); its first kLdsSlabs
// slabs are then parked in LDS once per block, so that most bias reads of the
// two passes are LDS reads instead of vector memory loads.  This matters
// because vector loads complete in issue order: a bias load issued after the
// next row's data loads could only be waited for together with all of them,
// while an LDS read waits for nothing but itself.
template <typename T, int CH, bool SB>
__global__ void __launch_bounds__(kRegRowBlock) regrow_softmax_kernel(const Args a) {
    static_assert(CH >= 1 && CH <= kRegRowChunks, "slabs per row");
    using E = Elem<T>;
    constexpr int V = E::kPerChunk;
    constexpr int W = kRegRowBlock / 64;
    constexpr int K0 = SB ? (CH < kLdsSlabs ? CH : kLdsSlabs) : 0;  // slabs whose bias is in LDS
    constexpr float kLog2e = 1.4426950408889634f;
    constexpr float kNegInf = -__builtin_inff();
    __shared__ float2 red[2][W];
    extern __shared__ u32x4 sbias[];  // K0 slabs of 1024 chunks

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int hv = a.hidden / V;
    const bool small_rows = a.rows <= 0xFFFFFFFFll;
    // No __restrict__: out may be the data (or an exact bias) itself.  Each
    // chunk is read and written by one lane only, data before output.
    const u32x4* X = static_cast<const u32x4*>(a.input);
    const u32x4* B = static_cast<const u32x4*>(a.skip);
    u32x4* O = static_cast<u32x4*>(a.out);
    const int row_bytes = hv * 16;
    const int lane_off = tid * 16;
    // System-scope stores (for launches writing at least kStoreThroughBytes)
    // only when the row is whole 16 KiB slabs: rows of 192-256 KiB measured
    // 5-10 % faster with them, every row with a ragged last slab 2-11 %
    // faster with plain non-temporal stores (the vocabulary softmax's
    // 128,256 float16 values: 381 against 390 us).
    const bool through = a.store_through != 0 && row_bytes % kSlabBytes == 0;

    // Slabs holding a chunk of this lane: chunk k exists for k < nk.
    const int nk_lane = (hv - tid + kRegRowBlock - 1) / kRegRowBlock;
    // Lane offset of chunk k: this lane's, or one the range check refuses.
    // `lofs` and `nk` are re-read at the top of each pass (through an empty
    // asm), so the compiler forms each offset where it is used instead of
    // keeping sixteen of them live across the row loop.
    int lofs = lane_off, nk = nk_lane;
    // The launch runs the smallest compiled slab count CH >= the row's
    // slabs, and consecutive counts differ by at most 2 from 4 up, so slabs
    // below CH - 2 are whole for every lane: no mask there.
    constexpr int kWhole = CH >= 4 ? CH - 2 : 0;
    auto lo = [&](int k) { return k < kWhole || k < nk ? lofs : kPastRow; };
    auto refresh = [&]() {
        lofs = lane_off;
        nk = nk_lane;
        asm volatile("" : "+v"(lofs), "+v"(nk));
    };
    refresh();

    if constexpr (SB) {
        // Each lane parks its own bias chunks; it alone reads them back, so
        // no barrier is needed.
        const __amdgpu_buffer_rsrc_t b0 = row_rsrc(B, row_bytes);
#pragma unroll
        for (int k = 0; k < K0; ++k)
            sbias[k * kRegRowBlock + tid] = __builtin_amdgcn_raw_buffer_load_b128(b0, lo(k), k * kSlabBytes, 0);
    }

    u32x4 d[CH];
    int64_t row = blockIdx.x;
    {
        const __amdgpu_buffer_rsrc_t xr = row_rsrc(X + row * hv, row < a.rows ? row_bytes : 0);
#pragma unroll
        for (int k = 0; k < CH; ++k)
            d[k] = __builtin_amdgcn_raw_buffer_load_b128(xr, lo(k), k * kSlabBytes, kNonTemporal);
    }

    int buf = 0;
    for (; row < a.rows; row += gridDim.x) {
        const __amdgpu_buffer_rsrc_t br = row_rsrc(B + skip_row_of(row, a, small_rows) * hv, row_bytes);
        // Bias of slabs K0 .. CH-1 through a ring of kBiasAhead registers,
        // each load issued kBiasAhead slabs ahead of its use.
        u32x4 bq[kBiasAhead];
        auto ring_start = [&]() {
#pragma unroll
            for (int j = 0; j < kBiasAhead; ++j)
                if (K0 + j < CH) bq[j] = __builtin_amdgcn_raw_buffer_load_b128(br, lo(K0 + j), (K0 + j) * kSlabBytes, 0);
        };
        auto bias_of = [&](int k) -> u32x4 {
            if (k < K0) return sbias[k * kRegRowBlock + tid];
            const int q = (k - K0) % kBiasAhead;
            const u32x4 v = bq[q];
            if (k + kBiasAhead < CH)
                bq[q] = __builtin_amdgcn_raw_buffer_load_b128(br, lo(k + kBiasAhead), (k + kBiasAhead) * kSlabBytes, 0);
            return v;
        };

        // Pass 1.  Terms are taken relative to r = m (0 while m is -inf, so
        // that -inf data gives 0 and NaN stays NaN); when m grows, s is
        // rescaled by 2^((m_old - m) log2 e), which is 0 for m_old = -inf.
        // Chunks past the row's end enter as -inf (no term, no maximum).
        float m = kNegInf, s = 0.0f;
        refresh();
        ring_start();
#pragma unroll
        for (int k = 0; k < CH; ++k) {
            const u32x4 bk = bias_of(k);
            float z[V];
            E::widen_add(d[k], bk, z);
            float cm = kNegInf;
#pragma unroll
            for (int e = 0; e < V; ++e) {
                z[e] = k < kWhole || k < nk ? z[e] : kNegInf;
                cm = __builtin_fmaxf(cm, z[e]);
            }
            const float mn = __builtin_fmaxf(m, cm);
            s = cm > m ? s * __builtin_amdgcn_exp2f((m - mn) * kLog2e) : s;
            m = mn;
            const float r = m != kNegInf ? m : 0.0f;
            float cs = 0.0f;
#pragma unroll
            for (int e = 0; e < V; ++e) cs += __builtin_amdgcn_exp2f((z[e] - r) * kLog2e);
            s += cs;
            // Keep the ring's loads kBiasAhead slabs ahead, not all hoisted
            // to the top (that would take 64 more VGPRs).
            __builtin_amdgcn_sched_barrier(0);
        }
        // Wavefront, then block: M = max m, S = sum s 2^((m - M) log2 e); a
        // part whose maximum is -inf holds only zeros (or NaN) and enters
        // with factor 0 (NaN * 0 stays NaN).
        const float mw = wave_max(m);
        const float sw = wave_sum(s * (m != kNegInf ? __builtin_amdgcn_exp2f((m - mw) * kLog2e) : 0.0f));
        if ((tid & 63) == 0) red[buf][wave] = make_float2(mw, sw);
        __syncthreads();
        float M = kNegInf;
#pragma unroll
        for (int w = 0; w < W; ++w) M = __builtin_fmaxf(M, red[buf][w].x);
        float S = 0.0f;
#pragma unroll
        for (int w = 0; w < W; ++w) {
            const float2 p = red[buf][w];
            S += p.y * (p.x != kNegInf ? __builtin_amdgcn_exp2f((p.x - M) * kLog2e) : 0.0f);
        }
        buf ^= 1;
        // M = -inf (no finite value) gives (z - M) = NaN below, as the
        // definition has it; a NaN S makes the row NaN.
        const float scale = 1.0f / S;
        // binary16 outputs take 1/S into the exponent, 2^(t - log2 S): one fma
        // instead of two products per element.  The added error (about
        // |log2 S| 2^-24 relative, S <= the row's length) is far below the
        // output's own rounding; binary32 outputs keep the product.
        const float lsc = -log2f(S);

        // Pass 2: outputs, then the next row's data into the freed registers
        // (an empty range when there is no next row: no memory access).
        // Every store of the row is issued before the first of the next
        // row's loads: reloading each slab right after its store, so that
        // reads and writes alternate, measured 3-4 % slower on rows of
        // 100,000-128,256 float16 values with one bias row (1-2 % with a bias
        // row per row or float32).  The ring's slabs (K0 ..) go first, then
        // the LDS slabs (on float16 rows with one bias row 2 % faster than
        // slab order).
        const int64_t next = row + gridDim.x;
        const __amdgpu_buffer_rsrc_t orow = row_rsrc(O + row * hv, row_bytes);
        const __amdgpu_buffer_rsrc_t nrow =
            row_rsrc(X + (next < a.rows ? next : row) * hv, next < a.rows ? row_bytes : 0);
        refresh();
        ring_start();
        auto emit = [&](int k) {
            const u32x4 bk = bias_of(k);
            float y[V];
            // Widen the raw chunk again rather than keep pass 1's binary32
            // copy of the whole row alive (it would not fit in registers).
            asm volatile("" : "+v"(d[k]));
            E::widen_add(d[k], bk, y);
#pragma unroll
            for (int e = 0; e < V; ++e) {
                if constexpr (sizeof(T) == 2)
                    y[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(y[e] - M, kLog2e, lsc));
                else
                    y[e] = __builtin_amdgcn_exp2f((y[e] - M) * kLog2e) * scale;
            }
            E::store(E::narrow(y), orow, lo(k), k * kSlabBytes, through);
            __builtin_amdgcn_sched_barrier(0);
        };
#pragma unroll
        for (int k = K0; k < CH; ++k) emit(k);
#pragma unroll
        for (int k = 0; k < K0; ++k) emit(k);
#pragma unroll
        for (int k = 0; k < CH; ++k)
            d[k] = __builtin_amdgcn_raw_buffer_load_b128(nrow, lo(k), k * kSlabBytes, kNonTemporal);
    }
}

template <typename T, int CH, bool SB>
hipError_t launch_regrow_ch(const Args& a, hipStream_t st) {
    constexpr int k0 = SB ? (CH < kLdsSlabs ? CH : kLdsSlabs) : 0;
    constexpr size_t lds = static_cast<size_t>(k0) * kSlabBytes;
    auto kernel = regrow_softmax_kernel<T, CH, SB>;
    static int occ_cache = 0;
    int occ = __atomic_load_n(&occ_cache, __ATOMIC_RELAXED);
    if (occ <= 0) {
        const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, kRegRowBlock, lds);
        if (e != hipSuccess) return e;
        if (occ < 1) return hipErrorInvalidConfiguration;
        __atomic_store_n(&occ_cache, occ, __ATOMIC_RELAXED);
    }
    int cus = 0;
    const hipError_t e = rowtile::cu_count(&cus);
    if (e != hipSuccess) return e;
    int64_t blocks = static_cast<int64_t>(cus) * occ;
    if (a.rows < blocks) blocks = a.rows;
    Args arg = a;
    void* params[] = {&arg};
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3(static_cast<unsigned>(blocks < 1 ? 1 : blocks)),
                           dim3(kRegRowBlock), params, lds, st);
}

template <typename T, bool SB>
hipError_t launch_regrow_sb(const Args& a, int n, hipStream_t st) {
    if (n <= 1) return launch_regrow_ch<T, 1, SB>(a, st);
    if (n <= 2) return launch_regrow_ch<T, 2, SB>(a, st);
    if (n <= 4) return launch_regrow_ch<T, 4, SB>(a, st);
    if (n <= 6) return launch_regrow_ch<T, 6, SB>(a, st);
    if (n <= 8) return launch_regrow_ch<T, 8, SB>(a, st);
    if (n <= 10) return launch_regrow_ch<T, 10, SB>(a, st);
    if (n <= 12) return launch_regrow_ch<T, 12, SB>(a, st);
    if (n <= 14) return launch_regrow_ch<T, 14, SB>(a, st);
    if (n <= 16) return launch_regrow_ch<T, 16, SB>(a, st);
    if (n <= 18) return launch_regrow_ch<T, 18, SB>(a, st);
    if (n <= kRegRowChunks) return launch_regrow_ch<T, kRegRowChunks, SB>(a, st);
    return hipErrorInvalidValue;
}

// Slab counts compiled: a row of n slabs runs the first count >= n (for
// counts of 4 and more, n >= count - 1: the kernel relies on it).
template <typename T>
hipError_t launch_regrow_t(const Args& a, hipStream_t st) {
    const int hv = a.hidden / Elem<T>::kPerChunk;
    const int n = (hv + kRegRowBlock - 1) / kRegRowBlock;
    // Every row reads bias row 0: one cyclic row, one group holding all
    // rows, or a single row.
    const bool shared = a.skip_rows == 1 || (a.skip_group > 0 && a.skip_group >= a.rows) || a.rows == 1;
    return shared ? launch_regrow_sb<T, true>(a, n, st) : launch_regrow_sb<T, false>(a, n, st);
}

}  // namespace

bool regrow_holds(int op, int64_t hidden, int dtype) {
    if (op == kOpLayerNorm || op == kOpSimplified) return regnorm_holds(op, hidden, dtype);
    const int v = dtype == 0 ? Elem<float>::kPerChunk : Elem<_Float16>::kPerChunk;
    return op == kOpBiasSoftmax && hidden > 0 && hidden % v == 0 &&
           hidden / v <= static_cast<int64_t>(kRegRowBlock) * kRegRowChunks;
}

hipError_t launch_regrow(const Args& a, int op, int dtype, hipStream_t st) {
    if (op == kOpLayerNorm || op == kOpSimplified) return launch_regnorm(a, op, dtype, st);
    if (op != kOpBiasSoftmax) return hipErrorInvalidValue;
    return dtype == 0 ? launch_regrow_t<float>(a, st) : launch_regrow_t<_Float16>(a, st);
}

}  // namespace skipln
