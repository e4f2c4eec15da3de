// Split-row kernels for gfx950: rows longer than one workgroup can hold.
//
// A row is cut into slices of kSliceChunks 16-byte chunks (4096 float32 or
// 8192 float16 values); every slice is one 256-lane workgroup, so a row of
// P slices spreads over P workgroups and the whole chip works on a handful of
// rows.  Two kernels per batch of rows:
//   split_stats_kernel: loads its slice once (x, skip, bias), stores the
//     residual, and writes the slice's partial result to the workspace:
//       layer norm   (n_p, mean of (s - shift_p), M2 about that mean, shift_p)
//       simplified   (n_p, sum of s^2)
//       BiasSoftmax  (n_p, slice maximum m_p, sum of exp(z - m_p))
//     shift_p is the slice's first sum (as the row-tile kernel shifts by a
//     value of the row), so the merge, relative to slice 0's shift, only adds
//     small numbers.
//   split_apply_kernel: every wavefront merges the row's P partials on its own
//     (Chan's update for (mean, M2); max and rescaled sums for the softmax),
//     reloads its slice, forms the same sums again and writes the output.
//     A workgroup reads only its own slice before writing it, so the output
//     may alias an input; the residual may not (the second pass re-reads x and
//     skip), and the selection sends such calls elsewhere.
// The second pass re-reads x and skip, so a launch moves one more read stream
// than the single-workgroup kernels (the cost of needing no inter-workgroup
// synchronization: no workgroup ever waits for another).  Rows are processed
// in batches of about 128 MiB of streamed inputs, half the 256 MiB
// last-level cache; measured on MI355X this beat both smaller batches (more
// launches, fewer workgroups in flight) and one batch for all rows.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "skipln_device.h"
#include "skipln_internal.h"

namespace skipln {
namespace {
using namespace device;

constexpr int kSplitBlock = 256;
constexpr int kSplitCh = 4;                             // chunks per lane and slice
constexpr int kSliceChunks = kSplitBlock * kSplitCh;    // 1024 chunks = 16 KiB per tensor
constexpr int kMaxSlices = 64;                          // partials merged by one wavefront
// Input bytes one batch streams before its second pass re-reads them.
constexpr int64_t kBatchInputBytes = 128ll << 20;

struct Split {
    float4* ws;      // [batch rows][slices] partials
    int32_t slices;  // P
    int64_t row0;    // first row of this batch
};

// The sum at column `col` of a row: input + skip (+ bias), formed with the
// operations of the slice loops, hence the same bits.
template <typename T>
__device__ __forceinline__ float sum_at(const Args& a, int64_t row, int64_t srow, int64_t col) {
    using E = Elem<T>;
    float v = E::load1(a.input, row * a.hidden + col) + E::load1(a.skip, srow * a.hidden + col);
    if (a.bias != nullptr) v = v + E::load1(a.bias, col);
    return v;
}

template <typename T, int OP>
__global__ void __launch_bounds__(kSplitBlock) split_stats_kernel(const Args a, const Split sp) {
    static_assert(OP == kOpLayerNorm || OP == kOpSimplified || OP == kOpBiasSoftmax, "row-reducing operations");
    using E = Elem<T>;
    constexpr int V = E::kPerChunk;
    constexpr int W = kSplitBlock / 64;
    __shared__ float red[2][W];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int64_t b = blockIdx.x;
    const int64_t row = sp.row0 + b / sp.slices;
    const int p = static_cast<int>(b % sp.slices);
    const int hv = a.hidden / V;
    const int c0 = p * kSliceChunks;
    const int n_chunks = hv - c0 < kSliceChunks ? hv - c0 : kSliceChunks;
    const float n_p = static_cast<float>(n_chunks * V);
    const bool small_rows = a.rows <= 0xFFFFFFFFll;
    const int64_t srow = skip_row_of(row, a, small_rows);
    const bool has_bias = OP != kOpBiasSoftmax && a.bias != nullptr;

    const u32x4* xp = static_cast<const u32x4*>(a.input) + row * hv + c0;
    const u32x4* spp = static_cast<const u32x4*>(a.skip) + srow * hv + c0;
    const u32x4* bp = static_cast<const u32x4*>(a.bias) + c0;

    u32x4 xr[kSplitCh], sr[kSplitCh], br[kSplitCh];
#pragma unroll
    for (int k = 0; k < kSplitCh; ++k) {
        const int c = k * kSplitBlock + tid;
        xr[k] = sr[k] = br[k] = u32x4{0, 0, 0, 0};
        if (c < n_chunks) {
            // Ordinary (cache-allocating) loads: the second pass reads the
            // same lines again.
            xr[k] = xp[c];
            sr[k] = spp[c];
            if (has_bias) br[k] = bp[c];
        }
    }

    auto block_reduce = [&](float v, int buf, auto op) {
        using Op = decltype(op);
        const float ws = wave_reduce<Op>(v);
        if ((tid & 63) == 0) red[buf][wave] = ws;
        __syncthreads();
        float t = Op::id();
#pragma unroll
        for (int w = 0; w < W; ++w) t = Op::apply(t, red[buf][w]);
        return t;
    };

    float s[kSplitCh][V];
#pragma unroll
    for (int k = 0; k < kSplitCh; ++k) {
        float xf[V], sf[V], bf[V];
        E::widen(xr[k], xf);
        E::widen(sr[k], sf);
        E::widen(br[k], bf);
#pragma unroll
        for (int e = 0; e < V; ++e) {
            float v = xf[e] + sf[e];
            if (has_bias) v = v + bf[e];
            s[k][e] = v;
        }
    }

    if (OP != kOpBiasSoftmax && a.residual != nullptr) {
        u32x4* rp = static_cast<u32x4*>(a.residual) + row * hv + c0;
#pragma unroll
        for (int k = 0; k < kSplitCh; ++k) {
            const int c = k * kSplitBlock + tid;
            if (c < n_chunks) __builtin_nontemporal_store(E::narrow(s[k]), rp + c);
        }
    }

    float4 out;
    if constexpr (OP == kOpLayerNorm) {
        const float shift = sum_at<T>(a, row, srow, static_cast<int64_t>(c0) * V);
        float part = 0.0f;
#pragma unroll
        for (int k = 0; k < kSplitCh; ++k)
            if (k * kSplitBlock + tid < n_chunks)
#pragma unroll
                for (int e = 0; e < V; ++e) part += s[k][e] - shift;
        const float dm = block_reduce(part, 0, SumOp{}) / n_p;
        float q = 0.0f;
#pragma unroll
        for (int k = 0; k < kSplitCh; ++k)
            if (k * kSplitBlock + tid < n_chunks)
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    const float d = (s[k][e] - shift) - dm;
                    q += d * d;
                }
        out = make_float4(n_p, dm, block_reduce(q, 1, SumOp{}), shift);
    } else if constexpr (OP == kOpSimplified) {
        float sq = 0.0f;
#pragma unroll
        for (int k = 0; k < kSplitCh; ++k)
            if (k * kSplitBlock + tid < n_chunks)
#pragma unroll
                for (int e = 0; e < V; ++e) sq += s[k][e] * s[k][e];
        out = make_float4(n_p, block_reduce(sq, 0, SumOp{}), 0.0f, 0.0f);
    } else {
        constexpr float kLog2e = 1.4426950408889634f;
        float mx = -__builtin_inff();
#pragma unroll
        for (int k = 0; k < kSplitCh; ++k)
            if (k * kSplitBlock + tid < n_chunks)
#pragma unroll
                for (int e = 0; e < V; ++e) mx = __builtin_fmaxf(mx, s[k][e]);
        const float m = block_reduce(mx, 0, MaxOp{});
        // A slice of -inf only: its exponentials are 0 whatever the reference.
        const float r = m != -__builtin_inff() ? m : 0.0f;
        float part = 0.0f;
#pragma unroll
        for (int k = 0; k < kSplitCh; ++k)
            if (k * kSplitBlock + tid < n_chunks)
#pragma unroll
                for (int e = 0; e < V; ++e) part += __builtin_amdgcn_exp2f((s[k][e] - r) * kLog2e);
        out = make_float4(n_p, m, block_reduce(part, 1, SumOp{}), 0.0f);
    }
    if (tid == 0) sp.ws[b] = out;
}

template <typename T, int OP>
__global__ void __launch_bounds__(kSplitBlock) split_apply_kernel(const Args a, const Split sp) {
    using E = Elem<T>;
    constexpr int V = E::kPerChunk;
    constexpr float kNegInf = -__builtin_inff();
    constexpr float kLog2e = 1.4426950408889634f;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int64_t b = blockIdx.x;
    const int64_t lrow = b / sp.slices;  // row within the batch
    const int64_t row = sp.row0 + lrow;
    const int p = static_cast<int>(b % sp.slices);
    const int hv = a.hidden / V;
    const int c0 = p * kSliceChunks;
    const int n_chunks = hv - c0 < kSliceChunks ? hv - c0 : kSliceChunks;
    const float h = static_cast<float>(a.hidden);
    const bool small_rows = a.rows <= 0xFFFFFFFFll;
    const int64_t srow = skip_row_of(row, a, small_rows);
    const bool has_bias = OP != kOpBiasSoftmax && a.bias != nullptr;
    const bool has_beta = a.beta != nullptr;

    // Merge the row's partials, each wavefront on its own (lane l holds
    // slice l's partial).
    const bool mine = lane < sp.slices;
    const float4 q = mine ? sp.ws[lrow * sp.slices + lane] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    float shift = 0.0f, off = 0.0f, scale, ref = 0.0f;
    if constexpr (OP == kOpLayerNorm) {
        // This slice's shift, read by every lane before any lane stores over
        // an aliased input; slice means relative to slice 0's shift.
        shift = sum_at<T>(a, row, srow, static_cast<int64_t>(c0) * V);
        __syncthreads();
        const float row_shift = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, q.w)));
        const float d = mine ? (q.w - row_shift) + q.y : 0.0f;
        const float dmean = wave_sum(q.x * d) / h;
        const float dd = d - dmean;
        const float m2 = wave_sum(mine ? q.z + q.x * dd * dd : 0.0f);
        // s - shift is centered on the row mean by subtracting
        // dmean - (shift - row_shift).
        off = dmean - (shift - row_shift);
        scale = rsqrtf(m2 / h + a.eps);
    } else if constexpr (OP == kOpSimplified) {
        scale = rsqrtf(wave_sum(q.y) / h + a.eps);
    } else {
        const float m = wave_max(mine ? q.y : kNegInf);
        const float f = (mine && q.y != kNegInf) ? __builtin_amdgcn_exp2f((q.y - m) * kLog2e) : 0.0f;
        scale = 1.0f / wave_sum(q.z * f);
        ref = m;
    }

    const u32x4* xp = static_cast<const u32x4*>(a.input) + row * hv + c0;
    const u32x4* spp = static_cast<const u32x4*>(a.skip) + srow * hv + c0;
    u32x4* op = static_cast<u32x4*>(a.out) + row * hv + c0;
    u32x4 xr[kSplitCh], sr[kSplitCh];
#pragma unroll
    for (int k = 0; k < kSplitCh; ++k) {
        const int c = k * kSplitBlock + tid;
        xr[k] = sr[k] = u32x4{0, 0, 0, 0};
        if (c < n_chunks) {
            xr[k] = __builtin_nontemporal_load(xp + c);
            sr[k] = __builtin_nontemporal_load(spp + c);
        }
    }
#pragma unroll
    for (int k = 0; k < kSplitCh; ++k) {
        const int c = k * kSplitBlock + tid;
        if (c >= n_chunks) continue;
        float xf[V], sf[V], y[V];
        E::widen(xr[k], xf);
        E::widen(sr[k], sf);
        if constexpr (OP == kOpBiasSoftmax) {
#pragma unroll
            for (int e = 0; e < V; ++e) y[e] = __builtin_amdgcn_exp2f(((xf[e] + sf[e]) - ref) * kLog2e) * scale;
        } else {
            float bf[V], gf[V], tf[V];
            E::widen(has_bias ? static_cast<const u32x4*>(a.bias)[c0 + c] : u32x4{0, 0, 0, 0}, bf);
            E::widen(static_cast<const u32x4*>(a.gamma)[c0 + c], gf);
            E::widen(has_beta ? static_cast<const u32x4*>(a.beta)[c0 + c] : u32x4{0, 0, 0, 0}, tf);
#pragma unroll
            for (int e = 0; e < V; ++e) {
                float v = xf[e] + sf[e];
                if (has_bias) v = v + bf[e];
                if constexpr (OP == kOpLayerNorm)
                    y[e] = ((v - shift) - off) * scale * gf[e] + tf[e];
                else
                    y[e] = v * scale * gf[e] + tf[e];
            }
        }
        __builtin_nontemporal_store(E::narrow(y), op + c);
    }
}

int slices_of(int64_t hidden, int dtype) {
    const int v = dtype == 0 ? Elem<float>::kPerChunk : Elem<_Float16>::kPerChunk;
    return static_cast<int>((hidden / v + kSliceChunks - 1) / kSliceChunks);
}

// Rows per batch: the inputs streamed per batch (x, and skip when it is not
// broadcast) within kBatchInputBytes, at least one row.
int64_t batch_rows_of(const Args& a, int dtype) {
    const int64_t row_bytes = static_cast<int64_t>(a.hidden) * (dtype == 0 ? 4 : 2);
    const bool exact_skip = a.skip_rows == 0 && a.skip_group == 0;
    const int64_t per_row = row_bytes * (exact_skip ? 2 : 1);
    int64_t n = kBatchInputBytes / per_row;
    if (n < 1) n = 1;
    return n < a.rows ? n : a.rows;
}

template <typename T, int OP>
hipError_t launch_split_t(const Args& a, float4* ws, hipStream_t st) {
    const int P = slices_of(a.hidden, sizeof(T) == 4 ? 0 : 1);
    const int64_t batch = batch_rows_of(a, sizeof(T) == 4 ? 0 : 1);
    for (int64_t row0 = 0; row0 < a.rows; row0 += batch) {
        const int64_t n = a.rows - row0 < batch ? a.rows - row0 : batch;
        Args arg = a;
        Split sp;
        sp.ws = ws;
        sp.slices = P;
        sp.row0 = row0;
        void* params[] = {&arg, &sp};
        // n * P * kSplitBlock work-items: a batch streams at most
        // kBatchInputBytes, i.e. at most 2^23 rows of 16 bytes, one slice each.
        const dim3 grid(static_cast<unsigned>(n * P));
        hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(split_stats_kernel<T, OP>), grid,
                                       dim3(kSplitBlock), params, 0, st);
        if (e != hipSuccess) return e;
        e = hipLaunchKernel(reinterpret_cast<const void*>(split_apply_kernel<T, OP>), grid, dim3(kSplitBlock), params,
                            0, st);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <typename T>
hipError_t launch_split_op(const Args& a, int op, float4* ws, hipStream_t st) {
    switch (op) {
        case kOpLayerNorm: return launch_split_t<T, kOpLayerNorm>(a, ws, st);
        case kOpSimplified: return launch_split_t<T, kOpSimplified>(a, ws, st);
        case kOpBiasSoftmax: return launch_split_t<T, kOpBiasSoftmax>(a, ws, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool split_holds(int op, int64_t hidden, int dtype) {
    const int v = dtype == 0 ? Elem<float>::kPerChunk : Elem<_Float16>::kPerChunk;
    return (op == kOpLayerNorm || op == kOpSimplified || op == kOpBiasSoftmax) && hidden > 0 && hidden % v == 0 &&
           slices_of(hidden, dtype) <= kMaxSlices;
}

int64_t split_workspace_bytes(const Args& a, int dtype) {
    if (a.rows <= 0) return 0;
    return batch_rows_of(a, dtype) * slices_of(a.hidden, dtype) * static_cast<int64_t>(sizeof(float4));
}

hipError_t launch_split(const Args& a, int op, int dtype, void* workspace, hipStream_t st) {
    float4* ws = static_cast<float4*>(workspace);
    return dtype == 0 ? launch_split_op<float>(a, op, ws, st) : launch_split_op<_Float16>(a, op, ws, st);
}

}  // namespace skipln
