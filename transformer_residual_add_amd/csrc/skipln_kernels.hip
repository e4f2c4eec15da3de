// Row kernels for gfx950 (CDNA4, wave64): SkipLayerNormalization, its
// root-mean-square form, BiasAdd and BiasSoftmax.
//
// SkipLayerNormalization (com.microsoft SkipLayerNormalization WebGPU
// manifest): `description` (skip addition fused with a layer normalization
// over the hidden axis), `inputs[skip]` (exact, or broadcast over the batch
// with numel(skip)/H rows, the `Params.skipRows` of the broadcast binding
// set), `inputs[bias]` (joins input + skip before the normalization),
// `inputs[gamma]` / `inputs[beta]`, `outputs[input_skip_bias_sum]`,
// `attributes.epsilon`.  Statistics are the population mean and variance of
// the binary32 sum; all arithmetic is binary32, float16 only at load/store.
// BiasAdd (com.microsoft BiasAdd manifest) is the same sum without the
// normalization, in the order (x + bias) + skip.  BiasSoftmax (com.microsoft
// BiasSoftmax manifest) is a softmax over each row of data + bias, the bias
// rows arriving through the skip slot (exact, cyclic, or grouped reuse).
//
// The work is bound by HBM bandwidth (about 1 flop per byte moved), so the
// kernels are organised around moving each byte once:
//   * rowtile_kernel: a group of G lanes owns one row at a time and keeps the
//     whole row in VGPRs between the reduction and the output, so x and skip
//     are read from HBM exactly once.  Every access is a 16-byte vector
//     load/store (4 fp32 or 8 fp16), coalesced across the group.  G is 4..32
//     (several rows per wavefront, short rows), 64 (one wavefront per row)
//     or 128..1024 (several wavefronts per row, partial results combined
//     through LDS with one barrier per row).  Each block walks row tiles
//     (contiguous, strided, or skip-stationary), loads gamma/beta/bias into
//     registers once, and issues the loads of its next tile before it
//     reduces and stores the current one, keeping HBM requests in flight
//     across the reduction.  Streaming tensors use non-temporal accesses so
//     they do not displace the broadcast skip and the parameters in L2.
//   * ldsrow_kernel: rows too long for registers, staged in LDS (160 KiB per
//     workgroup on gfx950), one 1024-lane block per row.
//   * generic_chunk_kernel: aligned rows of whole 16-byte chunks beyond the
//     other families' reach when no workspace is given, one 1024-lane block
//     per row, two passes (statistics, then output), the second taking the
//     row's first 40,832 sums from LDS and re-reading only the rest.
//   * generic_kernel: any H and any alignment, one 256-lane block per row,
//     several passes over the row with element accesses.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <cstdio>
#include <utility>

#include "skipln_device.h"
#include "skipln_internal.h"
#include "skipln_rowtile.h"

namespace skipln {
namespace {
using namespace device;
using rowtile::cu_count;
using rowtile::Geom;
using rowtile::kElemGeoms;
using rowtile::kGeoms;
using rowtile::kNumElemGeoms;
using rowtile::kNumGeoms;
using rowtile::launch_grid;
using rowtile::resident_blocks;

// ------------------------------------------------------------------------
// Long-row kernel: the row is staged in LDS.
// ------------------------------------------------------------------------
// One 1024-lane block per row at a time (persistent over rows).  Lane t owns
// chunks t, t + 1024, ...; it loads them (kLdsBatch chunks in flight per
// lane), forms the binary32 sums and parks them in LDS (the residual is
// stored with the output) -- up to 160 KiB, i.e. rows of up to ~40K values
// whatever T is -- so x and skip cross HBM once.  Each lane re-reads only the LDS words it wrote,
// so the row data needs no barrier; only the block reductions do.
constexpr int kLdsBlock = 1024;
constexpr int kLdsBatch = 4;

template <typename T, int OP>
__global__ void __launch_bounds__(kLdsBlock) ldsrow_kernel(const Args a) {
    static_assert(OP == kOpLayerNorm || OP == kOpSimplified || OP == kOpBiasSoftmax, "row-reducing operations");
    using E = Elem<T>;
    constexpr int V = E::kPerChunk;
    constexpr int Q = V / 4;  // float4 words of binary32 sums per chunk
    constexpr int W = kLdsBlock / 64;
    extern __shared__ float4 srow[];
    __shared__ float red[2][W];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int hv = a.hidden / V;
    const float h = static_cast<float>(a.hidden);
    const bool has_bias = OP != kOpBiasSoftmax && a.bias != nullptr;
    const bool has_beta = a.beta != nullptr;
    const bool bcast = a.skip_rows > 0 || a.skip_group > 0;
    const bool small_rows = a.rows <= 0xFFFFFFFFll;
    const u32x4* __restrict__ X = static_cast<const u32x4*>(a.input);
    const u32x4* __restrict__ S = static_cast<const u32x4*>(a.skip);
    const u32x4* __restrict__ Bz = static_cast<const u32x4*>(a.bias);
    const u32x4* __restrict__ Gm = static_cast<const u32x4*>(a.gamma);
    const u32x4* __restrict__ Bt = static_cast<const u32x4*>(a.beta);
    u32x4* __restrict__ R = static_cast<u32x4*>(a.residual);
    u32x4* __restrict__ O = static_cast<u32x4*>(a.out);

    // Block reduction (SumOp or MaxOp); `buf` alternates so that a slot is
    // rewritten only after a barrier every lane passes after reading it.
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
    auto block_sum = [&](float v, int buf) { return block_reduce(v, buf, SumOp{}); };

    int rms_buf = 0;
    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
        const int64_t srow_i = skip_row_of(row, a, small_rows);
        const u32x4* xp = X + row * hv;
        const u32x4* sp = S + srow_i * hv;

        if constexpr (OP == kOpBiasSoftmax) {
            // Softmax over the row of z = data + bias (bias through the skip
            // slot): z parked in LDS while the block finds the maximum M, then
            // replaced by 2^((z - M) log2 e) while the block sums them, then
            // scaled by 1 / sum.  Special values as in the row-tile kernel
            // (one reference, the row maximum).
            constexpr float kLog2e = 1.4426950408889634f;
            float mx = -__builtin_inff();
            for (int c0 = tid; c0 < hv; c0 += kLdsBlock * kLdsBatch) {
                u32x4 xr[kLdsBatch], sr[kLdsBatch];
#pragma unroll
                for (int b = 0; b < kLdsBatch; ++b) {
                    const int c = c0 + b * kLdsBlock;
                    xr[b] = sr[b] = u32x4{0, 0, 0, 0};
                    if (c < hv) {
                        xr[b] = __builtin_nontemporal_load(xp + c);
                        sr[b] = bcast ? sp[c] : __builtin_nontemporal_load(sp + c);
                    }
                }
#pragma unroll
                for (int b = 0; b < kLdsBatch; ++b) {
                    const int c = c0 + b * kLdsBlock;
                    if (c < hv) {
                        float xf[V], sf[V], zv[V];
                        E::widen(xr[b], xf);
                        E::widen(sr[b], sf);
#pragma unroll
                        for (int e = 0; e < V; ++e) {
                            zv[e] = xf[e] + sf[e];
                            mx = __builtin_fmaxf(mx, zv[e]);
                        }
#pragma unroll
                        for (int q = 0; q < Q; ++q)
                            srow[c * Q + q] = make_float4(zv[4 * q], zv[4 * q + 1], zv[4 * q + 2], zv[4 * q + 3]);
                    }
                }
            }
            const float m = block_reduce(mx, 0, MaxOp{});
            float part = 0.0f;
            for (int c = tid; c < hv; c += kLdsBlock) {
#pragma unroll
                for (int q = 0; q < Q; ++q) {
                    float4 v = srow[c * Q + q];
                    v.x = __builtin_amdgcn_exp2f((v.x - m) * kLog2e);
                    v.y = __builtin_amdgcn_exp2f((v.y - m) * kLog2e);
                    v.z = __builtin_amdgcn_exp2f((v.z - m) * kLog2e);
                    v.w = __builtin_amdgcn_exp2f((v.w - m) * kLog2e);
                    part += v.x + v.y + v.z + v.w;
                    srow[c * Q + q] = v;
                }
            }
            const float scale = 1.0f / block_sum(part, 1);
            for (int c = tid; c < hv; c += kLdsBlock) {
                float y[V];
#pragma unroll
                for (int q = 0; q < Q; ++q) {
                    const float4 v = srow[c * Q + q];
                    y[4 * q] = v.x * scale;
                    y[4 * q + 1] = v.y * scale;
                    y[4 * q + 2] = v.z * scale;
                    y[4 * q + 3] = v.w * scale;
                }
                __builtin_nontemporal_store(E::narrow(y), O + row * hv + c);
            }
            continue;
        }
        // Shift of the sums (see the row-tile kernel): the row's first sum,
        // formed by every lane with the same operations, hence the same bits.
        float shift = 0.0f;
        if constexpr (OP == kOpLayerNorm) {
            shift = E::load1(a.input, row * a.hidden) + E::load1(a.skip, srow_i * a.hidden);
            if (has_bias) shift = shift + E::load1(a.bias, 0);
            // Every lane has read the row's first sum before lane 0 may store
            // its residual over an aliased skip (or input).
            __syncthreads();
        }

        float part = 0.0f;
        for (int c0 = tid; c0 < hv; c0 += kLdsBlock * kLdsBatch) {
            u32x4 xr[kLdsBatch], sr[kLdsBatch], br[kLdsBatch];
#pragma unroll
            for (int b = 0; b < kLdsBatch; ++b) {
                const int c = c0 + b * kLdsBlock;
                xr[b] = sr[b] = br[b] = u32x4{0, 0, 0, 0};
                if (c < hv) {
                    xr[b] = __builtin_nontemporal_load(xp + c);
                    sr[b] = bcast ? sp[c] : __builtin_nontemporal_load(sp + c);
                    if (has_bias) br[b] = Bz[c];
                }
            }
#pragma unroll
            for (int b = 0; b < kLdsBatch; ++b) {
                const int c = c0 + b * kLdsBlock;
                if (c < hv) {
                    float xf[V], sf[V], bf[V], sv[V];
                    E::widen(xr[b], xf);
                    E::widen(sr[b], sf);
                    E::widen(br[b], bf);
#pragma unroll
                    for (int e = 0; e < V; ++e) {
                        float v = xf[e] + sf[e];
                        if (has_bias) v = v + bf[e];
                        sv[e] = v;
                        if constexpr (OP == kOpSimplified)
                            part += v * v;
                        else
                            part += v - shift;
                    }
#pragma unroll
                    for (int q = 0; q < Q; ++q)
                        srow[c * Q + q] = make_float4(sv[4 * q], sv[4 * q + 1], sv[4 * q + 2], sv[4 * q + 3]);
                }
            }
        }

        // The mean is kept as shift + dmean (see the row-tile kernel).
        float dmean = 0.0f, var;
        if constexpr (OP == kOpSimplified) {
            var = block_sum(part, rms_buf) / h;
            rms_buf ^= 1;
        } else {
            dmean = block_sum(part, 0) / h;
            float q2 = 0.0f;
            for (int c = tid; c < hv; c += kLdsBlock) {
#pragma unroll
                for (int q = 0; q < Q; ++q) {
                    const float4 v = srow[c * Q + q];
                    const float d0 = (v.x - shift) - dmean, d1 = (v.y - shift) - dmean;
                    const float d2 = (v.z - shift) - dmean, d3 = (v.w - shift) - dmean;
                    q2 += d0 * d0 + d1 * d1 + d2 * d2 + d3 * d3;
                }
            }
            var = block_sum(q2, 1) / h;
        }
        const float rstd = rsqrtf(var + a.eps);

        for (int c = tid; c < hv; c += kLdsBlock) {
            float gf[V], bf[V], y[V];
            // The residual goes out here, with the output, rather than while
            // the row is read: reads and writes in phases of their own
            // (rows of 32768 float32 values: 826 against 864 us).  The sums
            // are still in LDS, and every load of the row is done, so an
            // aliased input or skip is safe to overwrite.
            if (R != nullptr) {
                float sv[V];
#pragma unroll
                for (int q = 0; q < Q; ++q) {
                    const float4 v = srow[c * Q + q];
                    sv[4 * q] = v.x;
                    sv[4 * q + 1] = v.y;
                    sv[4 * q + 2] = v.z;
                    sv[4 * q + 3] = v.w;
                }
                __builtin_nontemporal_store(E::narrow(sv), R + row * hv + c);
            }
            E::widen(Gm[c], gf);
            if (has_beta) {
                E::widen(Bt[c], bf);
            } else {
#pragma unroll
                for (int e = 0; e < V; ++e) bf[e] = 0.0f;
            }
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                const float4 v = srow[c * Q + q];
                y[4 * q] = ((v.x - shift) - dmean) * rstd * gf[4 * q] + bf[4 * q];
                y[4 * q + 1] = ((v.y - shift) - dmean) * rstd * gf[4 * q + 1] + bf[4 * q + 1];
                y[4 * q + 2] = ((v.z - shift) - dmean) * rstd * gf[4 * q + 2] + bf[4 * q + 2];
                y[4 * q + 3] = ((v.w - shift) - dmean) * rstd * gf[4 * q + 3] + bf[4 * q + 3];
            }
            __builtin_nontemporal_store(E::narrow(y), O + row * hv + c);
        }
    }
}

// ------------------------------------------------------------------------
// Generic kernel: any hidden size and alignment.
// ------------------------------------------------------------------------
constexpr int kGenericBlock = 256;

template <typename T, int OP>
__global__ void __launch_bounds__(kGenericBlock) generic_kernel(const Args a) {
    using E = Elem<T>;
    constexpr int W = kGenericBlock / 64;
    __shared__ float red[2][W];
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int64_t H = a.hidden;
    const float h = static_cast<float>(a.hidden);
    int rms_slot = 0;

    const bool small_rows = a.rows <= 0xFFFFFFFFll;
    // Block reduction (SumOp or MaxOp) through LDS slot `buf`.
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

    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
        const int64_t srow = skip_row_of(row, a, small_rows);
        const int64_t xo = row * H, so = srow * H;
        // The same binary32 operations in every pass, hence the same bits.
        auto sum_at = [&](int64_t c) {
            float v;
            if constexpr (OP == kOpBiasAdd) {
                v = E::load1(a.input, xo + c) + E::load1(a.bias, c);
                v = v + E::load1(a.skip, so + c);
            } else {
                v = E::load1(a.input, xo + c) + E::load1(a.skip, so + c);
                if (OP != kOpBiasSoftmax && a.bias != nullptr) v = v + E::load1(a.bias, c);
            }
            return v;
        };

        if constexpr (OP == kOpBiasAdd) {
            for (int64_t c = tid; c < H; c += kGenericBlock) E::store1(a.out, xo + c, sum_at(c));
            continue;
        }
        if constexpr (OP == kOpBiasSoftmax) {
            // Softmax over the row of z = data + bias (bias through the skip
            // slot): the maximum M, then the sum of 2^((z - M) log2 e), then
            // the scaled exponentials, recomputed from the same bits in each
            // pass.  Slot 0 holds the maximum, slot 1 the sum: a slot is
            // rewritten only after the other slot's barrier, which every lane
            // passes after reading it.
            constexpr float kLog2e = 1.4426950408889634f;
            float mx = -__builtin_inff();
            for (int64_t c = tid; c < H; c += kGenericBlock) mx = __builtin_fmaxf(mx, sum_at(c));
            const float m = block_reduce(mx, 0, MaxOp{});
            float part = 0.0f;
            for (int64_t c = tid; c < H; c += kGenericBlock) part += __builtin_amdgcn_exp2f((sum_at(c) - m) * kLog2e);
            const float scale = 1.0f / block_reduce(part, 1, SumOp{});
            for (int64_t c = tid; c < H; c += kGenericBlock)
                E::store1(a.out, xo + c, __builtin_amdgcn_exp2f((sum_at(c) - m) * kLog2e) * scale);
            continue;
        }
        if constexpr (OP == kOpSimplified) {
            float sq = 0.0f;
            for (int64_t c = tid; c < H; c += kGenericBlock) {
                const float v = sum_at(c);
                sq += v * v;
            }
            // One barrier per row: consecutive rows use alternate LDS slots,
            // and a slot is rewritten two rows later, after a barrier that
            // every lane reaches only once it has read the slot.
            const float wsq = wave_sum(sq);
            if ((tid & 63) == 0) red[rms_slot][wave] = wsq;
            __syncthreads();
            float tot = 0.0f;
#pragma unroll
            for (int w = 0; w < W; ++w) tot += red[rms_slot][w];
            rms_slot ^= 1;
            const float rstd = rsqrtf(tot / h + a.eps);
            for (int64_t c = tid; c < H; c += kGenericBlock) {
                const float v = sum_at(c);
                if (a.residual != nullptr) E::store1(a.residual, xo + c, v);
                const float g = E::load1(a.gamma, c);
                const float b = a.beta != nullptr ? E::load1(a.beta, c) : 0.0f;
                E::store1(a.out, xo + c, v * rstd * g + b);
            }
            continue;
        }

        // Sums relative to the row's first sum (see the row-tile kernel).
        const float shift = sum_at(0);
        float part = 0.0f;
        for (int64_t c = tid; c < H; c += kGenericBlock) part += sum_at(c) - shift;
        float ws = wave_sum(part);
        if ((tid & 63) == 0) red[0][wave] = ws;
        __syncthreads();
        float tot = 0.0f;
#pragma unroll
        for (int w = 0; w < W; ++w) tot += red[0][w];
        const float dmean = tot / h;  // the mean is shift + dmean (see the row-tile kernel)

        float q = 0.0f;
        for (int64_t c = tid; c < H; c += kGenericBlock) {
            const float d = (sum_at(c) - shift) - dmean;
            q += d * d;
        }
        ws = wave_sum(q);
        if ((tid & 63) == 0) red[1][wave] = ws;
        __syncthreads();
        tot = 0.0f;
#pragma unroll
        for (int w = 0; w < W; ++w) tot += red[1][w];
        const float rstd = rsqrtf(tot / h + a.eps);

        // Each element is read and then written by the same lane, so exact
        // aliasing of an output with input or skip is safe.
        for (int64_t c = tid; c < H; c += kGenericBlock) {
            const float v = sum_at(c);
            if (a.residual != nullptr) E::store1(a.residual, xo + c, v);
            const float g = E::load1(a.gamma, c);
            const float b = a.beta != nullptr ? E::load1(a.beta, c) : 0.0f;
            E::store1(a.out, xo + c, ((v - shift) - dmean) * rstd * g + b);
        }
    }
}

// ------------------------------------------------------------------------
// Streaming copy (bandwidth reference): 16-byte chunks, persistent grid.
// ------------------------------------------------------------------------
constexpr int kCopyBlock = 256;
constexpr int kCopyUnroll = 4;

__global__ void __launch_bounds__(kCopyBlock) copy_kernel(u32x4* __restrict__ dst, const u32x4* __restrict__ src,
                                                          int64_t chunks) {
    const int64_t step = static_cast<int64_t>(gridDim.x) * kCopyBlock;
    int64_t i = static_cast<int64_t>(blockIdx.x) * kCopyBlock + threadIdx.x;
    for (; i + (kCopyUnroll - 1) * step < chunks; i += kCopyUnroll * step) {
        u32x4 v[kCopyUnroll];
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * step);
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) __builtin_nontemporal_store(v[u], dst + i + u * step);
    }
    for (; i < chunks; i += step) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}



// Automatic choice: the first entry whose capacity holds the row's chunks.
// Short rows are latency bound: one chunk per lane spreads a row over more
// lanes and shortens the per-lane load/reduce chain; rows of 8 chunks or
// fewer (e.g. attention rows of a few keys) pack 32 or 64 rows into a
// 256-lane block instead of leaving most of a 16-lane group idle.  Long rows use 256-lane
// groups (4 wavefronts; 1024-lane groups pay for 16-wavefront barriers).
// A broadcast skip uses the same geometries with skip-stationary tiling.
struct AutoEntry {
    int max_chunks, geom;
};
// Normalizations with an exact skip: rows of 65-128 chunks run one
// wavefront per row (2 chunks per lane, no cross-wave barrier), measured on
// two boxes 2-3 % faster than 128-lane groups with the buffer-store outputs
// (16384 x 1024 float16: 22.9 against 23.3-23.6 us, interleaved runs).  At
// 192 chunks the same change was 2.7 % faster on one box and 3.5 % slower on
// another for BERT-base (1024 x 768 float32), so 192-lane groups stay.
// Rows of 257-512 chunks run 128-lane groups of 4 chunks per lane, two rows
// per block: 3-7 % faster than 256 x 2 tiles at 16384-32768 rows (layer
// norm, float16 2560 / 3072 / 3584 / 4096 values at 32768 rows: 111.7 /
// 132.5 / 156.2 / 172.7 against 116.9 / 138.3 / 163.4 / 180.2 us; float32
// 1280 / 1536 / 2048: 109.2 / 133.0 / 172.4 against 117.4 / 141.0 / 182.4;
// RMS float16 3072: 132.0 against 140.3).  Launches of the single-tile form
// (rowtile_pick with the row count) keep 256 x 2 tiles, which that form runs
// at 4 blocks per CU (65536 x 4096 float16: 343.0 against 345.9).  Rows of
// 513-768 chunks run 256 x 4 tiles rather than 256 x 3: layer norm, float32
// 2560 / 3072 values 236.7 / 276.9 -> 226.6 / 264.8 us at 32768 rows (61.1 /
// 71.3 -> 58.9 / 68.2 at 8192), float16 6144 values 277.4 -> 268.5, float16
// 5120 within 1 % either way.
constexpr AutoEntry kAutoNorm[] = {
    {4, 17}, {8, 18}, {16, 0}, {32, 1}, {64, 2}, {128, 3}, {192, 15}, {256, 13}, {512, 5},
    {1024, 7}, {1536, 8}, {2048, 9}, {3072, 10}, {4096, 11},
};
constexpr int kGeom256x2 = 16;  // 256-lane groups of 2 chunks per lane
// Rows of 161-256 chunks in launches of 16384 rows or more (below the
// single-tile size) run one wavefront per row, 4 chunks per lane, instead of
// 192- or 256-lane groups: layer norm float16 1536 / 1792 / 2048 values at
// 32768 rows 70.0 / 84.0 / 94.3 -> 66.9 / 79.1 / 88.9 us, at 131072 rows
// 1536 / 1792: 278.0 / 339.2 -> 262.0 / 302.1; float32 768 at 131072 rows
// 276.5 -> 265.7; RMS float16 1792 at 131072 rows 329.2 -> 304.1.  At 8192
// rows the wider groups were 1-4 % faster, at 160 chunks (float16 1280) the
// two equal.  Large launches of 161-192 chunks take it too (262144 rows:
// layer norm float16 1536 / 1408 values 565.4 / 518.1 -> 531.6 / 495.2 us,
// float32 768 563.7 -> 534.0, RMS float16 1536 565.1 -> 523.1); those of
// 193-256 keep their single-tile 256 x 1 tiles (float32 1024 at 131072
// rows: 339.6 against 355.0).
constexpr int kGeom64x4 = 4;
// float32 layer norm rows of 1537-2048 chunks (whole 128-byte lines) run
// 1024 x 3 tiles in the single-tile form rather than 512 x 4 walking (which
// holds one block per CU), one process, walking -> single-tile at 4096 /
// 8192 / 32768 rows: 6400 values 84.4 / 168.4 / 636.3 -> 79.2 / 151.2 /
// 589.5 us, 7168 values 91.2 / 178.9 / 680.7 -> 86.2 / 163.7 / 641.4, 8192
// values 101.5 / 201.8 / 765.0 -> 97.0 / 188.6 / 735.9 (another box had 8192
// x 32768 at 807.3 against 815.8).  RMS (fewer registers) measured best on
// 512 x 4 walking.
constexpr int kGeom1024x3 = 10;
// BiasAdd (no reduction) keeps the wider groups: one wavefront per row was
// slower at 192 chunks (1024 x 768 float32: 3.74 against 3.54 us).
constexpr AutoEntry kAutoExact[] = {
    {4, 17}, {8, 18}, {16, 0}, {32, 1}, {64, 2}, {128, 12}, {192, 15}, {256, 13}, {512, 16},
    {768, 6}, {1024, 7}, {1536, 8}, {2048, 9}, {3072, 10}, {4096, 11},
};
// Normalizations with a skip broadcast over the batch (skip-stationary
// blocks): rows of 65-128 chunks one wavefront per row (2 chunks per lane),
// 193-256 one wavefront of 4 chunks per lane, 257-512 128-lane groups of 4:
// layer norm float16 (256, 128, 768) / (16, 4096, 2048) / (64, 512, 4096)
// 27.8 / 115.4 / 97.9 -> 21.8 / 96.5 / 96.2 us, float32 (64, 512, 1024) 51.3
// -> 49.8, against the 128 x 1 / 256 x 1 / 256 x 2 tiles.
constexpr AutoEntry kAutoBroadcast[] = {
    {4, 17}, {8, 18}, {16, 0}, {32, 1}, {64, 2}, {128, 3}, {192, 15}, {256, 4}, {512, 5},
    {768, 6}, {1024, 7}, {1536, 8}, {2048, 9}, {3072, 10}, {4096, 11},
};
// BiasSoftmax streams one tensor in and one out and has no per-column
// parameters; on MI355X it runs fastest with two to four chunks per lane
// (more independent loads in flight per lane, fewer lanes per reduction)
// until a row needs several wavefronts (measured over 2..2048 chunks).
constexpr AutoEntry kAutoSoftmax[] = {
    {4, 17},   {8, 18},   {16, 19},  {32, 20},   {64, 21},   {128, 22},  {256, 4},
    {512, 5},  {1024, 14}, {2048, 9}, {3072, 10}, {4096, 11},
};

// Automatic choice by elements per row (measured on MI355X: four elements
// per lane up to 512 per row, eight beyond).
constexpr AutoEntry kAutoElem[] = {
    {4, 0},    {8, 1},     {16, 2},    {32, 3},    {64, 4},    {128, 5},   {256, 6},
    {512, 7},  {1024, 8}, {2048, 9}, {4096, 10}, {8192, 11}, {16384, 12},
};

// Generic kernel, chunked form: rows of whole 16-byte chunks with every
// tensor 16-byte aligned (the automatic choice sends such rows here only
// when they are too long for the other families and no workspace came with
// the call).  One 1024-lane block per row (persistent), chunk c of the row
// on lane c mod 1024 in every pass, kGenChunkBatch chunks loaded per lane
// before they are used.  The normalizations read the row twice: pass 1
// forms the sums and their statistics relative to the row's first sum
// (per lane: count, mean and M2 of each chunk merged with Chan's update;
// then across the block), pass 2 forms the sums again, writes the residual
// and the output.  BiasSoftmax keeps a running maximum and rescaled sum per
// lane in pass 1 (at most one rescale per batch of 4 chunks), merged across
// the block before pass 2 writes the scaled exponentials.  BiasAdd is one
// pass.
// Pass 1 also parks the binary32 sums of the row's first chunks in LDS (as
// many as fit beside the reduction slots: 40,832 values), so pass 2 re-reads
// from HBM only the chunks beyond them.  Every chunk is read, parked and
// written by one lane, data before output, so an output may alias its input
// exactly and the parked sums need no barrier.
constexpr int kGenChunkBlock = 1024;
constexpr int kGenChunkBatch = 4;
constexpr int kGenParkBytes = 160 * 1024 - 2 * (kGenChunkBlock / 64) * 16;  // LDS beside `red`
// Chunks of a row whose sums the block parks: the row's, at most the LDS's.
template <typename T>
constexpr int gen_park_chunks(int hv) {
    constexpr int cap = kGenParkBytes / (4 * Elem<T>::kPerChunk);
    return hv < cap ? hv : cap;
}

struct Moments {  // count, mean and M2 of values relative to the row's shift
    float n, mean, m2;
};
__device__ __forceinline__ Moments merge_moments(Moments a, Moments b) {
    if (b.n == 0.0f) return a;
    if (a.n == 0.0f) return b;
    const float n = a.n + b.n;
    const float d = b.mean - a.mean;
    const float f = b.n / n;
    return Moments{n, a.mean + d * f, a.m2 + b.m2 + d * d * a.n * f};
}

template <typename T, int OP>
__global__ void __launch_bounds__(kGenChunkBlock) generic_chunk_kernel(const Args a) {
    using E = Elem<T>;
    using Raw = typename E::Raw;
    constexpr int V = E::kPerChunk;
    constexpr int W = kGenChunkBlock / 64;
    constexpr int B = kGenChunkBatch;
    constexpr float kLog2e = 1.4426950408889634f;
    constexpr float kNegInf = -__builtin_inff();
    constexpr int Q = V / 4;  // float4 words of binary32 sums per chunk
    __shared__ float4 red[2][W];
    extern __shared__ float4 park[];  // Q planes of lc chunks' sums
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int hv = a.hidden / V;
    const int lc = OP == kOpBiasAdd ? 0 : gen_park_chunks<T>(hv);
    const float h = static_cast<float>(a.hidden);
    const bool small_rows = a.rows <= 0xFFFFFFFFll;
    const bool bcast = a.skip_rows > 0 || a.skip_group > 0;
    const bool has_bias = a.bias != nullptr;
    const bool has_beta = a.beta != nullptr;
    const Raw* X = static_cast<const Raw*>(a.input);
    const Raw* S = static_cast<const Raw*>(a.skip);
    const Raw* Bz = static_cast<const Raw*>(a.bias);
    const Raw* Gm = static_cast<const Raw*>(a.gamma);
    const Raw* Bt = static_cast<const Raw*>(a.beta);
    Raw* O = static_cast<Raw*>(a.out);
    Raw* R = static_cast<Raw*>(a.residual);
    int buf = 0;
    auto put = [&](int c, const float* v) {
        if (c < lc) {
#pragma unroll
            for (int q = 0; q < Q; ++q) park[q * lc + c] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
        }
    };

    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
        const int64_t srow = skip_row_of(row, a, small_rows);
        const Raw* xp = X + row * hv;
        const Raw* sp = S + srow * hv;
        // The binary32 sums of chunk c, by the same operations in each pass.
        auto sums = [&](const Raw& xr, const Raw& sr, int c, float* v) {
            float xf[V], sf[V];
            E::widen(xr, xf);
            E::widen(sr, sf);
            if constexpr (OP == kOpBiasAdd) {
                float bf[V];
                E::widen(Bz[c], bf);
#pragma unroll
                for (int e = 0; e < V; ++e) v[e] = (xf[e] + bf[e]) + sf[e];
            } else {
#pragma unroll
                for (int e = 0; e < V; ++e) v[e] = xf[e] + sf[e];
                if (OP != kOpBiasSoftmax && has_bias) {
                    float bf[V];
                    E::widen(Bz[c], bf);
#pragma unroll
                    for (int e = 0; e < V; ++e) v[e] = v[e] + bf[e];
                }
            }
        };
        // Visit the lane's chunks in batches of B (chunks c0 + b * 1024):
        // every load of a batch is issued before the first is used.
        auto for_batches = [&](int start, auto&& body) {
#pragma unroll 1
            for (int c0 = start; c0 < hv; c0 += kGenChunkBlock * B) {
                Raw xr[B], sr[B];
#pragma unroll
                for (int b = 0; b < B; ++b) {
                    const int c = c0 + b * kGenChunkBlock;
                    xr[b] = sr[b] = E::zero();
                    if (c < hv) {
                        xr[b] = __builtin_nontemporal_load(xp + c);
                        sr[b] = bcast ? sp[c] : __builtin_nontemporal_load(sp + c);
                    }
                }
                float v[B][V];
#pragma unroll
                for (int b = 0; b < B; ++b)
                    if (c0 + b * kGenChunkBlock < hv) sums(xr[b], sr[b], c0 + b * kGenChunkBlock, v[b]);
                body(c0, v);
            }
        };
        auto for_chunks = [&](auto&& body) {
            for_batches(tid, [&](int c0, float (&v)[B][V]) {
#pragma unroll
                for (int b = 0; b < B; ++b)
                    if (c0 + b * kGenChunkBlock < hv) body(c0 + b * kGenChunkBlock, v[b]);
            });
        };
        // Pass 2: parked sums from LDS, then the rest formed again from HBM
        // in batches from the lane's first chunk past the parked ones.
        auto for_chunks_again = [&](auto&& body) {
#pragma unroll 1
            for (int c = tid; c < lc; c += kGenChunkBlock) {
                float v[V];
#pragma unroll
                for (int q = 0; q < Q; ++q) {
                    const float4 p = park[q * lc + c];
                    v[4 * q] = p.x;
                    v[4 * q + 1] = p.y;
                    v[4 * q + 2] = p.z;
                    v[4 * q + 3] = p.w;
                }
                body(c, v);
            }
            const int first = tid >= lc ? tid : tid + (lc - tid + kGenChunkBlock - 1) / kGenChunkBlock * kGenChunkBlock;
            for_batches(first, [&](int c0, float (&v)[B][V]) {
#pragma unroll
                for (int b = 0; b < B; ++b)
                    if (c0 + b * kGenChunkBlock < hv) body(c0 + b * kGenChunkBlock, v[b]);
            });
        };

        if constexpr (OP == kOpBiasAdd) {
            for_chunks([&](int c, const float* v) { __builtin_nontemporal_store(E::narrow(v), O + row * hv + c); });
            continue;
        }

        if constexpr (OP == kOpBiasSoftmax) {
            // Per lane: the running maximum m of its batches and the sum of
            // 2^((z - m) log2 e), rescaled once per batch that raises m.
            float m = kNegInf, sm = 0.0f;
            for_batches(tid, [&](int c0, float (&v)[B][V]) {
#pragma unroll
                for (int b = 0; b < B; ++b) {
                    const int c = c0 + b * kGenChunkBlock;
                    if (c < hv) {
                        put(c, v[b]);
                    } else {
#pragma unroll
                        for (int e = 0; e < V; ++e) v[b][e] = kNegInf;
                    }
                }
                float bm = kNegInf;
#pragma unroll
                for (int b = 0; b < B; ++b)
#pragma unroll
                    for (int e = 0; e < V; ++e) bm = __builtin_fmaxf(bm, v[b][e]);
                if (bm > m) {
                    sm = sm * __builtin_amdgcn_exp2f((m - bm) * kLog2e);
                    m = bm;
                }
                const float r = m != kNegInf ? m : 0.0f;
                float cs = 0.0f;
#pragma unroll
                for (int b = 0; b < B; ++b)
#pragma unroll
                    for (int e = 0; e < V; ++e) cs += __builtin_amdgcn_exp2f((v[b][e] - r) * kLog2e);
                sm += cs;
            });
            const float mw = wave_max(m);
            const float sw = wave_sum(sm * (m != kNegInf ? __builtin_amdgcn_exp2f((m - mw) * kLog2e) : 0.0f));
            if ((tid & 63) == 0) red[buf][wave] = make_float4(mw, sw, 0.0f, 0.0f);
            __syncthreads();
            float M = kNegInf;
#pragma unroll
            for (int w = 0; w < W; ++w) M = __builtin_fmaxf(M, red[buf][w].x);
            float tot = 0.0f;
#pragma unroll
            for (int w = 0; w < W; ++w) {
                const float4 p = red[buf][w];
                tot += p.y * (p.x != kNegInf ? __builtin_amdgcn_exp2f((p.x - M) * kLog2e) : 0.0f);
            }
            buf ^= 1;
            const float scale = 1.0f / tot;
            for_chunks_again([&](int c, const float* v) {
                float y[V];
#pragma unroll
                for (int e = 0; e < V; ++e) y[e] = __builtin_amdgcn_exp2f((v[e] - M) * kLog2e) * scale;
                __builtin_nontemporal_store(E::narrow(y), O + row * hv + c);
            });
            continue;
        }

        // Normalizations.  Layer norm takes its statistics relative to the
        // row's first sum, read by every lane before the block's first
        // barrier (which precedes every store of the row).
        float shift = 0.0f;
        if constexpr (OP == kOpLayerNorm) {
            shift = E::load1(a.input, row * a.hidden) + E::load1(a.skip, srow * a.hidden);
            if (has_bias) shift = shift + E::load1(a.bias, 0);
        }
        float mean_rel = 0.0f, var;
        if constexpr (OP == kOpSimplified) {
            float sq = 0.0f;
            for_chunks([&](int c, const float* v) {
                put(c, v);
#pragma unroll
                for (int e = 0; e < V; ++e) sq += v[e] * v[e];
            });
            const float ws = wave_sum(sq);
            if ((tid & 63) == 0) red[buf][wave] = make_float4(ws, 0.0f, 0.0f, 0.0f);
            __syncthreads();
            float tot = 0.0f;
#pragma unroll
            for (int w = 0; w < W; ++w) tot += red[buf][w].x;
            buf ^= 1;
            var = tot / h;
        } else {
            Moments mo{0.0f, 0.0f, 0.0f};
            for_chunks([&](int c, const float* v) {
                put(c, v);
                float cm = 0.0f;
#pragma unroll
                for (int e = 0; e < V; ++e) cm += v[e] - shift;
                cm *= 1.0f / V;
                float cq = 0.0f;
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    const float d = (v[e] - shift) - cm;
                    cq += d * d;
                }
                mo = merge_moments(mo, Moments{static_cast<float>(V), cm, cq});
            });
            // Across the wavefront (butterfly), then across the block.
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) {
                const Moments o{__shfl_xor(mo.n, off), __shfl_xor(mo.mean, off), __shfl_xor(mo.m2, off)};
                mo = merge_moments(mo, o);
            }
            if ((tid & 63) == 0) red[buf][wave] = make_float4(mo.n, mo.mean, mo.m2, 0.0f);
            __syncthreads();
            Moments t{0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int w = 0; w < W; ++w) {
                const float4 p = red[buf][w];
                t = merge_moments(t, Moments{p.x, p.y, p.z});
            }
            buf ^= 1;
            mean_rel = t.mean;
            var = t.m2 / h;
        }
        const float rstd = rsqrtf(var + a.eps);
        // Pass 2: the sums again, the residual and the output (writes only
        // after the row's statistics, i.e. after every read of pass 1).
        for_chunks_again([&](int c, const float* v) {
            if (R != nullptr) __builtin_nontemporal_store(E::narrow(v), R + row * hv + c);
            float gf[V], bf[V], y[V];
            E::widen(Gm[c], gf);
            if (has_beta) {
                E::widen(Bt[c], bf);
            } else {
#pragma unroll
                for (int e = 0; e < V; ++e) bf[e] = 0.0f;
            }
#pragma unroll
            for (int e = 0; e < V; ++e) {
                const float t = OP == kOpLayerNorm ? ((v[e] - shift) - mean_rel) * rstd : v[e] * rstd;
                y[e] = t * gf[e] + bf[e];
            }
            __builtin_nontemporal_store(E::narrow(y), O + row * hv + c);
        });
    }
}

template <typename T, int OP>
hipError_t launch_generic_t(const Args& a, hipStream_t st) {
    // Rows of whole 16-byte chunks with every tensor aligned: the chunked form.
    auto al = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
    if (a.hidden % Elem<T>::kPerChunk == 0 && al(a.input) && al(a.skip) && al(a.out) && al(a.residual) &&
        al(a.gamma) && al(a.beta) && al(a.bias)) {
        auto kernel = generic_chunk_kernel<T, OP>;
        const int lc = OP == kOpBiasAdd ? 0 : gen_park_chunks<T>(a.hidden / Elem<T>::kPerChunk);
        const size_t lds = static_cast<size_t>(lc) * Elem<T>::kPerChunk * sizeof(float);
        int cus = 0;
        hipError_t e = cu_count(&cus);
        if (e != hipSuccess) return e;
        int occ = 0;  // depends on the row's LDS footprint, so it is not cached
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, kGenChunkBlock, lds);
        if (e != hipSuccess) return e;
        if (occ < 1) return hipErrorInvalidConfiguration;
        int64_t blocks = static_cast<int64_t>(cus) * occ;
        if (a.rows < blocks) blocks = a.rows;
        Args arg = a;
        void* params[] = {&arg};
        return hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3(static_cast<unsigned>(blocks < 1 ? 1 : blocks)),
                               dim3(kGenChunkBlock), params, lds, st);
    }
    static int occ = 0;
    int64_t resident = 0;
    const hipError_t e = resident_blocks(generic_kernel<T, OP>, kGenericBlock, &occ, &resident);
    if (e != hipSuccess) return e;
    const int64_t blocks = a.rows < resident ? a.rows : resident;
    return launch_grid(generic_kernel<T, OP>, kGenericBlock, blocks < 1 ? 1 : blocks, a, st);
}

// Kernel names: "<op>generic_<t>", "<op>ldsrow_<t>", "<op>splitrow_<t>", "<op>regrow_<t>",
// "<op>rowtile_<t>_g<G>_c<CH>" and "<op>rowelem_<t>_g<G>_c<CH>" (element-wise
// row tiles), with "_b<block>" when the block is not the default max(256,
// G); <op> is empty
// for layer normalization, "rms_" for the simplified form, "biasadd_",
// "softmax_".
struct NameTable {
    char name[kNumOps][2][kIdsPerType][48];
    static void geom_name(char* dst, const char* op, const char* family, const char* type, const Geom& g) {
        const int default_block = g.g > 256 ? g.g : 256;
        if (g.block == default_block)
            snprintf(dst, 48, "%s%s_%s_g%d_c%d", op, family, type, g.g, g.ch);
        else
            snprintf(dst, 48, "%s%s_%s_g%d_c%d_b%d", op, family, type, g.g, g.ch, g.block);
    }
    NameTable() {
        const char* op_prefix[kNumOps] = {"", "rms_", "biasadd_", "softmax_"};
        const char* tn[2] = {"f32", "f16"};
        for (int op = 0; op < kNumOps; ++op) {
            for (int t = 0; t < 2; ++t) {
                for (int i = 0; i < kIdsPerType; ++i) {
                    char* dst = name[op][t][i];
                    const int gi = i - kRowtileFirst;
                    if (i == kGenericIndex) {
                        snprintf(dst, 48, "%sgeneric_%s", op_prefix[op], tn[t]);
                    } else if (i == kLdsRowIndex) {
                        snprintf(dst, 48, "%sldsrow_%s", op_prefix[op], tn[t]);
                    } else if (i == kSplitRowIndex) {
                        snprintf(dst, 48, "%ssplitrow_%s", op_prefix[op], tn[t]);
                    } else if (i == kRegRowIndex) {
                        snprintf(dst, 48, "%sregrow_%s", op_prefix[op], tn[t]);
                    } else if (gi >= 0 && gi < kNumGeoms) {
                        geom_name(dst, op_prefix[op], "rowtile", tn[t], kGeoms[gi]);
                    } else if (i >= kElemFirst && i < kElemFirst + kNumElemGeoms) {
                        geom_name(dst, op_prefix[op], "rowelem", tn[t], kElemGeoms[i - kElemFirst]);
                    } else if (Geom sg; i >= kSpanFirst &&
                               span_geometry(i - kSpanFirst, &sg.g, &sg.ch, &sg.block)) {
                        geom_name(dst, op_prefix[op], "span", tn[t], sg);
                    } else {
                        snprintf(dst, 48, "unknown");
                    }
                }
            }
        }
    }
};

}  // namespace

int rowtile_count() { return kNumGeoms; }

// The first entry of an automatic-choice table that holds `hv` chunks.
template <size_t N>
int auto_pick(const AutoEntry (&table)[N], int64_t hv) {
    for (const AutoEntry& e : table)
        if (hv <= e.max_chunks) return e.geom;
    return -1;
}

int rowtile_pick(int op, int64_t hidden, int dtype, bool broadcast, bool multiwave_only, int64_t rows) {
    const int v = dtype == 0 ? Elem<float>::kPerChunk : Elem<_Float16>::kPerChunk;
    if (hidden <= 0 || hidden % v != 0) return -1;
    const int64_t hv = hidden / v;
    const bool norm = !multiwave_only && !broadcast && (op == kOpLayerNorm || op == kOpSimplified);
    const bool large = single_tile_launch(rows, hidden, 16 / v);
    if (norm && hv > 256 && hv <= 512 && large) return kGeom256x2;
    if (norm && hv > 160 && hv <= 256 && rows >= 16384 && (hv <= 192 || !large)) return kGeom64x4;
    if (norm && op == kOpLayerNorm && v == 4 && hv > 1536 && hv <= 2048 && hidden * 4 % 128 == 0) return kGeom1024x3;
    if (!multiwave_only) {
        if (op == kOpBiasSoftmax) return auto_pick(kAutoSoftmax, hv);
        if (broadcast) return auto_pick(kAutoBroadcast, hv);
        return op == kOpBiasAdd ? auto_pick(kAutoExact, hv) : auto_pick(kAutoNorm, hv);
    }
    int best = -1;  // smallest capacity among groups of two or more wavefronts
    for (int i = 0; i < kNumGeoms; ++i) {
        if (kGeoms[i].g < 128) continue;
        const int64_t cap = static_cast<int64_t>(kGeoms[i].g) * kGeoms[i].ch;
        if (cap < hv) continue;
        if (best < 0 || cap < static_cast<int64_t>(kGeoms[best].g) * kGeoms[best].ch) best = i;
    }
    return best;
}

int elem_count() { return kNumElemGeoms; }

int elem_pick(int op, int64_t hidden) {
    (void)op;
    if (hidden <= 0) return -1;
    for (const AutoEntry& e : kAutoElem)
        if (hidden <= e.max_chunks) return e.geom;
    return -1;
}

Tiling elem_tiling(int geometry) {
    // Measured: two tiles per block walked in address order, except for
    // 1024-lane rows, which run best on a persistent grid.
    Tiling t;
    const bool wide = geometry >= 0 && geometry < kNumElemGeoms && kElemGeoms[geometry].g >= 1024;
    t.tiles_per_block = wide ? 0 : 2;
    t.mode = wide ? kTileStrided : kTileContiguous;
    return t;
}

bool elem_holds(int geometry, int64_t hidden) {
    if (geometry < 0 || geometry >= kNumElemGeoms || hidden <= 0) return false;
    return hidden <= static_cast<int64_t>(kElemGeoms[geometry].g) * kElemGeoms[geometry].ch;
}

bool rowtile_holds(int geometry, int64_t hidden, int dtype) {
    const int v = dtype == 0 ? Elem<float>::kPerChunk : Elem<_Float16>::kPerChunk;
    if (geometry < 0 || geometry >= kNumGeoms || hidden <= 0 || hidden % v != 0) return false;
    return hidden / v <= static_cast<int64_t>(kGeoms[geometry].g) * kGeoms[geometry].ch;
}

const char* kernel_name(int kernel_id) {
    static const NameTable table;  // built once, thread-safe initialization
    if (kernel_id < 0 || kernel_id >= kNumOps * 2 * kIdsPerType) return "unknown";
    const int op = kernel_id / (2 * kIdsPerType), t = kernel_id / kIdsPerType % 2;
    return table.name[op][t][kernel_id % kIdsPerType];
}

hipError_t launch_copy(void* dst, const void* src, int64_t chunks, hipStream_t st) {
    static int occ = 0;
    int64_t blocks = 0;
    const hipError_t e = resident_blocks(copy_kernel, kCopyBlock, &occ, &blocks);
    if (e != hipSuccess) return e;
    const int64_t need = (chunks + kCopyBlock - 1) / kCopyBlock;
    if (need < blocks) blocks = need;
    if (blocks < 1) blocks = 1;
    u32x4* d = static_cast<u32x4*>(dst);
    const u32x4* s = static_cast<const u32x4*>(src);
    void* params[] = {&d, &s, &chunks};
    return hipLaunchKernel(reinterpret_cast<const void*>(copy_kernel), dim3(static_cast<unsigned>(blocks)),
                           dim3(kCopyBlock), params, 0, st);
}

template <typename T, int OP>
hipError_t launch_ldsrow_t(const Args& a, hipStream_t st) {
    auto kernel = ldsrow_kernel<T, OP>;
    const size_t lds = static_cast<size_t>(a.hidden) * sizeof(float);
    int cus = 0;
    hipError_t e = cu_count(&cus);
    if (e != hipSuccess) return e;
    int occ = 0;  // depends on the row's LDS footprint, so it is not cached
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, kLdsBlock, lds);
    if (e != hipSuccess) return e;
    if (occ < 1) return hipErrorInvalidConfiguration;
    int64_t blocks = static_cast<int64_t>(cus) * occ;
    if (a.rows < blocks) blocks = a.rows;
    Args arg = a;
    void* params[] = {&arg};
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3(static_cast<unsigned>(blocks < 1 ? 1 : blocks)),
                           dim3(kLdsBlock), params, lds, st);
}

template <typename T>
hipError_t launch_generic_op(const Args& a, int op, hipStream_t st) {
    switch (op) {
        case kOpLayerNorm: return launch_generic_t<T, kOpLayerNorm>(a, st);
        case kOpSimplified: return launch_generic_t<T, kOpSimplified>(a, st);
        case kOpBiasAdd: return launch_generic_t<T, kOpBiasAdd>(a, st);
        case kOpBiasSoftmax: return launch_generic_t<T, kOpBiasSoftmax>(a, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_ldsrow(const Args& a, int op, int dtype, hipStream_t st) {
    if (op == kOpLayerNorm)
        return dtype == 0 ? launch_ldsrow_t<float, kOpLayerNorm>(a, st) : launch_ldsrow_t<_Float16, kOpLayerNorm>(a, st);
    if (op == kOpSimplified)
        return dtype == 0 ? launch_ldsrow_t<float, kOpSimplified>(a, st)
                          : launch_ldsrow_t<_Float16, kOpSimplified>(a, st);
    if (op == kOpBiasSoftmax)
        return dtype == 0 ? launch_ldsrow_t<float, kOpBiasSoftmax>(a, st)
                          : launch_ldsrow_t<_Float16, kOpBiasSoftmax>(a, st);
    return hipErrorInvalidValue;
}

bool ldsrow_holds(int op, int64_t hidden, int dtype) {
    const int v = dtype == 0 ? Elem<float>::kPerChunk : Elem<_Float16>::kPerChunk;
    return (op == kOpLayerNorm || op == kOpSimplified || op == kOpBiasSoftmax) && hidden > 0 && hidden % v == 0 &&
           hidden * static_cast<int64_t>(sizeof(float)) <= kLdsRowBytes;
}

hipError_t launch_generic(const Args& a, int op, int dtype, hipStream_t st) {
    return dtype == 0 ? launch_generic_op<float>(a, op, st) : launch_generic_op<_Float16>(a, op, st);
}

// The row tiles of each operation are compiled in their own translation unit
// (skipln_rowtile_op.hip, once per operation).
hipError_t launch_elem(const Args& a, int op, int dtype, int geometry, Tiling tiling, hipStream_t st) {
    switch (op) {
        case kOpLayerNorm: return launch_elem_for<kOpLayerNorm>(a, dtype, geometry, tiling, st);
        case kOpSimplified: return launch_elem_for<kOpSimplified>(a, dtype, geometry, tiling, st);
        case kOpBiasAdd: return launch_elem_for<kOpBiasAdd>(a, dtype, geometry, tiling, st);
        case kOpBiasSoftmax: return launch_elem_for<kOpBiasSoftmax>(a, dtype, geometry, tiling, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t rowtile_occupancy(int op, int dtype, int geometry, int form, int blocks_per_cu, int* out) {
    switch (op) {
        case kOpLayerNorm: return rowtile_occupancy_for<kOpLayerNorm>(dtype, geometry, form, blocks_per_cu, out);
        case kOpSimplified: return rowtile_occupancy_for<kOpSimplified>(dtype, geometry, form, blocks_per_cu, out);
        case kOpBiasAdd: return rowtile_occupancy_for<kOpBiasAdd>(dtype, geometry, form, blocks_per_cu, out);
        case kOpBiasSoftmax: return rowtile_occupancy_for<kOpBiasSoftmax>(dtype, geometry, form, blocks_per_cu, out);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_rowtile(const Args& a, int op, int dtype, int geometry, Tiling tiling, hipStream_t st) {
    switch (op) {
        case kOpLayerNorm: return launch_rowtile_for<kOpLayerNorm>(a, dtype, geometry, tiling, st);
        case kOpSimplified: return launch_rowtile_for<kOpSimplified>(a, dtype, geometry, tiling, st);
        case kOpBiasAdd: return launch_rowtile_for<kOpBiasAdd>(a, dtype, geometry, tiling, st);
        case kOpBiasSoftmax: return launch_rowtile_for<kOpBiasSoftmax>(a, dtype, geometry, tiling, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace skipln
