// Streaming probe: 0-2 input streams to 0-2 output streams with the access
// pattern of the row kernels (16-byte non-temporal vector loads, stores
// through buffer resources with either store policy of the row kernels, one
// tile of BLOCK lanes x U chunks per workgroup).  It measures the HBM rates a
// kernel of that pattern can reach for each mix of reads and writes -- the
// attainable ceilings the row kernels are compared with.
//
// Tile order.  The dispatcher deals workgroups round-robin over the eight
// XCDs (workgroup b runs on XCD b mod 8), so in address order consecutive
// tiles land on different XCDs.  With a granule of g tiles the mapping
// instead hands each XCD g consecutive tiles per round of 8g: the address
// granularity at which the XCDs share the streams becomes g tiles -- what a
// row kernel has when one workgroup owns whole rows.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "skipln_device.h"
#include "skipln_internal.h"

namespace skipln {
namespace {
using device::u32x4;

template <int NR, int NW, int BLOCK, int kStreamCh>
__global__ void __launch_bounds__(BLOCK)
    stream_kernel(const u32x4* __restrict__ s0, const u32x4* __restrict__ s1, u32x4* __restrict__ d0,
                  u32x4* __restrict__ d1, int64_t chunks, int64_t granule, int through) {
    constexpr int kStreamBlock = BLOCK;
    constexpr int kStreamTile = BLOCK * kStreamCh;
    const int64_t b = blockIdx.x;
    int64_t tile = b;
    if (granule > 1) {
        // Position q of block b in its round of 8g blocks goes to XCD q mod 8
        // as that XCD's (q div 8)-th block of the round: tile (q mod 8) g +
        // q div 8 of the round.  A last, partial round keeps address order.
        const int64_t per_round = 8 * granule;
        const int64_t round = b / per_round;
        if ((round + 1) * per_round <= static_cast<int64_t>(gridDim.x)) {
            const int64_t q = b - round * per_round;
            tile = round * per_round + (q % 8) * granule + q / 8;
        }
    }
    const int64_t base = tile * kStreamTile + threadIdx.x;
    u32x4 v[kStreamCh];
#pragma unroll
    for (int k = 0; k < kStreamCh; ++k) {
        const int64_t c = base + k * kStreamBlock;
        v[k] = u32x4{static_cast<unsigned>(c), 0u, 0u, 0u};
        if (c < chunks) {
            if constexpr (NR >= 1) v[k] = __builtin_nontemporal_load(s0 + c);
            if constexpr (NR == 2) v[k] ^= __builtin_nontemporal_load(s1 + c);
        }
    }
    if constexpr (NW == 0) {
        // Reads only: fold the data so the loads stay; the fold is written
        // only if it equals a value the probe's inputs never produce.
        u32x4 f = v[0];
#pragma unroll
        for (int k = 1; k < kStreamCh; ++k) f ^= v[k];
        if (f.x == 0x9E3779B9u && f.y == 0x7F4A7C15u && f.z == 0x94D049BBu && f.w == 0x3C6EF372u && d0 != nullptr)
            d0[0] = f;
    } else {
        // Stores through buffer resources over the tile, with the row
        // kernels' two store policies (non-temporal, or non-temporal with
        // system-scope coherence).
        const int64_t t0 = tile * kStreamTile;
        const int64_t left = chunks - t0;
        const int bytes = static_cast<int>((left < kStreamTile ? left : kStreamTile) * 16);
        const __amdgpu_buffer_rsrc_t r0 = device::buffer_rsrc(d0 + t0, bytes);
        const __amdgpu_buffer_rsrc_t r1 = device::buffer_rsrc(NW == 2 ? d1 + t0 : d0 + t0, bytes);
        // The whole offset in the vector offset, the scalar offset zero: the
        // compiler then keeps the data registers of each 16-byte store from
        // being overwritten by the next instruction (it does not when the
        // scalar offset is a register).
        const int voff = static_cast<int>(threadIdx.x) * 16;
#pragma unroll
        for (int k = 0; k < kStreamCh; ++k) {
            const int64_t c = base + k * kStreamBlock;
            if (c < chunks) {
                device::Elem<float>::store(v[k], r0, voff + k * kStreamBlock * 16, 0, through != 0);
                if constexpr (NW == 2)
                    device::Elem<float>::store(v[k] + u32x4{1u, 1u, 1u, 1u}, r1, voff + k * kStreamBlock * 16, 0,
                                               through != 0);
            }
        }
    }
}

template <int NR, int NW, int BLOCK, int U>
hipError_t launch_stream_t(const void* s0, const void* s1, void* d0, void* d1, int64_t chunks, int64_t granule,
                           int through, hipStream_t st) {
    const u32x4* a = static_cast<const u32x4*>(s0);
    const u32x4* b = static_cast<const u32x4*>(s1);
    u32x4* c = static_cast<u32x4*>(d0);
    u32x4* d = static_cast<u32x4*>(d1);
    void* params[] = {&a, &b, &c, &d, &chunks, &granule, &through};
    const int64_t blocks = (chunks + BLOCK * U - 1) / (BLOCK * U);
    // A dispatch counts its work-items in 32 bits.
    if (blocks > 0x7FFFFFFF || blocks * BLOCK > 0xFFFFFFFFll) return hipErrorInvalidValue;
    return hipLaunchKernel(reinterpret_cast<const void*>(stream_kernel<NR, NW, BLOCK, U>),
                           dim3(static_cast<unsigned>(blocks)), dim3(BLOCK), params, 0, st);
}

template <int NR, int NW>
hipError_t launch_stream_mix(int block, int per_lane, const void* s0, const void* s1, void* d0, void* d1,
                             int64_t chunks, int64_t granule, int through, hipStream_t st) {
    switch (block * 8 + per_lane) {
        case 64 * 8 + 1: return launch_stream_t<NR, NW, 64, 1>(s0, s1, d0, d1, chunks, granule, through, st);
        case 64 * 8 + 4: return launch_stream_t<NR, NW, 64, 4>(s0, s1, d0, d1, chunks, granule, through, st);
        case 256 * 8 + 1: return launch_stream_t<NR, NW, 256, 1>(s0, s1, d0, d1, chunks, granule, through, st);
        case 256 * 8 + 4: return launch_stream_t<NR, NW, 256, 4>(s0, s1, d0, d1, chunks, granule, through, st);
        case 1024 * 8 + 1: return launch_stream_t<NR, NW, 1024, 1>(s0, s1, d0, d1, chunks, granule, through, st);
        case 1024 * 8 + 4: return launch_stream_t<NR, NW, 1024, 4>(s0, s1, d0, d1, chunks, granule, through, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool stream_shape_ok(int block, int per_lane) {
    return (block == 64 || block == 256 || block == 1024) && (per_lane == 1 || per_lane == 4);
}

hipError_t launch_stream(int reads, int writes, int block, int per_lane, int64_t granule, int through,
                         const void* s0, const void* s1, void* d0, void* d1, int64_t chunks, hipStream_t st) {
    switch (reads * 3 + writes) {
        case 1: return launch_stream_mix<0, 1>(block, per_lane, s0, s1, d0, d1, chunks, granule, through, st);
        case 2: return launch_stream_mix<0, 2>(block, per_lane, s0, s1, d0, d1, chunks, granule, through, st);
        case 3: return launch_stream_mix<1, 0>(block, per_lane, s0, s1, d0, d1, chunks, granule, through, st);
        case 4: return launch_stream_mix<1, 1>(block, per_lane, s0, s1, d0, d1, chunks, granule, through, st);
        case 5: return launch_stream_mix<1, 2>(block, per_lane, s0, s1, d0, d1, chunks, granule, through, st);
        case 6: return launch_stream_mix<2, 0>(block, per_lane, s0, s1, d0, d1, chunks, granule, through, st);
        case 7: return launch_stream_mix<2, 1>(block, per_lane, s0, s1, d0, d1, chunks, granule, through, st);
        case 8: return launch_stream_mix<2, 2>(block, per_lane, s0, s1, d0, d1, chunks, granule, through, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace skipln
