// Device-side building blocks shared by the row kernels (gfx950, wave64):
// 16-byte chunk element types, DPP/swizzle cross-lane reductions, and the
// skip-row mapping.  Included by the kernel sources only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "skipln_internal.h"

namespace skipln {
namespace device {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Streaming outputs are written through buffer resources (a row tile's base
// and size in scalar registers) with one of two cache policies (bit 0 sc0,
// bit 1 nt, bit 4 sc1): non-temporal, or non-temporal with system-scope
// coherence (sc0 sc1).  Measured on MI355X, the second moves large
// read/write streams about 4 % faster (a 4 GiB two-read/two-write layer
// norm: 712 against 739 us) and small launches slower (12.6 MB: 4.9
// against 4.3 us); the launcher picks it by the bytes a launch writes
// (Args::store_through).
constexpr int kStoreStream = 2;
constexpr int kStoreThrough = 19;
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format

// Buffer resource over `bytes` bytes at `base` (bytes <= 2^31 - 1): accesses
// at or past `bytes` are dropped (stores) or read zero (loads).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), bytes, kRsrcWord3);
}

// ------------------------------------------------------------------------
// Element types: a 16-byte chunk holds kPerChunk elements.
// ------------------------------------------------------------------------
template <typename T>
struct Elem;

template <>
struct Elem<float> {
    typedef u32x4 Raw;
    static constexpr int kPerChunk = 4;
    __device__ __forceinline__ static Raw zero() { return u32x4{0, 0, 0, 0}; }
    // Components are passed by value: __builtin_bit_cast applied directly to
    // a vector component (r.y) reads component 0 with this compiler.
    __device__ __forceinline__ static void widen(const u32x4& r, float* f) {
        f[0] = __uint_as_float(r.x);
        f[1] = __uint_as_float(r.y);
        f[2] = __uint_as_float(r.z);
        f[3] = __uint_as_float(r.w);
    }
    // f = a + b and y = t g + b element by element (one rounding each); the
    // binary16 forms below round the same way.
    __device__ __forceinline__ static void widen_add(const u32x4& a, const u32x4& b, float* f) {
        f[0] = __uint_as_float(a.x) + __uint_as_float(b.x);
        f[1] = __uint_as_float(a.y) + __uint_as_float(b.y);
        f[2] = __uint_as_float(a.z) + __uint_as_float(b.z);
        f[3] = __uint_as_float(a.w) + __uint_as_float(b.w);
    }
    __device__ __forceinline__ static void widen_fma(const float* t, const u32x4& g, const u32x4& b, float* y) {
        y[0] = __builtin_fmaf(t[0], __uint_as_float(g.x), __uint_as_float(b.x));
        y[1] = __builtin_fmaf(t[1], __uint_as_float(g.y), __uint_as_float(b.y));
        y[2] = __builtin_fmaf(t[2], __uint_as_float(g.z), __uint_as_float(b.z));
        y[3] = __builtin_fmaf(t[3], __uint_as_float(g.w), __uint_as_float(b.w));
    }
    __device__ __forceinline__ static u32x4 narrow(const float* f) {
        u32x4 r;
        r.x = __float_as_uint(f[0]);
        r.y = __float_as_uint(f[1]);
        r.z = __float_as_uint(f[2]);
        r.w = __float_as_uint(f[3]);
        return r;
    }
    __device__ __forceinline__ static float load1(const void* p, int64_t i) {
        return static_cast<const float*>(p)[i];
    }
    __device__ __forceinline__ static void store(const Raw& v, __amdgpu_buffer_rsrc_t r, int voff, int soff,
                                                 bool through) {
        if (through)
            __builtin_amdgcn_raw_buffer_store_b128(v, r, voff, soff, kStoreThrough);
        else
            __builtin_amdgcn_raw_buffer_store_b128(v, r, voff, soff, kStoreStream);
    }
    __device__ __forceinline__ static void store1(void* p, int64_t i, float v) {
        static_cast<float*>(p)[i] = v;
    }
};

template <>
struct Elem<_Float16> {
    typedef u32x4 Raw;
    static constexpr int kPerChunk = 8;
    __device__ __forceinline__ static Raw zero() { return u32x4{0, 0, 0, 0}; }
    __device__ __forceinline__ static float lo(unsigned w) {
        return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<unsigned short>(w & 0xFFFFu)));
    }
    __device__ __forceinline__ static float hi(unsigned w) {
        return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<unsigned short>(w >> 16)));
    }
    // Round to nearest even: a two-element vector conversion, one packed
    // conversion instruction (v_cvt_pk_f16_f32, the default rounding mode)
    // instead of two conversions, a shift and an or.
    __device__ __forceinline__ static unsigned pack(float a, float b) {
        typedef float F2 __attribute__((ext_vector_type(2)));
        typedef _Float16 H2 __attribute__((ext_vector_type(2)));
        return __builtin_bit_cast(unsigned, __builtin_convertvector(F2{a, b}, H2));
    }
    __device__ __forceinline__ static void widen(const u32x4& r, float* f) {
        f[0] = lo(r.x); f[1] = hi(r.x);
        f[2] = lo(r.y); f[3] = hi(r.y);
        f[4] = lo(r.z); f[5] = hi(r.z);
        f[6] = lo(r.w); f[7] = hi(r.w);
    }
    // f = a + b element by element in binary32: one mixed-precision fma
    // a * 1 + b per element (v_fma_mix_f32 reads either half of a register
    // as a binary16 operand and widens it exactly), so each sum is rounded
    // once, as when both halves are widened and then added, in one
    // instruction instead of three.  The compiler folds a widening fma by 1
    // into a plain add and does not form this instruction by itself.
    __device__ __forceinline__ static float add_lo(unsigned a, unsigned b) {
        float r;
        asm("v_fma_mix_f32 %0, %1, 1.0, %2 op_sel_hi:[1,0,1]" : "=v"(r) : "v"(a), "v"(b));
        return r;
    }
    __device__ __forceinline__ static float add_hi(unsigned a, unsigned b) {
        float r;
        asm("v_fma_mix_f32 %0, %1, 1.0, %2 op_sel:[1,0,1] op_sel_hi:[1,0,1]" : "=v"(r) : "v"(a), "v"(b));
        return r;
    }
    __device__ __forceinline__ static void widen_add(const u32x4& a, const u32x4& b, float* f) {
        f[0] = add_lo(a.x, b.x); f[1] = add_hi(a.x, b.x);
        f[2] = add_lo(a.y, b.y); f[3] = add_hi(a.y, b.y);
        f[4] = add_lo(a.z, b.z); f[5] = add_hi(a.z, b.z);
        f[6] = add_lo(a.w, b.w); f[7] = add_hi(a.w, b.w);
    }
    // y = t g + b: the binary32 t times g's half plus b's half.
    __device__ __forceinline__ static float fma_lo(float t, unsigned g, unsigned b) {
        float r;
        asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel_hi:[0,1,1]" : "=v"(r) : "v"(t), "v"(g), "v"(b));
        return r;
    }
    __device__ __forceinline__ static float fma_hi(float t, unsigned g, unsigned b) {
        float r;
        asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[0,1,1] op_sel_hi:[0,1,1]" : "=v"(r) : "v"(t), "v"(g), "v"(b));
        return r;
    }
    __device__ __forceinline__ static void widen_fma(const float* t, const u32x4& g, const u32x4& b, float* y) {
        y[0] = fma_lo(t[0], g.x, b.x); y[1] = fma_hi(t[1], g.x, b.x);
        y[2] = fma_lo(t[2], g.y, b.y); y[3] = fma_hi(t[3], g.y, b.y);
        y[4] = fma_lo(t[4], g.z, b.z); y[5] = fma_hi(t[5], g.z, b.z);
        y[6] = fma_lo(t[6], g.w, b.w); y[7] = fma_hi(t[7], g.w, b.w);
    }
    __device__ __forceinline__ static u32x4 narrow(const float* f) {
        u32x4 r;
        r.x = pack(f[0], f[1]);
        r.y = pack(f[2], f[3]);
        r.z = pack(f[4], f[5]);
        r.w = pack(f[6], f[7]);
        return r;
    }
    __device__ __forceinline__ static float load1(const void* p, int64_t i) {
        return static_cast<float>(static_cast<const _Float16*>(p)[i]);
    }
    __device__ __forceinline__ static void store(const Raw& v, __amdgpu_buffer_rsrc_t r, int voff, int soff,
                                                 bool through) {
        if (through)
            __builtin_amdgcn_raw_buffer_store_b128(v, r, voff, soff, kStoreThrough);
        else
            __builtin_amdgcn_raw_buffer_store_b128(v, r, voff, soff, kStoreStream);
    }
    __device__ __forceinline__ static void store1(void* p, int64_t i, float v) {
        static_cast<_Float16*>(p)[i] = static_cast<_Float16>(v);
    }
};

// Element-wise access (rows that are not whole 16-byte chunks, or tensors
// not 16-byte aligned): a "chunk" of one element, loaded and stored on its
// own.  Same interface as Elem.
template <typename T>
struct Single;

template <>
struct Single<float> {
    typedef unsigned int Raw;
    static constexpr int kPerChunk = 1;
    __device__ __forceinline__ static Raw zero() { return 0u; }
    __device__ __forceinline__ static void widen(const Raw& r, float* f) { f[0] = __uint_as_float(r); }
    __device__ __forceinline__ static Raw narrow(const float* f) { return __float_as_uint(f[0]); }
    __device__ __forceinline__ static void widen_fma(const float* t, const Raw& g, const Raw& b, float* y) {
        float u, v;
        widen(g, &u);
        widen(b, &v);
        y[0] = __builtin_fmaf(t[0], u, v);
    }
    __device__ __forceinline__ static void store(const Raw& v, __amdgpu_buffer_rsrc_t r, int voff, int soff,
                                                 bool through) {
        if (through)
            __builtin_amdgcn_raw_buffer_store_b32(v, r, voff, soff, kStoreThrough);
        else
            __builtin_amdgcn_raw_buffer_store_b32(v, r, voff, soff, kStoreStream);
    }
};

template <>
struct Single<_Float16> {
    typedef unsigned short Raw;
    static constexpr int kPerChunk = 1;
    __device__ __forceinline__ static Raw zero() { return 0; }
    __device__ __forceinline__ static void widen(const Raw& r, float* f) {
        f[0] = static_cast<float>(__builtin_bit_cast(_Float16, r));
    }
    __device__ __forceinline__ static void widen_fma(const float* t, const Raw& g, const Raw& b, float* y) {
        float u, v;
        widen(g, &u);
        widen(b, &v);
        y[0] = __builtin_fmaf(t[0], u, v);
    }
    // Round to nearest even.
    __device__ __forceinline__ static Raw narrow(const float* f) {
        return __builtin_bit_cast(unsigned short, static_cast<_Float16>(f[0]));
    }
    __device__ __forceinline__ static void store(const Raw& v, __amdgpu_buffer_rsrc_t r, int voff, int soff,
                                                 bool through) {
        if (through)
            __builtin_amdgcn_raw_buffer_store_b16(v, r, voff, soff, kStoreThrough);
        else
            __builtin_amdgcn_raw_buffer_store_b16(v, r, voff, soff, kStoreStream);
    }
};

// ------------------------------------------------------------------------
// Cross-lane reductions with DPP (data-parallel primitives: a VALU operand
// read from another lane of the same row of 16 lanes, no LDS traffic).
// ------------------------------------------------------------------------
// Lanes that a DPP move does not write (rows outside row_mask) return `Id`,
// the identity of the reduction: 0 for sums, -inf for maxima.
template <int Ctrl, int RowMask = 0xF>
__device__ __forceinline__ float dpp(float v, float id) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, id),
                                                                 __builtin_bit_cast(int, v), Ctrl, RowMask, 0xF,
                                                                 false));
}

constexpr int kQuadSwap1 = 0xB1;    // quad_perm [1,0,3,2]: lane ^ 1
constexpr int kQuadSwap2 = 0x4E;    // quad_perm [2,3,0,1]: lane ^ 2
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;
constexpr int kRowBcast15 = 0x142;  // lane 15 of each row into the next row
constexpr int kRowBcast31 = 0x143;  // lane 31 into rows 2 and 3

struct SumOp {
    __device__ static float id() { return 0.0f; }
    __device__ static float apply(float a, float b) { return a + b; }
};
// IEEE maxNum (v_max_f32): a NaN operand yields the other one.
struct MaxOp {
    __device__ static float id() { return -__builtin_inff(); }
    __device__ static float apply(float a, float b) { return __builtin_fmaxf(a, b); }
};

// Reduction over aligned groups of G = 4, 8 or 16 lanes; every lane of a
// group gets the same bits (each step combines a commutative pair).
template <typename Op, int G>
__device__ __forceinline__ float reduce_upto16(float v) {
    static_assert(G == 4 || G == 8 || G == 16, "4, 8 or 16 lanes");
    v = Op::apply(v, dpp<kQuadSwap1>(v, Op::id()));
    v = Op::apply(v, dpp<kQuadSwap2>(v, Op::id()));
    if constexpr (G >= 8) v = Op::apply(v, dpp<kRowHalfMirror>(v, Op::id()));  // lane i <-> 7-i: other quad
    if constexpr (G >= 16) v = Op::apply(v, dpp<kRowMirror>(v, Op::id()));     // lane i <-> 15-i: other half
    return v;
}

// Reduction over the whole wavefront, returned as a wave-uniform value.
template <typename Op>
__device__ __forceinline__ float wave_reduce(float v) {
    v = reduce_upto16<Op, 16>(v);
    v = Op::apply(v, dpp<kRowBcast15, 0xA>(v, Op::id()));  // rows 1, 3 combine rows 0, 2
    v = Op::apply(v, dpp<kRowBcast31, 0xC>(v, Op::id()));  // rows 2, 3 combine rows 0+1
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

__device__ __forceinline__ float wave_sum(float v) { return wave_reduce<SumOp>(v); }
__device__ __forceinline__ float wave_max(float v) { return wave_reduce<MaxOp>(v); }

// Reduction over an aligned group of G lanes (G = 4, 8, 16, 32 or 64).
template <typename Op, int G>
__device__ __forceinline__ float group_reduce(float v) {
    static_assert(G == 4 || G == 8 || G == 16 || G == 32 || G == 64, "group of 4..64 lanes");
    if constexpr (G == 64) {
        return wave_reduce<Op>(v);
    } else if constexpr (G <= 16) {
        return reduce_upto16<Op, G>(v);
    } else {
        v = reduce_upto16<Op, 16>(v);
        // lane ^ 16 within each half-wave (swizzle bit mode: and 0x1F, xor 0x10)
        return Op::apply(v, __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F)));
    }
}

template <int G>
__device__ __forceinline__ float group_sum(float v) { return group_reduce<SumOp, G>(v); }

// Value of the first lane of each aligned group of G lanes (G <= 32: the
// group's lane 0; G >= 64: the wavefront's lane 0, wave-uniform).
template <int G>
__device__ __forceinline__ float group_first(float v) {
    if constexpr (G >= 64) {
        return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
    } else {
        // swizzle bit mode within 32 lanes: new lane = lane & and_mask
        constexpr int kPattern = G == 4 ? 0x001C : G == 8 ? 0x0018 : G == 16 ? 0x0010 : 0x0000;
        return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), kPattern));
    }
}

// Skip (bias) row read by data row `row`: the same row (exact), row mod
// skip_rows (cyclic reuse), or row / skip_group (consecutive groups of rows
// share one).  32-bit division whenever the row count fits.
__device__ __forceinline__ int64_t skip_row_of(int64_t row, const Args& a, bool small_rows) {
    if (a.skip_group > 0)
        return small_rows ? static_cast<int64_t>(static_cast<uint32_t>(row) / static_cast<uint32_t>(a.skip_group))
                          : row / a.skip_group;
    if (a.skip_rows > 0)
        return small_rows ? static_cast<int64_t>(static_cast<uint32_t>(row) % static_cast<uint32_t>(a.skip_rows))
                          : row % a.skip_rows;
    return row;
}

}  // namespace device
}  // namespace skipln
