// Device helpers shared by the kernels of this library (gfx950 only): bf16
// vector types, the MFMA wrappers and their operand layout, LDS fragment
// reads, bf16 conversions, DPP wave scans and raw buffer loads.
//
// MFMA operand layout (16x16 tiles, lane l, l16 = l % 16, lq = l / 16,
// r = 0..3):
//   A fragment (rows x k):  row l16, k = 4*lq + r
//   B fragment (k x cols):  col l16, k = 4*lq + r
//   C/D tile:               col l16, row = 4*lq + r
// so an MFMA result tile is directly the B fragment of the next product over
// its rows (and the A fragment of its transpose).  Every product runs on the
// 16x16x32 instruction used as two 16x16x16 products fused: lane slots 0-3
// carry one K16 block and slots 4-7 the next one, the same pairing on both
// operands.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdr_internal.h"

namespace gdr {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int v2u32 __attribute__((ext_vector_type(2)));
typedef unsigned int v4u32 __attribute__((ext_vector_type(4)));

constexpr int C = kChunk;
constexpr float kLog2e = 1.44269504088896340736f;

__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// one K16 block on the 16x16x32 instruction, upper slots zero
__device__ __forceinline__ f32x4 mfma16z(bf16x4 a, bf16x4 b, f32x4 c) {
    const bf16x4 z = {};
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_shufflevector(a, z, 0, 1, 2, 3, 4, 5, 6, 7),
                                                   __builtin_shufflevector(b, z, 0, 1, 2, 3, 4, 5, 6, 7),
                                                   c, 0, 0, 0);
}
// the 16x16x16 instruction, for the lane-layout self test only
__device__ __forceinline__ f32x4 mfma16(bf16x4 a, bf16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                     __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ bf16x4 ld4(const uint16_t *p) {   // 8-byte LDS read
    return *reinterpret_cast<const bf16x4 *>(p);
}
__device__ __forceinline__ bf16x4 cvt4(f32x4 x) {           // round to nearest even
    bf16x4 r;
    r[0] = (__bf16)x[0];
    r[1] = (__bf16)x[1];
    r[2] = (__bf16)x[2];
    r[3] = (__bf16)x[3];
    return r;
}
__device__ __forceinline__ f32x4 up4(bf16x4 x) {
    f32x4 r;
    r[0] = (float)x[0];
    r[1] = (float)x[1];
    r[2] = (float)x[2];
    r[3] = (float)x[3];
    return r;
}
__device__ __forceinline__ uint16_t bf16_bits(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
}
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }
template <int N>
struct IntC {
    static constexpr int value = N;
};
__device__ __forceinline__ bf16x4 neg4(bf16x4 x) {   // exact: flips the sign bits
    return __builtin_bit_cast(bf16x4, __builtin_bit_cast(v2u32, x) ^ 0x80008000u);
}

template <bool BF16>
__device__ __forceinline__ float load_scalar(const void *p, int64_t i) {
    if constexpr (BF16) {
        const uint16_t u = reinterpret_cast<const uint16_t *>(p)[i];
        return __uint_as_float(static_cast<uint32_t>(u) << 16);
    } else {
        return reinterpret_cast<const float *>(p)[i];
    }
}

// 8 consecutive elements of a row as 8 bf16 (16 bytes); f32 inputs are rounded.
template <bool BF16>
__device__ __forceinline__ uint4 load8(const void *p, int64_t i) {
    if constexpr (BF16) {
        return *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(p) + i);
    } else {
        const float4 x = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(p) + i);
        const float4 y = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(p) + i + 4);
        uint4 r;
        r.x = bf16_bits(x.x) | (static_cast<uint32_t>(bf16_bits(x.y)) << 16);
        r.y = bf16_bits(x.z) | (static_cast<uint32_t>(bf16_bits(x.w)) << 16);
        r.z = bf16_bits(y.x) | (static_cast<uint32_t>(bf16_bits(y.y)) << 16);
        r.w = bf16_bits(y.z) | (static_cast<uint32_t>(bf16_bits(y.w)) << 16);
        return r;
    }
}

// two 4-element pieces of a row as 8 bf16 (16 bytes); f32 inputs are rounded
template <bool BF16>
__device__ __forceinline__ uint4 load4x2(const void *p, int64_t i0, int64_t i1) {
    if constexpr (BF16) {
        const uint2 x = *reinterpret_cast<const uint2 *>(reinterpret_cast<const uint16_t *>(p) + i0);
        const uint2 y = *reinterpret_cast<const uint2 *>(reinterpret_cast<const uint16_t *>(p) + i1);
        return make_uint4(x.x, x.y, y.x, y.y);
    } else {
        const float4 x = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(p) + i0);
        const float4 y = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(p) + i1);
        uint4 r;
        r.x = bf16_bits(x.x) | (static_cast<uint32_t>(bf16_bits(x.y)) << 16);
        r.y = bf16_bits(x.z) | (static_cast<uint32_t>(bf16_bits(x.w)) << 16);
        r.z = bf16_bits(y.x) | (static_cast<uint32_t>(bf16_bits(y.y)) << 16);
        r.w = bf16_bits(y.z) | (static_cast<uint32_t>(bf16_bits(y.w)) << 16);
        return r;
    }
}

__device__ __forceinline__ uint16_t elem8(const uint4 &v, int e) {
    const uint32_t w = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
    return static_cast<uint16_t>((e & 1) ? (w >> 16) : (w & 0xFFFFu));
}

// x plus the value DPP control CTRL moves in (0 where no lane is moved in,
// or outside the rows ROW_MASK selects)
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add(float x) {
    return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xF, false));
}
// Inclusive prefix sum over the 64 lanes of a wave: scans within each
// 16-lane row (row shifts by 1, 2, 4, 8), then carries row totals with the
// row broadcasts of lane 15 (into rows 1 and 3) and lane 31 (into rows 2 and 3).
__device__ __forceinline__ float wave_inclusive_scan(float x) {
    x = dpp_add<0x111, 0xF>(x);
    x = dpp_add<0x112, 0xF>(x);
    x = dpp_add<0x114, 0xF>(x);
    x = dpp_add<0x118, 0xF>(x);
    x = dpp_add<0x142, 0xA>(x);
    x = dpp_add<0x143, 0xC>(x);
    return x;
}

__device__ __forceinline__ bf16x8 ld8(const uint16_t *p) {   // 16-byte LDS read
    return *reinterpret_cast<const bf16x8 *>(p);
}
__device__ __forceinline__ void st4(uint16_t *p, bf16x4 v) { *reinterpret_cast<bf16x4 *>(p) = v; }
// Transposing 8-byte LDS read (ds_read_b64_tr_b16): each lane names 8 bytes
// (4 elements); within every group of 16 lanes, slot r of lane i receives
// element i%4 of the piece named by lane 4r + i/4.
__device__ __forceinline__ bf16x4 ld4_tr(const uint16_t *p) {
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p)));
}
__device__ __forceinline__ bf16x8 ext8(bf16x4 a) { return __builtin_shufflevector(a, bf16x4{}, 0, 1, 2, 3, 4, 5, 6, 7); }

// wait until this wave's LDS accesses are complete (also a compiler barrier)
__device__ __forceinline__ void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Work-groups are dispatched round-robin over the 8 XCDs (each with its own
// L2), so blocks b and b + 8 run on one XCD at about the same time.  Over a
// grid of (item / hv, v-head item % hv) work items this renumbering gives
// such blocks the r = hv / hk v-heads that share a q/k head, so the second
// finds q and k in L2 (spans of 8 r items; a partial last span is left as is).
__device__ __forceinline__ int64_t gqa_xcd_item(int64_t item, int64_t grid, int hv, int hk) {
    const int64_t r = hv / hk;
    const int64_t span = 8 * r;
    const int64_t full = (grid / span) * span;
    if (r > 1 && item < full) {
        const int64_t w = item % span;
        item = (item - w) + (w % 8) * r + w / 8;
    }
    return item;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Raw buffer resource over [base, base + bytes): loads past the end return 0
// and stores past it are dropped, so one resource per chunk covers exactly the
// chunk's rows and the padding needs no branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t chunk_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), static_cast<short>(0),
                                             static_cast<int>(bytes), 0x00020000);
}
template <int BYTES>
__device__ __forceinline__ auto buf_load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    if constexpr (BYTES == 2) return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
    else if constexpr (BYTES == 4) return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
    else if constexpr (BYTES == 8) return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    else return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
// 4 consecutive elements at byte offset off as bf16 (f32 inputs are rounded).
// The loaded value is always bit-cast whole: indexing the builtin's result
// directly lets the compiler narrow the load to its first dword.
template <bool BF16>
__device__ __forceinline__ bf16x4 buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    if constexpr (BF16) return __builtin_bit_cast(bf16x4, buf_load<8>(r, off));
    else return cvt4(__builtin_bit_cast(f32x4, buf_load<16>(r, off)));
}
// 8 consecutive elements at byte offset off as bf16 (16 or 32 bytes)
template <bool BF16>
__device__ __forceinline__ bf16x8 buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    if constexpr (BF16) return __builtin_bit_cast(bf16x8, buf_load<16>(r, off));
    else return cat(buf_load4<false>(r, off), buf_load4<false>(r, off + 16));
}
template <bool BF16>
__device__ __forceinline__ float buf_load_scalar(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    if constexpr (BF16) return __uint_as_float(static_cast<uint32_t>(buf_load<2>(r, off)) << 16);
    else return __builtin_bit_cast(float, buf_load<4>(r, off));
}

// Column position of key index x within its block of 32 in a key-permuted LDS
// array: x = 16 h + 4 j + r is stored at 8 j + 4 h + r, so that one
// 16-byte read at 8 lq gives lane (l16, lq) the eight key slots of a 16x16x32
// MFMA operand, keys 4 lq + r and 16 + 4 lq + r, in the order of a C tile's
// rows (the same order on both operands, so the contraction is unchanged).
__device__ __forceinline__ int kpos(int x) { return (x & ~31) | ((x & 12) << 1) | ((x >> 2) & 4) | (x & 3); }
__device__ __forceinline__ bf16x8 kfrag8(const uint16_t *M, int pitch, int row0, int k0, int l16, int lq) {
    return ld8(M + (row0 + l16) * pitch + k0 + 8 * lq);
}
}  // namespace
}  // namespace gdr
