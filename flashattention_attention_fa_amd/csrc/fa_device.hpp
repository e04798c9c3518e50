// fa_device.hpp -- gfx950 device helpers shared by the attention kernels:
// MFMA operand types, 16-bit storage tags, lane exchanges, XCD-aware block
// remapping.  Device code only; nothing here is visible through the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 16-bit storage types.  mfma32: D = A*B + C on one 32x32x16 tile
// (v_mfma_f32_32x32x16_{bf16,f16}), fp32 accumulation.  Each lane holds 8
// consecutive contraction elements of A (row = lane%32) and of B
// (column = lane%32); lanes 32..63 hold the second half of the 16-wide
// contraction.  C: lane%32 is the column, register r of lane half h is row
// 8*(r/4) + 4*h + r%4.
// mfma16: D = A*B + C on one 16x16x32 tile (v_mfma_f32_16x16x32_*), same
// operand registers: lane group g = lane/16 holds contraction elements
// 8g..8g+7 of A row lane%16 and of B column lane%16; C: lane%16 is the
// column, register r is row 4g + r.
struct BF16 {
    typedef bf16x8 vec8;
    typedef __bf16 scalar;
    static __device__ __forceinline__ floatx16 mfma32(vec8 a, vec8 b, floatx16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ floatx4 mfma16(vec8 a, vec8 b, floatx4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};

struct FP16 {
    typedef f16x8 vec8;
    typedef _Float16 scalar;
    static __device__ __forceinline__ floatx16 mfma32(vec8 a, vec8 b, floatx16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ floatx4 mfma16(vec8 a, vec8 b, floatx4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
};

template <typename V>
__device__ __forceinline__ V as_vec8(u32x4 x) { return __builtin_bit_cast(V, x); }

__device__ __forceinline__ u32x4 zero4() { return u32x4{0u, 0u, 0u, 0u}; }

// Value held by lane (l ^ 32): the other half of the wave.
__device__ __forceinline__ float other_half(float x) { return __shfl_xor(x, 32, 64); }

// Raw buffer resource over [base, base + bytes): loads beyond `bytes` return
// zero in hardware, which gives free bounds handling for ragged tiles.
// 0x00020000 is the gfx9-family resource word 3 for untyped raw access.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// The same for a workgroup-uniform base and size that the compiler may hold
// in vector registers (e.g. after an integer division, which runs on the
// vector unit): reading them from the first lane keeps the resource in
// scalar registers instead of a loop over distinct lane values.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_uniform(const void *base,
                                                                   uint32_t bytes) {
    const uint64_t a = (uint64_t)(uintptr_t)base;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    return make_rsrc((const void *)(uintptr_t)(((uint64_t)hi << 32) | lo),
                     __builtin_amdgcn_readfirstlane(bytes));
}

__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 0);
}

// The same load marked non-temporal (cache policy sc0 nt) for data that is
// read exactly once, such as a key/value cache streamed by decode: it does
// not displace reusable lines and, measured on MI355X, streams about 14%
// faster than the default policy.
__device__ __forceinline__ u32x4 buffer_load16_stream(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 3);
}

// Direct global -> LDS copy of 16 bytes per lane (buffer_load_dwordx4 ... lds):
// lane i of the wave writes lds_base + 16*i; out-of-range reads store zeros.
// The LDS destination must be wave-uniform.  Completion is tracked by the
// vector-memory counter, like any load.
__device__ __forceinline__ void buffer_load16_lds(__amdgpu_buffer_rsrc_t r, uint32_t byte_off,
                                                  uint16_t *lds_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void *)lds_base, 16, (int)byte_off, 0, 0, 0);
}

// Wait until this wave's outstanding vector-memory operations (including
// direct-to-LDS copies) have completed: s_waitcnt vmcnt(0).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Transposing LDS read (ds_read_b64_tr_b16).  Within each 16-lane group, lane
// j supplies the address of 4 consecutive 16-bit elements M[j][0..3]; lane i
// receives M[4e + i/4][i%4] for e = 0..3.  With lane j pointing at
// X[r0 + j/4][c0 + 4*(j%4)] of a row-major tile X, lane i receives
// X[r0 + e][c0 + i], e = 0..3: four consecutive rows of one column.
__device__ __forceinline__ shortx4 lds_read_tr4(const uint16_t *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4 *)(p));
}

template <typename V>
__device__ __forceinline__ V join8(shortx4 lo, shortx4 hi) {
    typedef short shortx8 __attribute__((ext_vector_type(8)));
    const shortx8 x = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(V, x);
}

// max / sum of a value over the two halves of the wave (lanes l and l^32):
// v_permlane32_swap exchanges the halves without going through LDS.
__device__ __forceinline__ float max_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// max / sum over the four lane groups l, l^16, l^32, l^48 (the lanes that
// hold one column of a 16x16 MFMA result): the halves first, then
// v_permlane16_swap, which exchanges lane groups 0 and 1, and 2 and 3.
__device__ __forceinline__ float max_quarters(float x) {
    const float y = max_halves(x);
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y),
                                                    false, false);
    return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_quarters(float x) {
    const float y = sum_halves(x);
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y),
                                                    false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Workgroups are handed to the 8 XCDs round-robin (hardware id % 8).  Remap
// so that consecutive logical ids run on the same XCD and share its L2:
// hardware ids x, x+8, x+16, ... become one contiguous logical range.
__device__ __forceinline__ unsigned xcd_remap(unsigned id, unsigned total) {
    const unsigned kXcd = 8;
    const unsigned per = total / kXcd, rem = total % kXcd;
    const unsigned x = id % kXcd, idx = id / kXcd;
    return x < rem ? x * (per + 1) + idx : rem * (per + 1) + (x - rem) * per + idx;
}

}  // namespace fa
