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

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 16-bit storage types.  mfma32: D = A*B + C on one 32x32x16 tile
// (v_mfma_f32_32x32x16_{bf16,f16}), fp32 accumulation.  Each lane holds 8
// consecutive contraction elements of A (row = lane%32) and of B
// (column = lane%32); lanes 32..63 hold the second half of the 16-wide
// contraction.  C: lane%32 is the column, register r of lane half h is row
// 8*(r/4) + 4*h + r%4.
struct BF16 {
    typedef bf16x8 vec8;
    typedef __bf16 scalar;
    static __device__ __forceinline__ floatx16 mfma32(vec8 a, vec8 b, floatx16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};

struct FP16 {
    typedef f16x8 vec8;
    typedef _Float16 scalar;
    static __device__ __forceinline__ floatx16 mfma32(vec8 a, vec8 b, floatx16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};

template <typename V>
__device__ __forceinline__ V as_vec8(u32x4 x) { return __builtin_bit_cast(V, x); }

__device__ __forceinline__ u32x4 zero4() { return u32x4{0u, 0u, 0u, 0u}; }

// Value held by lane (l ^ 32): the other half of the wave.
__device__ __forceinline__ float other_half(float x) { return __shfl_xor(x, 32, 64); }

// Workgroups are handed to the 8 XCDs round-robin (hardware id % 8).  Remap
// so that consecutive logical ids run on the same XCD and share its L2:
// hardware ids x, x+8, x+16, ... become one contiguous logical range.
__device__ __forceinline__ unsigned xcd_remap(unsigned id, unsigned total) {
    const unsigned kXcd = 8;
    const unsigned per = total / kXcd, rem = total % kXcd;
    const unsigned x = id % kXcd, idx = id / kXcd;
    return x < rem ? x * (per + 1) + idx : rem * (per + 1) + (x - rem) * per + idx;
}

// Pack the 16-bit element e (0..7) of two 8-element rows into one dword:
// low half from row a, high half from row b.
template <int E>
__device__ __forceinline__ uint32_t pack_col(u32x4 a, u32x4 b) {
    const uint32_t x = a[E >> 1], y = b[E >> 1];
    return (E & 1) ? ((x >> 16) | (y & 0xffff0000u)) : ((x & 0xffffu) | (y << 16));
}

// Row index within a 32-key block whose score lands in S^T accumulator row i
// when K is fed as the A operand: swapping bits 2 and 3 makes accumulator
// registers 0..7 of lane half h hold keys 8h..8h+7 and registers 8..15 keys
// 16+8h..16+8h+7, which is exactly the contraction order the next MFMA
// (O^T += V^T P^T) wants for its B operand.
__device__ __forceinline__ int key_perm(int i) {
    return (i & 0x13) | ((i & 4) << 1) | ((i & 8) >> 1);
}

}  // namespace fa
