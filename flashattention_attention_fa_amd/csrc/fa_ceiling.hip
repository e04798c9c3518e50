// fa_ceiling.hip -- measurement kernels of libfa_ceiling.so (include/fa_ceiling.h):
// the matrix-core throughput and the HBM read bandwidth that gfx950 sustains
// when doing nothing else, the achievable ceilings against which the
// attention kernels' own rates can be read.
#include "fa_ceiling.h"
#include "fa_device.hpp"

namespace fa {

// Every wave runs four independent accumulation chains of 32x32x16 MFMAs on
// operands loaded once: the matrix core never waits for a previous result
// (three other products issue in between) and nothing else is issued in the
// loop but the loop counter.  Two workgroups of four waves per CU put two
// waves on every SIMD, as the forward kernel does.
template <typename T>
__global__ __launch_bounds__(256, 2) void fa_ceiling_mfma_kernel(const u32x4 *__restrict__ ops,
                                                                  float *__restrict__ out,
                                                                  int iters) {
    typedef typename T::vec8 vec8;
    const size_t lane = (size_t)blockIdx.x * 256 + threadIdx.x;
    const vec8 a = as_vec8<vec8>(ops[2 * lane]);
    const vec8 b = as_vec8<vec8>(ops[2 * lane + 1]);
    floatx16 c0, c1, c2, c3;
#pragma unroll
    for (int r = 0; r < 16; ++r) c0[r] = c1[r] = c2[r] = c3[r] = 0.f;
    for (int i = 0; i < iters; ++i) {
        c0 = T::mfma32(a, b, c0);
        c1 = T::mfma32(b, a, c1);
        c2 = T::mfma32(a, a, c2);
        c3 = T::mfma32(b, b, c3);
    }
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) s += (c0[r] + c1[r]) + (c2[r] + c3[r]);
    out[lane] = s;
}

__device__ __forceinline__ floatx4 mfma16(bf16x8 a, bf16x8 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma16(f16x8 a, f16x8 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// The same loop on the 16x16x32 16-bit product, which does half the work of
// a 32x32x16 one per instruction on the same operand registers but reads and
// writes a quarter of the accumulator: whether that moves the power-limited
// throughput decides between the two shapes for the forward's products.
template <typename T>
__global__ __launch_bounds__(256, 2) void fa_ceiling_mfma16_kernel(const u32x4 *__restrict__ ops,
                                                                    float *__restrict__ out,
                                                                    int iters) {
    typedef typename T::vec8 vec8;
    const size_t lane = (size_t)blockIdx.x * 256 + threadIdx.x;
    const vec8 a = as_vec8<vec8>(ops[2 * lane]);
    const vec8 b = as_vec8<vec8>(ops[2 * lane + 1]);
    floatx4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0, c2 = c0, c3 = c0;
    for (int i = 0; i < iters; ++i) {
        c0 = mfma16(a, b, c0);
        c1 = mfma16(b, a, c1);
        c2 = mfma16(a, a, c2);
        c3 = mfma16(b, b, c3);
    }
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) s += (c0[r] + c1[r]) + (c2[r] + c3[r]);
    out[lane] = s;
}

// The same loop on the FP8 product of the FP8 forward,
// v_mfma_scale_f32_32x32x64_f8f6f4 on E4M3 operands with neutral block
// scales (twice the flops of the 16-bit product per instruction).
typedef int i32x8 __attribute__((ext_vector_type(8)));

__global__ __launch_bounds__(256, 2) void fa_ceiling_mfma_fp8_kernel(const u32x4 *__restrict__ ops,
                                                                    float *__restrict__ out,
                                                                    int iters) {
    const size_t lane = (size_t)blockIdx.x * 256 + threadIdx.x;
    const u32x4 a0 = ops[4 * lane], a1 = ops[4 * lane + 1], b0 = ops[4 * lane + 2],
                b1 = ops[4 * lane + 3];
    const i32x8 a = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                     (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
    const i32x8 b = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3],
                     (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
    floatx16 c0, c1, c2, c3;
#pragma unroll
    for (int r = 0; r < 16; ++r) c0[r] = c1[r] = c2[r] = c3[r] = 0.f;
    for (int i = 0; i < iters; ++i) {
        c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c0, 0, 0, 0, 127, 0, 127);
        c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, c1, 0, 0, 0, 127, 0, 127);
        c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, a, c2, 0, 0, 0, 127, 0, 127);
        c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, b, c3, 0, 0, 0, 127, 0, 127);
    }
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) s += (c0[r] + c1[r]) + (c2[r] + c3[r]);
    out[lane] = s;
}

// Each workgroup streams one contiguous chunk of the buffer, as a decode
// workgroup streams its shard of the cache: 256 lanes x 16 bytes per load,
// four loads in flight per lane, through a buffer resource over the chunk
// (loads past its end return zero), folded into an XOR so that no load can
// be dropped.  STREAM selects the decode kernel's non-temporal policy.
template <bool STREAM>
__global__ __launch_bounds__(256) void fa_ceiling_read_kernel(const unsigned char *__restrict__ src,
                                                              size_t bytes, uint32_t chunk,
                                                              unsigned *__restrict__ out) {
    const size_t start = (size_t)blockIdx.x * chunk;
    const uint32_t n = start < bytes ? (uint32_t)min((size_t)chunk, bytes - start) : 0u;
    const __amdgpu_buffer_rsrc_t r = make_rsrc_uniform(src + start, n);
    auto load = [&](uint32_t off) __attribute__((always_inline)) {
        return STREAM ? buffer_load16_stream(r, off) : buffer_load16(r, off);
    };
    u32x4 x = zero4();
    for (uint32_t off = threadIdx.x * 16u; off < n; off += 4u * 4096u) {
        const u32x4 a = load(off), b = load(off + 4096u), c = load(off + 8192u),
                    d = load(off + 12288u);
        x ^= (a ^ b) ^ (c ^ d);
    }
    out[(size_t)blockIdx.x * 256 + threadIdx.x] = x[0] ^ x[1] ^ x[2] ^ x[3];
}

// LDS read bandwidth: a 64 KiB tile filled once, then read back over and
// over with the access patterns of the attention kernels' operand reads,
// eight independent reads in flight per wave.  MODE 0: ds_read_b128, 16
// consecutive 16-byte chunks per 16 lanes (a row read, conflict-free);
// MODE 1: ds_read_b64_tr_b16 (the transposing read), 512 contiguous bytes
// per instruction.
template <int MODE>
__global__ __launch_bounds__(256, 2) void fa_ceiling_lds_kernel(unsigned *__restrict__ out, int iters) {
    __shared__ __attribute__((aligned(16))) uint16_t tile[32768];
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int e = (i * 256 + tid) * 8;
        *(u32x4 *)(tile + e) = u32x4{(unsigned)e, (unsigned)e ^ 0x5555u, (unsigned)e + 7u,
                                     (unsigned)tid};
    }
    __syncthreads();
    const int wave = tid >> 6, lane = tid & 63;
    // Each of the four waves reads its own 16 KiB quarter of the tile.
    const int base = (wave & 3) * 8192;
    u32x4 x = zero4();
    for (int it = 0; it < iters; ++it) {
        const int rot = (it & 7) * 512;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            if constexpr (MODE == 0) {
                const int e = base + ((rot + r * 1024 + lane * 8) & 8191);
                x ^= *(const u32x4 *)(tile + e);
            } else {
                const int e = base + ((rot + r * 1024 + lane * 4) & 8191);
                const shortx4 t = lds_read_tr4(tile + e);
                x[r & 3] ^= (unsigned)(uint16_t)t[0] | ((unsigned)(uint16_t)t[3] << 16);
            }
        }
    }
    out[(size_t)blockIdx.x * 256 + tid] = x[0] ^ x[1] ^ x[2] ^ x[3];
}

}  // namespace fa

extern "C" {

int fa_ceiling_mfma(const void *operands, float *out, int workgroups, int iters, int dtype,
                    hipStream_t stream) {
    if (!operands || !out || workgroups < 1 || iters < 1 || dtype < 0 || dtype > 4 ||
        (reinterpret_cast<uintptr_t>(operands) & 15))
        return (int)hipErrorInvalidValue;
    const fa::u32x4 *ops = static_cast<const fa::u32x4 *>(operands);
    if (dtype == 4)
        hipLaunchKernelGGL(fa::fa_ceiling_mfma16_kernel<fa::FP16>, dim3(workgroups), dim3(256), 0,
                           stream, ops, out, iters);
    else if (dtype == 3)
        hipLaunchKernelGGL(fa::fa_ceiling_mfma16_kernel<fa::BF16>, dim3(workgroups), dim3(256), 0,
                           stream, ops, out, iters);
    else if (dtype == 2)
        hipLaunchKernelGGL(fa::fa_ceiling_mfma_fp8_kernel, dim3(workgroups), dim3(256), 0,
                           stream, ops, out, iters);
    else if (dtype == 1)
        hipLaunchKernelGGL(fa::fa_ceiling_mfma_kernel<fa::FP16>, dim3(workgroups), dim3(256), 0,
                           stream, ops, out, iters);
    else
        hipLaunchKernelGGL(fa::fa_ceiling_mfma_kernel<fa::BF16>, dim3(workgroups), dim3(256), 0,
                           stream, ops, out, iters);
    return (int)hipGetLastError();
}

int fa_ceiling_lds(unsigned *out, int workgroups, int iters, int mode, hipStream_t stream) {
    if (!out || workgroups < 1 || iters < 1 || mode < 0 || mode > 1)
        return (int)hipErrorInvalidValue;
    if (mode == 0)
        hipLaunchKernelGGL(fa::fa_ceiling_lds_kernel<0>, dim3(workgroups), dim3(256), 0, stream, out,
                           iters);
    else
        hipLaunchKernelGGL(fa::fa_ceiling_lds_kernel<1>, dim3(workgroups), dim3(256), 0, stream, out,
                           iters);
    return (int)hipGetLastError();
}

int fa_ceiling_read(const void *src, size_t bytes, unsigned *out, int workgroups,
                    int nontemporal, hipStream_t stream) {
    if (!src || !out || workgroups < 1 || bytes == 0 || (bytes & 15) ||
        (reinterpret_cast<uintptr_t>(src) & 15))
        return (int)hipErrorInvalidValue;
    // chunk: bytes / workgroups rounded up to 16 KiB (one round of four loads)
    const size_t chunk = ((bytes + workgroups - 1) / workgroups + 16383) / 16384 * 16384;
    if (chunk >= (size_t(1) << 31)) return (int)hipErrorInvalidValue;
    const unsigned char *p = static_cast<const unsigned char *>(src);
    if (nontemporal)
        hipLaunchKernelGGL(fa::fa_ceiling_read_kernel<true>, dim3(workgroups), dim3(256), 0,
                           stream, p, bytes, (uint32_t)chunk, out);
    else
        hipLaunchKernelGGL(fa::fa_ceiling_read_kernel<false>, dim3(workgroups), dim3(256), 0,
                           stream, p, bytes, (uint32_t)chunk, out);
    return (int)hipGetLastError();
}

}  // extern "C"
