// fa_launch.hpp -- host-side launchers implemented in the .hip files and
// called by the C ABI layer (fa_api.cpp) after it has validated arguments.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>

namespace fa {

struct FwdArgs {
    const void *q, *k, *v;  // [BH, N, d] 16-bit
    float *o;               // [BH, N, d]
    float *lse;             // [BH, N] or nullptr
    int BH, N, d;
    bool causal;
    float scale;
    int dtype;              // 0 bf16, 1 fp16
    // Packed variable-length batch (cu_seqlens != nullptr): q, k, v, o are
    // [T, H, d], BH = B*H, N = the longest sequence, lse is [H, T].
    const int *cu_seqlens = nullptr;   // [B + 1]
    int H = 0, T = 0;
};

hipError_t launch_fwd(const FwdArgs &a, hipStream_t stream);

// FP8 (E4M3) forward: q, k, v are [BH, N, d] bytes; the attention is that of
// the dequantized tensors qd*q, kd*k, vd*v.
struct FwdFp8Args {
    const void *q, *k, *v;
    float *o, *lse;
    int BH, N, d;
    bool causal;
    float scale, qd, kd, vd;
};

hipError_t launch_fwd_fp8(const FwdFp8Args &a, hipStream_t stream);

// Attention backward: gradients of the forward with upstream gradient dout.
struct BwdArgs {
    const void *q, *k, *v, *dout;   // [BH, N, d] 16-bit
    const float *o, *lse;           // forward outputs: [BH, N, d], [BH, N]
    float *dq, *dk, *dv;            // [BH, N, d]
    float *ws_lse2, *ws_dl;         // workspace: [BH, N] each
    int BH, N, d;
    bool causal;
    float scale;
    int dtype;                      // 0 bf16, 1 fp16
    // Packed variable-length batch (cu_seqlens != nullptr): tensors are
    // [T, H, d], BH = B*H, N = the longest sequence, lse and the workspace
    // arrays are [H, T].
    const int *cu_seqlens = nullptr;   // [B + 1]
    int H = 0, T = 0;
};

hipError_t launch_bwd(const BwdArgs &a, hipStream_t stream);

struct DecodeArgs {
    const void *q;          // [B, Hq, d] 16-bit
    const void *k, *v;      // [B, Hkv, L, d] 16-bit
    float *o;               // [B, Hq, d]
    float *lse;             // [B, Hq] or nullptr
    float *ws_o;            // [B, Hq, nsplit, d]
    float *ws_lse;          // [B, Hq, nsplit]
    int B, Hq, Hkv, L, d, nsplit, chunk;
    int dtype;
    // Paged caches (block_table != nullptr): k, v are [num_pages, page_size,
    // Hkv, d] pools, L is unused, each sequence has seq_lens[b] keys.
    const int *block_table = nullptr;   // [B, pages_per_seq]
    const int *seq_lens = nullptr;      // [B]
    int page_size = 0, pages_per_seq = 0, num_pages = 0;
};

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);

// The decode partials of fa_decode_noalloc live in a fixed device array of
// this many bytes (one per GPU, for the life of the process).
constexpr size_t kDecodeScratchBytes = size_t(8) << 20;

// Device address of that array on the current device (looked up once per
// device; no allocation).
hipError_t decode_scratch(void **ptr);

}  // namespace fa
