// fa_api.cpp -- the C ABI declared in include/fa.h: argument validation,
// the decode workspace, and dispatch to the HIP launchers.
//
// Validation touches no HIP API, so a rejected call enqueues nothing and can
// be exercised on a machine without a GPU.  No C++ exception crosses the ABI.
#include <climits>
#include <cmath>
#include <cstdint>
#include <mutex>
#include <new>
#include <vector>

#include "fa.h"
#include "fa_launch.hpp"

namespace {

// Per-head byte offsets are 32-bit (buffer addressing): seq_len * 128 * 2 < 2^32.
constexpr int kMaxSeq = 1 << 23;

static_assert(FA_DECODE_NOALLOC_MAX_BYTES == fa::kDecodeScratchBytes,
              "the header's no-alloc limit must match the device buffer");

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

// Workspace layout for nsplit partials: ws_o [B, Hq, nsplit, d] fp32, then
// ws_lse [B, Hq, nsplit] fp32, each 256-byte aligned.
bool decode_ws_layout(int B, int Hq, int d, int nsplit, size_t *o_bytes, size_t *total) {
    if (B < 0 || Hq < 0 || d < 1 || nsplit < 1) return false;
    const unsigned long long rows = (unsigned long long)B * Hq * nsplit;
    if (rows > (1ull << 40)) return false;
    *o_bytes = round256((size_t)rows * d * sizeof(float));
    *total = *o_bytes + round256((size_t)rows * sizeof(float));
    return true;
}

struct DeviceWorkspace {
    void *ptr = nullptr;
    size_t bytes = 0;
};

std::mutex g_ws_mutex;
std::vector<DeviceWorkspace> g_ws;   // indexed by HIP device id

fa_status_t check_decode(const void *q, const void *kc, const void *vc, const float *o,
                         const float *lse, int B, int Hq, int Hkv, int L, int d, int nsplit,
                         fa_dtype_t dtype) {
    if (B < 0 || Hq < 0 || Hkv < 1 || L < 1 || nsplit < 1 || d < 0) return FA_ERR_SHAPE;
    if (dtype != FA_BF16 && dtype != FA_FP16) return FA_ERR_UNSUPPORTED;
    if (Hq % Hkv != 0) return FA_ERR_SHAPE;
    if (!q || !kc || !vc || !o) return FA_ERR_NULL;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (!aligned(q, 16) || !aligned(kc, 16) || !aligned(vc, 16) || !aligned(o, 16) ||
        (lse && !aligned(lse, 4)))
        return FA_ERR_ALIGN;
    if (L > kMaxSeq || B > 65535) return FA_ERR_SHAPE;
    const int ncc = (Hq / Hkv + 15) / 16;
    if ((long long)Hkv * ncc > 65535) return FA_ERR_SHAPE;
    return FA_OK;
}

fa_status_t run_decode(const void *q, const void *kc, const void *vc, float *o, float *lse,
                       int B, int Hq, int Hkv, int L, int d, int nsplit, hipStream_t stream,
                       fa_dtype_t dtype, void *ws, size_t ws_bytes) {
    const int ns = nsplit > L ? L : nsplit;
    size_t o_bytes = 0, need = 0;
    if (!decode_ws_layout(B, Hq, d, ns, &o_bytes, &need)) return FA_ERR_SHAPE;
    if (!ws || ws_bytes < need || !aligned(ws, 256)) return FA_ERR_WORKSPACE;
    fa::DecodeArgs a;
    a.q = q;
    a.k = kc;
    a.v = vc;
    a.o = o;
    a.lse = lse;
    a.ws_o = static_cast<float *>(ws);
    a.ws_lse = reinterpret_cast<float *>(static_cast<char *>(ws) + o_bytes);
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.L = L;
    a.d = d;
    a.nsplit = ns;
    a.chunk = (L + ns - 1) / ns;
    a.dtype = dtype == FA_FP16 ? 1 : 0;
    return fa::launch_decode(a, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace

extern "C" {

fa_status_t fa_fwd(const void *q, const void *k, const void *v, float *o, float *lse, int B,
                   int H, int N, int d, int causal, float scale, hipStream_t stream,
                   fa_dtype_t dtype) {
    try {
        if (B < 0 || H < 0 || N < 0 || d < 0) return FA_ERR_SHAPE;
        if (dtype != FA_BF16 && dtype != FA_FP16) return FA_ERR_UNSUPPORTED;
        if (!std::isfinite(scale)) return FA_ERR_VALUE;
        if (B == 0 || H == 0 || N == 0) return FA_OK;
        if (!q || !k || !v || !o) return FA_ERR_NULL;
        if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
        if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
            (lse && !aligned(lse, 4)))
            return FA_ERR_ALIGN;
        const long long BH = (long long)B * H;
        if (N > kMaxSeq || BH > INT_MAX || BH * ((N + 127) / 128) > INT_MAX) return FA_ERR_SHAPE;
        fa::FwdArgs a;
        a.q = q;
        a.k = k;
        a.v = v;
        a.o = o;
        a.lse = lse;
        a.BH = (int)BH;
        a.N = N;
        a.d = d;
        a.causal = causal != 0;
        a.scale = scale;
        a.dtype = dtype == FA_FP16 ? 1 : 0;
        return fa::launch_fwd(a, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
    } catch (...) {
        return FA_ERR_INTERNAL;
    }
}

fa_status_t fa_fwd_varlen(const void *q, const void *k, const void *v, float *o, float *lse,
                          const int *cu_seqlens, int B, int H, int total_tokens, int max_seqlen,
                          int d, int causal, float scale, hipStream_t stream, fa_dtype_t dtype) {
    try {
        if (B < 0 || H < 0 || total_tokens < 0 || max_seqlen < 0 || d < 0) return FA_ERR_SHAPE;
        if (dtype != FA_BF16 && dtype != FA_FP16) return FA_ERR_UNSUPPORTED;
        if (!std::isfinite(scale)) return FA_ERR_VALUE;
        if (B == 0 || H == 0 || total_tokens == 0 || max_seqlen == 0) return FA_OK;
        if (!q || !k || !v || !o || !cu_seqlens) return FA_ERR_NULL;
        if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
        if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
            !aligned(cu_seqlens, 4) || (lse && !aligned(lse, 4)))
            return FA_ERR_ALIGN;
        const long long BH = (long long)B * H;
        if ((long long)max_seqlen * H * d >= (1ll << 30) || BH > INT_MAX ||
            BH * ((max_seqlen + 127) / 128) > INT_MAX)
            return FA_ERR_SHAPE;
        fa::FwdArgs a;
        a.q = q;
        a.k = k;
        a.v = v;
        a.o = o;
        a.lse = lse;
        a.BH = (int)BH;
        a.N = max_seqlen;
        a.d = d;
        a.causal = causal != 0;
        a.scale = scale;
        a.dtype = dtype == FA_FP16 ? 1 : 0;
        a.cu_seqlens = cu_seqlens;
        a.H = H;
        a.T = total_tokens;
        return fa::launch_fwd(a, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
    } catch (...) {
        return FA_ERR_INTERNAL;
    }
}

fa_status_t fa_fwd_fp8(const void *q, const void *k, const void *v, float *o, float *lse,
                       int B, int H, int N, int d, int causal, float scale, float q_descale,
                       float k_descale, float v_descale, hipStream_t stream) {
    try {
        if (B < 0 || H < 0 || N < 0 || d < 0) return FA_ERR_SHAPE;
        if (!std::isfinite(scale) || !std::isfinite(q_descale) || !std::isfinite(k_descale) ||
            !std::isfinite(v_descale))
            return FA_ERR_VALUE;
        if (B == 0 || H == 0 || N == 0) return FA_OK;
        if (!q || !k || !v || !o) return FA_ERR_NULL;
        if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
        if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
            (lse && !aligned(lse, 4)))
            return FA_ERR_ALIGN;
        const long long BH = (long long)B * H;
        if (N > kMaxSeq || BH > INT_MAX || BH * ((N + 127) / 128) > INT_MAX) return FA_ERR_SHAPE;
        fa::FwdFp8Args a;
        a.q = q;
        a.k = k;
        a.v = v;
        a.o = o;
        a.lse = lse;
        a.BH = (int)BH;
        a.N = N;
        a.d = d;
        a.causal = causal != 0;
        a.scale = scale;
        a.qd = q_descale;
        a.kd = k_descale;
        a.vd = v_descale;
        return fa::launch_fwd_fp8(a, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
    } catch (...) {
        return FA_ERR_INTERNAL;
    }
}

size_t fa_bwd_workspace_bytes(int B, int H, int N) {
    if (B < 0 || H < 0 || N < 0) return 0;
    const unsigned long long rows = (unsigned long long)B * H * N;
    if (rows > (1ull << 40)) return 0;
    return 2 * round256((size_t)rows * sizeof(float));
}

fa_status_t fa_bwd(const void *q, const void *k, const void *v, const float *o, const void *dout,
                   const float *lse, float *dq, float *dk, float *dv, int B, int H, int N, int d,
                   int causal, float scale, hipStream_t stream, fa_dtype_t dtype, void *workspace,
                   size_t workspace_bytes) {
    try {
        if (B < 0 || H < 0 || N < 0 || d < 0) return FA_ERR_SHAPE;
        if (dtype != FA_BF16 && dtype != FA_FP16) return FA_ERR_UNSUPPORTED;
        if (!std::isfinite(scale)) return FA_ERR_VALUE;
        if (B == 0 || H == 0 || N == 0) return FA_OK;
        if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return FA_ERR_NULL;
        if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
        if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
            !aligned(dout, 16) || !aligned(lse, 4) || !aligned(dq, 16) || !aligned(dk, 16) ||
            !aligned(dv, 16))
            return FA_ERR_ALIGN;
        const long long BH = (long long)B * H;
        if (N > kMaxSeq || BH > INT_MAX || BH * ((N + 127) / 128) > INT_MAX) return FA_ERR_SHAPE;
        const size_t need = fa_bwd_workspace_bytes(B, H, N);
        if (need == 0) return FA_ERR_SHAPE;
        if (!workspace || workspace_bytes < need || !aligned(workspace, 256))
            return FA_ERR_WORKSPACE;
        fa::BwdArgs a;
        a.q = q;
        a.k = k;
        a.v = v;
        a.dout = dout;
        a.o = o;
        a.lse = lse;
        a.dq = dq;
        a.dk = dk;
        a.dv = dv;
        a.ws_lse2 = static_cast<float *>(workspace);
        a.ws_dl = reinterpret_cast<float *>(static_cast<char *>(workspace) + need / 2);
        a.BH = (int)BH;
        a.N = N;
        a.d = d;
        a.causal = causal != 0;
        a.scale = scale;
        a.dtype = dtype == FA_FP16 ? 1 : 0;
        return fa::launch_bwd(a, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
    } catch (...) {
        return FA_ERR_INTERNAL;
    }
}

fa_status_t fa_bwd_varlen(const void *q, const void *k, const void *v, const float *o,
                          const void *dout, const float *lse, float *dq, float *dk, float *dv,
                          const int *cu_seqlens, int B, int H, int total_tokens, int max_seqlen,
                          int d, int causal, float scale, hipStream_t stream, fa_dtype_t dtype,
                          void *workspace, size_t workspace_bytes) {
    try {
        if (B < 0 || H < 0 || total_tokens < 0 || max_seqlen < 0 || d < 0) return FA_ERR_SHAPE;
        if (dtype != FA_BF16 && dtype != FA_FP16) return FA_ERR_UNSUPPORTED;
        if (!std::isfinite(scale)) return FA_ERR_VALUE;
        if (B == 0 || H == 0 || total_tokens == 0 || max_seqlen == 0) return FA_OK;
        if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !cu_seqlens)
            return FA_ERR_NULL;
        if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
        if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
            !aligned(dout, 16) || !aligned(lse, 4) || !aligned(dq, 16) || !aligned(dk, 16) ||
            !aligned(dv, 16) || !aligned(cu_seqlens, 4))
            return FA_ERR_ALIGN;
        const long long BH = (long long)B * H;
        if ((long long)max_seqlen * H * d >= (1ll << 30) || BH > INT_MAX ||
            BH * ((max_seqlen + 127) / 128) > INT_MAX)
            return FA_ERR_SHAPE;
        const size_t need = fa_bwd_workspace_bytes(1, H, total_tokens);
        if (need == 0) return FA_ERR_SHAPE;
        if (!workspace || workspace_bytes < need || !aligned(workspace, 256))
            return FA_ERR_WORKSPACE;
        fa::BwdArgs a;
        a.q = q;
        a.k = k;
        a.v = v;
        a.dout = dout;
        a.o = o;
        a.lse = lse;
        a.dq = dq;
        a.dk = dk;
        a.dv = dv;
        a.ws_lse2 = static_cast<float *>(workspace);
        a.ws_dl = reinterpret_cast<float *>(static_cast<char *>(workspace) + need / 2);
        a.BH = (int)BH;
        a.N = max_seqlen;
        a.d = d;
        a.causal = causal != 0;
        a.scale = scale;
        a.dtype = dtype == FA_FP16 ? 1 : 0;
        a.cu_seqlens = cu_seqlens;
        a.H = H;
        a.T = total_tokens;
        return fa::launch_bwd(a, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
    } catch (...) {
        return FA_ERR_INTERNAL;
    }
}

size_t fa_decode_workspace_bytes(int B, int Hq, int d, int nsplit) {
    size_t o_bytes = 0, total = 0;
    if (d != 64 && d != 128) return 0;
    return decode_ws_layout(B, Hq, d, nsplit, &o_bytes, &total) ? total : 0;
}

fa_status_t fa_decode_ex(const void *q, const void *kcache, const void *vcache, float *o,
                         float *lse, int B, int Hq, int Hkv, int L, int d, int nsplit,
                         hipStream_t stream, fa_dtype_t dtype, void *workspace,
                         size_t workspace_bytes) {
    try {
        if (B == 0 || Hq == 0) {
            if (B < 0 || Hq < 0 || Hkv < 1 || L < 1 || nsplit < 1) return FA_ERR_SHAPE;
            return FA_OK;
        }
        fa_status_t st = check_decode(q, kcache, vcache, o, lse, B, Hq, Hkv, L, d, nsplit, dtype);
        if (st != FA_OK) return st;
        return run_decode(q, kcache, vcache, o, lse, B, Hq, Hkv, L, d, nsplit, stream, dtype,
                          workspace, workspace_bytes);
    } catch (...) {
        return FA_ERR_INTERNAL;
    }
}

fa_status_t fa_decode_paged(const void *q, const void *kpages, const void *vpages,
                            const int *block_table, const int *seq_lens, float *o, float *lse,
                            int B, int Hq, int Hkv, int page_size, int pages_per_seq,
                            int num_pages, int d, int nsplit, hipStream_t stream,
                            fa_dtype_t dtype, void *workspace, size_t workspace_bytes) {
    try {
        if (B < 0 || Hq < 0 || Hkv < 1 || nsplit < 1 || d < 0) return FA_ERR_SHAPE;
        if (page_size < 16 || page_size % 16 != 0 || pages_per_seq < 1 || num_pages < 1)
            return FA_ERR_SHAPE;
        if (B == 0 || Hq == 0) return FA_OK;
        if (dtype != FA_BF16 && dtype != FA_FP16) return FA_ERR_UNSUPPORTED;
        if (Hq % Hkv != 0) return FA_ERR_SHAPE;
        if (!q || !kpages || !vpages || !block_table || !seq_lens || !o) return FA_ERR_NULL;
        if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
        if (!aligned(q, 16) || !aligned(kpages, 16) || !aligned(vpages, 16) || !aligned(o, 16) ||
            !aligned(block_table, 4) || !aligned(seq_lens, 4) || (lse && !aligned(lse, 4)))
            return FA_ERR_ALIGN;
        if (B > 65535 || (long long)pages_per_seq * page_size > kMaxSeq) return FA_ERR_SHAPE;
        const int ncc = (Hq / Hkv + 15) / 16;
        if ((long long)Hkv * ncc > 65535) return FA_ERR_SHAPE;
        size_t o_bytes = 0, need = 0;
        if (!decode_ws_layout(B, Hq, d, nsplit, &o_bytes, &need)) return FA_ERR_SHAPE;
        if (!workspace || workspace_bytes < need || !aligned(workspace, 256))
            return FA_ERR_WORKSPACE;
        fa::DecodeArgs a;
        a.q = q;
        a.k = kpages;
        a.v = vpages;
        a.o = o;
        a.lse = lse;
        a.ws_o = static_cast<float *>(workspace);
        a.ws_lse = reinterpret_cast<float *>(static_cast<char *>(workspace) + o_bytes);
        a.B = B;
        a.Hq = Hq;
        a.Hkv = Hkv;
        a.L = 0;
        a.d = d;
        a.nsplit = nsplit;
        a.chunk = 0;
        a.dtype = dtype == FA_FP16 ? 1 : 0;
        a.block_table = block_table;
        a.seq_lens = seq_lens;
        a.page_size = page_size;
        a.pages_per_seq = pages_per_seq;
        a.num_pages = num_pages;
        return fa::launch_decode(a, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
    } catch (...) {
        return FA_ERR_INTERNAL;
    }
}

fa_status_t fa_decode_noalloc(const void *q, const void *kcache, const void *vcache, float *o,
                              float *lse, int B, int Hq, int Hkv, int L, int d, int nsplit,
                              hipStream_t stream, fa_dtype_t dtype) {
    try {
        if (B == 0 || Hq == 0) {
            if (B < 0 || Hq < 0 || Hkv < 1 || L < 1 || nsplit < 1) return FA_ERR_SHAPE;
            return FA_OK;
        }
        fa_status_t st = check_decode(q, kcache, vcache, o, lse, B, Hq, Hkv, L, d, nsplit, dtype);
        if (st != FA_OK) return st;
        const int ns = nsplit > L ? L : nsplit;
        const size_t need = fa_decode_workspace_bytes(B, Hq, d, ns);
        if (need == 0) return FA_ERR_SHAPE;
        if (need > fa::kDecodeScratchBytes) return FA_ERR_WORKSPACE;
        void *ws = nullptr;
        if (fa::decode_scratch(&ws) != hipSuccess) return FA_ERR_HIP;
        return run_decode(q, kcache, vcache, o, lse, B, Hq, Hkv, L, d, ns, stream, dtype, ws,
                          fa::kDecodeScratchBytes);
    } catch (...) {
        return FA_ERR_INTERNAL;
    }
}

fa_status_t fa_decode(const void *q, const void *kcache, const void *vcache, float *o, int B,
                      int Hq, int Hkv, int L, int d, int nsplit, hipStream_t stream,
                      fa_dtype_t dtype) {
    try {
        if (B == 0 || Hq == 0) {
            if (B < 0 || Hq < 0 || Hkv < 1 || L < 1 || nsplit < 1) return FA_ERR_SHAPE;
            return FA_OK;
        }
        fa_status_t st =
            check_decode(q, kcache, vcache, o, nullptr, B, Hq, Hkv, L, d, nsplit, dtype);
        if (st != FA_OK) return st;
        const int ns = nsplit > L ? L : nsplit;
        const size_t need = fa_decode_workspace_bytes(B, Hq, d, ns);
        if (need == 0) return FA_ERR_SHAPE;
        std::lock_guard<std::mutex> lock(g_ws_mutex);
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess || dev < 0) return FA_ERR_HIP;
        if ((size_t)dev >= g_ws.size()) g_ws.resize((size_t)dev + 1);
        DeviceWorkspace &w = g_ws[(size_t)dev];
        if (w.bytes < need) {
            if (w.ptr) {
                if (hipFree(w.ptr) != hipSuccess) return FA_ERR_HIP;
                w.ptr = nullptr;
                w.bytes = 0;
            }
            void *p = nullptr;
            if (hipMalloc(&p, need) != hipSuccess) return FA_ERR_HIP;
            w.ptr = p;
            w.bytes = need;
        }
        return run_decode(q, kcache, vcache, o, nullptr, B, Hq, Hkv, L, d, ns, stream, dtype,
                          w.ptr, w.bytes);
    } catch (...) {
        return FA_ERR_INTERNAL;
    }
}

const char *fa_status_string(fa_status_t status) {
    switch (status) {
        case FA_OK: return "ok";
        case FA_ERR_NULL: return "a required pointer is NULL";
        case FA_ERR_SHAPE: return "a size is negative, inconsistent or too large";
        case FA_ERR_UNSUPPORTED: return "unsupported head_dim (need 64 or 128) or dtype";
        case FA_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
        case FA_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        case FA_ERR_HIP: return "a HIP runtime call or kernel launch failed";
        case FA_ERR_INTERNAL: return "internal error";
        case FA_ERR_VALUE: return "scale or a dequantization factor is not finite";
    }
    return "unknown status";
}

int fa_version(void) { return 300; }

}  // extern "C"
