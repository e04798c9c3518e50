// fa_decode.hip -- split-KV flash-decode for gfx950 (MI355X).
//
// One new query token per sequence attends to a key/value cache of length L.
// The cache is cut into nsplit contiguous shards; each shard yields a partial
// output O_s (already normalised by its own softmax denominator) and its
// log-sum-exp lse_s.  A second, tiny kernel combines the shards:
//     lse = log sum_s exp(lse_s),   O = sum_s exp(lse_s - lse) O_s
// Shard outputs cannot simply be summed because every shard has its own
// denominator; the lse carried with each shard is what lets the combine
// re-normalise (post.smzdm.com digest on Triton warp specialisation,
// section 5, describing sequence-parallel flash-decode).
//
// Split kernel: one workgroup per (shard, kv-head, batch[, column chunk]).
// The query heads that share a kv-head (grouped-query attention) are the
// columns of the score tile, so every K/V byte is read from HBM once for all
// of them.  The 4 waves take interleaved 32-key blocks of the shard; each
// wave keeps its own online-softmax state and the 4 states are merged through
// LDS at the end.  This kernel is bound by HBM bandwidth: MFMA and VALU work
// hide under the K/V stream, and the next block's loads are issued before
// the current block is computed.
//
// MFMA 16x16x32 (16 columns = up to 16 query heads of one group):
//   S^T (16 keys x 16 heads) = K (16 x 32 dims) Q^T;  K rows are fed in the
//   order that makes two S^T blocks together equal the B-operand layout of
//   O^T (16 dims x 16 heads) += V^T (16 dims x 32 keys) P^T (32 keys x 16).
#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// 16x16x32 MFMA: A lane (i + 16g) holds row i, contraction 8g..8g+7; B lane
// (j + 16g) holds column j, contraction 8g..8g+7; C lane (j + 16g) register
// r holds row 4g + r, column j.
struct BF16x16 {
    typedef bf16x8 vec8;
    typedef __bf16 scalar;
    static __device__ __forceinline__ floatx4 mfma16(vec8 a, vec8 b, floatx4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};
struct FP16x16 {
    typedef f16x8 vec8;
    typedef _Float16 scalar;
    static __device__ __forceinline__ floatx4 mfma16(vec8 a, vec8 b, floatx4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
};

template <int D>
struct DecTile {
    static constexpr int THREADS = 256;
    static constexpr int WAVES = 4;
    static constexpr int BK = 32;                 // keys per wave step
    static constexpr int COLS = 16;               // query heads per workgroup
    static constexpr int VLD = BK + 8;            // V^T row stride (elements)
    static constexpr int KCH = D / 8;             // 16-byte chunks per row
    static constexpr int KPL = BK * KCH / 64;     // V rows loaded per lane
    static constexpr int V_ELEMS = D * VLD;       // per wave
    static_assert(KPL == 4 || KPL == 8, "V row grouping");
};

template <int D>
struct DecBuf {
    u32x4 kf[2][D / 32];           // K A-operands, 2 S^T blocks x D/32 steps
    u32x4 vr[DecTile<D>::KPL];     // V rows for the LDS transpose
};

template <typename T, int D>
__global__ __launch_bounds__(256, 2) void fa_decode_split_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, float *__restrict__ ws_o,
    float *__restrict__ ws_lse, int Hq, int Hkv, int L, int nsplit, int chunk,
    int ncc, float c) {
    typedef DecTile<D> C;
    typedef typename T::vec8 vec8;
    typedef typename T::scalar scalar;

    // V^T staging, one slab per wave; reused for the final merge.
    __shared__ __attribute__((aligned(16))) uint16_t Vt[C::WAVES][C::V_ELEMS];
    __shared__ float sm_m[C::WAVES][C::COLS], sm_l[C::WAVES][C::COLS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int lj = lane & 15;   // column (query head) / A-operand row
    const int lg = lane >> 4;   // contraction group 0..3

    const int s = blockIdx.x;
    const int g = blockIdx.y / ncc, cc = blockIdx.y % ncc;
    const int b = blockIdx.z;
    const int G = Hq / Hkv;
    const int hq0 = g * G + cc * C::COLS;
    const int ncol = min(C::COLS, G - cc * C::COLS);

    const int k_lo = s * chunk;
    const int k_hi = min(L, k_lo + chunk);
    const int nblk = k_hi > k_lo ? (k_hi - k_lo + C::BK - 1) / C::BK : 0;

    const size_t kvhead = ((size_t)b * Hkv + g) * (size_t)L * D;
    const uint16_t *kh = k + kvhead, *vh = v + kvhead;

    // Q^T fragments: B operand, lane (lj, lg) holds head hq0+lj, dims 32t+8lg..+8.
    vec8 qf[D / 32];
    {
        const bool ok = lj < ncol;
        const uint16_t *src = q + ((size_t)b * Hq + hq0 + (ok ? lj : 0)) * D + 8 * lg;
#pragma unroll
        for (int t = 0; t < D / 32; ++t)
            qf[t] = as_vec8<vec8>(ok ? *(const u32x4 *)(src + 32 * t) : zero4());
    }

    // S^T block beta, A row i holds key 8*(i/4) + 4*beta + i%4 of the 32-key
    // block, so lane group lg ends up with keys 8lg..8lg+7 in the order the
    // P^T operand needs (registers 0..3 of block 0, then of block 1).
    const int krow0 = 8 * (lj >> 2) + (lj & 3);
    // V transpose: lane (dc, vg) loads rows vg*KPL .. +KPL of dim chunk dc.
    const int dc = lane % C::KCH, vg = lane / C::KCH;

    auto load = [&](DecBuf<D> &bf, int n) {
        const int key0 = k_lo + C::BK * n;
#pragma unroll
        for (int beta = 0; beta < 2; ++beta) {
            const int key = key0 + krow0 + 4 * beta;
            const bool ok = key < k_hi;
            const uint16_t *src = kh + (size_t)(ok ? key : 0) * D + 8 * lg;
#pragma unroll
            for (int t = 0; t < D / 32; ++t)
                bf.kf[beta][t] = ok ? *(const u32x4 *)(src + 32 * t) : zero4();
        }
#pragma unroll
        for (int r = 0; r < C::KPL; ++r) {
            const int key = key0 + vg * C::KPL + r;
            bf.vr[r] = key < k_hi ? *(const u32x4 *)(vh + (size_t)key * D + 8 * dc) : zero4();
        }
    };

    floatx4 oacc[D / 16];
#pragma unroll
    for (int db = 0; db < D / 16; ++db) oacc[db] = floatx4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;
    uint16_t *vt = Vt[wave];

    auto compute = [&](const DecBuf<D> &bf, int n) {
        const int key0 = k_lo + C::BK * n;
        floatx4 sc[2];
#pragma unroll
        for (int beta = 0; beta < 2; ++beta) {
            sc[beta] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < D / 32; ++t)
                sc[beta] = T::mfma16(as_vec8<vec8>(bf.kf[beta][t]), qf[t], sc[beta]);
        }
        // Stage V^T for this block: dims 8dc..8dc+7, keys vg*KPL..+KPL.
        {
            uint16_t *dst = vt + (8 * dc) * C::VLD + vg * C::KPL;
#define FA_DEC_VT(E)                                                             \
    if constexpr (C::KPL == 8)                                                   \
        *(u32x4 *)(dst + (E) * C::VLD) = u32x4{                                  \
            pack_col<E>(bf.vr[0], bf.vr[1]), pack_col<E>(bf.vr[2], bf.vr[3]),    \
            pack_col<E>(bf.vr[4], bf.vr[5]), pack_col<E>(bf.vr[6], bf.vr[7])};   \
    else                                                                         \
        *(u32x2 *)(dst + (E) * C::VLD) =                                         \
            u32x2{pack_col<E>(bf.vr[0], bf.vr[1]), pack_col<E>(bf.vr[2], bf.vr[3])};
            FA_DEC_VT(0) FA_DEC_VT(1) FA_DEC_VT(2) FA_DEC_VT(3)
            FA_DEC_VT(4) FA_DEC_VT(5) FA_DEC_VT(6) FA_DEC_VT(7)
#undef FA_DEC_VT
        }
        // key of (block beta, register r) in lane group lg: 8lg + 4beta + r
        if (key0 + C::BK > k_hi) {
#pragma unroll
            for (int beta = 0; beta < 2; ++beta)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (key0 + 8 * lg + 4 * beta + r >= k_hi) sc[beta][r] = -INFINITY;
        }
        float mx = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                         fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float m_new = fmaxf(m_run, mx * c);
        const float mb = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - mb);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < D / 16; ++db) oacc[db] *= alpha;
        vec8 pb;
#pragma unroll
        for (int beta = 0; beta < 2; ++beta)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float p = __builtin_amdgcn_exp2f(fmaf(sc[beta][r], c, -mb));
                l_run += p;
                pb[4 * beta + r] = (scalar)p;
            }
        // The V^T slab is private to this wave: order its LDS writes before
        // the reads below (LDS operations of one wave complete in order).
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const uint16_t *va = vt + lj * C::VLD + 8 * lg;
#pragma unroll
        for (int db = 0; db < D / 16; ++db)
            oacc[db] = T::mfma16(as_vec8<vec8>(*(const u32x4 *)(va + 16 * db * C::VLD)), pb, oacc[db]);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };

    {
        DecBuf<D> A, B;
        int n = wave;
        if (n < nblk) load(A, n);
        for (; n < nblk; n += 2 * C::WAVES) {
            if (n + C::WAVES < nblk) load(B, n + C::WAVES);
            compute(A, n);
            if (n + C::WAVES >= nblk) break;
            if (n + 2 * C::WAVES < nblk) load(A, n + 2 * C::WAVES);
            compute(B, n + C::WAVES);
        }
    }

    // Merge the 4 wave states.  Per column: M = max_w m_w,
    // Lsum = sum_w l_w 2^(m_w - M), O = sum_w 2^(m_w - M) O_w / Lsum.
    float l_w = l_run + __shfl_xor(l_run, 16, 64);
    l_w += __shfl_xor(l_w, 32, 64);
    if (lg == 0) {
        sm_m[wave][lj] = m_run;
        sm_l[wave][lj] = l_w;
    }
    __syncthreads();
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < C::WAVES; ++w) M = fmaxf(M, sm_m[w][lj]);
    const float Mb = M == -INFINITY ? 0.f : M;
    float Lsum = 0.f;
#pragma unroll
    for (int w = 0; w < C::WAVES; ++w)
        Lsum += sm_l[w][lj] * __builtin_amdgcn_exp2f(sm_m[w][lj] - Mb);
    const float f = Lsum > 0.f ? __builtin_amdgcn_exp2f(m_run - Mb) / Lsum : 0.f;
    // Scaled wave outputs go to LDS as part[w][col][d] (reusing the V^T slabs).
    float *part = reinterpret_cast<float *>(&Vt[0][0]);
    static_assert(C::WAVES * C::COLS * D * 4 <= (int)sizeof(Vt), "merge buffer");
    __syncthreads();
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
        *(floatx4 *)&part[(wave * C::COLS + lj) * D + 16 * db + 4 * lg] = oacc[db] * f;
    __syncthreads();
    for (int idx = tid; idx < ncol * D; idx += C::THREADS) {
        const int col = idx / D, d = idx % D;
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < C::WAVES; ++w) acc += part[(w * C::COLS + col) * D + d];
        ws_o[(((size_t)b * Hq + hq0 + col) * nsplit + s) * D + d] = acc;
    }
    if (tid < ncol)
        ws_lse[((size_t)b * Hq + hq0 + tid) * nsplit + s] =
            Lsum > 0.f ? (M + log2f(Lsum)) * kLn2 : -INFINITY;
}

// Combine: one workgroup per (batch, query head), one thread per dim.
__global__ __launch_bounds__(128) void fa_decode_combine_kernel(
    const float *__restrict__ ws_o, const float *__restrict__ ws_lse,
    float *__restrict__ o, float *__restrict__ lse, int D, int nsplit) {
    const size_t row = blockIdx.x;
    const float *pl = ws_lse + row * nsplit;
    const float *po = ws_o + row * (size_t)nsplit * D;
    float M = -INFINITY;
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, pl[s]);
    float total = -INFINITY;
    if (M != -INFINITY) {
        float wsum = 0.f;
        for (int s = 0; s < nsplit; ++s) wsum += expf(pl[s] - M);
        total = M + logf(wsum);
    }
    for (int d = threadIdx.x; d < D; d += blockDim.x) {
        float acc = 0.f;
        if (total != -INFINITY)
            for (int s = 0; s < nsplit; ++s) {
                const float w = expf(pl[s] - total);
                if (w > 0.f) acc += w * po[(size_t)s * D + d];
            }
        o[row * D + d] = acc;
    }
    if (lse != nullptr && threadIdx.x == 0) lse[row] = total;
}

template <typename T, int D>
static hipError_t launch(const DecodeArgs &a, hipStream_t stream) {
    typedef DecTile<D> C;
    const int G = a.Hq / a.Hkv;
    const int ncc = (G + C::COLS - 1) / C::COLS;
    const float c = kLog2e / sqrtf((float)D);
    if ((long long)a.Hkv * ncc > 65535 || a.B > 65535) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((fa_decode_split_kernel<T, D>), dim3(a.nsplit, a.Hkv * ncc, a.B),
                       dim3(C::THREADS), 0, stream, (const uint16_t *)a.q,
                       (const uint16_t *)a.k, (const uint16_t *)a.v, a.ws_o, a.ws_lse,
                       a.Hq, a.Hkv, a.L, a.nsplit, a.chunk, ncc, c);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(fa_decode_combine_kernel, dim3(a.B * a.Hq), dim3(128), 0, stream,
                       a.ws_o, a.ws_lse, a.o, a.lse, D, a.nsplit);
    return hipGetLastError();
}

template <typename T>
static hipError_t launch_dtype(const DecodeArgs &a, hipStream_t s) {
    if (a.d == 128) return launch<T, 128>(a, s);
    if (a.d == 64) return launch<T, 64>(a, s);
    return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream) {
    return a.dtype == 1 ? launch_dtype<FP16x16>(a, stream) : launch_dtype<BF16x16>(a, stream);
}

}  // namespace fa
