// fa_fwd.hip -- exact attention forward for gfx950 (MI355X).
//
// What it computes: softmax(scale * Q K^T [+ causal mask]) V and the per-row
// natural log-sum-exp, tile by tile, never writing the N x N score matrix
// (dailyaiworld page "FlashAttention-3 vs Triton Kernels", introduction).
// The running-max / running-sum rescaling is the "online normalisation"
// the smzdm digest (section 6) tells multi-GPU users to check first.
//
// Work split: one workgroup = 4 waves = 128 queries of one (batch, head);
// each wave owns 32 queries.  Keys stream through LDS in tiles of 64, double
// buffered: while the waves run MFMA on tile j, the next tile's K and V rows
// are already in flight from global memory into registers, and are written
// to the other LDS buffer afterwards (one barrier per tile).  The dailyaiworld
// page's Hopper design gives loading and math to different warps; here every
// wave does both, in program order, and the overlap comes from the in-flight
// loads plus two resident workgroups per CU interleaving their MFMA and
// softmax phases.
//
// Per wave and tile (32 queries x 64 keys):
//   S^T = K Q^T   4 x 8 MFMA 32x32x16; Q lives in registers for the whole
//                 loop (B operand), K rows come from LDS (A operand).  Each
//                 lane then owns the scores of ONE query (its column), so the
//                 row max / row sum are in-lane plus one exchange with the
//                 other lane half.
//   online softmax in the exp2 domain with c = scale*log2(e):
//                 m' = max(m, c*max_j s_j);  alpha = 2^(m - m');
//                 p_j = 2^(c*s_j - m');  l = alpha*l + sum p_j;  O *= alpha
//   O^T += V^T P^T  P^T is the S^T accumulator converted to 16 bits in
//                 place (the key order of K rows makes the accumulator layout
//                 equal the B-operand layout), V^T is read from LDS where the
//                 V tile was stored transposed.
// Epilogue: O /= l, lse = (m + log2 l) * ln 2, both fp32.
#include <type_traits>

#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {

template <int D>
struct FwdTile {
    static constexpr int BM = 128;                // queries per workgroup
    static constexpr int BN = 64;                 // keys per tile
    static constexpr int THREADS = 256;
    // LDS row strides (elements).  K rows are read 16 bytes per lane, 32
    // consecutive rows per instruction; V rows are read by the transposing
    // read, 4 rows x 32 bytes per 16 lanes.  The paddings keep both patterns
    // free of bank conflicts.
    static constexpr int LDK = D + 8;
    static constexpr int LDV = D + 32;
    static constexpr int KCH = D / 8;             // 16-byte chunks per row
    static constexpr int LOADS = BN * KCH / THREADS;   // per thread, per tensor, per tile
    static constexpr int K_ELEMS = BN * LDK;
    static constexpr int V_ELEMS = BN * LDV;
    static_assert(BN * KCH % THREADS == 0, "tile must split evenly over the threads");
};

// Rescale slack in log2 units: the running max m is only raised (and O, l
// rescaled) when some query's tile max exceeds m by more than this, so the
// unnormalised weights stay below 2^8 and fit bf16/fp16 with room to spare.
constexpr float kRescaleSlack = 8.0f;

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void fa_fwd_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, float *__restrict__ o,
    float *__restrict__ lse, int BH, int N, int nq, float c, uint32_t qand,
    uint32_t qxor) {
    typedef FwdTile<D> C;
    typedef typename T::vec8 vec8;
    typedef typename T::scalar scalar;
    constexpr int BM = C::BM, BN = C::BN, LDK = C::LDK, LDV = C::LDV;

    __shared__ __attribute__((aligned(16))) uint16_t Ks[2][C::K_ELEMS];
    __shared__ __attribute__((aligned(16))) uint16_t Vs[2][C::V_ELEMS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int li = lane & 31;   // query column inside the wave's 32
    const int lh = lane >> 5;   // lane half

    // Block -> (head, q-tile).  Consecutive logical ids walk the q-tiles of
    // one head, so the workgroups resident on one XCD share that head's K/V
    // in their L2.  Causal: each head's q-tiles run longest (most keys) first,
    // so the short ones fill the tail.
    const unsigned id = xcd_remap(blockIdx.x, gridDim.x);
    const int bh = (int)(id / (unsigned)nq);
    const int qt = CAUSAL ? nq - 1 - (int)(id % (unsigned)nq) : (int)(id % (unsigned)nq);
    const size_t head = (size_t)bh * N * D;
    const uint32_t head_bytes = (uint32_t)N * D * 2;
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(q + head, head_bytes);
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(k + head, head_bytes);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(v + head, head_bytes);
    const int q0 = qt * BM;
    const int qw = q0 + wave * 32;   // first query of this wave
    const int my_q = qw + li;

    // Q fragments: B operand, lane (li, lh) holds row my_q, dims 16t+8lh..+8
    // (rows past N read as zero).
    vec8 qf[D / 16];
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
        u32x4 x = buffer_load16(qr, (uint32_t)(my_q * D + 16 * t + 8 * lh) * 2u);
        // scale < 0: flip the sign of q (exact) and use |scale|;
        // scale == 0: every visible score is 0, i.e. q = 0.
        x = (x & qand) ^ qxor;
        qf[t] = as_vec8<vec8>(x);
    }

    const int kv_end = CAUSAL ? min(N, q0 + BM) : N;
    const int ntiles = (kv_end + BN - 1) / BN;

    // Global -> register staging of one K and one V tile; rows past N read
    // as zero (buffer range check), and are masked out of the softmax.
    u32x4 kreg[C::LOADS], vreg[C::LOADS];
    auto load_tile = [&](int kv0) {
#pragma unroll
        for (int r = 0; r < C::LOADS; ++r) {
            const int ch = tid + C::THREADS * r;
            const uint32_t off = (uint32_t)((kv0 + ch / C::KCH) * D + (ch % C::KCH) * 8) * 2u;
            kreg[r] = buffer_load16(kr, off);
            vreg[r] = buffer_load16(vr, off);
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int r = 0; r < C::LOADS; ++r) {
            const int ch = tid + C::THREADS * r;
            const int row = ch / C::KCH, col = (ch % C::KCH) * 8;
            *(u32x4 *)&Ks[buf][row * LDK + col] = kreg[r];
            *(u32x4 *)&Vs[buf][row * LDV + col] = vreg[r];
        }
    };

    floatx16 oacc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    load_tile(0);
    store_tile(0);
    __syncthreads();

    // ds_read_b64_tr_b16 addressing for the V^T operand: lane j of each
    // 16-lane group points at row (j/4), column 16*(group&1) + 4*(j%4).
    const int tr_row = (lane & 15) >> 2;
    const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

    // One KV tile.  MASK is a compile-time flag so that interior tiles carry
    // no per-element compare at all; only the diagonal tiles (causal) and the
    // ragged last tile run the masked variant.
    auto step = [&](int j, auto mask_tag) {
        constexpr bool MASK = decltype(mask_tag)::value;
        const int buf = j & 1;
        const int kv0 = j * BN;
        if (j + 1 < ntiles) load_tile(kv0 + BN);

        // Causal: a wave whose queries all precede the tile has nothing to do.
        const bool active = !(CAUSAL && MASK) || kv0 <= qw + 31;
        if (active) {
            // S^T = K Q^T: lane (li, lh), register r of block kb holds the
            // score of query my_q against key kv0 + 32kb + 8(r/4) + 4lh + r%4.
            floatx16 s[BN / 32];
#pragma unroll
            for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
                const uint16_t *ka = &Ks[buf][(32 * kb + li) * LDK + 8 * lh];
#pragma unroll
                for (int t = 0; t < D / 16; ++t)
                    s[kb] = T::mfma32(as_vec8<vec8>(*(const u32x4 *)(ka + 16 * t)), qf[t], s[kb]);
            }

            if constexpr (MASK) {
                // keys past the end, and (causal) keys after the query
                const int lim = CAUSAL ? min(N - 1, my_q) : N - 1;
#pragma unroll
                for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = kv0 + 32 * kb + 8 * (r >> 2) + 4 * lh + (r & 3);
                        if (key > lim) s[kb][r] = -INFINITY;
                    }
            }

            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
            mx = fmaxf(mx, other_half(mx));
            const float mt = mx * c;
            if (__any(mt > m_run + kRescaleSlack)) {
                const float m_new = fmaxf(m_run, mt);
                const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
                m_run = m_new;
                l_run *= alpha;
#pragma unroll
                for (int db = 0; db < D / 32; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
            }
            const float mb = m_run == -INFINITY ? 0.f : m_run;

#pragma unroll
            for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][r], c, -mb));
                    s[kb][r] = p;
                    l_run += p;
                }

            // O^T += V^T P^T.  MFMA u of key block kb contracts over keys
            // 32kb + 16u + 8(e/4) + 4lh + e%4 (e = 0..7): P^T is registers
            // 8u..8u+7 of s[kb]; V^T comes from two transposing reads of 4
            // keys each.
#pragma unroll
            for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    vec8 pb;
#pragma unroll
                    for (int e = 0; e < 8; ++e) pb[e] = (scalar)s[kb][8 * u + e];
                    const uint16_t *va = &Vs[buf][(32 * kb + 16 * u + 4 * lh + tr_row) * LDV + tr_col];
#pragma unroll
                    for (int db = 0; db < D / 32; ++db) {
                        const vec8 vt = join8<vec8>(lds_read_tr4(va + 32 * db),
                                                    lds_read_tr4(va + 8 * LDV + 32 * db));
                        oacc[db] = T::mfma32(vt, pb, oacc[db]);
                    }
                }
        }

        if (j + 1 < ntiles) store_tile(buf ^ 1);
        __syncthreads();
    };

    // Tiles before n_full need no mask for any query of the workgroup: all
    // their keys exist and (causal) precede the workgroup's first query.
    int n_full = N / BN;
    if (CAUSAL) n_full = min(n_full, q0 / BN);
    n_full = min(n_full, ntiles);
    for (int j = 0; j < n_full; ++j) step(j, std::false_type{});
    for (int j = n_full; j < ntiles; ++j) step(j, std::true_type{});

    // Epilogue.  O^T accumulator: lane (li, lh), register r of block db holds
    // dim 32*db + 8*(r/4) + 4*lh + r%4 of query my_q.
    const float l_tot = l_run + other_half(l_run);
    if (my_q < N) {
        const float inv = 1.f / l_tot;
        float *orow = o + head + (size_t)my_q * D + 4 * lh;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int a = 0; a < 4; ++a)
                *(floatx4 *)(orow + 32 * db + 8 * a) =
                    floatx4{oacc[db][4 * a] * inv, oacc[db][4 * a + 1] * inv,
                            oacc[db][4 * a + 2] * inv, oacc[db][4 * a + 3] * inv};
        if (lse != nullptr && lh == 0)
            lse[(size_t)bh * N + my_q] = (m_run + log2f(l_tot)) * kLn2;
    }
}

template <typename T, int D, bool CAUSAL>
static hipError_t launch(const FwdArgs &a, hipStream_t stream) {
    typedef FwdTile<D> C;
    const int nq = (a.N + C::BM - 1) / C::BM;
    const long long blocks = (long long)nq * a.BH;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const bool zero = a.scale == 0.f;
    const float c = zero ? kLog2e : fabsf(a.scale) * kLog2e;
    const uint32_t qand = zero ? 0u : 0xffffffffu;
    const uint32_t qxor = a.scale < 0.f ? 0x80008000u : 0u;
    hipLaunchKernelGGL((fa_fwd_kernel<T, D, CAUSAL>), dim3((unsigned)blocks), dim3(C::THREADS),
                       0, stream, (const uint16_t *)a.q, (const uint16_t *)a.k,
                       (const uint16_t *)a.v, a.o, a.lse, a.BH, a.N, nq, c, qand, qxor);
    return hipGetLastError();
}

template <typename T>
static hipError_t launch_dtype(const FwdArgs &a, hipStream_t s) {
    if (a.d == 128) return a.causal ? launch<T, 128, true>(a, s) : launch<T, 128, false>(a, s);
    if (a.d == 64) return a.causal ? launch<T, 64, true>(a, s) : launch<T, 64, false>(a, s);
    return hipErrorInvalidValue;
}

hipError_t launch_fwd(const FwdArgs &a, hipStream_t stream) {
    return a.dtype == 1 ? launch_dtype<FP16>(a, stream) : launch_dtype<BF16>(a, stream);
}

}  // namespace fa
