// fa_bwd.hip -- gradients of exact attention for gfx950 (MI355X).
//
// What it computes: for self-attention O = softmax(scale * Q K^T [+ causal
// mask]) V with upstream gradient dO, the gradients dQ, dK, dV.  The pages
// list the attention backward as the next kernel after the forward ("Warp
// Specialization in Triton: Design and Roadmap", roadmap section); the
// formulas are the chain rule through the forward's definition:
//     P_ij  = exp(scale s_ij - lse_i)            (lse from the forward)
//     dV_j  = sum_i P_ij dO_i
//     dP_ij = <dO_i, v_j>
//     dS_ij = P_ij (dP_ij - D_i),   D_i = <dO_i, O_i> = sum_k P_ik dP_ik
//     dQ_i  = scale sum_j dS_ij k_j,  dK_j = scale sum_i dS_ij q_i
// Like the forward, nothing of size N x N is stored: P and dS are rebuilt
// tile by tile from Q, K and the forward's lse.
//
// Two kernels, no atomics (results are deterministic):
//  fa_bwd_dq_kernel    each wave owns 32 queries; K and V tiles of 64 keys
//                      stream through LDS.  Per tile: S^T = K Q^T and
//                      dP^T = V dO^T (Q, dO in registers as the B operand),
//                      then dQ^T += K^T dS^T with K^T from the transposing
//                      LDS read.  First it computes D_i from dO and O and
//                      writes D and lse*log2(e) to the workspace.
//  fa_bwd_dkdv_kernel  each pair of waves owns 32 keys; Q, dO and the
//                      per-query lse and D of 64 queries stream through LDS.
//                      One wave of the pair holds K: S = Q K^T, P, and
//                      dV^T += dO^T P; the other holds V: dP = dO V^T,
//                      dS = P (dP - D) with P handed over through LDS, and
//                      dK^T += Q^T dS.  dO^T and Q^T come from transposing
//                      LDS reads.
// The dQ kernel must run first (the second reads its D and lse).  S and dP
// are formed in both kernels: 7 matrix products per tile pair instead of the
// 5 of a single pass that accumulates dQ with atomics.
#include <type_traits>

#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {

// LDS chunk swizzle for tiles that are read both row-wise (16-byte reads,
// 16 consecutive rows per 16 lanes) and transposed (ds_read_b64_tr_b16:
// 4 consecutive rows x 4 consecutive chunks per 32 lanes).  Chunk c of row r
// is stored at c ^ swz_kt(r), with
//   swz_kt(r) = (g % (KCH/4)) << 2 | (g / (KCH/4)) % 4,   g = r / ROWS_PER_LINE.
// Row-wise: over 16 aligned rows the swizzle takes every value once per bank
// line position, so the 16 lanes hit 16 distinct chunk positions.
// Transposed: the 4 rows of a group differ in the high bits (the chunk
// quadruple), so their 4-chunk runs land on disjoint banks.
template <int D>
__device__ __forceinline__ int swz_kt(int r) {
    constexpr int KCH = D / 8, RPL = 16 / KCH, Q4 = KCH / 4;
    const int g = r / RPL;
    return ((g % Q4) << 2) | ((g / Q4) % 4);
}

// Tile shape shared by both kernels: 4 waves of 32 rows (queries for dQ,
// keys for dK/dV) and streamed tiles of 64 rows.
template <int D>
struct BwdTile {
    static constexpr int WAVES = 4;
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int BM = 32 * WAVES;      // rows owned by a workgroup
    static constexpr int BN = 64;              // rows per streamed tile
    static constexpr int NB = BN / 32;         // 32-row blocks per tile
    static constexpr int KCH = D / 8;          // 16-byte chunks per row
    static constexpr int RPI = 64 / KCH;       // rows per wave copy instruction
    static constexpr int ROWS = BN / WAVES;    // tile rows each wave copies
    static constexpr int LOADS = ROWS / RPI;   // copy instructions per wave and tensor
    static constexpr int ELEMS = BN * D;
    static constexpr int KSTEPS = D / 16;      // MFMAs per 32x32 score block
    static constexpr int DB = D / 32;          // 32-dim blocks of an accumulator
    static_assert(ROWS % RPI == 0, "tile must split evenly over the waves");
};

// Buffer resource for a streamed tile: base advanced to the tile, range cut
// at the end of the head (rows past the end read as zero).  Uniform values
// are forced into scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc_at(const void *head_base,
                                                               uint32_t off, uint32_t head_bytes) {
    const uint64_t addr = (uint64_t)(uintptr_t)head_base + off;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)addr);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(addr >> 32));
    const uint32_t n = __builtin_amdgcn_readfirstlane(off < head_bytes ? head_bytes - off : 0u);
    return make_rsrc((const void *)(uintptr_t)(((uint64_t)hi << 32) | lo), n);
}

// Packed variable-length batches (VARLEN): q, k, v, dO, o and the gradients
// are [T, H, D] with sequence b at rows [cu[b], cu[b+1]); lse and the
// workspace statistics are [H, T].
struct BwdSeqs {
    const int *cu;   // [B + 1]
    int H, T;
};

// One (sequence, head) as a kernel sees it: N rows starting at element
// `head`, consecutive rows RS elements apart, statistics of row i at
// srow0 + i.  Varlen bounds read from cu are clamped to [0, T] and to Nmax.
// Consecutive (sequence, head) pairs of the grid are ordered head-major
// across sequences, so that each XCD's contiguous range of workgroups holds
// an equal share of every sequence.
template <int D, bool VARLEN>
struct BwdHead {
    int bh, N;
    size_t head, srow0;
    static constexpr int rs(const BwdSeqs &vl) { return VARLEN ? vl.H * D : D; }
    __device__ BwdHead(int pair_id, int npairs, int Nmax, const BwdSeqs &vl) {
        bh = pair_id;
        N = Nmax;
        head = (size_t)bh * Nmax * D;
        srow0 = (size_t)bh * Nmax;
        if constexpr (VARLEN) {
            const int nseq = npairs / vl.H;
            bh = (pair_id % nseq) * vl.H + pair_id / nseq;
            const int b = bh / vl.H, h = bh % vl.H;
            const int s0 = min(max(vl.cu[b], 0), vl.T);
            const int e = min(max(vl.cu[b + 1], s0), vl.T);
            N = min(e - s0, Nmax);
            head = ((size_t)s0 * vl.H + h) * D;
            srow0 = (size_t)h * vl.T + s0;
        }
    }
};

// ---------------------------------------------------------------------------
// dQ (and D, lse2) kernel
// ---------------------------------------------------------------------------
template <typename T, int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(256, 2) void fa_bwd_dq_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, const float *__restrict__ o,
    const uint16_t *__restrict__ dout, const float *__restrict__ lse,
    float *__restrict__ dq, float *__restrict__ ws_lse2, float *__restrict__ ws_dl, int Nmax,
    int nq, float c, float scale, BwdSeqs vl) {
    typedef BwdTile<D> C;
    typedef typename T::vec8 vec8;
    typedef typename T::scalar scalar;
    constexpr int BN = C::BN, NB = C::NB, KSTEPS = C::KSTEPS, DB = C::DB;

    __shared__ __attribute__((aligned(16))) uint16_t K0[C::ELEMS], K1[C::ELEMS];
    __shared__ __attribute__((aligned(16))) uint16_t V0[C::ELEMS], V1[C::ELEMS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 31, lh = lane >> 5;

    // Block -> (head, q-tile): consecutive ids walk one head's q-tiles (they
    // share its K and V in the XCD's L2); causal: longest rows first.
    const unsigned id = xcd_remap(blockIdx.x, gridDim.x);
    const int qt = CAUSAL ? nq - 1 - (int)(id % (unsigned)nq) : (int)(id % (unsigned)nq);
    const int q0 = qt * C::BM;
    const BwdHead<D, VARLEN> hd((int)(id / (unsigned)nq), (int)(gridDim.x / (unsigned)nq), Nmax, vl);
    const int N = hd.N;
    const size_t head = hd.head;
    const int RS = BwdHead<D, VARLEN>::rs(vl);
    if (VARLEN && q0 >= N) return;   // past this sequence: leave before any barrier
    const uint32_t head_bytes = (uint32_t)((N > 0 ? (size_t)(N - 1) * RS + D : 0) * 2);
    const int my_q = q0 + wave * 32 + li;
    const bool q_ok = my_q < N;

    // Q and dO fragments (B operand): lane (li, lh) holds row my_q, dims
    // 16t + 8lh .. +8; rows past N read as zero.
    const __amdgpu_buffer_rsrc_t qr = make_rsrc_uniform(q + head, head_bytes);
    const __amdgpu_buffer_rsrc_t dr = make_rsrc_uniform(dout + head, head_bytes);
    vec8 qf[KSTEPS], df[KSTEPS];
    float dl = 0.f;
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) {
        const uint32_t off = (uint32_t)(my_q * RS + 16 * t + 8 * lh) * 2u;
        qf[t] = as_vec8<vec8>(buffer_load16(qr, off));
        df[t] = as_vec8<vec8>(buffer_load16(dr, off));
    }
    // D_i = <dO_i, O_i> with dO as stored (16 bit) and O in fp32.
    if (q_ok) {
        const float *orow = o + head + (size_t)my_q * RS + 8 * lh;
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t) {
            const floatx4 a = *(const floatx4 *)(orow + 16 * t);
            const floatx4 b = *(const floatx4 *)(orow + 16 * t + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                dl = fmaf((float)df[t][e], a[e], dl);
                dl = fmaf((float)df[t][4 + e], b[e], dl);
            }
        }
    }
    dl = sum_halves(dl);
    const float lse2 = q_ok ? lse[hd.srow0 + my_q] * kLog2e : 0.f;
    if (q_ok && lh == 0) {
        ws_lse2[hd.srow0 + my_q] = lse2;
        ws_dl[hd.srow0 + my_q] = dl;
    }

    const int kv_end = CAUSAL ? min(N, q0 + C::BM) : N;
    const int ntiles = (kv_end + BN - 1) / BN;

    // Tile copies: wave w copies rows [w*ROWS, (w+1)*ROWS); K with the
    // two-way swizzle (read row-wise and transposed), V with the row-wise one.
    uint32_t koff[C::LOADS], voff[C::LOADS];
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
        const int row = wave * C::ROWS + i * C::RPI + lane / C::KCH;
        const int pos = lane % C::KCH;
        koff[i] = (uint32_t)(row * RS + 8 * (pos ^ swz_kt<D>(row))) * 2u;
        voff[i] = (uint32_t)(row * RS + 8 * (pos ^ swz_kt<D>(row))) * 2u;
    }
    auto load_tile = [&](int tile, uint16_t *kbuf, uint16_t *vbuf) __attribute__((always_inline)) {
        const uint32_t off = (uint32_t)tile * (uint32_t)(BN * RS * 2);
        const __amdgpu_buffer_rsrc_t rk = tile_rsrc_at(k + head, off, head_bytes);
        const __amdgpu_buffer_rsrc_t rv = tile_rsrc_at(v + head, off, head_bytes);
#pragma unroll
        for (int i = 0; i < C::LOADS; ++i) {
            buffer_load16_lds(rk, koff[i], kbuf + (wave * C::ROWS + i * C::RPI) * D);
            buffer_load16_lds(rv, voff[i], vbuf + (wave * C::ROWS + i * C::RPI) * D);
        }
    };

    // Row-wise operand (A): row 32kb + li, logical chunk 2t + lh.
    int rcol[KSTEPS];
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) rcol[t] = li * D + 8 * ((2 * t + lh) ^ swz_kt<D>(li));
    auto read_rows = [&](const uint16_t *buf, int kb, int t) __attribute__((always_inline)) {
        return as_vec8<vec8>(*(const u32x4 *)(buf + 32 * kb * D + rcol[t]));
    };
    // Transposed operand (A of dQ^T += K^T dS^T): two transposing reads give
    // lane (li, lh) K[32kb + 16u + 8(e/4) + 4lh + e%4][32db + li], e = 0..7.
    // The swizzle repeats every 16 rows, so one offset serves every 16-row
    // group; rows tr_row and tr_row + 8 each need their own.
    const int tr_row = 4 * lh + ((lane & 15) >> 2);
    int tcol[DB], tcol8[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        const int col = 32 * db + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
        tcol[db] = tr_row * D + 8 * ((col >> 3) ^ swz_kt<D>(tr_row)) + (col & 7);
        tcol8[db] = (tr_row + 8) * D + 8 * ((col >> 3) ^ swz_kt<D>(tr_row + 8)) + (col & 7);
    }
    auto read_tr = [&](const uint16_t *buf, int kb, int u, int db) __attribute__((always_inline)) {
        const uint16_t *p = buf + (32 * kb + 16 * u) * D;
        return join8<vec8>(lds_read_tr4(p + tcol[db]), lds_read_tr4(p + tcol8[db]));
    };

    floatx16 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
    const floatx16 zero16 = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f,
                             0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};

    // Tiles from n_full on hold keys past the end or (causal) after some
    // query of the workgroup: their weights are masked.
    int n_full = N / BN;
    if (CAUSAL) n_full = min(n_full, q0 / BN);
    const int lim = CAUSAL ? min(N - 1, my_q) : N - 1;

    // MASK is a compile-time tag: tiles without masked keys carry no mask code.
    auto tile_step = [&](int j, const uint16_t *kbuf, const uint16_t *vbuf, auto mask_tag)
                         __attribute__((always_inline)) {
        constexpr bool MASK = decltype(mask_tag)::value;
        static_assert(NB == 2, "two 32-key blocks per tile");
        vec8 dsb[NB][2];
        // S^T and dP^T blocks: lane (li, lh), register r holds key
        // 32kb + 8(r/4) + 4lh + r%4 of query my_q.
        floatx16 s[NB], dp[NB];
        auto products = [&](int kb) __attribute__((always_inline)) {
#pragma unroll
            for (int t = 0; t < KSTEPS; ++t) {
                s[kb] = T::mfma32(read_rows(kbuf, kb, t), qf[t], t == 0 ? zero16 : s[kb]);
                dp[kb] = T::mfma32(read_rows(vbuf, kb, t), df[t], t == 0 ? zero16 : dp[kb]);
            }
        };
        auto weights = [&](int kb) __attribute__((always_inline)) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float p = __builtin_amdgcn_exp2f(fmaf(s[kb][r], c, -lse2));
                if constexpr (MASK) {
                    const int key = j * BN + 32 * kb + 8 * (r >> 2) + 4 * lh + (r & 3);
                    if (key > lim) p = 0.f;
                }
                dsb[kb][r >> 3][r & 7] = (scalar)(p * (dp[kb][r] - dl));
            }
        };
        auto dq_part = [&](int kb) __attribute__((always_inline)) {
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int db = 0; db < DB; ++db)
                    acc[db] = T::mfma32(read_tr(kbuf, kb, u, db), dsb[kb][u], acc[db]);
        };
        // Each block's vector work runs next to the other block's MFMAs.
        products(0);
        __builtin_amdgcn_sched_barrier(0);
        products(1);
        weights(0);
        __builtin_amdgcn_sched_barrier(0);
        dq_part(0);
        weights(1);
        __builtin_amdgcn_sched_barrier(0);
        dq_part(1);
    };

    // Tile j sits in buffer j % 2; tile j+1 is copied while j is computed.
    typedef std::integral_constant<int, 0> B0;
    typedef std::integral_constant<int, 1> B1;
    auto iter = [&](int j, auto par, auto mask_tag) __attribute__((always_inline)) {
        constexpr int PAR = decltype(par)::value;
        if (j + 1 < ntiles) load_tile(j + 1, PAR ? K0 : K1, PAR ? V0 : V1);
        tile_step(j, PAR ? K1 : K0, PAR ? V1 : V0, mask_tag);
        wait_vmem();
        __syncthreads();
    };
    // Tiles [j0, j1), unrolled by two so that buffer parities are static.
    auto run = [&](int j0, int j1, auto mask_tag) __attribute__((always_inline)) {
        int j = j0;
        if (j < j1 && (j & 1)) iter(j++, B1{}, mask_tag);
        for (; j + 1 < j1; j += 2) {
            iter(j, B0{}, mask_tag);
            iter(j + 1, B1{}, mask_tag);
        }
        if (j < j1) iter(j, B0{}, mask_tag);
    };
    if (ntiles > 0) load_tile(0, K0, V0);
    wait_vmem();
    __syncthreads();
    const int split = max(0, min(n_full, ntiles));
    run(0, split, std::false_type{});
    run(split, ntiles, std::true_type{});

    // dQ^T accumulator: lane (li, lh), register r of block db holds dim
    // 32db + 8(r/4) + 4lh + r%4 of query my_q.
    if (q_ok) {
        float *row = dq + head + (size_t)my_q * RS + 4 * lh;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int a = 0; a < 4; ++a)
                *(floatx4 *)(row + 32 * db + 8 * a) =
                    floatx4{acc[db][4 * a] * scale, acc[db][4 * a + 1] * scale,
                            acc[db][4 * a + 2] * scale, acc[db][4 * a + 3] * scale};
    }
}

// ---------------------------------------------------------------------------
// dK, dV kernel
// ---------------------------------------------------------------------------
// Eight waves in two roles.  Wave pair p (waves p and p + 4, which share a
// SIMD) owns keys k0 + 32p .. +32:
//   P wave  (role 0): holds K; S = Q K^T, P = exp2(c S - lse2), masked; hands
//                     P (16 bit) to its partner through LDS; dV^T += dO^T P.
//   dS wave (role 1): holds V; dP = dO V^T; reads P; dS = P (dP - D);
//                     dK^T += Q^T dS.
// Each role keeps one operand and one accumulator in registers, so two waves
// fit on a SIMD, and each does half of the tile's matrix products.  The two
// roles run one query tile apart: in step j the P wave works on tile j and
// the dS wave on tile j - 1, whose P the barrier ending step j - 1 published.
// Nothing inside a step waits on the partner, so one wave's exponentials and
// LDS waits hide under the other's products.  Query tiles, their statistics
// and P rotate through three LDS buffers (tile j - 1 read by dS waves, tile j
// by P waves, tile j + 1 being copied in).
template <int D>
struct BwdKvTile {
    static constexpr int WAVES = 8;
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int PAIRS = 4;
    static constexpr int BM = 32 * PAIRS;      // keys owned by a workgroup
    static constexpr int BN = 64;              // queries per streamed tile
    static constexpr int NB = BN / 32;
    static constexpr int KCH = D / 8;
    static constexpr int RPI = 64 / KCH;
    static constexpr int ROWS = BN / WAVES;
    static constexpr int LOADS = ROWS / RPI;
    static constexpr int ELEMS = BN * D;
    static constexpr int PSLOTS = PAIRS * NB * 2 * 64;   // 16-byte P slots per buffer
    static constexpr int KSTEPS = D / 16;
    static constexpr int DB = D / 32;
    static_assert(ROWS % RPI == 0, "tile must split evenly over the waves");
};

template <typename T, int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(512, 1) void fa_bwd_dkdv_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, const uint16_t *__restrict__ dout,
    const float *__restrict__ ws_lse2, const float *__restrict__ ws_dl,
    float *__restrict__ dk, float *__restrict__ dv, int Nmax, int nk, float c, float scale,
    BwdSeqs vl) {
    typedef BwdKvTile<D> C;
    typedef typename T::vec8 vec8;
    typedef typename T::scalar scalar;
    constexpr int BN = C::BN, NB = C::NB, KSTEPS = C::KSTEPS, DB = C::DB;

    // Three rotating buffers of each kind, each its own LDS object so that
    // every access names its buffer at compile time.
    __shared__ __attribute__((aligned(16))) uint16_t Q0[C::ELEMS], Q1[C::ELEMS], Q2[C::ELEMS];
    __shared__ __attribute__((aligned(16))) uint16_t G0[C::ELEMS], G1[C::ELEMS], G2[C::ELEMS];
    __shared__ __attribute__((aligned(16))) float L0[BN], L1[BN], L2[BN];   // lse2
    __shared__ __attribute__((aligned(16))) float E0[BN], E1[BN], E2[BN];   // D
    // P from each P wave to its partner: [pair][qb][u][lane], 16 bytes.
    __shared__ __attribute__((aligned(16))) u32x4 P0[C::PSLOTS], P1[C::PSLOTS], P2[C::PSLOTS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int role = wave >> 2, pair = wave & 3;
    const int li = lane & 31, lh = lane >> 5;

    // Block -> (head, key tile): consecutive ids walk one head's key tiles
    // (sharing its Q and dO in L2); causal: the first key tiles see the most
    // queries, so ascending order runs the longest first.
    const unsigned id = xcd_remap(blockIdx.x, gridDim.x);
    const int kt = (int)(id % (unsigned)nk);
    const int k0 = kt * C::BM;
    const BwdHead<D, VARLEN> hd((int)(id / (unsigned)nk), (int)(gridDim.x / (unsigned)nk), Nmax, vl);
    const int N = hd.N;
    const size_t head = hd.head;
    const int RS = BwdHead<D, VARLEN>::rs(vl);
    if (VARLEN && k0 >= N) return;   // past this sequence: leave before any barrier
    const uint32_t head_bytes = (uint32_t)((N > 0 ? (size_t)(N - 1) * RS + D : 0) * 2);
    const uint32_t stat_bytes = (uint32_t)((size_t)N * 4);
    const int my_k = k0 + 32 * pair + li;

    // The role's operand (B): K rows for P waves, V rows for dS waves; lane
    // (li, lh) holds key my_k, dims 16t + 8lh .. +8 (zero past N).
    const __amdgpu_buffer_rsrc_t kr = make_rsrc_uniform((role ? v : k) + head, head_bytes);
    vec8 kv[KSTEPS];
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t)
        kv[t] = as_vec8<vec8>(buffer_load16(kr, (uint32_t)(my_k * RS + 16 * t + 8 * lh) * 2u));

    // Query tiles [qt0, nqt): causal skips the tiles wholly before k0.
    const int qt0 = CAUSAL ? k0 / BN : 0;
    const int nqt = (N + BN - 1) / BN;

    uint32_t toff[C::LOADS];
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
        const int row = wave * C::ROWS + i * C::RPI + lane / C::KCH;
        toff[i] = (uint32_t)(row * RS + 8 * ((lane % C::KCH) ^ swz_kt<D>(row))) * 2u;
    }
    // Waves 0 and 1 also copy the tile's lse2 and D (one dword per lane;
    // past N reads as zero and is masked).
    auto load_tile = [&](int tile, uint16_t *qbuf, uint16_t *gbuf, float *lbuf, float *ebuf)
                         __attribute__((always_inline)) {
        const uint32_t off = (uint32_t)tile * (uint32_t)(BN * RS * 2);
        const __amdgpu_buffer_rsrc_t rq = tile_rsrc_at(q + head, off, head_bytes);
        const __amdgpu_buffer_rsrc_t rg = tile_rsrc_at(dout + head, off, head_bytes);
#pragma unroll
        for (int i = 0; i < C::LOADS; ++i) {
            buffer_load16_lds(rq, toff[i], qbuf + (wave * C::ROWS + i * C::RPI) * D);
            buffer_load16_lds(rg, toff[i], gbuf + (wave * C::ROWS + i * C::RPI) * D);
        }
        if (wave < 2) {
            const uint32_t soff = (uint32_t)tile * (uint32_t)(BN * 4);
            const float *src = wave == 0 ? ws_lse2 : ws_dl;
            const __amdgpu_buffer_rsrc_t rs = tile_rsrc_at(src + hd.srow0, soff, stat_bytes);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rs, (__attribute__((address_space(3))) void *)(wave == 0 ? lbuf : ebuf), 4,
                (int)(lane * 4), 0, 0, 0);
        }
    };

    int rcol[KSTEPS];
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) rcol[t] = li * D + 8 * ((2 * t + lh) ^ swz_kt<D>(li));
    auto read_rows = [&](const uint16_t *buf, int qb, int t) __attribute__((always_inline)) {
        return as_vec8<vec8>(*(const u32x4 *)(buf + 32 * qb * D + rcol[t]));
    };
    const int tr_row = 4 * lh + ((lane & 15) >> 2);
    int tcol[DB], tcol8[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        const int col = 32 * db + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
        tcol[db] = tr_row * D + 8 * ((col >> 3) ^ swz_kt<D>(tr_row)) + (col & 7);
        tcol8[db] = (tr_row + 8) * D + 8 * ((col >> 3) ^ swz_kt<D>(tr_row + 8)) + (col & 7);
    }
    auto read_tr = [&](const uint16_t *buf, int qb, int u, int db) __attribute__((always_inline)) {
        const uint16_t *p = buf + (32 * qb + 16 * u) * D;
        return join8<vec8>(lds_read_tr4(p + tcol[db]), lds_read_tr4(p + tcol8[db]));
    };
    const int pbase = pair * (NB * 2 * 64) + lane;   // slot (qb, u): pbase + (2qb + u) * 64

    // Scheduling patterns for the matrix-product phases: keep several LDS
    // operand reads in flight ahead of the products that consume them (left
    // to itself the scheduler issues one read, waits, then multiplies).
    // Measured on MI355X: 5 % faster without the mask, 3-5 % slower with
    // it, so only the unmasked kernel uses them.
    constexpr bool kSched = !CAUSAL;
    auto fence = [&]() __attribute__((always_inline)) {
        if constexpr (kSched) __builtin_amdgcn_sched_barrier(0);
    };
    auto sched_chain = [&]() __attribute__((always_inline)) {   // KSTEPS reads, KSTEPS MFMAs
        if constexpr (kSched) {
            __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);   // LDS reads
#pragma unroll
            for (int i = 0; i < KSTEPS - 3; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
        }
    };
    auto sched_tr = [&]() __attribute__((always_inline)) {      // 4*DB reads, 2*DB MFMAs
        if constexpr (kSched) {
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
            for (int i = 0; i < 2 * DB - 2; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        }
    };

    // dV^T (P waves) or dK^T (dS waves): lane (li, lh), register r of block
    // db holds dim 32db + 8(r/4) + 4lh + r%4 of key my_k.
    floatx16 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
    const floatx16 zero16 = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f,
                             0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};

    // Tiles that need a mask: (causal) queries before some key of the
    // workgroup, or queries past N.
    const int mask_lo = CAUSAL ? (k0 + C::BM + BN - 1) / BN : 0;
    const int mask_hi = N / BN;

    // S / dP blocks: lane (li, lh), register r holds query
    // 32qb + 8(r/4) + 4lh + r%4 against key my_k.
    auto p_work = [&](int j, const uint16_t *qbuf, const uint16_t *gbuf, const float *lbuf,
                      u32x4 *pbuf, auto mask_tag) __attribute__((always_inline)) {
        constexpr bool MASK = decltype(mask_tag)::value;
#pragma unroll
        for (int qb = 0; qb < NB; ++qb) {
            floatx16 s;
            fence();
#pragma unroll
            for (int t = 0; t < KSTEPS; ++t)
                s = T::mfma32(read_rows(qbuf, qb, t), kv[t], t == 0 ? zero16 : s);
            sched_chain();
            fence();
            vec8 pb[2];
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const floatx4 l4 = *(const floatx4 *)(lbuf + 32 * qb + 8 * a + 4 * lh);
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const int r = 4 * a + x;
                    float p = __builtin_amdgcn_exp2f(fmaf(s[r], c, -l4[x]));
                    if constexpr (MASK) {
                        const int qi = j * BN + 32 * qb + 8 * a + 4 * lh + x;
                        if (qi >= N || (CAUSAL && qi < my_k)) p = 0.f;
                    }
                    pb[r >> 3][r & 7] = (scalar)p;
                }
            }
            fence();
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                pbuf[pbase + (2 * qb + u) * 64] = __builtin_bit_cast(u32x4, pb[u]);
#pragma unroll
                for (int db = 0; db < DB; ++db)
                    acc[db] = T::mfma32(read_tr(gbuf, qb, u, db), pb[u], acc[db]);
            }
            sched_tr();
            fence();
        }
    };
    auto ds_work = [&](const uint16_t *qbuf, const uint16_t *gbuf, const float *ebuf,
                       const u32x4 *pbuf) __attribute__((always_inline)) {
#pragma unroll
        for (int qb = 0; qb < NB; ++qb) {
            floatx16 dp;
            fence();
#pragma unroll
            for (int t = 0; t < KSTEPS; ++t)
                dp = T::mfma32(read_rows(gbuf, qb, t), kv[t], t == 0 ? zero16 : dp);
            sched_chain();
            fence();
            auto make_ds = [&](int u) __attribute__((always_inline)) {
                const vec8 pv = __builtin_bit_cast(vec8, pbuf[pbase + (2 * qb + u) * 64]);
                const floatx4 e0 = *(const floatx4 *)(ebuf + 32 * qb + 16 * u + 4 * lh);
                const floatx4 e1 = *(const floatx4 *)(ebuf + 32 * qb + 16 * u + 8 + 4 * lh);
                vec8 ds;
#pragma unroll
                for (int x = 0; x < 8; ++x) {
                    const float e = x < 4 ? e0[x] : e1[x - 4];
                    // Written as an FMA with a zero addend (same rounding as the
                    // product) so that fp16 P is widened inside v_fma_mix_f32.
                    ds[x] = (scalar)__builtin_fmaf((float)pv[x], dp[8 * u + x] - e, 0.f);
                }
                return ds;
            };
            if constexpr (kSched) {
                // Both halves first, then one scheduled product phase.
                const vec8 dsb[2] = {make_ds(0), make_ds(1)};
                fence();
#pragma unroll
                for (int u = 0; u < 2; ++u)
#pragma unroll
                    for (int db = 0; db < DB; ++db)
                        acc[db] = T::mfma32(read_tr(qbuf, qb, u, db), dsb[u], acc[db]);
                sched_tr();
                fence();
            } else {
                // Half by half (fewer live registers).
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const vec8 dsb = make_ds(u);
#pragma unroll
                    for (int db = 0; db < DB; ++db)
                        acc[db] = T::mfma32(read_tr(qbuf, qb, u, db), dsb, acc[db]);
                }
            }
        }
    };

    // Step j: copy tile j + 1, P waves on tile j, dS waves on tile j - 1.
    // Buffer set b holds tiles j with (j - qt0) % 3 == b.
    auto step = [&](int j, auto par, auto role_tag, auto mask_tag) __attribute__((always_inline)) {
        constexpr int B = decltype(par)::value;
        constexpr int ROLE = decltype(role_tag)::value;
        uint16_t *const qc = B == 0 ? Q0 : B == 1 ? Q1 : Q2;   // tile j
        uint16_t *const gc = B == 0 ? G0 : B == 1 ? G1 : G2;
        float *const lc = B == 0 ? L0 : B == 1 ? L1 : L2;
        u32x4 *const pc = B == 0 ? P0 : B == 1 ? P1 : P2;
        uint16_t *const qp = B == 0 ? Q2 : B == 1 ? Q0 : Q1;   // tile j - 1
        uint16_t *const gp = B == 0 ? G2 : B == 1 ? G0 : G1;
        float *const ep = B == 0 ? E2 : B == 1 ? E0 : E1;
        u32x4 *const pp = B == 0 ? P2 : B == 1 ? P0 : P1;
        uint16_t *const qn = B == 0 ? Q1 : B == 1 ? Q2 : Q0;   // tile j + 1
        uint16_t *const gn = B == 0 ? G1 : B == 1 ? G2 : G0;
        float *const ln = B == 0 ? L1 : B == 1 ? L2 : L0;
        float *const en = B == 0 ? E1 : B == 1 ? E2 : E0;
        if (j + 1 < nqt) load_tile(j + 1, qn, gn, ln, en);
        if constexpr (ROLE == 0) {
            if (j < nqt) p_work(j, qc, gc, lc, pc, mask_tag);
        } else {
            if (j > qt0) ds_work(qp, gp, ep, pp);
        }
        wait_vmem();
        __syncthreads();
    };

    load_tile(qt0, Q0, G0, L0, E0);
    wait_vmem();
    __syncthreads();
    typedef std::integral_constant<int, 0> S0;
    typedef std::integral_constant<int, 1> S1;
    typedef std::integral_constant<int, 2> S2;
    // nqt - qt0 + 1 steps: the dS waves finish one step after the P waves.
    // One loop per role (the role is uniform in each wave), so each keeps its
    // accumulator in one place; both loops pass the same barriers.
    // Steps [j0, j1) with a static buffer phase (j - qt0) % 3; the P waves'
    // tiles in [mask_lo, mask_hi) need no mask and run without mask code.
    auto range = [&](int j0, int j1, auto role_tag, auto mask_tag) __attribute__((always_inline)) {
        int j = j0;
        if (j < j1 && (j - qt0) % 3 == 1) step(j++, S1{}, role_tag, mask_tag);
        if (j < j1 && (j - qt0) % 3 == 2) step(j++, S2{}, role_tag, mask_tag);
        for (; j + 2 < j1; j += 3) {
            step(j, S0{}, role_tag, mask_tag);
            step(j + 1, S1{}, role_tag, mask_tag);
            step(j + 2, S2{}, role_tag, mask_tag);
        }
        if (j < j1) step(j++, S0{}, role_tag, mask_tag);
        if (j < j1) step(j++, S1{}, role_tag, mask_tag);
    };
    const int lo = max(qt0, min(mask_lo, nqt + 1));
    const int hi = max(lo, min(mask_hi, nqt + 1));
    auto run = [&](auto role_tag) __attribute__((always_inline)) {
        range(qt0, lo, role_tag, std::true_type{});
        range(lo, hi, role_tag, std::false_type{});
        range(hi, nqt + 1, role_tag, std::true_type{});
    };
    if (role == 0)
        run(std::integral_constant<int, 0>{});
    else
        run(std::integral_constant<int, 1>{});

    if (my_k < N) {
        float *row = (role ? dk : dv) + head + (size_t)my_k * RS + 4 * lh;
        const float f = role ? scale : 1.f;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int a = 0; a < 4; ++a)
                *(floatx4 *)(row + 32 * db + 8 * a) =
                    floatx4{acc[db][4 * a] * f, acc[db][4 * a + 1] * f, acc[db][4 * a + 2] * f,
                            acc[db][4 * a + 3] * f};
    }
}

template <typename T, int D, bool CAUSAL, bool VARLEN>
static hipError_t launch_kernels(const BwdArgs &a, int nt, unsigned blocks, int ntk,
                                 unsigned blocks_k, hipStream_t stream) {
    typedef BwdTile<D> C;
    typedef BwdKvTile<D> CK;
    const float c = a.scale * kLog2e;
    const BwdSeqs vl = {a.cu_seqlens, a.H, a.T};
    hipLaunchKernelGGL((fa_bwd_dq_kernel<T, D, CAUSAL, VARLEN>), dim3(blocks), dim3(C::THREADS), 0,
                       stream, (const uint16_t *)a.q, (const uint16_t *)a.k,
                       (const uint16_t *)a.v, a.o, (const uint16_t *)a.dout, a.lse, a.dq,
                       a.ws_lse2, a.ws_dl, a.N, nt, c, a.scale, vl);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((fa_bwd_dkdv_kernel<T, D, CAUSAL, VARLEN>), dim3(blocks_k),
                       dim3(CK::THREADS), 0, stream, (const uint16_t *)a.q,
                       (const uint16_t *)a.k, (const uint16_t *)a.v,
                       (const uint16_t *)a.dout, a.ws_lse2, a.ws_dl, a.dk, a.dv, a.N, ntk, c,
                       a.scale, vl);
    return hipGetLastError();
}

template <typename T, int D, bool CAUSAL>
static hipError_t launch(const BwdArgs &a, hipStream_t stream) {
    typedef BwdTile<D> C;
    typedef BwdKvTile<D> CK;
    const int nt = (a.N + C::BM - 1) / C::BM;
    const long long blocks = (long long)nt * a.BH;
    const int ntk = (a.N + CK::BM - 1) / CK::BM;
    const long long blocks_k = (long long)ntk * a.BH;
    if (blocks > 0x7fffffffLL || blocks_k > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    // N = the longest sequence when varlen; BH = B * H.
    if (a.cu_seqlens != nullptr)
        return launch_kernels<T, D, CAUSAL, true>(a, nt, (unsigned)blocks, ntk,
                                                  (unsigned)blocks_k, stream);
    return launch_kernels<T, D, CAUSAL, false>(a, nt, (unsigned)blocks, ntk, (unsigned)blocks_k,
                                               stream);
}

template <typename T>
static hipError_t launch_dtype(const BwdArgs &a, hipStream_t s) {
    if (a.d == 128) return a.causal ? launch<T, 128, true>(a, s) : launch<T, 128, false>(a, s);
    if (a.d == 64) return a.causal ? launch<T, 64, true>(a, s) : launch<T, 64, false>(a, s);
    return hipErrorInvalidValue;
}

hipError_t launch_bwd(const BwdArgs &a, hipStream_t stream) {
    return a.dtype == 1 ? launch_dtype<FP16>(a, stream) : launch_dtype<BF16>(a, stream);
}

}  // namespace fa
