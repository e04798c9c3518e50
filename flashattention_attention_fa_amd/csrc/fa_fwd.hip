// fa_fwd.hip -- exact attention forward for gfx950 (MI355X).
//
// What it computes: softmax(scale * Q K^T [+ causal mask]) V and the per-row
// natural log-sum-exp, tile by tile, never writing the N x N score matrix
// (dailyaiworld page "FlashAttention-3 vs Triton Kernels", introduction).
// The running-max / running-sum rescaling is the "online normalisation"
// the smzdm digest (section 6) tells multi-GPU users to check first.
//
// Work split: one workgroup = 4 waves = 256 queries of one (batch, head);
// each wave owns 64 queries as two 32-query blocks, so every K or V operand
// read from LDS feeds two MFMAs (LDS traffic per flop is what limits a
// 32-query wave on this chip).  Keys stream through LDS in tiles of 64: the
// K and V tiles of the coming iterations are copied from global memory
// straight into the LDS buffers that just became free while the current tile
// is computed (one barrier per tile).
//
// The loop is software pipelined inside each wave (the pages contrast this
// "different iterations of one role" schedule with warp specialisation):
// iteration j issues the QK^T MFMAs of tile j+1 next to the exponentials of
// tile j, then the PV MFMAs of tile j next to the row maxima of tile j+1, so
// the matrix cores and the vector ALUs always have independent work.
//
// Per wave and tile (64 queries x 64 keys), for each 32-query block:
//   S^T = K Q^T   MFMA 32x32x16; Q lives in registers for the whole loop
//                 (B operand), K rows come from LDS (A operand).  Each lane
//                 owns the scores of ONE query (its column): row max and row
//                 sum are in-lane plus one swap with the other lane half.
//   online softmax in the exp2 domain with c = scale*log2(e):
//                 m' = max(m, c*max_j s_j);  alpha = 2^(m - m');
//                 p_j = 2^(c*s_j - m');  l = alpha*l + sum p_j;  O *= alpha
//                 (m is only raised when the tile max exceeds it by more than
//                 a slack, which skips most O rescales exactly)
//   O^T += V^T P^T  P^T is the S^T accumulator converted to 16 bits in
//                 place; V^T comes from the row-major V tile through the
//                 transposing LDS read.
// Epilogue: O /= l, lse = (m + log2 l) * ln 2, both fp32.
#include <type_traits>

#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {

template <int D>
struct FwdTile {
    static constexpr int QB = 2;                  // 32-query blocks per wave
    static constexpr int BM = 4 * 32 * QB;        // queries per workgroup
    static constexpr int BN = 32;                 // keys per tile
    static constexpr int KB = BN / 32;            // 32-key blocks per tile
    static constexpr int THREADS = 256;
    static constexpr int KCH = D / 8;             // 16-byte chunks per row
    static constexpr int RPI = 64 / KCH;          // rows one wave copy instruction covers
    static constexpr int LOADS = BN / 4 / RPI;    // copy instructions per wave, per tensor, per tile
    static constexpr int ELEMS = BN * D;
    // Rows that share a bank line: 64 banks hold 16 chunks, i.e. 16/KCH rows.
    static constexpr int ROWS_PER_LINE = 16 / KCH;
    static_assert(BN % (4 * RPI) == 0, "tile must split evenly over the waves");
};

// LDS tiles are unpadded (direct copies write 1 KB contiguous per wave
// instruction); bank conflicts are avoided by permuting the 16-byte chunks of
// each row.  Chunk c of row r is stored at chunk position c ^ swz(r).
//  K tile, read 16 bytes per lane with 32 consecutive rows per instruction:
//    swz = (r / ROWS_PER_LINE) % KCH spreads 16 consecutive rows over all 16
//    chunk positions of a bank line.
//  V tile, read by the transposing read (4 rows x 32 bytes per 16 lanes):
//    swz = 4 * ((r / ROWS_PER_LINE) % (KCH / 4)) gives the 4 rows of a group
//    disjoint chunk quadruples.
template <int D>
__device__ __forceinline__ int swz_k(int r) {
    typedef FwdTile<D> C;
    return (r / C::ROWS_PER_LINE) % C::KCH;
}
template <int D>
__device__ __forceinline__ int swz_v(int r) {
    typedef FwdTile<D> C;
    return 4 * ((r / C::ROWS_PER_LINE) % (C::KCH / 4));
}

// Rescale slack in log2 units: the running max m is only raised (and O, l
// rescaled) when some query's tile max exceeds m by more than this, so the
// unnormalised weights stay below 2^8 and fit bf16/fp16 with room to spare.
constexpr float kRescaleSlack = 8.0f;

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

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void fa_fwd_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, float *__restrict__ o,
    float *__restrict__ lse, int N, int nq, float c, uint32_t qand, uint32_t qxor) {
    typedef FwdTile<D> C;
    typedef typename T::vec8 vec8;
    typedef typename T::scalar scalar;
    constexpr int QB = C::QB, BM = C::BM, BN = C::BN, KCH = C::KCH;
    constexpr int KSTEPS = D / 16;         // QK^T MFMAs per 32-query block and tile
    constexpr int DB = D / 32;             // 32-dim blocks of O
    static_assert(BN == 32 && QB == 2, "the schedule below is written for 32-key tiles");

    // Two K and two V tile buffers, each its own LDS object: every access
    // below names its buffer at compile time, so the compiler can tell that
    // the copies in flight into one buffer do not alias reads of the other.
    __shared__ __attribute__((aligned(16))) uint16_t K0[C::ELEMS], K1[C::ELEMS];
    __shared__ __attribute__((aligned(16))) uint16_t V0[C::ELEMS], V1[C::ELEMS];
    typedef std::integral_constant<int, 0> P0;
    typedef std::integral_constant<int, 1> P1;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 31;   // query column inside a 32-query block
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
    const int qw = q0 + wave * 32 * QB;   // first query of this wave

    // Q fragments: B operand, lane (li, lh) of block qb holds query
    // qw + 32qb + li, dims 16t+8lh..+8 (rows past N read as zero).
    vec8 qf[QB][KSTEPS];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t) {
            u32x4 x = buffer_load16(qr, (uint32_t)((qw + 32 * qb + li) * D + 16 * t + 8 * lh) * 2u);
            // scale < 0: flip the sign of q (exact) and use |scale|;
            // scale == 0: every visible score is 0, i.e. q = 0.
            x = (x & qand) ^ qxor;
            qf[qb][t] = as_vec8<vec8>(x);
            // Q is only ever an MFMA operand: keep it in accumulation
            // registers and leave the vector registers to S, P and operands.
            asm volatile("" : "+a"(qf[qb][t]));
        }

    const int kv_end = CAUSAL ? min(N, q0 + BM) : N;
    const int ntiles = (kv_end + BN - 1) / BN;

    // Tile copies go straight from global memory into LDS.  Wave w copies
    // rows [w*BN/4, (w+1)*BN/4) of a tile, RPI rows per instruction; lane l
    // fills chunk position l%KCH of its row with the source chunk that the
    // swizzle puts there.  Rows past N read as zero (buffer range check) and
    // are masked out of the softmax; tiles past the last one are copied the
    // same way and never read.
    uint32_t koff[C::LOADS], voff[C::LOADS];
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
        const int row = wave * (BN / 4) + i * C::RPI + lane / KCH;
        const int pos = lane % KCH;
        koff[i] = (uint32_t)(row * D + 8 * (pos ^ swz_k<D>(row))) * 2u;
        voff[i] = (uint32_t)(row * D + 8 * (pos ^ swz_v<D>(row))) * 2u;
    }
    auto load_tiles = [&](int ktile, uint16_t *kbuf, int vtile, uint16_t *vbuf)
        __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < C::LOADS; ++i) {
            const int dst = (wave * (BN / 4) + i * C::RPI) * D;
            buffer_load16_lds(kr, koff[i] + (uint32_t)ktile * (BN * D * 2), kbuf + dst);
            buffer_load16_lds(vr, voff[i] + (uint32_t)vtile * (BN * D * 2), vbuf + dst);
        }
    };

    // K operand: logical chunk 2t + lh of row li (swizzled).
    int kcol[KSTEPS];
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) kcol[t] = li * D + 8 * ((2 * t + lh) ^ swz_k<D>(li));
    auto read_k = [&](const uint16_t *buf, int t) __attribute__((always_inline)) {
        return as_vec8<vec8>(*(const u32x4 *)(buf + kcol[t]));
    };
    // V^T operand of PV MFMA u, dim block db, by two transposing reads: lane
    // j of each 16-lane group points at row 16u + 4lh + j/4 (+8 for the
    // second read) and logical column 32db + 16*(group&1) + 4*(j%4).  The
    // row swizzle is the same for all those rows.
    const int tr_row = 4 * lh + ((lane & 15) >> 2);
    int vcol[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        const int col = 32 * db + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
        vcol[db] = tr_row * D + 8 * ((col >> 3) ^ swz_v<D>(tr_row)) + (col & 7);
    }
    auto read_v = [&](const uint16_t *buf, int u, int db) __attribute__((always_inline)) {
        const uint16_t *p = buf + 16 * u * D + vcol[db];
        return join8<vec8>(lds_read_tr4(p), lds_read_tr4(p + 8 * D));
    };

    floatx16 oacc[QB][DB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[qb][db][r] = 0.f;
    float m_run[QB], l_run[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        m_run[qb] = -INFINITY;
        l_run[qb] = 0.f;
    }
    const floatx16 zero16 = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f,
                             0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};

    // S^T of one tile, two register sets used alternately (tile parity):
    // lane (li, lh), register r of block qb holds the score of query
    // qw + 32qb + li against key tile*BN + 8(r/4) + 4lh + r%4.
    floatx16 sA[QB], sB[QB];

    // Keys past the end and (causal) keys after the query get -inf.
    auto mask = [&](floatx16 (&x)[QB], int tile) __attribute__((always_inline)) {
        const int kv0 = tile * BN;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const int my_q = qw + 32 * qb + li;
            const int lim = CAUSAL ? min(N - 1, my_q) : N - 1;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = kv0 + 8 * (r >> 2) + 4 * lh + (r & 3);
                if (key > lim) x[qb][r] = -INFINITY;
            }
        }
    };
    // Row maxima of a tile, in log2 units.
    float mt[QB];
    // (maximum, not fmaxf: no NaN can occur here, and maximum maps straight
    // onto v_maximum3_f32 without canonicalising every MFMA result first.)
    auto row_max = [&](const floatx16 (&x)[QB], int qb) __attribute__((always_inline)) {
        float mx = __builtin_elementwise_maximum(x[qb][0], x[qb][1]);
#pragma unroll
        for (int r = 2; r < 16; ++r) mx = __builtin_elementwise_maximum(mx, x[qb][r]);
        mt[qb] = max_halves(mx) * c;
    };
    // Raise m (and rescale O, l) only when a tile max passes the slack.
    auto raise_max = [&]() __attribute__((always_inline)) {
        bool need = false;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) need |= mt[qb] > m_run[qb] + kRescaleSlack;
        if (__any(need)) {
            // Rare path: keep it a real branch (the compiler would otherwise
            // turn it into unconditional multiplies of the whole O tile).
            asm volatile("" ::: "memory");
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const float m_new = fmaxf(m_run[qb], mt[qb]);
                const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - m_new);
                m_run[qb] = m_new;
                l_run[qb] *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[qb][db][r] *= alpha;
            }
        }
    };

    // P^T operands: register r of block qb becomes element r%8 of operand
    // pb[qb][r/8]; MFMA u contracts over keys 8(e/4) + 4lh + e%4 + 16u.
    vec8 pb[QB][2];
    float mb[QB];
    auto softmax_part = [&](const floatx16 (&x)[QB], int qb, int r0, int n)
        __attribute__((always_inline)) {
#pragma unroll
        for (int r = r0; r < r0 + n; ++r) {
            const float p = __builtin_amdgcn_exp2f(fmaf(x[qb][r], c, -mb[qb]));
            if constexpr (!T::kSumP) l_run[qb] += p;
            pb[qb][r >> 3][r & 7] = (scalar)p;
        }
    };
    auto sum_p = [&](int qb, int u) __attribute__((always_inline)) {
        if constexpr (T::kSumP) l_run[qb] = T::sum8(pb[qb][u], l_run[qb]);
    };
    // m is finite from tile 0 on (every query sees key 0), so the softmax
    // needs no guard against an infinite base.
    auto set_mb = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) mb[qb] = m_run[qb];
    };
    auto pin_o = [&]() __attribute__((always_inline)) {
        // O is only touched by the PV MFMAs (and the rare rescale): keep it in
        // accumulation registers, so that those MFMAs accumulate there and
        // the vector registers hold S, P and the operands in flight.
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int db = 0; db < DB; ++db) asm volatile("" : "+a"(oacc[qb][db]));
    };

    // Tiles before n_full need no mask for any query of the workgroup: all
    // their keys exist and (causal) precede the workgroup's first query.
    int n_full = N / BN;
    if (CAUSAL) n_full = min(n_full, q0 / BN);
    n_full = min(n_full, ntiles);

    // Prologue: K(0), K(1), V(0) into LDS; scores and maxima of tile 0.
    load_tiles(0, K0, 0, V0);
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i)
        buffer_load16_lds(kr, koff[i] + (uint32_t)(BN * D * 2), K1 + (wave * (BN / 4) + i * C::RPI) * D);
    wait_vmem();
    __syncthreads();
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) {
        const vec8 a = read_k(K0, t);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) sA[qb] = T::mfma32(a, qf[qb][t], t == 0 ? zero16 : sA[qb]);
    }
    if (n_full == 0) mask(sA, 0);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) row_max(sA, qb);
    raise_max();
    // Iteration 0 overwrites K0; every wave must be done reading K(0).
    __syncthreads();

    // Iteration j (parity PAR = j % 2): softmax of tile j and QK^T of tile
    // j+1, then PV of tile j and the row maxima of tile j+1.  LDS holds K(j+1)
    // in K[1-PAR] and V(j) in V[PAR]; K(j+2) and V(j+1) are copied meanwhile
    // into K[PAR] and V[1-PAR], which iteration j-1 finished reading, and the
    // barrier at the end publishes them.
    //
    // The instruction order is spelled out and fenced with sched_barrier:
    // with one wave per SIMD, the matrix core only stays busy if every MFMA
    // is issued next to independent vector work (the softmax of the previous
    // tile, the row maxima of the next) and its operands were requested from
    // LDS well before.
    auto iteration = [&](int j, auto par, auto mask_tag, floatx16 (&cur)[QB],
                         floatx16 (&nxt)[QB]) __attribute__((always_inline)) {
        constexpr bool MASK_NEXT = decltype(mask_tag)::value;
        constexpr int PAR = decltype(par)::value;
        uint16_t *const kb_next = PAR ? K0 : K1;   // holds K(j+1)
        uint16_t *const kb_fill = PAR ? K1 : K0;   // receives K(j+2)
        uint16_t *const vb_cur = PAR ? V1 : V0;    // holds V(j)
        uint16_t *const vb_fill = PAR ? V0 : V1;   // receives V(j+1)

        vec8 kop[KSTEPS];
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t) kop[t] = read_k(kb_next, t);
        load_tiles(j + 2, kb_fill, j + 1, vb_fill);
        set_mb();
        __builtin_amdgcn_sched_barrier(0);

        // Phase 1: QK^T(j+1) | first half of softmax(j) (P operand u = 0) |
        // V^T(j) reads.
        vec8 vop[2][DB];
        constexpr int PER_STEP = 2 * 8 / KSTEPS;    // u = 0 elements per QK step
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
                nxt[qb] = T::mfma32(kop[t], qf[qb][t], t == 0 ? zero16 : nxt[qb]);
            const int e0 = t * PER_STEP;            // over (qb, r < 8)
            softmax_part(cur, e0 / 8, e0 % 8, PER_STEP);
            vop[t / DB][t % DB] = read_v(vb_cur, t / DB, t % DB);
            __builtin_amdgcn_sched_barrier(0);
        }

        // Phase 2a: PV(j) over keys 0..15 | second half of softmax(j).
        constexpr int PER_DB = 2 * 8 / DB;           // u = 1 elements per PV step
#pragma unroll
        for (int db = 0; db < DB; ++db) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
                oacc[qb][db] = T::mfma32(vop[0][db], pb[qb][0], oacc[qb][db]);
            const int e0 = db * PER_DB;             // over (qb, 8 <= r < 16)
            softmax_part(cur, e0 / 8, 8 + e0 % 8, PER_DB);
            if (db < QB) sum_p(db, 0);
            __builtin_amdgcn_sched_barrier(0);
        }

        // Phase 2b: PV(j) over keys 16..31 | row maxima of tile j+1.
        if constexpr (MASK_NEXT) mask(nxt, j + 1);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
                oacc[qb][db] = T::mfma32(vop[1][db], pb[qb][1], oacc[qb][db]);
            if (db < QB) sum_p(db, 1), row_max(nxt, db);
            __builtin_amdgcn_sched_barrier(0);
        }
        pin_o();
        raise_max();
        wait_vmem();
        __syncthreads();
    };
    // Iterations [j0, j1), unrolled by two so that buffer and register-set
    // parities are static.
    auto run = [&](int j0, int j1, auto mask_tag) __attribute__((always_inline)) {
        int j = j0;
        if (j < j1 && (j & 1)) iteration(j++, P1{}, mask_tag, sB, sA);
        for (; j + 1 < j1; j += 2) {
            iteration(j, P0{}, mask_tag, sA, sB);
            iteration(j + 1, P1{}, mask_tag, sB, sA);
        }
        if (j < j1) iteration(j, P0{}, mask_tag, sA, sB);
    };
    const int split = max(0, min(n_full - 1, ntiles - 1));
    run(0, split, std::false_type{});
    run(split, ntiles - 1, std::true_type{});

    // Last tile: softmax and PV only.
    auto last = [&](floatx16 (&cur)[QB], const uint16_t *vb) __attribute__((always_inline)) {
        set_mb();
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            softmax_part(cur, qb, 0, 16);
            sum_p(qb, 0);
            sum_p(qb, 1);
        }
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const vec8 vt = read_v(vb, u, db);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
                    oacc[qb][db] = T::mfma32(vt, pb[qb][u], oacc[qb][db]);
            }
    };
    if ((ntiles - 1) & 1) last(sB, V1); else last(sA, V0);

    // Epilogue.  O^T accumulator: lane (li, lh), register r of block db holds
    // dim 32*db + 8*(r/4) + 4*lh + r%4 of query qw + 32qb + li.
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int my_q = qw + 32 * qb + li;
        const float l_tot = sum_halves(l_run[qb]);
        if (my_q < N) {
            const float inv = 1.f / l_tot;
            float *orow = o + head + (size_t)my_q * D + 4 * lh;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int a = 0; a < 4; ++a)
                    *(floatx4 *)(orow + 32 * db + 8 * a) =
                        floatx4{oacc[qb][db][4 * a] * inv, oacc[qb][db][4 * a + 1] * inv,
                                oacc[qb][db][4 * a + 2] * inv, oacc[qb][db][4 * a + 3] * inv};
            if (lse != nullptr && lh == 0)
                lse[(size_t)bh * N + my_q] = (m_run[qb] + log2f(l_tot)) * kLn2;
        }
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
                       (const uint16_t *)a.v, a.o, a.lse, a.N, nq, c, qand, qxor);
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
