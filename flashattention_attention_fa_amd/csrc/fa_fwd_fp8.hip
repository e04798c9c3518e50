// fa_fwd_fp8.hip -- exact attention forward on FP8 (OCP E4M3) inputs for
// gfx950 (MI355X).
//
// What it computes: the attention of the dequantized tensors
// q = qd*q8, k = kd*k8, v = vd*v8 (per-tensor factors), softmax(scale*QK^T
// [+ causal mask]) V and the per-row natural log-sum-exp, tile by tile.  FP8
// is the variant that the dailyaiworld page "FlashAttention-3 vs Triton
// Kernels" features for its headline throughput (introduction, and the
// pipeline figure's FP8 note).
//
// Both products run on v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 x E4M3, fp32
// accumulation, neutral block scales), twice the fp16 rate; 32 queries per
// wave, two waves per SIMD, 64-key tiles copied global->LDS by DMA.  With
// four times fewer MFMAs per score than the 16-bit kernels, this kernel is
// bound by its vector work (exponentials, row sums, conversions), so the
// pipeline keeps MFMAs next to that work in every wave: iteration j forms
// the softmax of tile j between the MFMAs of QK^T(j+1) and of PV(j-1) (PV
// trails by one tile; V(j) is copied during iteration j and read in j+1).
// When every wave of the workgroup runs the PV MFMAs of a tile together
// after its softmax, as the 16-bit kernels do, the per-tile barrier keeps
// the two waves of a SIMD in step and the vector unit idles through them.
// What else changes:
//
//  * S^T = K Q^T contracts 64 dims per MFMA.  Lane (i, h) of the A operand
//    holds 32 consecutive dims of one key row; lane (j, h) of the B operand
//    the same 32 dims of query j (h = lane half selects dims 32h..32h+31 of
//    the 64).  The key that A row i carries is permuted, key(i) =
//    16*(i/16) + 8*((i/4)%2) + 4*((i/8)%2) + i%4, so that in the S^T
//    accumulator (lane half h holds rows 8a + 4h + b) each lane half owns
//    runs of 8 consecutive keys: registers 0..7 hold keys 8h..8h+7 of the
//    block, registers 8..15 keys 16+8h..16+8h+7.
//  * P is rounded to E4M3 as the B operand of O^T += V^T P^T (64 keys per
//    MFMA): byte t of lane (query, h) is the weight of key
//    32*(t/16) + 16*((t%16)/8) + 8h + t%8 of the tile.  The A operand V^T
//    gets exactly those keys from four 8-byte transposing LDS reads
//    (ds_read_b64_tr_b8: each yields 8 consecutive keys of one dim).
//  * The weights are scaled by 2^4 before rounding, p' = 2^(c*s - m + 4), so
//    that weights down to 2^-10 of the row maximum sit in E4M3's normal
//    range instead of its subnormals.  l sums the fp32 p' (the scale cancels
//    in O = sum p'v / l; lse subtracts it).  E4M3's largest value is
//    448 = 2^8.8, so every p' must stay at or below it: the running max m is
//    taken exactly from the first tile.  A weight is at most its lane's sum
//    of the tile, so a tile whose lane sums all stay within 448 is accepted
//    as is (with weights of at most 16 at the row maximum, the rule); only
//    otherwise is the tile's row maximum formed, and if a score passes
//    m + 4.8 (log2 units, i.e. p' could pass 448), m is raised to it (O and
//    l rescaled) and the tile recomputed.  (With a 2^6 scale the lane sums
//    pass 448 on almost every tile, and tracking each lane's largest score
//    instead costs a vector instruction per two scores.)
#include <type_traits>

#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

// D = A*B + C on one 32x32x64 E4M3 tile; block scales 127 (= 2^0).  Each
// product of two E4M3 values is exact, but the matrix core adds the products
// of 8 consecutive contraction elements aligned to the largest of them and
// drops the bits below 2^-13 of its leading bit (measured on MI355X): a
// score can fall short of the exact dot product by that much per product.
__device__ __forceinline__ floatx16 mfma_fp8(i32x8 a, i32x8 b, floatx16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Transposing 8-byte LDS read (ds_read_b64_tr_b8).  Within each 16-lane
// group, lane j points at X[r0 + j/2][c0 + 8*(j%2)] of a row-major byte tile
// X; lane i then receives X[r0 + e][c0 + i] for e = 0..7.
__device__ __forceinline__ i32x2 lds_read_tr8(const uint8_t *p) {
    return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2 *)(p));
}

// Four fp32 values rounded (to nearest even) to E4M3, packed into the bytes
// of one dword in order.  The first conversion writes the low half of a
// register whose high half the second one overwrites, so its previous
// content is irrelevant: it comes from an empty asm statement (a constant
// would cost one register move per dword).
__device__ __forceinline__ int cvt_fp8x4(float a, float b, float c2, float d) {
    int any;
    asm volatile("" : "=v"(any));
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, any, false);
    return __builtin_amdgcn_cvt_pk_fp8_f32(c2, d, lo, true);
}

// The weight scale 2^kPShift.  m is raised when a score passes m + kRaise
// (log2 units): 2^(kRaise + kPShift) stays below 448, E4M3's largest value.
// Every weight is at most its lane's tile sum, so a lane sum up to 448 rules
// out any overflow without looking at the scores; with weights of at most
// 2^4 at the row maximum such sums are the rule.
constexpr float kPShift = 4.0f;
constexpr float kRaise = 4.8f;
constexpr float kE4M3Max = 448.0f;

template <int D, bool CAUSAL>
struct Fp8Tile {
    static constexpr int WAVES = CAUSAL ? 4 : 8;
    static constexpr int BM = 32 * WAVES;        // queries per workgroup
    static constexpr int KB = 2;                 // 32-key blocks per tile
    static constexpr int BN = 32 * KB;           // keys per tile
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int KCH = D / 16;           // 16-byte chunks per row
    static constexpr int RPL = 16 / KCH;         // rows per 256-byte bank line
    static constexpr int INSTR = BN * KCH / 64;  // copy instructions per tensor and tile
    static constexpr int COPY_WAVES = INSTR < WAVES ? INSTR : WAVES;
    static constexpr int LOADS = INSTR / COPY_WAVES;
    static constexpr int RPI = 64 / KCH;         // rows per copy instruction
    static constexpr int ELEMS = BN * D;         // bytes per tile
    static_assert(INSTR % COPY_WAVES == 0, "copies must split evenly over the waves");
};

// Chunk c of row r is stored at chunk position c ^ swz(r), with g = r / RPL
// (the row's bank line) and Q = KCH / 2 aligned chunk pairs per row:
//   swz(r) = 2 (g mod Q) + (g div Q) mod 2.
// K (16-byte reads, 16 consecutive rows at one logical chunk): over 2Q
// consecutive lines swz takes every value once, so the rows land in
// distinct bank slots.  V (transposing byte reads, 8 consecutive rows at the
// two chunks of one aligned pair): rows in different lines get different
// pairs (swz / 2 differs), so the 8 rows x 2 chunks fill distinct slots.
// (The plainer (g mod KCH) maps both chunks of a pair onto one pair for
// neighbouring lines: a 2-way conflict on every V read, measured 1 % slower.)
template <int D>
__device__ __forceinline__ int swz8(int r) {
    constexpr int KCH = D / 16, RPL = 16 / KCH, Q = KCH / 2;
    const int g = r / RPL;
    return 2 * (g % Q) + (g / Q) % 2;
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(CAUSAL ? 256 : 512, CAUSAL ? 2 : 1) void fa_fwd_fp8_kernel(
    const uint8_t *__restrict__ q, const uint8_t *__restrict__ k,
    const uint8_t *__restrict__ v, float *__restrict__ o, float *__restrict__ lse,
    int N, int nq, float c, uint32_t qand, uint32_t qxor, float vd) {
    typedef Fp8Tile<D, CAUSAL> C;
    static_assert(C::THREADS == (CAUSAL ? 256 : 512), "launch bounds must match the tile shape");
    constexpr int BM = C::BM, BN = C::BN, KB = C::KB, KCH = C::KCH;
    constexpr int KT = D / 64;   // QK^T MFMAs per 32-key block
    constexpr int DB = D / 32;   // 32-dim blocks of O

    __shared__ __attribute__((aligned(16))) uint8_t K0[C::ELEMS], K1[C::ELEMS];
    __shared__ __attribute__((aligned(16))) uint8_t V0[C::ELEMS], V1[C::ELEMS];
    typedef std::integral_constant<int, 0> P0;
    typedef std::integral_constant<int, 1> P1;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 31;
    const int lh = lane >> 5;

    const unsigned id = xcd_remap(blockIdx.x, gridDim.x);
    const int bh = (int)(id / (unsigned)nq);
    const int qt = CAUSAL ? nq - 1 - (int)(id % (unsigned)nq) : (int)(id % (unsigned)nq);
    const size_t head = (size_t)bh * N * D;
    const uint32_t head_bytes = (uint32_t)N * D;
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(q + head, head_bytes);
    const int q0 = qt * BM;
    const int my_q = q0 + wave * 32 + li;

    // Q^T fragments (B operand): lane (li, lh), MFMA t holds dims
    // 64t + 32lh .. +32 of query my_q (zero past N).
    i32x8 qf[KT];
#pragma unroll
    for (int t = 0; t < KT; ++t) {
        const uint32_t off = (uint32_t)(my_q * D + 64 * t + 32 * lh);
        u32x4 x0 = (buffer_load16(qr, off) & qand) ^ qxor;
        u32x4 x1 = (buffer_load16(qr, off + 16) & qand) ^ qxor;
        qf[t] = i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                      (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
    }

    const int kv_end = CAUSAL ? min(N, q0 + BM) : N;
    const int ntiles = (kv_end + BN - 1) / BN;

    // Tile copies straight into LDS; waves below COPY_WAVES copy LOADS
    // instructions of RPI rows each per tensor and tile.
    const bool copier = wave < C::COPY_WAVES;
    uint32_t koff[C::LOADS];
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
        const int row = (wave * C::LOADS + i) * C::RPI + lane / KCH;
        const int pos = lane % KCH;
        koff[i] = (uint32_t)(row * D + 16 * (pos ^ swz8<D>(row)));
    }
    auto tile_rsrc = [&](const uint8_t *base, int tile) __attribute__((always_inline)) {
        const uint32_t off = (uint32_t)tile * (BN * D);
        const uint64_t addr = (uint64_t)(uintptr_t)base + off;
        const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)addr);
        const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(addr >> 32));
        const uint32_t n = __builtin_amdgcn_readfirstlane(off < head_bytes ? head_bytes - off : 0u);
        return make_rsrc((const void *)(uintptr_t)(((uint64_t)hi << 32) | lo), n);
    };
    auto load_tile = [&](const uint8_t *src, int tile, uint8_t *buf) __attribute__((always_inline)) {
        if (copier) {
            const __amdgpu_buffer_rsrc_t r = tile_rsrc(src + head, tile);
#pragma unroll
            for (int i = 0; i < C::LOADS; ++i)
                buffer_load16_lds(r, koff[i], (uint16_t *)(buf + (wave * C::LOADS + i) * C::RPI * D));
        }
    };

    // K operand of block kb, MFMA t: row key(li) of the block, logical
    // chunks 4t + 2lh and 4t + 2lh + 1.
    const int krow = 16 * (li / 16) + 8 * ((li >> 2) & 1) + 4 * ((li >> 3) & 1) + (li & 3);
    int kcol[2 * KT];
#pragma unroll
    for (int t = 0; t < KT; ++t)
#pragma unroll
        for (int s = 0; s < 2; ++s)
            kcol[2 * t + s] = krow * D + 16 * ((4 * t + 2 * lh + s) ^ swz8<D>(krow));
    auto read_k = [&](const uint8_t *buf, int kb, int t) __attribute__((always_inline)) {
        const u32x4 a = *(const u32x4 *)(buf + 32 * kb * D + kcol[2 * t]);
        const u32x4 b = *(const u32x4 *)(buf + 32 * kb * D + kcol[2 * t + 1]);
        return i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3],
                     (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
    };
    // V^T operand of PV MFMA db: run s (s = 0..3) covers keys
    // 32(s/2) + 16(s%2) + 8lh .. +8 of the tile.  Lane j of 16-lane group g
    // points at row (run start + j/2), byte column 32db + 16(g%2) + 8(j%2).
    const int g2 = (lane >> 4) & 1;
    const int jr = (lane & 15) >> 1, jc = lane & 1;
    int vcol[4][DB];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const int row = 32 * (s / 2) + 16 * (s % 2) + 8 * lh + jr;
            const int col = 32 * db + 16 * g2 + 8 * jc;
            vcol[s][db] = row * D + 16 * ((col >> 4) ^ swz8<D>(row)) + (col & 15);
        }
    auto read_v = [&](const uint8_t *buf, int db) __attribute__((always_inline)) {
        const i32x2 r0 = lds_read_tr8(buf + vcol[0][db]);
        const i32x2 r1 = lds_read_tr8(buf + vcol[1][db]);
        const i32x2 r2 = lds_read_tr8(buf + vcol[2][db]);
        const i32x2 r3 = lds_read_tr8(buf + vcol[3][db]);
        return i32x8{r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
    };

    floatx16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;
    const floatx16 zero16 = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f,
                             0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    floatx16 sA[KB], sB[KB];

    // Key of register r of block kb for this lane half, within the tile.
    auto key_of = [&](int kb, int r) __attribute__((always_inline)) {
        return 32 * kb + 16 * (r >> 3) + 8 * lh + (r & 7);
    };
    auto mask = [&](floatx16 (&x)[KB], int tile) __attribute__((always_inline)) {
        const int kv0 = tile * BN;
        const int lim = CAUSAL ? min(N - 1, my_q) : N - 1;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (kv0 + key_of(kb, r) > lim) x[kb][r] = -INFINITY;
    };
    float mt = 0.f;
    auto row_max = [&](const floatx16 (&x)[KB]) __attribute__((always_inline)) {
        float mx = __builtin_elementwise_maximum(x[0][0], x[0][1]);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r = kb == 0 ? 2 : 0; r < 16; ++r) mx = __builtin_elementwise_maximum(mx, x[kb][r]);
        mt = max_halves(mx) * c;
    };
    auto raise_max = [&]() __attribute__((always_inline)) {
        const float m_new = fmaxf(m_run, mt);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    };

    // P^T operand bytes: dword w = 4kb + (r/4) of pb holds registers
    // 4(w%4) .. +3 of block kb.
    i32x8 pbA, pbB;
    float tsum = 0.f;
    auto softmax_part = [&](const floatx16 (&x)[KB], i32x8 &pb, int kb, int half) __attribute__((always_inline)) {
        if (kb == 0 && half == 0) tsum = 0.f;
        const float bias = kPShift - m_run;
#pragma unroll
        for (int w = 0; w < 2; ++w) {
            const int r0 = 8 * half + 4 * w;
            float p[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                p[e] = __builtin_amdgcn_exp2f(fmaf(x[kb][r0 + e], c, bias));
                tsum += p[e];
            }
            pb[4 * kb + r0 / 4] = cvt_fp8x4(p[0], p[1], p[2], p[3]);
        }
    };
    // Accept the tile's weights when every lane sum is within E4M3's range
    // (the negated test also catches an infinite sum); otherwise look at the
    // tile's row maximum and, if a score passes m + kRaise, raise m to it,
    // rescale O and l, and recompute the weights.
    auto accept = [&](const floatx16 (&x)[KB], i32x8 &pb) __attribute__((always_inline)) {
        if (__any(!(tsum <= kE4M3Max))) {
            asm volatile("" ::: "memory");
            row_max(x);
            if (__any(!(mt <= m_run + kRaise))) {
                raise_max();
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int h = 0; h < 2; ++h) softmax_part(x, pb, kb, h);
            }
        }
        l_run += tsum;
    };

    int n_full = N / BN;
    if (CAUSAL) n_full = min(n_full, q0 / BN);
    n_full = min(n_full, ntiles);

    load_tile(k, 0, K0);
    load_tile(k, 1, K1);
    wait_vmem();
    __syncthreads();
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int t = 0; t < KT; ++t)
            sA[kb] = mfma_fp8(read_k(K0, kb, t), qf[t], t == 0 ? zero16 : sA[kb]);
    if (n_full == 0) mask(sA, 0);
    row_max(sA);
    raise_max();
    __syncthreads();

    // Iteration j (parity PAR): softmax(j) next to QK^T(j+1) and PV(j-1),
    // copies of K(j+2) and V(j) in flight meanwhile.  PV trails the softmax
    // by one tile so that its MFMAs overlap this wave's vector work.
    auto iteration = [&](int j, auto par, auto mask_tag, auto first_tag, floatx16 (&cur)[KB],
                         floatx16 (&nxt)[KB]) __attribute__((always_inline)) {
        constexpr bool MASK_NEXT = decltype(mask_tag)::value;
        constexpr bool FIRST = decltype(first_tag)::value;
        constexpr int PAR = decltype(par)::value;
        uint8_t *const kb_next = PAR ? K0 : K1;
        uint8_t *const kb_fill = PAR ? K1 : K0;
        uint8_t *const vb_prev = PAR ? V0 : V1;
        uint8_t *const vb_fill = PAR ? V1 : V0;
        i32x8 &pb_cur = PAR ? pbB : pbA;
        i32x8 &pb_prev = PAR ? pbA : pbB;

        load_tile(k, j + 2, kb_fill);
        load_tile(v, j, vb_fill);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int t = 0; t < KT; ++t) {
                nxt[kb] = mfma_fp8(read_k(kb_next, kb, t), qf[t], t == 0 ? zero16 : nxt[kb]);
                if (t == 0) softmax_part(cur, pb_cur, kb, 0);
                if constexpr (!FIRST) {
                    constexpr int PER = DB / (KB * KT) > 0 ? DB / (KB * KT) : 1;
#pragma unroll
                    for (int e = 0; e < PER; ++e) {
                        const int db = (kb * KT + t) * PER + e;
                        if (db < DB) oacc[db] = mfma_fp8(read_v(vb_prev, db), pb_prev, oacc[db]);
                    }
                }
                if (t == KT - 1) softmax_part(cur, pb_cur, kb, 1);
            }
        __builtin_amdgcn_sched_barrier(0);
        accept(cur, pb_cur);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (MASK_NEXT) mask(nxt, j + 1);
        wait_vmem();
        __syncthreads();
    };
    typedef std::false_type NF;
    typedef std::true_type YF;
    auto run = [&](int j0, int j1, auto mask_tag) __attribute__((always_inline)) {
        int j = j0;
        if (j < j1 && (j & 1)) iteration(j++, P1{}, mask_tag, NF{}, sB, sA);
        for (; j + 1 < j1; j += 2) {
            iteration(j, P0{}, mask_tag, NF{}, sA, sB);
            iteration(j + 1, P1{}, mask_tag, NF{}, sB, sA);
        }
        if (j < j1) iteration(j, P0{}, mask_tag, NF{}, sA, sB);
    };
    const int split = max(0, min(n_full - 1, ntiles - 1));
    int j_start = 0;
    if (ntiles > 1) {
        if (split > 0) iteration(0, P0{}, std::false_type{}, YF{}, sA, sB);
        else iteration(0, P0{}, std::true_type{}, YF{}, sA, sB);
        j_start = 1;
    }
    run(j_start, max(j_start, split), std::false_type{});
    run(max(j_start, split), ntiles - 1, std::true_type{});

    // Last tile L: V(L) copied now; softmax(L) next to PV(L-1), then PV(L).
    auto last = [&](floatx16 (&cur)[KB], auto par, auto first_tag) __attribute__((always_inline)) {
        constexpr bool FIRST = decltype(first_tag)::value;
        constexpr int PAR = decltype(par)::value;
        uint8_t *const vb_prev = PAR ? V0 : V1;
        uint8_t *const vb_cur = PAR ? V1 : V0;
        i32x8 &pb_cur = PAR ? pbB : pbA;
        i32x8 &pb_prev = PAR ? pbA : pbB;
        load_tile(v, ntiles - 1, vb_cur);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int h = 0; h < 2; ++h) softmax_part(cur, pb_cur, kb, h);
        if constexpr (!FIRST) {
#pragma unroll
            for (int db = 0; db < DB; ++db) oacc[db] = mfma_fp8(read_v(vb_prev, db), pb_prev, oacc[db]);
        }
        __builtin_amdgcn_sched_barrier(0);
        accept(cur, pb_cur);
        __builtin_amdgcn_sched_barrier(0);
        wait_vmem();
        __syncthreads();
        // One V operand in flight at a time here: the registers of the
        // pipeline are free, but the compiler would otherwise read all of
        // V at once and spill.
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            oacc[db] = mfma_fp8(read_v(vb_cur, db), pb_cur, oacc[db]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    if (ntiles == 1) last(sA, P0{}, YF{});
    else if ((ntiles - 1) & 1) last(sB, P1{}, NF{});
    else last(sA, P0{}, NF{});

    // Epilogue: O = vd * sum p'v / sum p'; lse = (m - kPShift + log2 l') ln 2.
    const float l_tot = sum_halves(l_run);
    if (my_q < N) {
        const float inv = vd / l_tot;
        float *orow = o + head + (size_t)my_q * D + 4 * lh;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int a = 0; a < 4; ++a)
                *(floatx4 *)(orow + 32 * db + 8 * a) =
                    floatx4{oacc[db][4 * a] * inv, oacc[db][4 * a + 1] * inv,
                            oacc[db][4 * a + 2] * inv, oacc[db][4 * a + 3] * inv};
        if (lse != nullptr && lh == 0)
            lse[(size_t)bh * N + my_q] = (m_run - kPShift + log2f(l_tot)) * kLn2;
    }
}

template <int D, bool CAUSAL>
static hipError_t launch(const FwdFp8Args &a, hipStream_t stream) {
    typedef Fp8Tile<D, CAUSAL> C;
    const int nq = (a.N + C::BM - 1) / C::BM;
    const long long blocks = (long long)nq * a.BH;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    // Scores are scale*qd*kd*<q8, k8>.  A negative factor flips the sign of
    // q8 (exact: the E4M3 sign bit); a zero factor makes every score 0.
    const float f = a.scale * a.qd * a.kd;
    const bool zero = f == 0.f;
    const float c = zero ? kLog2e : fabsf(f) * kLog2e;
    const uint32_t qand = zero ? 0u : 0xffffffffu;
    const uint32_t qxor = f < 0.f ? 0x80808080u : 0u;
    hipLaunchKernelGGL((fa_fwd_fp8_kernel<D, CAUSAL>), dim3((unsigned)blocks), dim3(C::THREADS),
                       0, stream, (const uint8_t *)a.q, (const uint8_t *)a.k,
                       (const uint8_t *)a.v, a.o, a.lse, a.N, nq, c, qand, qxor, a.vd);
    return hipGetLastError();
}

hipError_t launch_fwd_fp8(const FwdFp8Args &a, hipStream_t stream) {
    if (a.d == 128) return a.causal ? launch<128, true>(a, stream) : launch<128, false>(a, stream);
    if (a.d == 64) return a.causal ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace fa
