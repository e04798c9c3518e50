// fa_fwd.hip -- exact attention forward for gfx950 (MI355X).
//
// What it computes: softmax(scale * Q K^T [+ causal mask]) V and the per-row
// natural log-sum-exp, tile by tile, never writing the N x N score matrix
// (dailyaiworld page "FlashAttention-3 vs Triton Kernels", introduction).
// The running-max / running-sum rescaling is the "online normalisation"
// the smzdm digest (section 6) tells multi-GPU users to check first.
//
// Work split: each wave owns 32 queries of one (batch, head); a workgroup
// is 8 waves (256 queries) without a mask at d = 128 and 4 waves (128
// queries) otherwise.  Every SIMD runs two waves (at most 256 registers each):
// while one wave computes exponentials the other keeps the matrix core
// busy.  Keys stream through
// LDS in tiles of 64: the K and V tiles of the coming iterations are copied
// from global memory straight into the LDS buffers that just became free
// while the current tile is computed (one barrier per tile).
//
// The loop is also software pipelined inside each wave (the pages contrast
// this "different iterations of one role" schedule with warp
// specialisation): iteration j issues the QK^T MFMAs of tile j+1 next to the
// exponentials of tile j, then the PV MFMAs of tile j next to the exponents
// (c*s - m) of tile j+1, so that both MFMA phases carry vector work.
//
// Per wave and tile (32 queries x 64 keys), on 16x16x32 MFMAs:
//   S^T = K Q^T   4 key blocks x 2 query blocks of 16x16, contraction over
//                 the head dim in steps of 32; Q lives in registers for the
//                 whole loop (B operand), K rows come from LDS (A operand,
//                 each read serves both query blocks).  A lane holds 16
//                 scores of each of TWO queries; the four lane groups that
//                 share a query combine their maxima and sums with two lane
//                 swaps, needed only at the end and on the rare path.
//   online softmax in the exp2 domain with c = scale*log2(e):
//                 m' = max(m, c*max_j s_j);  alpha = 2^(m - m');
//                 p_j = 2^(c*s_j - m');  l = alpha*l + sum p_j;  O *= alpha
//                 m is taken exactly from the first tile; later tiles keep it
//                 unless their weights, computed with it, grow past a bound
//                 (then m, O and l are updated as above and the tile's
//                 weights recomputed).  Any m that keeps the weights finite
//                 gives the same O and lse; the bound keeps them small.
//   O^T += V^T P^T  P^T is the S^T accumulator converted to 16 bits in
//                 place: two score blocks make one 32-key contraction (the
//                 key order inside it is the accumulator's, matched by the V
//                 operand); V^T comes from the V tile through the transposing
//                 LDS read.
// The 16x16x32 product reads and writes a quarter of the accumulator per
// instruction that the 32x32x16 one does, for half its work: measured alone
// on MI355X (two boxes), under the board's power limit, it sustains 9-12 %
// more fp16 and 2-6 % more bf16 throughput, and the forward follows.
// Epilogue: O /= l, lse = (m + log2 l) * ln 2, both fp32.  With bf16 weights
//                 O is divided by l plus a correction that swaps in the
//                 rounded weights of tiles that could dominate the row (see
//                 rounded_sum below).
#include <type_traits>

#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {

// Workgroup shape.  Every wave owns 32 queries and every SIMD runs two
// waves.  Without a mask and at d = 128 the workgroup is 8 waves (256
// queries, one per CU), so each K/V tile copied into LDS serves twice the
// queries; with the causal mask it is 4 waves (128 queries, two per CU),
// which keeps the diagonal tiles that a workgroup must visit, and the tail
// of the grid, small.  At d = 64 (half the MFMA work per tile) 4 waves are
// faster without a mask too.  All picked by measurement on MI355X.
template <int D, bool CAUSAL>
constexpr int fwd_waves() { return (CAUSAL || D == 64) ? 4 : 8; }

template <int D, bool CAUSAL>
struct FwdTile {
    static constexpr int WAVES = fwd_waves<D, CAUSAL>();
    static constexpr int BM = 32 * WAVES;         // queries per workgroup
    static constexpr int KB = 2;                  // 32-key blocks per tile
    static constexpr int BN = 32 * KB;            // keys per tile
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int BLOCKS_PER_CU = 8 / WAVES;
    static constexpr int KCH = D / 8;             // 16-byte chunks per row
    static constexpr int RPI = 64 / KCH;          // rows one wave copy instruction covers
    static constexpr int ROWS = BN / WAVES;       // rows of a tile each wave copies
    static constexpr int LOADS = ROWS / RPI;      // copy instructions per wave, per tensor, per tile
    static constexpr int ELEMS = BN * D;
    // Rows that share a bank line: 64 banks hold 16 chunks, i.e. 16/KCH rows.
    static constexpr int ROWS_PER_LINE = 16 / KCH;
    static_assert(ROWS % RPI == 0, "tile must split evenly over the waves");
};

// LDS tiles are unpadded: a direct copy writes 1 KB contiguous per wave
// instruction, 16 bytes per lane, each lane from any global address.
//  K tile, row-major, read 16 bytes per lane, 16 consecutive rows per
//    16-lane group.  Chunk c of row r is stored at chunk position c ^ swz_k(r);
//    swz_k = (r / ROWS_PER_LINE) % KCH spreads 16 consecutive rows over all
//    16 chunk positions of a bank line.
//  V tile, in 32-byte slabs: slab (q, r) holds dims 16q..16q+15 of key row
//    r, at element (q * BN + r) * 16.  A transposing read takes 4 rows x 32
//    bytes per 16 lanes and 16 consecutive rows per wave: 16 consecutive
//    slabs, 512 contiguous bytes, each half wave on distinct banks.  Every
//    read address is one per-lane register plus a compile-time offset (dim
//    block, key step), where a row-major tile with a row swizzle needs one
//    register per dim block.
template <int D>
__device__ __forceinline__ int swz_k(int r) {
    constexpr int KCH = D / 8, ROWS_PER_LINE = 16 / KCH;
    return (r / ROWS_PER_LINE) % KCH;
}

// Bound on one lane's sum of the unnormalised weights of a tile.  The running
// max m is taken exactly from the first tile and afterwards only raised when a
// tile's weights, computed with the current m, sum past this bound in some
// lane (which includes any weight that overflowed).  Below the bound every
// weight is at most 2^10: well inside fp16 and bf16, and O and l stay exact
// in fp32.  Random data essentially never comes near it, so the row maximum
// of a tile is computed only on that rare path.
constexpr float kTileSumLimit = 1024.0f;

// bf16 weights keep 8 significant bits, so rounding one for the PV product
// can move it by 2^-8 of itself (fp16: 2^-11).  If its key dominates the
// row's softmax, O inherits that error almost whole (up to 2^-8 * |v|) when
// the numerator sums rounded weights and the denominator l exact ones.  With
// bf16 the kernel therefore keeps, next to l, a correction: for every tile in
// which some lane's weights sum to more than that lane's running sum (the
// only tiles in which a weight can hold more than half of its row), the sum
// of the weights as rounded minus their exact sum.  O is divided by l plus
// the correction, so such a tile's weights enter numerator and denominator
// rounded alike and a dominant weight's rounding cancels; lse keeps the
// exact l.  The other tiles' weights each hold at most half of their row.

// Packed variable-length batches (VARLEN): q, k, v, o are [T, H, D] with
// sequence b at rows [cu[b], cu[b+1]); lse is [H, T].
struct Varlen {
    const int *cu;   // [B + 1]
    int H, T;
};

template <typename T, int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__((64 * fwd_waves<D, CAUSAL>()), (8 / fwd_waves<D, CAUSAL>())) void fa_fwd_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, float *__restrict__ o,
    float *__restrict__ lse, int Nmax, int nq, float c, uint32_t qand, uint32_t qxor,
    Varlen vl) {
    typedef FwdTile<D, CAUSAL> C;
    static_assert(C::THREADS == 64 * fwd_waves<D, CAUSAL>() &&
                      C::BLOCKS_PER_CU == 8 / fwd_waves<D, CAUSAL>(),
                  "launch bounds must match the tile shape");
    typedef typename T::vec8 vec8;
    typedef typename T::scalar scalar;
    constexpr int BM = C::BM, BN = C::BN, KCH = C::KCH;
    constexpr int KB = BN / 16;            // 16-key blocks per tile
    constexpr int QB = 2;                  // 16-query blocks per wave
    constexpr int KST = D / 32;            // QK^T MFMAs per (key block, query block)
    constexpr int DB = D / 16;             // 16-dim blocks of O
    constexpr int PS = BN / 32;            // PV MFMAs per (dim block, query block)
    // Normalisation by the rounded weights of dominant tiles (bf16 only).
    constexpr bool RCORR = std::is_same<T, BF16>::value;

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
    const int li = lane & 15;   // column (query) inside a 16-query block
    const int lg = lane >> 4;   // lane group: rows 4lg..4lg+3 of each 16-row block

    // Block -> (head, q-tile).  Consecutive logical ids walk the q-tiles of
    // one head, so the workgroups resident on one XCD share that head's K/V
    // in their L2.  Causal: each head's q-tiles run longest (most keys) first,
    // so the short ones fill the tail.
    // Varlen: sequences differ in length, and each XCD takes a contiguous
    // range of (sequence, head) pairs, so the pairs are ordered head-major
    // across sequences: every XCD gets an equal share of every sequence's
    // heads, while the q-tiles of one head stay together on one XCD.
    const unsigned id = xcd_remap(blockIdx.x, gridDim.x);
    int bh = (int)(id / (unsigned)nq);
    const int qt = CAUSAL ? nq - 1 - (int)(id % (unsigned)nq) : (int)(id % (unsigned)nq);
    if constexpr (VARLEN) {
        const int nseq = (int)(gridDim.x / (unsigned)nq) / vl.H;
        bh = (bh % nseq) * vl.H + bh / nseq;
    }
    const int q0 = qt * BM;
    // This (sequence, head): N keys = N queries, row 0 at element `head`,
    // consecutive rows RS elements apart, lse of row i at lse_row0 + i.
    // Varlen: bounds read from cu are clamped to [0, T] and to Nmax, and
    // workgroups past the sequence end leave at once (before any barrier).
    int N = Nmax;
    size_t head = (size_t)bh * Nmax * D, lse_row0 = (size_t)bh * Nmax;
    const int RS = VARLEN ? vl.H * D : D;
    if constexpr (VARLEN) {
        const int b = bh / vl.H, h = bh % vl.H;
        const int s0 = min(max(vl.cu[b], 0), vl.T);
        const int e = min(max(vl.cu[b + 1], s0), vl.T);
        N = min(e - s0, Nmax);
        head = ((size_t)s0 * vl.H + h) * D;
        lse_row0 = (size_t)h * vl.T + s0;
        if (q0 >= N) return;
    }
    const uint32_t head_bytes = (uint32_t)((N > 0 ? (size_t)(N - 1) * RS + D : 0) * 2);
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(q + head, head_bytes);
    const int qw = q0 + wave * 32;    // first query of this wave
    int my_q[QB];                     // this lane's queries (column li of each block)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) my_q[qb] = qw + 16 * qb + li;

    // Q fragments: B operand of block qb, step t: lane (li, lg) holds query
    // my_q[qb], dims 32t+8lg..+8 (rows past N read as zero).
    vec8 qf[QB][KST];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int t = 0; t < KST; ++t) {
            u32x4 x = buffer_load16(qr, (uint32_t)(my_q[qb] * RS + 32 * t + 8 * lg) * 2u);
            // scale < 0: flip the sign of q (exact) and use |scale|;
            // scale == 0: every visible score is 0, i.e. q = 0.
            x = (x & qand) ^ qxor;
            qf[qb][t] = as_vec8<vec8>(x);
        }

    const int kv_end = CAUSAL ? min(N, q0 + BM) : N;
    const int ntiles = (kv_end + BN - 1) / BN;

    // Tile copies go straight from global memory into LDS.  Copy
    // instruction n = wave*LOADS + i of a tile fills elements
    // [512n, 512n + 512) of its buffer.  K: rows [RPI*n, RPI*(n+1)); lane l
    // fills chunk position l%KCH of its row with the source chunk that the
    // swizzle puts there.  V: 32-byte slabs [32n, 32n + 32); lane l fills
    // half l%2 of slab 32n + l/2, and slab s holds dims 16(s/BN)..+16 of key
    // row s%BN.  Rows past N read as zero (buffer range check) and are
    // masked out of the softmax; tiles past the last one are copied the same
    // way and never read.
    static_assert(C::RPI * D == 512, "one copy instruction fills 512 elements");
    // V: instruction n reads rows 32(n%2) + lane/2 of dim block n/2.  With
    // the packed layout's run-time row stride, its per-lane offset is kept
    // as one register (voff0) plus a uniform part that goes into the
    // instruction's buffer resource; with the dense layout the offsets are
    // cheap to keep per instruction.
    static_assert(BN == 64, "two V copy instructions per dim block");
    uint32_t koff[C::LOADS], voff[C::LOADS];
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
        const int n = wave * C::LOADS + i;
        const int row = n * C::RPI + lane / KCH;
        const int pos = lane % KCH;
        koff[i] = (uint32_t)(row * RS + 8 * (pos ^ swz_k<D>(row))) * 2u;
        voff[i] = (uint32_t)((32 * (n % 2) + lane / 2) * RS + 16 * (n / 2) + 8 * (lane % 2)) * 2u;
    }
    const uint32_t voff0 = (uint32_t)((lane / 2) * RS + 8 * (lane % 2)) * 2u;
    auto vpart = [&](int i) __attribute__((always_inline)) {
        const int n = wave * C::LOADS + i;
        return (uint32_t)((n % 2) * 32 * RS + 16 * (n / 2)) * 2u;
    };
    // The tile's base goes into the (scalar) buffer resource, so the
    // per-lane offsets stay fixed and the range check still covers the end of
    // the head: a resource past the end has zero records and reads zeros.
    auto tile_rsrc = [&](const uint16_t *base, int tile, uint32_t extra = 0u) __attribute__((always_inline)) {
        const uint32_t off = (uint32_t)tile * (uint32_t)(BN * RS * 2) + extra;
        const uint64_t addr = (uint64_t)(uintptr_t)base + off;
        // Uniform values: keep the resource in scalar registers.
        const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)addr);
        const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(addr >> 32));
        const uint32_t n = __builtin_amdgcn_readfirstlane(off < head_bytes ? head_bytes - off : 0u);
        return make_rsrc((const void *)(uintptr_t)(((uint64_t)hi << 32) | lo), n);
    };
    auto load_k = [&](int tile, uint16_t *buf) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t r = tile_rsrc(k + head, tile);
#pragma unroll
        for (int i = 0; i < C::LOADS; ++i)
            buffer_load16_lds(r, koff[i], buf + 512 * (wave * C::LOADS + i));
    };
    auto load_v = [&](int tile, uint16_t *buf) __attribute__((always_inline)) {
        if constexpr (VARLEN) {
#pragma unroll
            for (int i = 0; i < C::LOADS; ++i)
                buffer_load16_lds(tile_rsrc(v + head, tile, vpart(i)), voff0,
                                  buf + 512 * (wave * C::LOADS + i));
        } else {
            const __amdgpu_buffer_rsrc_t r = tile_rsrc(v + head, tile);
#pragma unroll
            for (int i = 0; i < C::LOADS; ++i)
                buffer_load16_lds(r, voff[i], buf + 512 * (wave * C::LOADS + i));
        }
    };

    // K operand of key block kb, step t: lane (li, lg) holds key row
    // 16kb + li, logical chunk 4t + lg.  The swizzle of row 16kb + li
    // depends on li only, so one register per step serves every key block.
    int kcol[KST];
#pragma unroll
    for (int t = 0; t < KST; ++t) kcol[t] = li * D + 8 * ((4 * t + lg) ^ swz_k<D>(li));
    auto read_k = [&](const uint16_t *buf, int kb, int t) __attribute__((always_inline)) {
        return as_vec8<vec8>(*(const u32x4 *)(buf + 16 * kb * D + kcol[t]));
    };
    // V^T operand of PV MFMA (db, s): contraction element e of lane group lg
    // is key 32s + 16(e/4) + 4lg + e%4, the key the P operand below puts
    // there.  Two transposing reads: lane j of group lg points at row
    // 32s + 16h + 4lg + j/4 (read h) and dims 16db + 4(j%4) of slab
    // (db, row), and receives dim 16db + j of its group's four rows.  The 16
    // rows of one read are 16 consecutive slabs, 512 contiguous bytes.
    const int vlane = (4 * lg + (li >> 2)) * 16 + 4 * (li & 3);
    auto read_v = [&](const uint16_t *buf, int db, int s) __attribute__((always_inline)) {
        const uint16_t *p = buf + (db * BN + 32 * s) * 16 + vlane;
        return join8<vec8>(lds_read_tr4(p), lds_read_tr4(p + 16 * 16));
    };

    floatx4 oacc[DB][QB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) oacc[db][qb] = floatx4{0.f, 0.f, 0.f, 0.f};
    float m_run[QB], l_run[QB], corr[QB];   // corr: rounded minus exact weights of dominant tiles
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) { m_run[qb] = -INFINITY; l_run[qb] = 0.f; corr[qb] = 0.f; }
    const floatx4 zero4v = {0.f, 0.f, 0.f, 0.f};

    // S^T of one tile, two register sets used alternately (tile parity):
    // lane (li, lg), register r of block (kb, qb) holds the score of query
    // my_q[qb] against key tile*BN + 16kb + 4lg + r.
    floatx4 sA[KB][QB], sB[KB][QB];

    // Keys past the end and (causal) keys after the query get -inf.
    auto mask = [&](floatx4 (&x)[KB][QB], int tile) __attribute__((always_inline)) {
        const int kv0 = tile * BN;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const int lim = CAUSAL ? min(N - 1, my_q[qb]) : N - 1;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int key = kv0 + 16 * kb + 4 * lg + r;
                    if (key > lim) x[kb][qb][r] = -INFINITY;
                }
        }
    };
    // Largest of x over this lane's values of block qb and the three other
    // lane groups holding the same query.  (maximum, not fmaxf: no NaN can
    // occur here, and maximum maps onto v_maximum3_f32.)
    auto row_max = [&](const floatx4 (&x)[KB][QB], int qb) __attribute__((always_inline)) {
        float mx = __builtin_elementwise_maximum(x[0][qb][0], x[0][qb][1]);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r = kb == 0 ? 2 : 0; r < 4; ++r) mx = __builtin_elementwise_maximum(mx, x[kb][qb][r]);
        return max_quarters(mx);
    };
    auto rescale = [&](int qb, float alpha) __attribute__((always_inline)) {
        l_run[qb] *= alpha;
        corr[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[db][qb] *= alpha;
    };

    // P^T operands: pb[s][qb] element e is the weight of key
    // 32s + 16(e/4) + 4lg + e%4, i.e. register e%4 of score block 2s + e/4.
    vec8 pb[PS][QB];
    // The softmax reads a tile's scores as exponents x = c*s - m, formed in
    // place by shift() while the previous tile's PV MFMAs run (the vector
    // ALU is otherwise idle there).  m is finite from tile 0 on (every query
    // sees key 0), so x never involves an infinite base.  tsum collects this
    // lane's part of the tile's row sums, from the fp32 weights (the 16-bit
    // rounding of P, up to 2^-8 relative for bf16 and 2^-11 for fp16, stays
    // out of l and lse).
    auto shift = [&](floatx4 (&x)[KB][QB], int idx) __attribute__((always_inline)) {
        const int kb = idx / (4 * QB), qb = (idx / 4) % QB, r = idx % 4;
        x[kb][qb][r] = fmaf(x[kb][qb][r], c, -m_run[qb]);
    };
    float tsum[QB];
    auto softmax_part = [&](const floatx4 (&x)[KB][QB], int kb, int qb) __attribute__((always_inline)) {
        if (kb == 0) tsum[qb] = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float p = __builtin_amdgcn_exp2f(x[kb][qb][r]);
            tsum[qb] += p;
            pb[kb / 2][qb][4 * (kb % 2) + r] = (scalar)p;
        }
    };
    // bf16: this lane's part of block qb's weight sum as rounded for the PV
    // product (pairs summed exactly in fp32 by the dot-product instruction).
    auto rounded_sum = [&](int qb) __attribute__((always_inline)) {
        float rs = 0.f;
        if constexpr (RCORR) {
            typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
            const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
            for (int s = 0; s < PS; ++s) {
                const vec8 w = pb[s][qb];
                rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(w, w, 0, 1), one, rs, false);
                rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(w, w, 2, 3), one, rs, false);
                rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(w, w, 4, 5), one, rs, false);
                rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(w, w, 6, 7), one, rs, false);
            }
        }
        return rs;
    };
    // Accept the tile's weights, or (rare) raise m by the tile's largest
    // exponent (to the tile's exact row maximum), rescale O and l, shift the
    // exponents and recompute the weights.  The negated test also catches an
    // infinite sum.  Then, for bf16, the correction of a tile that may hold a
    // dominant weight (see the note on bf16 weights above).
    auto accept = [&](floatx4 (&x)[KB][QB]) __attribute__((always_inline)) {
        if (__any(!(tsum[0] <= kTileSumLimit) || !(tsum[1] <= kTileSumLimit))) {
            // Keep this a real branch: the compiler would otherwise turn it
            // into unconditional work on every tile.
            asm volatile("" ::: "memory");
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                // delta >= 0; a query whose keys are all masked has -inf.
                const float delta = fmaxf(row_max(x, qb), 0.f);
                m_run[qb] += delta;
                rescale(qb, __builtin_amdgcn_exp2f(-delta));
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) x[kb][qb] -= delta;
            }
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) softmax_part(x, kb, qb);
        }
        if constexpr (RCORR) {
            if (__any(tsum[0] > l_run[0] || tsum[1] > l_run[1])) {
                asm volatile("" ::: "memory");
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) corr[qb] += rounded_sum(qb) - tsum[qb];
            }
        }
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) l_run[qb] += tsum[qb];
    };

    // Tiles before n_full need no mask for any query of the workgroup: all
    // their keys exist and (causal) precede the workgroup's first query.
    int n_full = N / BN;
    if (CAUSAL) n_full = min(n_full, q0 / BN);
    n_full = min(n_full, ntiles);

    // Prologue: K(0), K(1), V(0) into LDS; scores and maxima of tile 0.
    load_k(0, K0);
    load_v(0, V0);
    load_k(1, K1);
    wait_vmem();
    __syncthreads();
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int t = 0; t < KST; ++t) {
            const vec8 kop = read_k(K0, kb, t);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
                sA[kb][qb] = T::mfma16(kop, qf[qb][t], t == 0 ? zero4v : sA[kb][qb]);
        }
    if (n_full == 0) mask(sA, 0);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        m_run[qb] = row_max(sA, qb) * c;
#pragma unroll
        for (int i = 0; i < 4 * KB; ++i) shift(sA, (i / 4) * 4 * QB + qb * 4 + i % 4);
    }
    // Iteration 0 overwrites K0; every wave must be done reading K(0).
    __syncthreads();

    // Iteration j (parity PAR = j % 2): softmax of tile j next to QK^T of
    // tile j+1, then PV of tile j.  LDS holds K(j+1) in K[1-PAR] and V(j) in
    // V[PAR]; K(j+2) and V(j+1) are copied meanwhile into K[PAR] and V[1-PAR],
    // which iteration j-1 finished reading, and the barrier at the end
    // publishes them.  Two waves share each SIMD, so one wave's exponentials
    // run under the other's MFMAs; inside a wave, the exponentials of tile j
    // are also independent of the QK^T MFMAs next to them.  Phase boundaries
    // are fenced so the compiler keeps that order.
    auto iteration = [&](int j, auto par, auto mask_tag, floatx4 (&cur)[KB][QB],
                         floatx4 (&nxt)[KB][QB]) __attribute__((always_inline)) {
        constexpr bool MASK_NEXT = decltype(mask_tag)::value;
        constexpr int PAR = decltype(par)::value;
        uint16_t *const kb_next = PAR ? K0 : K1;   // holds K(j+1)
        uint16_t *const kb_fill = PAR ? K1 : K0;   // receives K(j+2)
        uint16_t *const vb_cur = PAR ? V1 : V0;    // holds V(j)
        uint16_t *const vb_fill = PAR ? V0 : V1;   // receives V(j+1)

        load_k(j + 2, kb_fill);
        load_v(j + 1, vb_fill);
        // Phase 1: QK^T(j+1) | softmax(j): the KB*QB softmax blocks spread
        // over the KB*KST*QB MFMAs.
        constexpr int NM1 = KB * KST * QB, SB1 = KB * QB;
        static_assert(NM1 % SB1 == 0, "phase 1 spreads whole softmax blocks");
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int t = 0; t < KST; ++t) {
                const vec8 kop = read_k(kb_next, kb, t);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    nxt[kb][qb] = T::mfma16(kop, qf[qb][t], t == 0 ? zero4v : nxt[kb][qb]);
                    const int m = (kb * KST + t) * QB + qb;
                    if (m % (NM1 / SB1) == 0) {
                        const int sb = m / (NM1 / SB1);
                        softmax_part(cur, sb / QB, sb % QB);
                    }
                }
            }
        __builtin_amdgcn_sched_barrier(0);
        accept(cur);
        __builtin_amdgcn_sched_barrier(0);
        // Phase 2: PV(j) | mask and exponents of tile j+1, SPM scores next
        // to each of the DB*PS*QB MFMAs.
        if constexpr (MASK_NEXT) mask(nxt, j + 1);
        constexpr int NM2 = DB * PS * QB, SPM = 4 * KB * QB / NM2;
        static_assert(SPM * NM2 == 4 * KB * QB, "phase 2 must cover every score once");
#pragma unroll
        for (int s = 0; s < PS; ++s)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const vec8 vop = read_v(vb_cur, db, s);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    oacc[db][qb] = T::mfma16(vop, pb[s][qb], oacc[db][qb]);
                    const int i = SPM * ((s * DB + db) * QB + qb);
#pragma unroll
                    for (int e = 0; e < SPM; ++e) shift(nxt, i + e);
                }
            }
        // Causal kernels: at most four V reads ahead of the PV MFMAs (left to
        // itself the scheduler issues them all early, and these kernels,
        // with their mask state, then spill).
        if constexpr (CAUSAL) {
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
            for (int i = 0; i < NM2 / 2 - 2; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
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
    auto last = [&](floatx4 (&cur)[KB][QB], const uint16_t *vb) __attribute__((always_inline)) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) softmax_part(cur, kb, qb);
        accept(cur);
#pragma unroll
        for (int s = 0; s < PS; ++s)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const vec8 vop = read_v(vb, db, s);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) oacc[db][qb] = T::mfma16(vop, pb[s][qb], oacc[db][qb]);
            }
    };
    if ((ntiles - 1) & 1) last(sB, V1); else last(sA, V0);

    // Epilogue.  O^T accumulator: lane (li, lg), register r of block
    // (db, qb) holds dim 16db + 4lg + r of query my_q[qb].  O is written
    // through LDS (the K/V tile buffers are free once every wave is past the
    // last tile), so that each store instruction writes whole rows: straight
    // from the accumulator, one instruction would put 16 bytes into each of
    // 64 rows, and where rows lie far apart (the H*d stride of packed
    // variable-length tensors) such partly written lines are evicted and
    // written back more than once.
    // Packed variable-length layout: the lane index is recomputed from the
    // execution mask, so nothing needs to carry it, or this lane's query
    // numbers, through the loop (its kernels otherwise spilled them).
    const int lane_e =
        VARLEN ? (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)) : lane;
    float inv[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float l_tot = sum_quarters(l_run[qb]);
        inv[qb] = 1.f / (RCORR ? l_tot + sum_quarters(corr[qb]) : l_tot);
        const int qe = qw + 16 * qb + (lane_e & 15);
        if (lse != nullptr && lane_e < 16 && qe < N)
            lse[lse_row0 + qe] = (m_run[qb] + log2f(l_tot)) * kLn2;
    }
    // Each wave stages its 32 rows, CPR 16-byte chunks (4*CPR dims) per
    // pass, in its share of one tile buffer: chunk c of row r is stored at
    // position c ^ (r % 16), which keeps the column writes and the row reads
    // on distinct banks.
    constexpr int WPB = C::WAVES / 4;                       // waves per tile buffer
    constexpr int CPR = C::ELEMS * 2 / WPB / 32 / 16;       // chunks per staged row
    constexpr int RPI = 64 / CPR;                           // rows per store instruction
    constexpr int NPASS = D / 4 / CPR;
    static_assert(CPR >= 16 && CPR % 4 == 0 && NPASS * CPR * 4 == D && 64 % CPR == 0,
                  "staging must fit a tile buffer");
    uint16_t *const sbuf = (wave % 4) == 0 ? K0 : (wave % 4) == 1 ? K1 : (wave % 4) == 2 ? V0 : V1;
    floatx4 *const stage = (floatx4 *)sbuf + (wave / 4) * 32 * CPR;
    __syncthreads();
    // The staging addresses depend on the lane only; taken from an opaque
    // copy of the recomputed lane index, the compiler cannot compute them
    // before the loop (where they would stay live, and spill, across it).
    int el = lane_e;
    asm volatile("" : "+v"(el));
    const int eli = el & 15, elg = el >> 4;
#pragma unroll
    for (int pass = 0; pass < NPASS; ++pass) {
#pragma unroll
        for (int dl = 0; dl < CPR / 4; ++dl)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const int db = pass * (CPR / 4) + dl;
                const int row = 16 * qb + eli, ch = 4 * dl + elg;
                stage[row * CPR + (ch ^ eli)] = oacc[db][qb] * inv[qb];
            }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int i = 0; i < 32 / RPI; ++i) {
            const int r = i * RPI + el / CPR, ch = el % CPR;
            const floatx4 x = stage[r * CPR + (ch ^ (r % 16))];
            if (qw + r < N)
                *(floatx4 *)(o + head + (size_t)(qw + r) * RS + 4 * (CPR * pass + ch)) = x;
        }
        __builtin_amdgcn_wave_barrier();
    }
}

template <typename T, int D, bool CAUSAL>
static hipError_t launch(const FwdArgs &a, hipStream_t stream) {
    typedef FwdTile<D, CAUSAL> C;
    const int nq = (a.N + C::BM - 1) / C::BM;   // N = longest sequence when varlen
    const long long blocks = (long long)nq * a.BH;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const bool zero = a.scale == 0.f;
    const float c = zero ? kLog2e : fabsf(a.scale) * kLog2e;
    const uint32_t qand = zero ? 0u : 0xffffffffu;
    const uint32_t qxor = a.scale < 0.f ? 0x80008000u : 0u;
    const Varlen vl = {a.cu_seqlens, a.H, a.T};
    if (a.cu_seqlens != nullptr)
        hipLaunchKernelGGL((fa_fwd_kernel<T, D, CAUSAL, true>), dim3((unsigned)blocks),
                           dim3(C::THREADS), 0, stream, (const uint16_t *)a.q,
                           (const uint16_t *)a.k, (const uint16_t *)a.v, a.o, a.lse, a.N, nq, c,
                           qand, qxor, vl);
    else
        hipLaunchKernelGGL((fa_fwd_kernel<T, D, CAUSAL, false>), dim3((unsigned)blocks),
                           dim3(C::THREADS), 0, stream, (const uint16_t *)a.q,
                           (const uint16_t *)a.k, (const uint16_t *)a.v, a.o, a.lse, a.N, nq, c,
                           qand, qxor, vl);
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
