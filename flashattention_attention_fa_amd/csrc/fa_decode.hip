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
// hide under the K/V stream, the next block's loads are issued before the
// current block is computed, and the cache is read with non-temporal loads
// (every byte of it is used once).
//
// MFMA 16x16x32 (16 columns = up to 16 query heads of one group):
//   S^T (16 keys x 16 heads) = K (16 x 32 dims) Q^T, K straight from global
//   memory into A-operand registers (paged caches: K rows staged through LDS
//   like V, see load()); two S^T blocks (32 keys) form the P^T
//   operand of O^T (16 dims x 16 heads) += V^T (16 dims x 32 keys) P^T, with
//   V^T read from a row-major LDS copy of the V rows by transposing reads.
#include <mutex>
#include <type_traits>
#include <vector>

#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {

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
    static constexpr int BK = 32;                  // keys per wave step
    static constexpr int COLS = 16;                // query heads per workgroup
    static constexpr int LD = D + 8;               // V tile row stride (elements)
    static constexpr int KCH = D / 8;              // 16-byte chunks per row
    static constexpr int VROWS = 64 / KCH;         // V rows covered by one wave load
    static constexpr int VLOADS = BK / VROWS;      // V loads per lane per step
    static constexpr int V_ELEMS = BK * LD;        // per wave
};

template <int D, bool PAGED>
struct DecBuf {
    u32x4 kf[2][D / 32];               // K A-operands, 2 S^T blocks x D/32 steps
    u32x4 vr[DecTile<D>::VLOADS];      // V rows, staged to LDS
};
// Paged: K rows are loaded whole, like V, and staged through LDS as well.
template <int D>
struct DecBuf<D, true> {
    u32x4 kr[DecTile<D>::VLOADS];      // K rows, staged to LDS
    u32x4 vr[DecTile<D>::VLOADS];      // V rows, staged to LDS
};

// Paged caches (PAGED): k and v are pools [num_pages, page_size, Hkv, d];
// sequence b owns seq_lens[b] keys, key j stored in page
// block_table[b][j / page_size], slot j % page_size.
struct PagedCache {
    const int *block_table;   // [B, pages_per_seq]
    const int *seq_lens;      // [B]
    int page_size, pages_per_seq, num_pages;
};

// Paged caches store the rows of all Hkv heads of a token next to each
// other, so one head's rows are Hkv*D*2 bytes apart.  A paged workgroup
// takes HG adjacent kv heads of the shard with WH waves each: its waves then
// read HG*D*2 contiguous bytes of every token row instead of one head's
// D*2 bytes, which DRAM serves far better.  8 waves fill a CU.
template <typename T, int D, bool PAGED, int HG, int WH>
__global__ __launch_bounds__(64 * HG * WH, 8 / (HG * WH)) void fa_decode_split_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, float *__restrict__ ws_o,
    float *__restrict__ ws_lse, int Hq, int Hkv, int L, int nsplit, int chunk,
    int ncc, float c, PagedCache pc) {
    typedef DecTile<D> C;
    typedef typename T::vec8 vec8;
    typedef typename T::scalar scalar;
    constexpr int LD = C::LD;

    static_assert((HG == 1 && WH == C::WAVES) || PAGED, "head groups are for paged caches");
    constexpr int NW = WH * HG;           // waves of the workgroup
    constexpr int NT = 64 * NW;

    // V tile staging, one slab per wave; reused for the final merge.
    __shared__ __attribute__((aligned(16))) uint16_t Vs[NW][C::V_ELEMS];
    // Paged: the K rows of the step, same layout as the V slab.
    __shared__ __attribute__((aligned(16))) uint16_t Ks[PAGED ? NW : 1][PAGED ? C::V_ELEMS : 1];
    __shared__ float sm_m[NW][C::COLS], sm_l[NW][C::COLS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave_id = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar block-table reads
    const int hh = wave_id / WH;   // kv head of the group
    const int wave = wave_id % WH;   // wave among the head's WH
    const int lj = lane & 15;   // column (query head) / A-operand row
    const int lg = lane >> 4;   // contraction group 0..3

    const int s = blockIdx.x;
    const int g = (blockIdx.y / ncc) * HG + hh, cc = blockIdx.y % ncc;
    const int b = blockIdx.z;
    const int G = Hq / Hkv;
    const int hq0 = g * G + cc * C::COLS;
    const int ncol = min(C::COLS, G - cc * C::COLS);

    // Keys of this sequence and this shard.  Paged: the sequence's own
    // length (clamped to what its block-table row can address), and shards
    // of whole 32-key blocks, so that each 16-key half block lies in one page.
    int Lb = L, chunkb = chunk;
    if constexpr (PAGED) {
        Lb = min(max(pc.seq_lens[b], 0), pc.pages_per_seq * pc.page_size);
        chunkb = (((Lb + nsplit - 1) / nsplit) + C::BK - 1) / C::BK * C::BK;
    }
    const int k_lo = min(s * chunkb, Lb);
    const int k_hi = min(Lb, k_lo + chunkb);
    const int nblk = k_hi > k_lo ? (k_hi - k_lo + C::BK - 1) / C::BK : 0;

    const size_t kvhead = PAGED ? 0 : ((size_t)b * Hkv + g) * (size_t)L * D;
    const uint32_t head_bytes = PAGED ? 0u : (uint32_t)L * D * 2;
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(k + kvhead, head_bytes);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(v + kvhead, head_bytes);
    // Paged: element offset of the first row of 16-key half block h of the
    // block at key0 (page of its first key, clamped to the sequence's last
    // key so masked rows stay inside a valid page; page ids clamped to the
    // pool).  Rows of a half block are Hkv*D elements apart.
    const size_t prow = (size_t)Hkv * D;
    auto half_base = [&](int key0, int h) __attribute__((always_inline)) {
        const int kh = key0 + 16 * h;
        const int kc = min(kh, Lb - 1);
        int pg = pc.block_table[(size_t)b * pc.pages_per_seq + kc / pc.page_size];
        pg = min(max(pg, 0), pc.num_pages - 1);
        return ((size_t)pg * pc.page_size + (kh % pc.page_size)) * prow + (size_t)g * D;
    };

    // Q^T fragments: B operand, lane (lj, lg) holds head hq0+lj, dims 32t+8lg..+8.
    vec8 qf[D / 32];
    {
        const bool ok = lj < ncol;
        const uint16_t *src = q + ((size_t)b * Hq + hq0 + (ok ? lj : 0)) * D + 8 * lg;
#pragma unroll
        for (int t = 0; t < D / 32; ++t)
            qf[t] = as_vec8<vec8>(ok ? *(const u32x4 *)(src + 32 * t) : zero4());
    }

    // V staging: lane (dc, vrow) loads chunk dc of rows vrow + VROWS*r.
    const int dc = lane % C::KCH, vrow = lane / C::KCH;

    // Keys past L read as zero (buffer range check); keys past the shard end
    // are masked out of the softmax below.
    auto load = [&](DecBuf<D, PAGED> &bf, int n) {
        const int key0 = k_lo + C::BK * n;
        if constexpr (PAGED) {
            // Whole 2*D-byte rows per 16 lanes for both K and V: a head's rows
            // are Hkv*D elements apart in the pool, and loading each row in
            // one go keeps its bytes together in the memory requests.
            const size_t hb[2] = {half_base(key0, 0), half_base(key0, 1)};
#pragma unroll
            for (int r = 0; r < C::VLOADS; ++r) {
                const int row = vrow + C::VROWS * r;   // row / 16 is static per r
                const size_t off = hb[row >> 4] + (row & 15) * prow + 8 * dc;
                bf.kr[r] = __builtin_nontemporal_load((const u32x4 *)(k + off));
                bf.vr[r] = __builtin_nontemporal_load((const u32x4 *)(v + off));
            }
        } else {
#pragma unroll
            for (int beta = 0; beta < 2; ++beta)
#pragma unroll
                for (int t = 0; t < D / 32; ++t)
                    bf.kf[beta][t] = buffer_load16_stream(
                        kr, (uint32_t)((key0 + 16 * beta + lj) * D + 32 * t + 8 * lg) * 2u);
#pragma unroll
            for (int r = 0; r < C::VLOADS; ++r)
                bf.vr[r] = buffer_load16_stream(vr, (uint32_t)((key0 + vrow + C::VROWS * r) * D + 8 * dc) * 2u);
        }
    };

    floatx4 oacc[D / 16];
#pragma unroll
    for (int db = 0; db < D / 16; ++db) oacc[db] = floatx4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;
    uint16_t *vt = Vs[wave_id];
    uint16_t *kt = Ks[PAGED ? wave_id : 0];
    // ds_read_b64_tr_b16 addressing: lane j of group lg points at row
    // 4*lg + j/4, column 4*(j%4) (plus the 16-dim block offset).
    const uint16_t *va = vt + (4 * lg + (lj >> 2)) * LD + 4 * (lj & 3);

    auto compute = [&](const DecBuf<D, PAGED> &bf, int n) {
        const int key0 = k_lo + C::BK * n;
#pragma unroll
        for (int r = 0; r < C::VLOADS; ++r)
            *(u32x4 *)(vt + (vrow + C::VROWS * r) * LD + 8 * dc) = bf.vr[r];
        // K A-operands: lane (lj, lg) holds key 16beta + lj, dims 32t + 8lg..+8.
        u32x4 kf[2][D / 32];
        if constexpr (PAGED) {
#pragma unroll
            for (int r = 0; r < C::VLOADS; ++r)
                *(u32x4 *)(kt + (vrow + C::VROWS * r) * LD + 8 * dc) = bf.kr[r];
            // The K slab is private to this wave (see the V slab below).
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
            for (int beta = 0; beta < 2; ++beta)
#pragma unroll
                for (int t = 0; t < D / 32; ++t)
                    kf[beta][t] = *(const u32x4 *)(kt + (16 * beta + lj) * LD + 32 * t + 8 * lg);
        } else {
#pragma unroll
            for (int beta = 0; beta < 2; ++beta)
#pragma unroll
                for (int t = 0; t < D / 32; ++t) kf[beta][t] = bf.kf[beta][t];
        }
        // S^T block beta: lane (lj, lg), register r holds key key0 + 16beta + 4lg + r.
        floatx4 sc[2];
#pragma unroll
        for (int beta = 0; beta < 2; ++beta) {
            sc[beta] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < D / 32; ++t)
                sc[beta] = T::mfma16(as_vec8<vec8>(kf[beta][t]), qf[t], sc[beta]);
        }
        if (key0 + C::BK > k_hi) {
#pragma unroll
            for (int beta = 0; beta < 2; ++beta)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (key0 + 16 * beta + 4 * lg + r >= k_hi) sc[beta][r] = -INFINITY;
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
        // P^T operand: element e holds key 4lg + e (block 0) for e < 4 and
        // key 16 + 4lg + e - 4 (block 1) for e >= 4.
        vec8 pb;
#pragma unroll
        for (int beta = 0; beta < 2; ++beta)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float p = __builtin_amdgcn_exp2f(fmaf(sc[beta][r], c, -mb));
                l_run += p;
                pb[4 * beta + r] = (scalar)p;
            }
        // The V slab is private to this wave: order its LDS writes before the
        // reads below (LDS operations of one wave complete in order).
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int db = 0; db < D / 16; ++db) {
            const vec8 vtp = join8<vec8>(lds_read_tr4(va + 16 * db), lds_read_tr4(va + 16 * LD + 16 * db));
            oacc[db] = T::mfma16(vtp, pb, oacc[db]);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };

    {
        DecBuf<D, PAGED> A, B;
        int n = wave;
        if (n < nblk) load(A, n);
        for (; n < nblk; n += 2 * WH) {
            if (n + WH < nblk) load(B, n + WH);
            compute(A, n);
            if (n + WH >= nblk) break;
            if (n + 2 * WH < nblk) load(A, n + 2 * WH);
            compute(B, n + WH);
        }
    }

    // Merge the WH wave states of each head.  Per column: M = max_w m_w,
    // Lsum = sum_w l_w 2^(m_w - M), O = sum_w 2^(m_w - M) O_w / Lsum.
    float l_w = l_run + __shfl_xor(l_run, 16, 64);
    l_w += __shfl_xor(l_w, 32, 64);
    if (lg == 0) {
        sm_m[wave_id][lj] = m_run;
        sm_l[wave_id][lj] = l_w;
    }
    __syncthreads();
    const int w0 = hh * WH;   // first wave of this head
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < WH; ++w) M = fmaxf(M, sm_m[w0 + w][lj]);
    const float Mb = M == -INFINITY ? 0.f : M;
    float Lsum = 0.f;
#pragma unroll
    for (int w = 0; w < WH; ++w)
        Lsum += sm_l[w0 + w][lj] * __builtin_amdgcn_exp2f(sm_m[w0 + w][lj] - Mb);
    const float f = Lsum > 0.f ? __builtin_amdgcn_exp2f(m_run - Mb) / Lsum : 0.f;
    // Scaled wave outputs go to LDS as part[wave][col][d] (reusing the V
    // slabs).  O^T accumulator: lane (lj, lg), register r of block db holds
    // dim 16db + 4lg + r of head hq0 + lj.
    float *part = reinterpret_cast<float *>(&Vs[0][0]);
    static_assert(NW * C::COLS * D * 4 <= (int)sizeof(Vs), "merge buffer");
    __syncthreads();
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
        *(floatx4 *)&part[(wave_id * C::COLS + lj) * D + 16 * db + 4 * lg] = oacc[db] * f;
    __syncthreads();
    // Head x of the group writes query heads hq0 - hh*G + x*G + col.
    for (int idx = tid; idx < HG * ncol * D; idx += NT) {
        const int x = idx / (ncol * D), col = (idx / D) % ncol, d = idx % D;
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < WH; ++w) acc += part[((x * WH + w) * C::COLS + col) * D + d];
        ws_o[(((size_t)b * Hq + hq0 + (x - hh) * G + col) * nsplit + s) * D + d] = acc;
    }
    if (wave == 0 && lane < ncol)
        ws_lse[((size_t)b * Hq + hq0 + lane) * nsplit + s] =
            Lsum > 0.f ? (M + log2f(Lsum)) * kLn2 : -INFINITY;
}

__device__ __forceinline__ float block_max128(float x, float *red) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
    __syncthreads();
    x = fmaxf(red[0], red[1]);
    __syncthreads();
    return x;
}

__device__ __forceinline__ float block_sum128(float x, float *red) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
    __syncthreads();
    x = red[0] + red[1];
    __syncthreads();
    return x;
}

// Combine for at most NS shards: every thread loads all shard lse values and
// its output dim of every shard at once (one memory round trip) and forms
// the weights itself (base-2 exponentials of log2(e)-scaled differences).
template <int NS>
__global__ __launch_bounds__(128) void fa_decode_combine_few_kernel(
    const float *__restrict__ ws_o, const float *__restrict__ ws_lse,
    float *__restrict__ o, float *__restrict__ lse, int D, int nsplit) {
    const int tid = threadIdx.x;
    const size_t row = blockIdx.x;
    const float *pl = ws_lse + row * nsplit;
    const float *po = ws_o + row * (size_t)nsplit * D;
    const bool mine = tid < D;
    float lv[NS], ov[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        lv[s] = s < nsplit ? pl[s] : -INFINITY;
        ov[s] = (s < nsplit && mine) ? po[(size_t)s * D + tid] : 0.f;
    }
    float M = -INFINITY;
#pragma unroll
    for (int s = 0; s < NS; ++s) M = fmaxf(M, lv[s]);
    const float mb = M == -INFINITY ? 0.f : M;
    float wsum = 0.f, acc = 0.f;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const float w = __builtin_amdgcn_exp2f((lv[s] - mb) * kLog2e);
        wsum += w;
        acc = fmaf(w, ov[s], acc);
    }
    if (mine) o[row * D + tid] = M == -INFINITY ? 0.f : acc / wsum;
    if (lse != nullptr && tid == 0) lse[row] = M == -INFINITY ? -INFINITY : M + logf(wsum);
}

// Combine: one 128-thread workgroup per (batch, query head).  The shard
// weights exp(lse_s - lse) are computed once per shard and shared via LDS;
// each thread then sums one output dim over the shards.
__global__ __launch_bounds__(128) void fa_decode_combine_kernel(
    const float *__restrict__ ws_o, const float *__restrict__ ws_lse,
    float *__restrict__ o, float *__restrict__ lse, int D, int nsplit) {
    constexpr int kChunk = 256;
    __shared__ float w[kChunk];
    __shared__ float red[2];
    const int tid = threadIdx.x;
    const size_t row = blockIdx.x;
    const float *pl = ws_lse + row * nsplit;
    const float *po = ws_o + row * (size_t)nsplit * D;

    float M = -INFINITY;
    for (int s = tid; s < nsplit; s += 128) M = fmaxf(M, pl[s]);
    M = block_max128(M, red);
    float wsum = 0.f;
    if (M != -INFINITY)
        for (int s = tid; s < nsplit; s += 128) wsum += expf(pl[s] - M);
    wsum = block_sum128(wsum, red);
    const float total = M == -INFINITY ? -INFINITY : M + logf(wsum);

    float acc = 0.f;
    for (int s0 = 0; s0 < nsplit; s0 += kChunk) {
        const int n = min(kChunk, nsplit - s0);
        for (int s = tid; s < n; s += 128)
            w[s] = total == -INFINITY ? 0.f : expf(pl[s0 + s] - total);
        __syncthreads();
        // No branch on the weight: shards without keys hold O_s = 0 and
        // weight 0, and a branch-free loop lets the loads issue together.
        if (tid < D) {
            const float *pp = po + (size_t)s0 * D + tid;
#pragma unroll 8
            for (int s = 0; s < n; ++s) acc += w[s] * pp[(size_t)s * D];
        }
        __syncthreads();
    }
    if (tid < D) o[row * D + tid] = acc;
    if (lse != nullptr && tid == 0) lse[row] = total;
}

// Workgroups a paged launch keeps at least (one per CU of MI355X), when it
// chooses how many kv heads one workgroup takes.
constexpr long long kDecodeMinWorkgroups = 256;

template <typename T, int D>
static hipError_t launch(const DecodeArgs &a, hipStream_t stream) {
    typedef DecTile<D> C;
    const int G = a.Hq / a.Hkv;
    const int ncc = (G + C::COLS - 1) / C::COLS;
    const float c = kLog2e / sqrtf((float)D);
    if ((long long)a.Hkv * ncc > 65535 || a.B > 65535) return hipErrorInvalidConfiguration;
    PagedCache pc = {a.block_table, a.seq_lens, a.page_size, a.pages_per_seq, a.num_pages};
    auto split = [&](auto paged, auto hg, auto wh) {
        constexpr int HG = decltype(hg)::value, WH = decltype(wh)::value;
        hipLaunchKernelGGL((fa_decode_split_kernel<T, D, decltype(paged)::value, HG, WH>),
                           dim3(a.nsplit, a.Hkv / HG * ncc, a.B), dim3(64 * HG * WH), 0, stream,
                           (const uint16_t *)a.q, (const uint16_t *)a.k, (const uint16_t *)a.v,
                           a.ws_o, a.ws_lse, a.Hq, a.Hkv, a.L, a.nsplit, a.chunk, ncc, c, pc);
    };
    typedef std::integral_constant<int, 1> I1;
    typedef std::integral_constant<int, 2> I2;
    typedef std::integral_constant<int, 4> I4;
    // Paged: the largest head group that divides Hkv and still gives every
    // CU a workgroup.
    const long long units = (long long)a.nsplit * a.B * ncc;
    if (a.block_table == nullptr)
        split(std::false_type{}, I1{}, I4{});
    else if (a.Hkv % 4 == 0 && units * (a.Hkv / 4) >= kDecodeMinWorkgroups)
        split(std::true_type{}, I4{}, I2{});
    else if (a.Hkv % 2 == 0)
        split(std::true_type{}, I2{}, I4{});
    else
        split(std::true_type{}, I1{}, I4{});
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.nsplit <= 16)
        hipLaunchKernelGGL(fa_decode_combine_few_kernel<16>, dim3(a.B * a.Hq), dim3(128), 0, stream,
                           a.ws_o, a.ws_lse, a.o, a.lse, D, a.nsplit);
    else if (a.nsplit <= 32)
        hipLaunchKernelGGL(fa_decode_combine_few_kernel<32>, dim3(a.B * a.Hq), dim3(128), 0, stream,
                           a.ws_o, a.ws_lse, a.o, a.lse, D, a.nsplit);
    else
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

// Fixed partial-result buffer for callers that cannot allocate: every GPU the
// library runs on holds one copy from the module load until the process
// ends.  In host code `scratch` names a host-side stand-in, not the device
// copy, so the kernels get the device address that hipGetSymbolAddress
// returns for the current device, looked up once per device.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

namespace {
std::mutex g_scratch_mutex;
std::vector<void *> g_scratch;   // device address of `scratch`, by HIP device id
}  // namespace

hipError_t decode_scratch(void **ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if ((size_t)dev >= g_scratch.size()) g_scratch.resize((size_t)dev + 1, nullptr);
    if (g_scratch[(size_t)dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch[(size_t)dev] = p;
    }
    *ptr = g_scratch[(size_t)dev];
    return hipSuccess;
}

}  // namespace fa
