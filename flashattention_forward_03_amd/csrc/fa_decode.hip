// Decode attention over a paged KV cache for gfx950 (MI355X).
//
// One query per (sequence, head) attends to every cached token of its
// sequence; token t of sequence s sits in page page_table[s][t / 16], row
// t % 16 (inference kernel cookbook page, recipe 03 "Paged Attention": fixed
// size pages reached through a page table, scattered physical pages giving
// the same result).  The arithmetic is the forward's with one query row:
// scores, online softmax (running max and normaliser, NanoInfer page "Online
// Softmax"), rescaled accumulation of p * V.
//
// With one K/V head per query head (or a few query heads per K/V head) the
// work is bandwidth bound (one FMA per byte of K/V per query head), and the
// split kernel below uses packed dot products, laid out for HBM streaming.
// Wide grouped-query batches (many query heads per K/V head) go to the
// matrix-core kernel further down.
//   * Split-KV: work items of (sequence, chunk of 8 pages = 128 tokens,
//     K/V head, slice of up to 8 of the query heads that share it
//     (grouped-query attention, llm-kernel-lib page, "Ablation Study"));
//     enough of them fill the 256 CUs even when a batch mixes short and
//     long sequences (measured on MI355X: 8-page chunks beat 16 and 4 for
//     both multi-head and grouped-query batches).  Chunk boundaries depend
//     only on logical token positions.
//   * One wave per item, four items of consecutive K/V heads per workgroup.
//     The pool is [page, K/V head, 16, d], so the four waves' rows of one
//     page are 4 * 16 * d * 2 bytes contiguous (16 KB at d = 128): HBM sees
//     contiguous 16 KB reads instead of scattered 4 KB ones (measured:
//     random 4 KB blocks read at ~5.2 TB/s, 16 KB blocks at ~6.1).  Splitting
//     a chunk's pages over the waves instead (more waves, 4 KB blocks) was
//     measured slower except for single-sequence grouped-query batches.
//   * Within a wave, token row r = lane / (d/8) with 8 consecutive head dims
//     per lane: each wave step is one fully coalesced 16-byte load per lane
//     for K and one for V; up to sixteen steps are loaded before any is used.
//     Every loaded K/V row serves all query heads of the wave's slice, so a
//     K/V row is read once per slice, not once per query head.
//   * q.k uses packed dot2 instructions on the raw f16/bf16 pairs, reduced
//     over the d/8 lanes of a row with DPP moves; every lane keeps its own
//     online-softmax state per query head for its token stream; the streams
//     of a wave are merged with cross-lane moves at the end of the chunk
//     with the log-sum-exp rule.
//   * Chunks of one (sequence, head) are merged by a second small kernel with
//     the same rule; a sequence with a single chunk is finished directly.
#include "fa_common.h"
#include "fa_internal.h"
#include "fa_tile.h"

namespace fa {
namespace {

constexpr int PAGE = 16;
static_assert(NTHREADS == 256, "four waves per workgroup");
constexpr int STEPS_IN_FLIGHT = 16;  // wave steps loaded before any is used
constexpr int GROUP = NTHREADS / 64;  // heads per workgroup, one per wave

template <bool BF16>
__device__ __forceinline__ void widen8(const u32x4_t &w, float *f)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = lo16<BF16>(w[i]);
        f[2 * i + 1] = hi16<BF16>(w[i]);
    }
}

// Dot product of 8 packed head dims (two per dword): products are exact in
// fp32 (8- or 11-bit significands), sums rounded to fp32.  The dwords are
// copied out of the vectors before the bit casts: a bit cast applied to a
// vector element directly was compiled to read element 0 every time.
template <bool BF16>
__device__ __forceinline__ float dot8(const u32x4_t &a, const u32x4_t &b)
{
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t ai = a[i], bi = b[i];
        if constexpr (BF16)
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, ai), __builtin_bit_cast(bf16x2_t, bi),
                                                  acc, false);
        else
            acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, ai), __builtin_bit_cast(f16x2_t, bi), acc, false);
    }
    return acc;
}

// Sum / max over the token rows of a wave: lanes that differ only in the
// bits above log2(TPR) (the same 8 head dims of different rows).
template <int TPR>
__device__ __forceinline__ float rows_sum(float x)
{
    if constexpr (TPR == 8)
        x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));  // lane ^ 8
    x += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F));                          // lane ^ 16
    return x + other_half(x);                                                                            // lane ^ 32
}
template <int TPR>
__device__ __forceinline__ float rows_max(float x)
{
    if constexpr (TPR == 8)
        x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false)));
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F)));
    return fmaxf(x, other_half(x));
}

// Split-KV pass.  Work item of one wave: (sequence, chunk, K/V head, slice of
// up to QPW of the query heads that read that K/V head).  Every K/V row the
// wave loads serves all QPW query heads, so grouped-query heads cost no
// extra K/V traffic.
template <int D, bool BF16, int QPW>
__global__ __launch_bounds__(NTHREADS) void decode_split_kernel(
    const uint16_t *__restrict__ Qp, const uint16_t *__restrict__ Kp, const uint16_t *__restrict__ Vp,
    const int32_t *__restrict__ page_table, const int32_t *__restrict__ kv_lens, float *__restrict__ O,
    float *__restrict__ LSE, float *__restrict__ part_o, float *__restrict__ part_ml, int H, int Hkv, int group,
    int n_slices, int n_items, int n_wgroups, int max_pages, int num_pages, int max_chunks, float c_log2)
{
    constexpr int TPR = D / 8;              // lanes per token row (8 head dims each)
    constexpr int RPW = 64 / TPR;           // token rows per wave step (4 or 8)
    constexpr int SPP = PAGE / RPW;         // wave steps per page (4 or 2)
    constexpr int CHUNK = kDecodeChunkPages;
    constexpr int SIF = QPW <= 2 ? STEPS_IN_FLIGHT : (QPW == 4 ? STEPS_IN_FLIGHT / 2 : STEPS_IN_FLIGHT / 4);

    const int chunk = blockIdx.x % max_chunks;
    const int swg = blockIdx.x / max_chunks;
    const int s = swg / n_wgroups, wg = swg - s * n_wgroups;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int item = wg * GROUP + wave;
    const bool item_ok = item < n_items;
    const int kvh = item_ok ? item / n_slices : 0;
    const int h0 = kvh * group + (item_ok ? item - kvh * n_slices : 0) * QPW;   // first query head
    const int nq = item_ok ? min(QPW, kvh * group + group - h0) : 0;          // query heads in the slice

    int kvlen = kv_lens[s];
    kvlen = kvlen < 0 ? 0 : (kvlen > max_pages * PAGE ? max_pages * PAGE : kvlen);
    const int npages = (kvlen + PAGE - 1) / PAGE;
    const int nchunks = (npages + CHUNK - 1) / CHUNK;
    if (chunk >= nchunks)   // uniform over the workgroup (depends on s only)
        return;
    const int p_begin = chunk * CHUNK;
    const int p_end = min(p_begin + CHUNK, npages);
    const int nsteps = nq > 0 ? (p_end - p_begin) * SPP : 0;

    const int r = lane / TPR;      // token row within a wave step
    const int gd = lane - r * TPR; // which 8 head dims

    u32x4_t qv[QPW];
#pragma unroll
    for (int j = 0; j < QPW; ++j)
        qv[j] = load16(Qp + ((size_t)s * H + h0 + min(j, max(nq - 1, 0))) * D + 8 * gd);

    float m[QPW], l[QPW], acc[QPW][8];
#pragma unroll
    for (int j = 0; j < QPW; ++j) {
        m[j] = -INFINITY;
        l[j] = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            acc[j][i] = 0.f;
    }

    // the chunk's physical page ids, one per lane (CHUNK <= 64), read once so
    // that the K/V loads of each step do not wait behind a page-table load
    static_assert(CHUNK <= 64, "one page id per lane");
    int phys_lane = 0;
    if (lane < p_end - p_begin) {
        phys_lane = page_table[(size_t)s * max_pages + p_begin + lane];
        phys_lane = phys_lane < 0 ? 0 : (phys_lane >= num_pages ? num_pages - 1 : phys_lane);
    }
    const size_t head_off = (size_t)kvh * PAGE * D + 8 * gd;
    const size_t page_stride = (size_t)Hkv * PAGE * D;

    for (int k0 = 0; k0 < nsteps; k0 += SIF) {
        u32x4_t kr[SIF], vr[SIF];
        bool ok[SIF];
#pragma unroll
        for (int u = 0; u < SIF; ++u) {
            const int step = k0 + u;
            const int page = p_begin + step / SPP;
            const int row = (step % SPP) * RPW + r;
            const int tok = page * PAGE + row;
            ok[u] = step < nsteps && tok < kvlen;
            const int phys = __builtin_amdgcn_readlane(phys_lane, min(step / SPP, CHUNK - 1));
            if (ok[u]) {
                const size_t off = (size_t)phys * page_stride + head_off + (size_t)row * D;
                kr[u] = load16(Kp + off);
                vr[u] = load16(Vp + off);
            } else {
                kr[u] = u32x4_t{0, 0, 0, 0};
                vr[u] = u32x4_t{0, 0, 0, 0};
            }
        }
        // base-2 scores of every query head, then one rescale per head
        float t[QPW][SIF], mref[QPW];
#pragma unroll
        for (int j = 0; j < QPW; ++j) {
            float mx = -INFINITY;
#pragma unroll
            for (int u = 0; u < SIF; ++u) {
                float dot = dot8<BF16>(qv[j], kr[u]);
                dot = (TPR == 16) ? row16_sum(dot) : row8_sum(dot);
                t[j][u] = ok[u] ? dot * c_log2 : -INFINITY;
                mx = fmaxf(mx, t[j][u]);
            }
            const float m_new = fmaxf(m[j], mx);
            mref[j] = m_new == -INFINITY ? 0.f : m_new;   // rows with no valid token yet stay at zero
            const float alpha = fast_exp2(m[j] - mref[j]);
            l[j] *= alpha;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                acc[j][i] *= alpha;
            m[j] = m_new;
        }
#pragma unroll
        for (int u = 0; u < SIF; ++u) {
            float vf[8];
            widen8<BF16>(vr[u], vf);
#pragma unroll
            for (int j = 0; j < QPW; ++j) {
                const float p = fast_exp2(t[j][u] - mref[j]);
                l[j] += p;
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    acc[j][i] = fmaf(p, vf[i], acc[j][i]);
            }
        }
    }

    // ---- merge the RPW token streams of each head (log-sum-exp rule); the
    // lanes of row 0 write the chunk's result, 8 head dims each
    const bool writer = r == 0;
#pragma unroll
    for (int j = 0; j < QPW; ++j) {
        if (j >= nq)
            break;
        const float M = rows_max<TPR>(m[j]);
        const float w = m[j] == -INFINITY ? 0.f : fast_exp2(m[j] - M);
        const float L = rows_sum<TPR>(w * l[j]);
        float o[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            o[i] = rows_sum<TPR>(w * acc[j][i]);
        const size_t sh = (size_t)s * H + h0 + j;
        float *dst;
        float sc;
        if (nchunks == 1) {
            dst = O + sh * D;
            sc = 1.f / L;
        } else {
            dst = part_o + (sh * max_chunks + chunk) * D;
            sc = 1.f;
        }
        if (writer) {
            *reinterpret_cast<f32x4_t *>(dst + 8 * gd) = f32x4_t{o[0] * sc, o[1] * sc, o[2] * sc, o[3] * sc};
            *reinterpret_cast<f32x4_t *>(dst + 8 * gd + 4) = f32x4_t{o[4] * sc, o[5] * sc, o[6] * sc, o[7] * sc};
        }
        if (lane == 0) {
            if (nchunks == 1) {
                LSE[sh] = (M + __log2f(L)) * kLn2;
            } else {
                const size_t slot = sh * max_chunks + chunk;
                part_ml[2 * slot] = M;
                part_ml[2 * slot + 1] = L;
            }
        }
    }
}

// Grouped-query split-KV pass on the matrix cores.  When several query heads
// read one K/V head, the scores of a 32-token sub-tile for all of them form a
// small matrix product, S^T = K Q^T with the query heads as the 32 MFMA
// columns (unused columns are zero), and the outputs another, O^T = V^T P^T:
// the forward's tile machinery with 32 keys per tile.  Work item of one wave:
// (sequence, chunk of 8 pages, K/V head, slice of up to 32 of its query
// heads); four waves of consecutive K/V heads per workgroup, so that their
// copies of one page are 16 KB contiguous at d = 128.  Each wave copies its
// own sub-tiles (two pages of K and of V) into a private two-slot LDS ring
// with buffer-to-LDS loads, one buffer resource per page whose range ends at
// the sequence's last token (rows past it read as zero, whatever the slot
// holds); no barrier is needed.  The online softmax is the forward's (lazy
// running max), with the row sums kept per query head.
constexpr int MQ_HEADS = 32;   // query heads per wave (MFMA columns)

template <int D, bool BF16, int NW, int SLOTS>
__global__ __launch_bounds__(NW * 64) void decode_mfma_kernel(
    const uint16_t *__restrict__ Qp, const uint16_t *__restrict__ Kp, const uint16_t *__restrict__ Vp,
    const int32_t *__restrict__ page_table, const int32_t *__restrict__ kv_lens, float *__restrict__ O,
    float *__restrict__ LSE, float *__restrict__ part_o, float *__restrict__ part_ml, int H, int Hkv, int group,
    int n_slices, int n_items, int n_wgroups, int max_pages, int num_pages, int max_chunks, float c_log2)
{
    using G = Geometry<D>;
    static_assert(G::BN == 2 * PAGE, "a sub-tile is two pages");
    constexpr int PPP = PAGE * D * 2 / 1024;   // 1 KB copy pieces per page (4 at d = 128, 2 at d = 64)
    constexpr int ROWS_PP = 1024 / (D * 2);     // token rows per piece
    __shared__ __attribute__((aligned(1024))) unsigned char kring[NW][SLOTS][G::TILE];
    __shared__ __attribute__((aligned(1024))) unsigned char vring[NW][SLOTS][G::TILE];

    const int chunk = blockIdx.x % max_chunks;
    const int swg = blockIdx.x / max_chunks;
    const int s = swg / n_wgroups, wg = swg - s * n_wgroups;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int item = wg * NW + wave;
    if (item >= n_items)   // wave-uniform; no barrier follows
        return;
    const int kvh = item / n_slices;
    const int h0 = kvh * group + (item - kvh * n_slices) * MQ_HEADS;   // first query head
    const int nq = min(MQ_HEADS, kvh * group + group - h0);            // query heads in the slice

    int kvlen = kv_lens[s];
    kvlen = kvlen < 0 ? 0 : (kvlen > max_pages * PAGE ? max_pages * PAGE : kvlen);
    const int npages = (kvlen + PAGE - 1) / PAGE;
    const int nchunks = (npages + kDecodeChunkPages - 1) / kDecodeChunkPages;
    if (chunk >= nchunks)
        return;
    const int p_begin = chunk * kDecodeChunkPages;
    const int p_count = min(kDecodeChunkPages, npages - p_begin);
    const int nsub = (p_count + 1) / 2;

    const int l32 = lane & 31, hh = lane >> 5;
    // Q of query head h0 + l32 (zero for columns past the slice), B-operand layout
    u32x4_t qf[G::KSTEPS];
    {
        const bool qok = l32 < nq;
        const uint16_t *qp = Qp + ((size_t)s * H + h0 + (qok ? l32 : 0)) * D + 8 * hh;
#pragma unroll
        for (int c = 0; c < G::KSTEPS; ++c)
            qf[c] = qok ? load16(qp + 16 * c) : u32x4_t{0, 0, 0, 0};
    }
    int phys_lane = 0;
    if (lane < p_count) {
        phys_lane = page_table[(size_t)s * max_pages + p_begin + lane];
        phys_lane = phys_lane < 0 ? 0 : (phys_lane >= num_pages ? num_pages - 1 : phys_lane);
    }
    // this lane's byte offsets inside one (page, K/V head) block for its pieces:
    // piece u covers rows ROWS_PP u .., lane -> row + lane / (D / 8), LDS slot lane % (D / 8)
    unsigned koff[PPP], voff[PPP];
#pragma unroll
    for (int u = 0; u < PPP; ++u) {
        const int row = u * ROWS_PP + lane / G::DC;   // row in the page (= row in the sub-tile mod 16)
        const int pc = lane % G::DC;
        koff[u] = (unsigned)row * (D * 2) + (unsigned)swz_slot<G::DC>(pc, swz_k(row)) * 16u;
        voff[u] = (unsigned)row * (D * 2) + (unsigned)swz_slot<G::DC>(pc, swz_v(row)) * 16u;
    }
    const size_t page_elems = (size_t)Hkv * PAGE * D;
    const size_t head_elems = (size_t)kvh * PAGE * D;
    const uint32_t klds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void *)&kring[wave][0][0]);
    const uint32_t vlds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void *)&vring[wave][0][0]);
    // copies of sub-tile t (pages 2t, 2t + 1 of the chunk) into ring slot t % SLOTS
    auto issue = [&](int t) {
#pragma unroll
        for (int pg = 0; pg < 2; ++pg) {
            const int pi = 2 * t + pg;   // page within the chunk
            const int phys = __builtin_amdgcn_readlane(phys_lane, min(pi, kDecodeChunkPages - 1));
            const int tok0 = (p_begin + pi) * PAGE;
            const int rows = pi < p_count ? min(PAGE, kvlen - tok0) : 0;   // valid rows of this page
            const size_t base = (size_t)phys * page_elems + head_elems;
            const u32x4s_t kr = make_rsrc(Kp + base, rows * D * 2);
            const u32x4s_t vr = make_rsrc(Vp + base, rows * D * 2);
            const uint32_t slot = (uint32_t)(t % SLOTS) * G::TILE + (uint32_t)pg * (PAGE * D * 2);
#pragma unroll
            for (int u = 0; u < PPP; ++u) {
                const uint32_t kl = klds + slot + u * 1024, vl = vlds + slot + u * 1024;
                asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %2, 0 offen lds"
                             :
                             : "v"(koff[u]), "s"(kl), "s"(kr)
                             : "memory", "m0");
                asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %2, 0 offen lds"
                             :
                             : "v"(voff[u]), "s"(vl), "s"(vr)
                             : "memory", "m0");
            }
        }
    };

    f32x16_t oacc[G::DB];
#pragma unroll
    for (int db = 0; db < G::DB; ++db)
        oacc[db] = f32x16_t{};
    RowState st{-INFINITY, 0.f, -INFINITY};
    const float tau_log2 = kRescaleLog2<BF16>;
    const int krow_in_blk = sigma(l32);
    // SLOTS - 1 sub-tiles in flight ahead of the one being computed; a slot is
    // refilled only after this wave's reads of it (the previous iteration) are done
#pragma unroll
    for (int i = 0; i < SLOTS - 1; ++i)
        if (i < nsub)
            issue(i);
    for (int t = 0; t < nsub; ++t) {
        if (t + SLOTS - 1 < nsub)
            issue(t + SLOTS - 1);
        // sub-tile t landed once at most the copies of the later ones issued remain
        const int later = min(SLOTS - 1, nsub - 1 - t);
        static_assert(SLOTS <= 4, "wait counts below cover up to three later sub-tiles");
        if (later >= 3)
            wait_vmcnt<12 * PPP>();
        else if (later == 2)
            wait_vmcnt<8 * PPP>();
        else if (later == 1)
            wait_vmcnt<4 * PPP>();
        else
            wait_vmcnt<0>();
        const unsigned char *kc = &kring[wave][t % SLOTS][0];
        const unsigned char *vc = &vring[wave][t % SLOTS][0];
        f32x16_t sc[G::NBLK];
        qk_tile<D, BF16>(kc, krow_in_blk, hh, qf, sc);
        const int tok0 = (p_begin + 2 * t) * PAGE;
        if (tok0 + G::BN > kvlen)
            mask_tile<D>(sc, kvlen - (tok0 + 8 * hh));
        u32x4_t pf[G::PCH];
        float alpha;
        if (__builtin_expect(softmax_tile<D, BF16>(sc, st, pf, c_log2, tau_log2, alpha), 0))
            rescale_acc<D>(oacc, alpha);
        pv_tile<D, BF16>(vc, lane, hh, pf, oacc);
    }

    // this slice's partial (or final) rows: query head h0 + l32 in both halves
    const float L = st.l + other_half(st.l);
    const float M = st.m == -INFINITY ? 0.f : st.mc;   // running max in base-2 units (m * c)
    if (l32 >= nq)
        return;
    const size_t sh = (size_t)s * H + h0 + l32;
    float *dst;
    float scl;
    if (nchunks == 1) {
        dst = O + sh * D;
        scl = 1.f / L;
    } else {
        dst = part_o + (sh * max_chunks + chunk) * D;
        scl = 1.f;
    }
#pragma unroll
    for (int db = 0; db < G::DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int dim0 = 32 * db + 8 * g + 4 * hh;
            *reinterpret_cast<f32x4_t *>(dst + dim0) =
                f32x4_t{oacc[db][4 * g] * scl, oacc[db][4 * g + 1] * scl, oacc[db][4 * g + 2] * scl,
                        oacc[db][4 * g + 3] * scl};
        }
    if (hh == 0) {
        if (nchunks == 1) {
            LSE[sh] = (M + __log2f(L)) * kLn2;
        } else {
            const size_t slot = sh * max_chunks + chunk;
            part_ml[2 * slot] = M;
            part_ml[2 * slot + 1] = L;
        }
    }
}

// Wave-wide max / sum (all 64 lanes hold the result).
__device__ __forceinline__ float wave_max(float x)
{
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false)));
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false)));
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false)));
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false)));
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F)));   // xor 16
    return fmaxf(x, other_half(x));
}
__device__ __forceinline__ float wave_sum(float x)
{
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F));
    return x + other_half(x);
}

// Merge the chunk partials of each (sequence, head) with the log-sum-exp
// rule; write empty sequences.  One workgroup per (sequence, group of 4
// heads), one wave per head: the lanes load all chunks' (m, l) at once, and
// the chunk weights are broadcast with readlane for the weighted sum of the
// partial outputs (lanes over head dims).
template <int D>
__global__ __launch_bounds__(NTHREADS) void decode_combine_kernel(const int32_t *__restrict__ kv_lens,
                                                                  const float *__restrict__ part_o,
                                                                  const float *__restrict__ part_ml,
                                                                  float *__restrict__ O, float *__restrict__ LSE,
                                                                  int H, int n_hgroups, int max_pages, int max_chunks)
{
    constexpr int DPL = D / 64;
    const int s = blockIdx.x / n_hgroups, hg = blockIdx.x - s * n_hgroups;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int h = hg * GROUP + wave;
    if (h >= H)
        return;
    const size_t sh = (size_t)s * H + h;
    int kvlen = kv_lens[s];
    kvlen = kvlen < 0 ? 0 : (kvlen > max_pages * PAGE ? max_pages * PAGE : kvlen);
    const int npages = (kvlen + PAGE - 1) / PAGE;
    const int nchunks = (npages + kDecodeChunkPages - 1) / kDecodeChunkPages;
    if (nchunks == 1)
        return;   // finished by the split kernel
    if (nchunks == 0) {
#pragma unroll
        for (int k = 0; k < DPL; ++k)
            O[sh * D + lane + 64 * k] = 0.f;
        if (lane == 0)
            LSE[sh] = -INFINITY;
        return;
    }
    const float *ml = part_ml + sh * max_chunks * 2;
    const float *po = part_o + sh * max_chunks * D;
    float acc[DPL];
#pragma unroll
    for (int k = 0; k < DPL; ++k)
        acc[k] = 0.f;
    // chunks in groups of 64 (one per lane); M over all chunks first
    float M = -INFINITY;
    for (int c0 = 0; c0 < nchunks; c0 += 64)
        M = fmaxf(M, wave_max(c0 + lane < nchunks ? ml[2 * (c0 + lane)] : -INFINITY));
    float L = 0.f;
    for (int c0 = 0; c0 < nchunks; c0 += 64) {
        const int c = c0 + lane;
        const float w = c < nchunks ? fast_exp2(ml[2 * c] - M) : 0.f;
        L += wave_sum(c < nchunks ? w * ml[2 * c + 1] : 0.f);
        const int n = min(64, nchunks - c0);
        // 16 chunks' partial rows are loaded before any is used
        for (int j0 = 0; j0 < n; j0 += 16) {
            float v[16][DPL];
#pragma unroll
            for (int j = 0; j < 16; ++j)
#pragma unroll
                for (int k = 0; k < DPL; ++k)
                    v[j][k] = j0 + j < n ? po[(size_t)(c0 + j0 + j) * D + lane + 64 * k] : 0.f;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const float wj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), j0 + j));
#pragma unroll
                for (int k = 0; k < DPL; ++k)
                    acc[k] = fmaf(wj, v[j][k], acc[k]);
            }
        }
    }
    const float inv = 1.f / L;
#pragma unroll
    for (int k = 0; k < DPL; ++k)
        O[sh * D + lane + 64 * k] = acc[k] * inv;
    if (lane == 0)
        LSE[sh] = (M + __log2f(L)) * kLn2;
}

template <int D, bool BF16, int QPW>
hipError_t launch(const DecodeArgs &a, hipStream_t stream)
{
    const int max_chunks = decode_max_chunks(a.max_pages);
    const int group = a.H / a.Hkv;
    const int n_slices = (group + QPW - 1) / QPW;
    const int n_items = a.Hkv * n_slices;
    const int n_wgroups = (n_items + GROUP - 1) / GROUP;
    const long long grid = (long long)a.S * n_wgroups * max_chunks;
    hipLaunchKernelGGL((decode_split_kernel<D, BF16, QPW>), dim3((unsigned)grid), dim3(NTHREADS), 0, stream,
                       (const uint16_t *)a.q, (const uint16_t *)a.k_pages, (const uint16_t *)a.v_pages,
                       a.page_table, a.kv_lens, a.o, a.lse, a.part_o, a.part_ml, a.H, a.Hkv, group, n_slices,
                       n_items, n_wgroups, a.max_pages, a.num_pages, max_chunks, a.scale * kLog2e);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const int n_hgroups = (a.H + GROUP - 1) / GROUP;
    hipLaunchKernelGGL((decode_combine_kernel<D>), dim3((unsigned)(a.S * n_hgroups)), dim3(NTHREADS), 0, stream,
                       a.kv_lens, a.part_o, a.part_ml, a.o, a.lse, a.H, n_hgroups, a.max_pages, max_chunks);
    return hipGetLastError();
}

template <int D, bool BF16, int NW, int SLOTS>
hipError_t launch_mfma(const DecodeArgs &a, hipStream_t stream)
{
    const int max_chunks = decode_max_chunks(a.max_pages);
    const int group = a.H / a.Hkv;
    const int n_slices = (group + MQ_HEADS - 1) / MQ_HEADS;
    const int n_items = a.Hkv * n_slices;
    const int n_wgroups = (n_items + NW - 1) / NW;
    const long long grid = (long long)a.S * n_wgroups * max_chunks;
    hipLaunchKernelGGL((decode_mfma_kernel<D, BF16, NW, SLOTS>), dim3((unsigned)grid), dim3(NW * 64), 0, stream,
                       (const uint16_t *)a.q, (const uint16_t *)a.k_pages, (const uint16_t *)a.v_pages,
                       a.page_table, a.kv_lens, a.o, a.lse, a.part_o, a.part_ml, a.H, a.Hkv, group, n_slices,
                       n_items, n_wgroups, a.max_pages, a.num_pages, max_chunks, a.scale * kLog2e);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const int n_hgroups = (a.H + GROUP - 1) / GROUP;
    hipLaunchKernelGGL((decode_combine_kernel<D>), dim3((unsigned)(a.S * n_hgroups)), dim3(NTHREADS), 0, stream,
                       a.kv_lens, a.part_o, a.part_ml, a.o, a.lse, a.H, n_hgroups, a.max_pages, max_chunks);
    return hipGetLastError();
}

// Which kernel a grouped-query batch uses (measured on MI355X, S32 and S1
// batches of 512..8192 tokens, d = 128): the matrix-core kernel is 1.8x
// faster at 8 query heads per K/V head and 2.3x for multi-query heads, and
// faster at 4 heads for a few sequences; at 4 heads over many (sequence, K/V
// head) pairs the dot-product kernel keeps more copies in flight (it holds no
// LDS) and streams ~10 % faster.
bool use_mfma_decode(int S, int Hkv, int group)
{
    if (group >= kDecodeMfmaGroup)
        return true;
    return group >= 4 && (long long)S * Hkv <= 64;
}

// Query heads per wave: the whole group when it has at most 8 heads (padded
// to 1, 2, 4 or 8), else slices of 8.
template <int D, bool BF16>
hipError_t launch_qpw(const DecodeArgs &a, hipStream_t stream)
{
    const int group = a.H / a.Hkv;
    if (use_mfma_decode(a.S, a.Hkv, group)) {
        // as many waves per workgroup as it has work items (LDS is per wave)
        const int items = a.Hkv * ((group + MQ_HEADS - 1) / MQ_HEADS);
        if (items >= 4)
            return launch_mfma<D, BF16, 4, 2>(a, stream);
        if (items >= 2)
            return launch_mfma<D, BF16, 2, 2>(a, stream);
        return launch_mfma<D, BF16, 1, 2>(a, stream);
    }
    if (group == 1)
        return launch<D, BF16, 1>(a, stream);
    if (group == 2)
        return launch<D, BF16, 2>(a, stream);
    if (group <= 4)
        return launch<D, BF16, 4>(a, stream);
    return launch<D, BF16, 8>(a, stream);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream)
{
    if (a.d == 64)
        return a.bf16 ? launch_qpw<64, true>(a, stream) : launch_qpw<64, false>(a, stream);
    return a.bf16 ? launch_qpw<128, true>(a, stream) : launch_qpw<128, false>(a, stream);
}

}  // namespace fa
