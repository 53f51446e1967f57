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
// The work is bandwidth bound: every cached K and V byte is read once and
// serves all the query heads that share its K/V head (grouped-query
// attention, llm-kernel-lib page, "Ablation Study").  Both kernels below form
// the scores and the output on the matrix cores, with the query heads of one
// K/V head as the MFMA columns:
//   * up to 16 query heads per K/V head (multi-head attention included): one
//     page of 16 tokens per step on 16x16 tiles, a two-page LDS ring per
//     wave, one wave per workgroup, so that many waves each keep a page in
//     flight (decode_mfma16_kernel);
//   * wider groups (multi-query): 32-token sub-tiles on 32x32 tiles, the
//     forward's tile machinery (decode_mfma_kernel).
// Split-KV: a work item is (sequence, chunk of consecutive pages, K/V head,
// slice of its query heads); chunk boundaries depend only on logical token
// positions, so the result does not depend on where the pages sit.  The
// chunks of one (sequence, head) are merged by a second small kernel with the
// log-sum-exp rule; a sequence with a single chunk is finished directly.
#include "fa_common.h"
#include "fa_internal.h"
#include "fa_tile.h"

namespace fa {
namespace {

constexpr int PAGE = 16;
static_assert(NTHREADS == 256, "four waves per workgroup");
constexpr int GROUP = NTHREADS / 64;  // heads per combine workgroup, one per wave

// Split-KV pass for wide query-head groups (more than 16 query heads per K/V
// head, e.g. multi-query) on 32x32 matrix-core tiles: the scores of a
// 32-token sub-tile for all the group's heads form a small matrix product,
// S^T = K Q^T with the query heads as the 32 MFMA columns (unused columns are
// zero), and the outputs another, O^T = V^T P^T: the forward's tile machinery
// with 32 keys per tile.  Work item of one wave: (sequence, chunk of 8 pages,
// K/V head, slice of up to 32 of its query heads); four waves of consecutive K/V heads per workgroup, so that their
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
    RowState st{INFINITY, 0.f};
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
        softmax_tile<D, BF16>(sc, st, pf, c_log2, tau_log2, oacc);
        pv_tile<D, BF16>(vc, lane, hh, pf, oacc);
    }

    // this slice's partial (or final) rows: query head h0 + l32 in both halves
    const float L = st.l + other_half(st.l);
    const float M = st.nmc == INFINITY ? 0.f : -st.nmc;   // running max in base-2 units (m * c)
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

// Split-KV pass for up to 16 query heads per K/V head (one: multi-head
// attention) on 16x16 matrix-core tiles, one page (16 tokens) per step.  Work
// item of one wave: (sequence, chunk of CHUNK pages, K/V head, slice of up to
// 16 of its query heads).  Per page: S^T = K Q^T with
// v_mfma_f32_16x16x32 (16 tokens x 16 query heads, d/32 k-steps), the lazy
// online softmax on each lane's four scores, then O^T += V^T P^T with
// v_mfma_f32_16x16x16 (the lane's four probabilities are exactly its B
// operand, and the transposing LDS read yields V^T's A operand).  Each lane
// holds one query head (lane % 16) and four of the page's tokens; the four
// lanes of a head keep one shared running max and their own partial sums.
// Pages are copied by buffer-to-LDS loads into a private SLOTS-page ring per
// wave, SLOTS - 1 pages ahead (SLOTS = 1: each page is copied, then used),
// each page's buffer range ending at the sequence's last token (rows past it
// read as zero); no barrier is needed.  A page in flight costs 8 KB of LDS
// at d = 128, so many waves, each with its page in flight, share a CU.
constexpr int MQ16_HEADS = 16;   // query heads per wave (MFMA columns)

// LDS slot of 16-byte chunk c of page row r (rows of D * 2 bytes): an XOR
// that keeps the 16 rows' chunk reads and the transposing reads spread over
// the banks.
template <int D>
__device__ __forceinline__ int pg_slot(int c, int r)
{
    return D == 128 ? (c ^ (r & 15)) : (c ^ ((r >> 1) & 7));
}

template <int D, bool BF16, int NW, int SLOTS, int CHUNK>
__global__ __launch_bounds__(NW * 64, 4) void decode_mfma16_kernel(
    const uint16_t *__restrict__ Qp, const uint16_t *__restrict__ Kp, const uint16_t *__restrict__ Vp,
    const int32_t *__restrict__ page_table, const int32_t *__restrict__ kv_lens, float *__restrict__ O,
    float *__restrict__ LSE, float *__restrict__ part_o, float *__restrict__ part_ml, int H, int Hkv, int group,
    int n_slices, int n_items, int n_wgroups, int max_pages, int num_pages, int max_chunks, float c_log2)
{
    static_assert(D == 64 || D == 128, "head dim");
    static_assert(SLOTS >= 1 && SLOTS <= 4, "ring depth");
    constexpr int DC = D / 8;                  // 16-byte chunks per row
    constexpr int PB = PAGE * D * 2;           // bytes of one (page, head) block
    constexpr int PIECES = PB / 1024;          // 1 KB copy pieces per block (2 or 4)
    constexpr int RPP = 64 / DC;               // rows per piece
    constexpr int KSTEPS = D / 32;             // 16x16x32 k-steps
    constexpr int DBLK = D / 16;               // 16-row blocks of O^T
    __shared__ __attribute__((aligned(1024))) unsigned char kring[NW][SLOTS][PB];
    __shared__ __attribute__((aligned(1024))) unsigned char vring[NW][SLOTS][PB];

    // chunk-major order: the chunks that exist for every sequence come first,
    // the (mostly empty) high chunk indices of the long sequences last
    const int n_sw = gridDim.x / max_chunks;
    const int chunk = blockIdx.x / n_sw;
    const int swg = blockIdx.x - chunk * n_sw;
    const int s = swg / n_wgroups, wg = swg - s * n_wgroups;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int item = wg * NW + wave;
    if (item >= n_items)   // wave-uniform; no barrier follows
        return;
    const int kvh = item / n_slices;
    const int h0 = kvh * group + (item - kvh * n_slices) * MQ16_HEADS;   // first query head
    const int nq = min(MQ16_HEADS, kvh * group + group - h0);             // query heads in the slice
    const int p_begin = chunk * CHUNK;

    // the chunk's table entries (page ids, one per lane) are loaded beside
    // kv_len instead of after it; entries past the sequence are not used
    static_assert(CHUNK <= 64, "one page id per lane");
    int phys_lane = 0;
    if (lane < CHUNK)
        phys_lane = page_table[(size_t)s * max_pages + min(p_begin + lane, max_pages - 1)];
    int kvlen = kv_lens[s];
    kvlen = kvlen < 0 ? 0 : (kvlen > max_pages * PAGE ? max_pages * PAGE : kvlen);
    const int npages = (kvlen + PAGE - 1) / PAGE;
    const int nchunks = (npages + CHUNK - 1) / CHUNK;
    if (chunk >= nchunks)
        return;
    const int p_count = min(CHUNK, npages - p_begin);
    phys_lane = phys_lane < 0 ? 0 : (phys_lane >= num_pages ? num_pages - 1 : phys_lane);

    const int l16 = lane & 15, g4 = lane >> 4;   // query head column, token group (tokens 4 g4 .. + 3)
    // Q of query head h0 + l16 (zero past the slice): B operand, d = 32 kk + 8 g4 .. + 7
    u32x4_t qf[KSTEPS];
    {
        const bool qok = l16 < nq;
        const uint16_t *qp = Qp + ((size_t)s * H + h0 + (qok ? l16 : 0)) * D + 8 * g4;
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk)
            qf[kk] = qok ? load16(qp + 32 * kk) : u32x4_t{0, 0, 0, 0};
    }
    // copy offsets: piece u, lane -> LDS row RPP u + lane / DC, slot lane % DC,
    // holding the row's chunk slot ^ swizzle (its own inverse)
    unsigned off[PIECES];
#pragma unroll
    for (int u = 0; u < PIECES; ++u) {
        const int row = u * RPP + lane / DC;
        off[u] = (unsigned)row * (D * 2) + (unsigned)pg_slot<D>(lane % DC, row) * 16u;
    }
    // operand read offsets inside a page slot: K rows (A of S^T), row l16,
    // chunk 4 kk + g4; V^T blocks by the transposing read, group g4 reads
    // tokens 4 g4 + (l16 >> 2) at head dims 16 db + 4 (l16 & 3) .. + 3
    int kro[KSTEPS], vro[DBLK];
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk)
        kro[kk] = l16 * (D * 2) + pg_slot<D>(4 * kk + g4, l16) * 16;
    {
        const int vr = 4 * g4 + (l16 >> 2);
#pragma unroll
        for (int db = 0; db < DBLK; ++db) {
            const int col = 16 * db + 4 * (l16 & 3);
            vro[db] = vr * (D * 2) + pg_slot<D>(col >> 3, vr) * 16 + (col & 7) * 2;
        }
    }
    const size_t page_elems = (size_t)Hkv * PAGE * D;
    const size_t head_elems = (size_t)kvh * PAGE * D;
    const uint32_t klds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void *)&kring[wave][0][0]);
    const uint32_t vlds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void *)&vring[wave][0][0]);
    auto issue = [&](int pi) {   // page pi of the chunk into slot pi % SLOTS
        const int phys = __builtin_amdgcn_readlane(phys_lane, pi);
        const int rows = min(PAGE, kvlen - (p_begin + pi) * PAGE);   // valid rows of this page
        const size_t base = (size_t)phys * page_elems + head_elems;
        const u32x4s_t kr = make_rsrc(Kp + base, rows * D * 2);
        const u32x4s_t vr = make_rsrc(Vp + base, rows * D * 2);
        const uint32_t slot = (uint32_t)(pi % SLOTS) * PB;
#pragma unroll
        for (int u = 0; u < PIECES; ++u) {
            asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %2, 0 offen lds"
                         :
                         : "v"(off[u]), "s"(klds + slot + u * 1024), "s"(kr)
                         : "memory", "m0");
            asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %2, 0 offen lds"
                         :
                         : "v"(off[u]), "s"(vlds + slot + u * 1024), "s"(vr)
                         : "memory", "m0");
        }
    };

    f32x4_t oacc[DBLK];
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
        oacc[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, mc = -INFINITY, l = 0.f;   // per head (shared by its 4 lanes); l: this lane's tokens
    const float limit = exp2f(kRescaleLog2<BF16>);
#pragma unroll
    for (int i = 0; i < SLOTS - 1; ++i)
        if (i < p_count)
            issue(i);
    for (int pi = 0; pi < p_count; ++pi) {
        // a slot is refilled only after this wave's reads of it (the previous
        // page's MFMAs consumed them) are done
        if (pi + SLOTS - 1 < p_count)
            issue(pi + SLOTS - 1);
        // page pi landed once at most the copies of the later pages remain
        const int later = min(SLOTS - 1, p_count - 1 - pi);
        if (SLOTS > 3 && later >= 3)
            wait_vmcnt<6 * PIECES>();
        else if (SLOTS > 2 && later == 2)
            wait_vmcnt<4 * PIECES>();
        else if (SLOTS > 1 && later == 1)
            wait_vmcnt<2 * PIECES>();
        else
            wait_vmcnt<0>();
        const unsigned char *kc = &kring[wave][pi % SLOTS][0];
        const unsigned char *vc = &vring[wave][pi % SLOTS][0];
        f32x4_t sc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) {
            const u32x4_t ka = *reinterpret_cast<const u32x4_t *>(kc + kro[kk]);
            if constexpr (BF16)
                sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ka),
                                                             __builtin_bit_cast(bf16x8_t, qf[kk]), sc, 0, 0, 0);
            else
                sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, ka),
                                                            __builtin_bit_cast(f16x8_t, qf[kk]), sc, 0, 0, 0);
        }
        // tokens past the sequence (last page) do not count
        const int tok = (p_begin + pi) * PAGE + 4 * g4;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            sc[i] = tok + i < kvlen ? sc[i] : -INFINITY;
        // lazy online softmax (see softmax_tile): p against the current max,
        // the exact update only when some row sum leaves [0, 2^tau]
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            p[i] = fast_exp2(fmaf(sc[i], c_log2, -mc));
        float psum = (p[0] + p[1]) + (p[2] + p[3]);
        if (__builtin_expect(__builtin_amdgcn_ballot_w64(!(psum <= limit)) != 0, 0)) {
            float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
            mx = fmaxf(mx, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(mx), 0x401F)));   // lane ^ 16
            mx = fmaxf(mx, other_half(mx));                                                            // lane ^ 32
            const float m_new = fmaxf(m, mx);
            const float alpha = m_new == -INFINITY ? 1.f : fast_exp2((m - m_new) * c_log2);
            m = m_new;
            mc = m_new * c_log2;
            const float mref = m_new == -INFINITY ? 0.f : mc;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                p[i] = fast_exp2(fmaf(sc[i], c_log2, -mref));
            psum = (p[0] + p[1]) + (p[2] + p[3]);
            l *= alpha;
#pragma unroll
            for (int db = 0; db < DBLK; ++db)
                oacc[db] *= alpha;
        }
        l += psum;
        const u32x2_t pb = u32x2_t{pack2<BF16>(p[0], p[1]), pack2<BF16>(p[2], p[3])};
#pragma unroll
        for (int db = 0; db < DBLK; ++db) {
            const u32x2_t va =
                __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(vc + vro[db])));
            if constexpr (BF16)
                oacc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, va),
                                                                      __builtin_bit_cast(i16x4_t, pb), oacc[db], 0,
                                                                      0, 0);
            else
                oacc[db] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, va),
                                                                 __builtin_bit_cast(f16x4_t, pb), oacc[db], 0, 0, 0);
        }
    }

    // head l16's row: the four token groups' sums; O^T rows 16 db + 4 g4 .. + 3
    float L = l + __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(l), 0x401F));
    L += other_half(L);
    const float M = m == -INFINITY ? 0.f : mc;   // running max in base-2 units
    if (l16 >= nq)
        return;
    const size_t sh = (size_t)s * H + h0 + l16;
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
    for (int db = 0; db < DBLK; ++db)
        *reinterpret_cast<f32x4_t *>(dst + 16 * db + 4 * g4) = oacc[db] * scl;
    if (g4 == 0) {
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
                                                                  int H, int n_hgroups, int max_pages, int max_chunks,
                                                                  int chunk_pages)
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
    const int nchunks = (npages + chunk_pages - 1) / chunk_pages;
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
    // chunks in groups of 64 (one (m, l) pair per lane); the pairs and the
    // first 32 chunks' partial rows are loaded together, so that a group costs
    // one memory round trip (two past 32 chunks); a later group that raises
    // the maximum rescales what is summed so far
    float M = -INFINITY, L = 0.f;
    for (int c0 = 0; c0 < nchunks; c0 += 64) {
        const int c = c0 + lane;
        const int n = min(64, nchunks - c0);
        const float mv = c < nchunks ? ml[2 * c] : -INFINITY;
        const float lv = c < nchunks ? ml[2 * c + 1] : 0.f;
        float v[32][DPL];
#pragma unroll
        for (int j = 0; j < 32; ++j)
#pragma unroll
            for (int k = 0; k < DPL; ++k)
                v[j][k] = j < n ? po[(size_t)(c0 + j) * D + lane + 64 * k] : 0.f;
        const float Mn = fmaxf(M, wave_max(mv));
        const float r = M == -INFINITY ? 0.f : fast_exp2(M - Mn);
        L *= r;
#pragma unroll
        for (int k = 0; k < DPL; ++k)
            acc[k] *= r;
        M = Mn;
        const float w = c < nchunks ? fast_exp2(mv - M) : 0.f;
        L += wave_sum(w * lv);
#pragma unroll
        for (int j = 0; j < 32; ++j) {
            const float wj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), j));
#pragma unroll
            for (int k = 0; k < DPL; ++k)
                acc[k] = fmaf(wj, v[j][k], acc[k]);
        }
        if (n > 32) {
#pragma unroll
            for (int j = 0; j < 32; ++j)
#pragma unroll
                for (int k = 0; k < DPL; ++k)
                    v[j][k] = 32 + j < n ? po[(size_t)(c0 + 32 + j) * D + lane + 64 * k] : 0.f;
#pragma unroll
            for (int j = 0; j < 32; ++j) {
                const float wj =
                    __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), 32 + j));
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
                       a.kv_lens, a.part_o, a.part_ml, a.o, a.lse, a.H, n_hgroups, a.max_pages, max_chunks,
                       kDecodeChunkPages);
    return hipGetLastError();
}

template <int D, bool BF16, int NW, int SLOTS, int CHUNK>
hipError_t launch_mfma16(const DecodeArgs &a, hipStream_t stream)
{
    static_assert(CHUNK >= kDecodeChunkPages, "the workspace holds the partials of 8-page chunks");
    const int max_chunks = (a.max_pages + CHUNK - 1) / CHUNK;
    const int group = a.H / a.Hkv;
    const int n_slices = (group + MQ16_HEADS - 1) / MQ16_HEADS;
    const int n_items = a.Hkv * n_slices;
    const int n_wgroups = (n_items + NW - 1) / NW;
    const long long grid = (long long)a.S * n_wgroups * max_chunks;
    hipLaunchKernelGGL((decode_mfma16_kernel<D, BF16, NW, SLOTS, CHUNK>), dim3((unsigned)grid), dim3(NW * 64), 0,
                       stream, (const uint16_t *)a.q, (const uint16_t *)a.k_pages, (const uint16_t *)a.v_pages,
                       a.page_table, a.kv_lens, a.o, a.lse, a.part_o, a.part_ml, a.H, a.Hkv, group, n_slices,
                       n_items, n_wgroups, a.max_pages, a.num_pages, max_chunks, a.scale * kLog2e);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const int n_hgroups = (a.H + GROUP - 1) / GROUP;
    hipLaunchKernelGGL((decode_combine_kernel<D>), dim3((unsigned)(a.S * n_hgroups)), dim3(NTHREADS), 0, stream,
                       a.kv_lens, a.part_o, a.part_ml, a.o, a.lse, a.H, n_hgroups, a.max_pages, max_chunks, CHUNK);
    return hipGetLastError();
}

// Kernel choice: up to 16 query heads per K/V head, the 16x16 page-step
// kernel (measured on MI355X against the earlier dot-product kernel and the
// 32x32 kernel on S32 H32 d128 batches of 512..8192 tokens: 5.7 TB/s vs 5.3
// at one head per K/V head, 4.7 vs 3.9 at 4, 5.0 vs 3.3 at 8, 5.3 vs 4.4 at
// 2); wider groups, the 32x32 kernel (one read of the pages for 32 heads).
// Chunks of 32 pages when there are at least 256 (sequence, work item)
// pairs, else 16 (more chunks in flight for small batches): longer chunks
// amortise each wave's start and halve the partials to merge (measured:
// 16 / 32 / 64-page chunks; the workspace is sized for 8-page chunks).
template <int D, bool BF16>
hipError_t launch_kind(const DecodeArgs &a, hipStream_t stream)
{
    const int group = a.H / a.Hkv;
    if (group <= MQ16_HEADS) {
        if ((long long)a.S * a.Hkv >= 256)
            return launch_mfma16<D, BF16, 1, 2, 32>(a, stream);
        return launch_mfma16<D, BF16, 1, 2, 16>(a, stream);
    }
    // as many waves per workgroup as it has work items (LDS is per wave)
    const int items = a.Hkv * ((group + MQ_HEADS - 1) / MQ_HEADS);
    if (items >= 4)
        return launch_mfma<D, BF16, 4, 2>(a, stream);
    if (items >= 2)
        return launch_mfma<D, BF16, 2, 2>(a, stream);
    return launch_mfma<D, BF16, 1, 2>(a, stream);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream)
{
    if (a.d == 64)
        return a.bf16 ? launch_kind<64, true>(a, stream) : launch_kind<64, false>(a, stream);
    return a.bf16 ? launch_kind<128, true>(a, stream) : launch_kind<128, false>(a, stream);
}

}  // namespace fa
