// Exact attention forward for gfx950 (MI355X).
//
// Method (Kernel-Inference-Engine page, tile dataflow chart; gpu-inference
// page, section 02): a tile of query rows stays on chip while tiles of K and
// V stream through LDS; for each key tile the scores S = Q K^T are formed,
// masked (causal / key padding), folded into a running row max m and
// normaliser l (online softmax, NanoInfer page "Online Softmax" section),
// the accumulator is rescaled by exp(m_old - m_new), and P V is added.  The
// score matrix never leaves registers.  Key tiles that lie entirely above the
// causal diagonal or past the padded length are never visited (flash-attn-
// from-scratch page, kernel 1: causal tile-level skipping).
//
// gfx950 mapping:
//   * workgroup = 4 waves = BM = 128 query rows (32 per wave) of one (b, h);
//     four workgroups per CU at d = 64 (one wave of each per SIMD), three at
//     d = 128, two at d = 96; causal tiles are dispatched heaviest first;
//   * key tiles of 32 rows at d = 64 / 128, 64 at d = 32 / 96.  K and V tiles
//     are copied HBM/L2 -> LDS by the buffer-to-LDS load (16 bytes per lane,
//     no VGPR staging); each lane fetches the chunk that belongs at its
//     XOR-swizzled LDS slot, and rows past the valid keys (and columns past d) fall
//     outside the buffer range and read as zero.  The LDS ring holds three K
//     and three V tiles (two at d = 128), filled two tiles ahead of use;
//   * scores are formed transposed, S^T = K Q^T, with the 32x32x16 MFMA so
//     that each lane owns ONE query row (lane % 32) and half of its tile scores:
//     the row sum is lane-local plus one permlane32 swap, and the
//     accumulator registers are directly the B operand of the second MFMA;
//   * O^T = V^T P^T with the same MFMA; V^T fragments come straight from the
//     row-major LDS tile through the gfx950 transposing read ds_read_b64_tr_b16;
//   * softmax in base 2: p = exp2(s * scale * log2(e) - m * scale * log2(e)),
//     one FMA + one v_exp_f32 per score; l accumulates p in fp32 before it is
//     rounded to 16 bits for the MFMA (a bf16-rounded sum would put up to
//     2^-9 of error into ln l);
//   * the running max m is moved only when needed: p is formed against the
//     current m and the row sums are checked; only a tile whose sum exceeds
//     2^32 (bf16) or 2^15 (f16) in some row, or a row without a finite m yet,
//     takes the exact update (tile max, rescale of l and O).  The result is
//     the same softmax, since m cancels in O = sum p v / sum p and in
//     LSE = m + ln l, and the max and the O rescale are skipped on almost
//     every tile;
//   * O is written in fp32 [B, H, Nq, d], LSE = m * scale + ln(l) in fp32.
#include <cstdlib>

#include "fa_common.h"
#include "fa_internal.h"
#include "fa_tile.h"

namespace fa {
namespace {

constexpr int BM = 128;
template <int D>
struct Pipe {
    static constexpr int STAGES = D == 128 ? 2 : 3;            // LDS ring depth (tiles)
    static constexpr int DMA_PER_TILE = 2 * Geometry<D>::PIECES_PER_WAVE;   // per thread: K + V
};

// Store 4 consecutive O values of one row in the output element type.
__device__ __forceinline__ void store_o4(void *row, int dim0, int o_kind, float a, float b, float c, float e)
{
    if (o_kind == FA_O_F32) {
        *reinterpret_cast<f32x4_t *>(static_cast<float *>(row) + dim0) = f32x4_t{a, b, c, e};
    } else {
        const u32x2_t v = o_kind == FA_O_BF16 ? u32x2_t{pack2<true>(a, b), pack2<true>(c, e)}
                                              : u32x2_t{pack2<false>(a, b), pack2<false>(c, e)};
        *reinterpret_cast<u32x2_t *>(static_cast<uint16_t *>(row) + dim0) = v;
    }
}

// One query tile (BM rows of one (b, h)) against its key tiles.  Qb, Kb, Vb,
// Ob, LSEb point at row 0 of this (b, h); qsn / osn are row strides in
// elements, krs / vrs in bytes.
template <int D, bool BF16>
__device__ __forceinline__ void attend_qtile(
    const uint16_t *__restrict__ Qb, long long qsn, const uint16_t *__restrict__ Kb, unsigned krs,
    const uint16_t *__restrict__ Vb, unsigned vrs, void *__restrict__ Ob, long long osn, int o_kind,
    float *__restrict__ LSEb, int d, int Nq, int Nk, int kvlen, int q0,
    float c_log2, bool causal, unsigned char *const (&kbuf)[Pipe<D>::STAGES],
    unsigned char *const (&vbuf)[Pipe<D>::STAGES], int wave, int lane)
{
    using G = Geometry<D>;
    constexpr int ST = Pipe<D>::STAGES;
    constexpr int PER = Pipe<D>::DMA_PER_TILE;
    const int l32 = lane & 31;
    const int hh = lane >> 5;
    const int dq = Nk - Nq;   // causal: row i sees keys j <= i + dq
    const int wave_first_row = q0 + wave * 32;
    int key_end = kvlen;
    int wave_key_end = kvlen;
    if (causal) {
        const int last = min(q0 + BM, Nq) - 1;
        key_end = min(key_end, max(last + dq + 1, 0));
        const int wlast = min(wave_first_row + 32, Nq) - 1;
        wave_key_end = min(wave_key_end, max(wlast + dq + 1, 0));
    }
    constexpr int BN = G::BN;
    const int n_tiles = __builtin_amdgcn_readfirstlane((key_end + BN - 1) / BN);
    const int wave_tiles = min(n_tiles, (wave_key_end + BN - 1) / BN);

    // first tile that needs the mask (both conditions only grow with t): the
    // one that reaches past kvlen, or (causal) whose last key passes the
    // wave's first row
    int mask_t = kvlen / BN;
    if (causal) {
        const int x1 = wave_first_row + dq + 1;
        mask_t = min(mask_t, x1 <= 0 ? 0 : x1 / BN);
    }
    const int qrow = wave_first_row + l32;
    int lim = kvlen;   // keys j < lim are valid for this lane's row
    if (causal)
        lim = min(lim, qrow + dq + 1);

    f32x16_t oacc[G::DB];
#pragma unroll
    for (int db = 0; db < G::DB; ++db)
        oacc[db] = f32x16_t{};
    RowState st{INFINITY, 0.f};
    const float tau_log2 = kRescaleLog2<BF16>;
    int ko[G::NBLK][G::KSTEPS];   // K operand read offsets inside a tile
    qk_offsets<D>(sigma(l32), hh, ko);
    // The K/V ranges end at the last valid key (kvlen), not at Nk: rows
    // [kvlen, Nk) are masked, but the P V product would still multiply their
    // zero probabilities by whatever the caller left there (0 * NaN = NaN),
    // so they must read as zero.  The issued tiles all start below kvlen, so
    // the range moved per copy stays positive.
    const u32x4s_t krsrc = make_rsrc(Kb, kvlen * krs), vrsrc = make_rsrc(Vb, kvlen * vrs);
    unsigned koff[G::PIECES_PER_WAVE], voff[G::PIECES_PER_WAVE];
    dma_offsets<D, true>(wave, lane, d, krs, koff);
    dma_offsets<D, false>(wave, lane, d, vrs, voff);

    // Copies of the next tile into ring slot `slot` (tiles are copied in
    // order): buffer resources at the tile's first key, advanced by one tile
    // per copy in scalar registers, so the lane offsets stay those of tile 0
    // (keys past kvlen are out of range); ring slots as 32-bit LDS addresses.
    uint64_t kb_next = ((uint64_t)krsrc[1] << 32) | krsrc[0];
    uint64_t vb_next = ((uint64_t)vrsrc[1] << 32) | vrsrc[0];
    uint32_t kr_next = krsrc[2], vr_next = vrsrc[2];
    const uint32_t kstep_t = (uint32_t)BN * krs, vstep_t = (uint32_t)BN * vrs;
    uint32_t klds[ST], vlds[ST];
#pragma unroll
    for (int i = 0; i < ST; ++i) {
        klds[i] = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void *)(kbuf[i] + wave * 1024));
        vlds[i] = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void *)(vbuf[i] + wave * 1024));
    }
    auto issue = [&](int slot) {
        const u32x4s_t kr = {(uint32_t)kb_next, (uint32_t)(kb_next >> 32), kr_next, krsrc[3]};
        const u32x4s_t vr = {(uint32_t)vb_next, (uint32_t)(vb_next >> 32), vr_next, vrsrc[3]};
        dma_tile_lds<D>(kr, koff, klds[slot]);
        dma_tile_lds<D>(vr, voff, vlds[slot]);
        kb_next += kstep_t;
        vb_next += vstep_t;
        kr_next -= kstep_t;
        vr_next -= vstep_t;
    };
    // prologue: the first ST-1 tiles in flight
#pragma unroll
    for (int i = 0; i < ST - 1; ++i)
        if (i < n_tiles)
            issue(i);

    // Q after the prologue copies; the empty asm makes the compiler wait for
    // it here, once, instead of at the loop head on every iteration
    u32x4_t qf[G::KSTEPS];
    {
        const uint16_t *qp = Qb + (qrow < Nq ? qrow : 0) * qsn + 8 * hh;
#pragma unroll
        for (int c = 0; c < G::KSTEPS; ++c)
            qf[c] = (qrow < Nq && 16 * c + 8 * hh < d) ? load16(qp + 16 * c) : u32x4_t{0, 0, 0, 0};
#pragma unroll
        for (int c = 0; c < G::KSTEPS; ++c)
            asm volatile("" : "+v"(qf[c]));
    }

    // Iteration t (tile t in ring slot cur): wait for tile t (own loads,
    // then everyone's via the barrier), refill slot `fill`, freed by tile
    // t-1, with tile t+ST-1, then S = K Q^T, masks, online softmax, O += P V
    // on tile t.  The K operand reads go out before the copy is issued, so
    // its scalar work overlaps their LDS round trip (d = 128: after it; the
    // operands held across the copy spill there).
    // With the fast tag the caller guarantees that this wave computes tile
    // t, that the tile needs no mask and that tile t+ST-1 exists, so the
    // iteration takes none of those checks.
    auto iter = [&](int t, int cur, int fill, auto fast_tag) {
        constexpr bool fast = decltype(fast_tag)::value;
        constexpr bool early = D <= 96;
        if (fast || t + ST - 2 < n_tiles)
            wait_vmcnt<(ST - 2) * PER>();
        else
            wait_vmcnt<0>();
        __syncthreads();
        const bool comp = fast || t < wave_tiles;
        u32x4_t ka[G::NBLK][G::KSTEPS];
        if (early && comp)
            qk_read<D>(kbuf[cur], ko, ka);
        __builtin_amdgcn_sched_barrier(0);
        if (fast || t + ST - 1 < n_tiles)
            issue(fill);
        __builtin_amdgcn_sched_barrier(0);
        if (comp) {
            const int kt0 = t * BN;
            f32x16_t s[G::NBLK];
            if (!early)
                qk_read<D>(kbuf[cur], ko, ka);
            qk_mma<D, BF16>(ka, qf, s);
            __builtin_amdgcn_sched_barrier(0);
            if (!fast && t >= mask_t)
                mask_tile<D>(s, lim - (kt0 + 8 * hh));
            u32x4_t pf[G::PCH];
            softmax_tile<D, BF16>(s, st, pf, c_log2, tau_log2, oacc);
            // keep the V operand reads after the softmax (register pressure)
            __builtin_amdgcn_sched_barrier(0);
            pv_tile<D, BF16>(vbuf[cur], lane, hh, pf, oacc);
        }
    };

    // Tiles below fast_end run the check-free iteration; every wave still
    // passes one barrier per tile, whichever loop it is in.
    const LoopTag<true> F;
    const LoopTag<false> C;
    const int fast_end = __builtin_amdgcn_readfirstlane(min(min(n_tiles - (ST - 1), wave_tiles), mask_t));
    int t = 0;
    if constexpr (ST == 3) {
        for (; t + 2 < fast_end; t += 3) {
            iter(t, 0, 2, F);
            iter(t + 1, 1, 0, F);
            iter(t + 2, 2, 1, F);
        }
        for (; t + 2 < n_tiles; t += 3) {
            iter(t, 0, 2, C);
            iter(t + 1, 1, 0, C);
            iter(t + 2, 2, 1, C);
        }
        if (t < n_tiles)
            iter(t, 0, 2, C);
        if (t + 1 < n_tiles)
            iter(t + 1, 1, 0, C);
    } else {
        for (; t + 1 < fast_end; t += 2) {
            iter(t, 0, 1, F);
            iter(t + 1, 1, 0, F);
        }
        for (; t + 1 < n_tiles; t += 2) {
            iter(t, 0, 1, C);
            iter(t + 1, 1, 0, C);
        }
        if (t < n_tiles)
            iter(t, 0, 1, C);
    }
    __syncthreads();   // the ring is reused by the next query tile of this workgroup

    // ---- epilogue: O = O_acc / l (columns < d, in the output type),
    // LSE = m * scale + ln(l) = (m*c + log2(l)) * ln(2)
    const float l_tot = st.l + other_half(st.l);
    if (qrow < Nq) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        void *orow = o_kind == FA_O_F32 ? (void *)(static_cast<float *>(Ob) + qrow * osn)
                                        : (void *)(static_cast<uint16_t *>(Ob) + qrow * osn);
#pragma unroll
        for (int db = 0; db < G::DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int dim0 = 32 * db + 8 * g + 4 * hh;
                if (dim0 < d)
                    store_o4(orow, dim0, o_kind, oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv,
                             oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
            }
        if (hh == 0)
            LSEb[qrow] = l_tot > 0.f ? (__log2f(l_tot) - st.nmc) * kLn2 : -INFINITY;
    }
}

// Work decomposition: one workgroup per (b, h, query tile).  Causal: tile
// qt = n_qtiles-1 - blockIdx / (B*H), so the heaviest tiles (most key tiles)
// are dispatched first and the dispatcher fills the GPU longest job first;
// the light diagonal-corner tiles form the tail.  blockIdx % (B*H) picks the
// head; workgroups go to XCD blockIdx % 8, and when B*H is a multiple of 8
// the heads are renumbered so that each XCD holds a contiguous range of them:
// all tiles of a head, and the query heads that share a K/V head, then share
// one XCD and its L2.  For long sequences (many workgroups) the heads of an
// XCD are further taken in groups, each group heaviest first.  Non-causal:
// work ids are renumbered so that each XCD receives a contiguous range.
// The causal flag is a runtime argument: both modes share one code path.
template <int D, bool BF16>
__global__ __launch_bounds__(NTHREADS, D == 64 ? 4 : (D == 96 ? 2 : 3)) void fwd_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
    void *__restrict__ O, float *__restrict__ LSE, FwdLayout lay, int H, int Hkv, int Nq, int Nk, int n_qtiles,
    int n_units, float c_log2, int causal_flag, const int32_t *__restrict__ kv_lens)
{
    using G = Geometry<D>;
    constexpr int ST = Pipe<D>::STAGES;
    __shared__ __attribute__((aligned(1024))) unsigned char lds_k0[G::TILE];
    __shared__ __attribute__((aligned(1024))) unsigned char lds_k1[G::TILE];
    __shared__ __attribute__((aligned(1024))) unsigned char lds_k2[ST > 2 ? G::TILE : 16];
    __shared__ __attribute__((aligned(1024))) unsigned char lds_v0[G::TILE];
    __shared__ __attribute__((aligned(1024))) unsigned char lds_v1[G::TILE];
    __shared__ __attribute__((aligned(1024))) unsigned char lds_v2[ST > 2 ? G::TILE : 16];
    unsigned char *const kbuf3[3] = {lds_k0, lds_k1, lds_k2};
    unsigned char *const vbuf3[3] = {lds_v0, lds_v1, lds_v2};
    unsigned char *const (&kbuf)[ST] = *reinterpret_cast<unsigned char *const(*)[ST]>(&kbuf3);
    unsigned char *const (&vbuf)[ST] = *reinterpret_cast<unsigned char *const(*)[ST]>(&vbuf3);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool causal = causal_flag != 0;

    int bhi, qt;
    if (causal) {
        const int BHn = gridDim.x / n_qtiles;
        // Long sequences: each XCD takes its heads in ng groups, one group's
        // query tiles (heaviest first) after the other's, so that fewer heads'
        // K/V rows compete for its L2; a group keeps at least 2048 workgroups
        // (two rounds of the resident slots at d = 64), so that heaviest-first
        // still balances inside it.
        int ng = 1;
        while (ng < 8 && BHn % (16 * ng) == 0 && (int)gridDim.x / (2 * ng) >= 2048)
            ng *= 2;
        const int per = gridDim.x / ng;   // workgroups of one group
        const int grp = blockIdx.x / per;
        const int r = blockIdx.x - grp * per;
        const int BHg = BHn / ng;
        const int slot = r % BHg;
        bhi = (BHn & 7) ? slot : (slot & 7) * (BHn >> 3) + grp * (BHg >> 3) + (slot >> 3);
        qt = n_qtiles - 1 - r / BHg;
    } else {
        const int logical = xcd_contiguous_id(blockIdx.x, gridDim.x);
        bhi = logical / n_units;
        qt = logical - bhi * n_units;
    }
    const int b = bhi / H;
    const int h = bhi - b * H;
    const int kvh = h / (H / Hkv);   // K/V head of this query head
    int kvlen = Nk;
    if (kv_lens) {
        kvlen = kv_lens[b];
        kvlen = kvlen < 0 ? 0 : (kvlen > Nk ? Nk : kvlen);
    }
    const uint16_t *Qb = Q + b * lay.qs[0] + h * lay.qs[1];
    const uint16_t *Kb = K + b * lay.ks[0] + kvh * lay.ks[1];
    const uint16_t *Vb = V + b * lay.vs[0] + kvh * lay.vs[1];
    const long long oe = b * lay.os[0] + h * lay.os[1];
    void *Ob = lay.o_kind == FA_O_F32 ? (void *)(static_cast<float *>(O) + oe) : (void *)(static_cast<uint16_t *>(O) + oe);

    attend_qtile<D, BF16>(Qb, lay.qs[2], Kb, (unsigned)(lay.ks[2] * 2), Vb, (unsigned)(lay.vs[2] * 2), Ob, lay.os[2],
                          lay.o_kind, LSE + (size_t)bhi * Nq, lay.d, Nq, Nk, kvlen, qt * BM, c_log2, causal,
                          kbuf, vbuf, wave, lane);
}

// Small grids (few heads, short or single sequences): the tiled kernel above
// gives each (b, h, 128-row query tile) to one workgroup, which leaves most
// of the 256 CUs idle and makes every wave walk all keys of its rows in one
// chain.  Here a workgroup owns one 32-row query block and its NW waves (4,
// or 8 on the smallest grids at d <= 64) split the block's key tiles between
// them (tile t goes to wave t % NW), each with its own two-slot LDS ring and
// no barrier in the loop; at the end the NW partial (O, m, l) are merged
// through LDS with the log-sum-exp rule, as the split-KV decode merges its
// chunks (NanoInfer page "Online Softmax": the same recurrence over blocks).
constexpr int SPLIT_ROWS = 32;
constexpr int SPLIT_ST = 2;   // ring slots per wave

template <int D, bool BF16, int NW>
__global__ __launch_bounds__(64 * NW, 1) void fwd_split_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
    void *__restrict__ O, float *__restrict__ LSE, FwdLayout lay, int H, int Hkv, int Nq, int Nk, int n_qblocks,
    float c_log2, int causal_flag, const int32_t *__restrict__ kv_lens)
{
    using G = Geometry<D>;
    constexpr int PPW = G::PIECES_PER_WAVE;
    static_assert(NW * SPLIT_ST * 2 * G::TILE <= 160 * 1024, "LDS");
    static_assert(NW * SPLIT_ROWS * D * 4 <= NW * SPLIT_ST * 2 * G::TILE, "merge staging fits the rings");
    __shared__ __attribute__((aligned(1024))) unsigned char ring[NW][SPLIT_ST][2][G::TILE];  // [wave][slot][K, V]
    __shared__ float mls[2][NW][SPLIT_ROWS];                                                  // m * c, l per wave

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int hh = lane >> 5;
    const bool causal = causal_flag != 0;

    const int logical = xcd_contiguous_id(blockIdx.x, gridDim.x);
    const int bhi = logical / n_qblocks;
    const int qb = logical - bhi * n_qblocks;
    const int b = bhi / H;
    const int h = bhi - b * H;
    const int kvh = h / (H / Hkv);
    int kvlen = Nk;
    if (kv_lens) {
        kvlen = kv_lens[b];
        kvlen = kvlen < 0 ? 0 : (kvlen > Nk ? Nk : kvlen);
    }
    const uint16_t *Qb = Q + b * lay.qs[0] + h * lay.qs[1];
    const uint16_t *Kb = K + b * lay.ks[0] + kvh * lay.ks[1];
    const uint16_t *Vb = V + b * lay.vs[0] + kvh * lay.vs[1];
    const long long oe = b * lay.os[0] + h * lay.os[1];
    const int d = lay.d;
    const unsigned krs = (unsigned)(lay.ks[2] * 2), vrs = (unsigned)(lay.vs[2] * 2);

    const int q0 = qb * SPLIT_ROWS;
    const int dq = Nk - Nq;
    const int qrow = q0 + l32;
    constexpr int BN = G::BN;
    int key_end = kvlen;
    if (causal)
        key_end = min(key_end, max(min(q0 + SPLIT_ROWS, Nq) - 1 + dq + 1, 0));
    const int n_tiles = __builtin_amdgcn_readfirstlane((key_end + BN - 1) / BN);
    int mask_t = kvlen / BN;   // first tile that needs the mask
    if (causal) {
        const int x1 = q0 + dq + 1;
        mask_t = min(mask_t, x1 <= 0 ? 0 : x1 / BN);
    }
    int lim = kvlen;
    if (causal)
        lim = min(lim, qrow + dq + 1);
    // this wave's tiles: t = wave, wave + NW, ...
    const int my_tiles = n_tiles > wave ? (n_tiles - wave + NW - 1) / NW : 0;

    f32x16_t oacc[G::DB];
#pragma unroll
    for (int db = 0; db < G::DB; ++db)
        oacc[db] = f32x16_t{};
    RowState st{INFINITY, 0.f};
    const float tau_log2 = kRescaleLog2<BF16>;
    int ko[G::NBLK][G::KSTEPS];
    qk_offsets<D>(sigma(l32), hh, ko);
    const u32x4s_t krsrc = make_rsrc(Kb, kvlen * krs), vrsrc = make_rsrc(Vb, kvlen * vrs);
    // the whole tile is copied by this wave: the pieces of the four copy
    // lanes sets of the tiled kernel (piece u of set w lands at w * 1 KB + u * 4 KB)
    unsigned koff[4][PPW], voff[4][PPW];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        dma_offsets<D, true>(w, lane, d, krs, koff[w]);
        dma_offsets<D, false>(w, lane, d, vrs, voff[w]);
    }
    uint32_t klds[SPLIT_ST], vlds[SPLIT_ST];
#pragma unroll
    for (int i = 0; i < SPLIT_ST; ++i) {
        klds[i] = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void *)&ring[wave][i][0][0]);
        vlds[i] = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void *)&ring[wave][i][1][0]);
    }
    auto issue = [&](int t, int slot) {   // key tile t into this wave's slot
        const uint64_t kb = (((uint64_t)krsrc[1] << 32) | krsrc[0]) + (uint64_t)t * BN * krs;
        const uint64_t vb = (((uint64_t)vrsrc[1] << 32) | vrsrc[0]) + (uint64_t)t * BN * vrs;
        const u32x4s_t kr = {(uint32_t)kb, (uint32_t)(kb >> 32), krsrc[2] - (uint32_t)(t * BN) * krs, krsrc[3]};
        const u32x4s_t vr = {(uint32_t)vb, (uint32_t)(vb >> 32), vrsrc[2] - (uint32_t)(t * BN) * vrs, vrsrc[3]};
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            dma_tile_lds<D>(kr, koff[w], klds[slot] + w * 1024);
            dma_tile_lds<D>(vr, voff[w], vlds[slot] + w * 1024);
        }
    };
    if (my_tiles > 0)
        issue(wave, 0);

    u32x4_t qf[G::KSTEPS];
    {
        const uint16_t *qp = Qb + (qrow < Nq ? qrow : 0) * lay.qs[2] + 8 * hh;
#pragma unroll
        for (int c = 0; c < G::KSTEPS; ++c)
            qf[c] = (qrow < Nq && 16 * c + 8 * hh < d) ? load16(qp + 16 * c) : u32x4_t{0, 0, 0, 0};
#pragma unroll
        for (int c = 0; c < G::KSTEPS; ++c)
            asm volatile("" : "+v"(qf[c]));
    }

    for (int j = 0; j < my_tiles; ++j) {
        const int t = wave + NW * j;
        const int slot = j & 1;
        // the other slot was read by this wave's previous tile (its MFMAs
        // consumed the reads), so it can be refilled now
        if (j + 1 < my_tiles) {
            issue(t + NW, slot ^ 1);
            wait_vmcnt<8 * PPW>();   // this tile's copies done, the next tile's in flight
        } else {
            wait_vmcnt<0>();
        }
        const unsigned char *kc = &ring[wave][slot][0][0];
        const unsigned char *vc = &ring[wave][slot][1][0];
        u32x4_t ka[G::NBLK][G::KSTEPS];
        qk_read<D>(kc, ko, ka);
        f32x16_t s[G::NBLK];
        qk_mma<D, BF16>(ka, qf, s);
        if (t >= mask_t)
            mask_tile<D>(s, lim - (t * BN + 8 * hh));
        u32x4_t pf[G::PCH];
        softmax_tile<D, BF16>(s, st, pf, c_log2, tau_log2, oacc);
        pv_tile<D, BF16>(vc, lane, hh, pf, oacc);
    }

    // ---- merge of the NW waves' partials: m*c and l per row, then O
    const float l_tot = st.l + other_half(st.l);
    __syncthreads();   // every wave is done with its ring: it becomes the staging area
    if (hh == 0) {
        mls[0][wave][l32] = -st.nmc;   // m*c (-inf: no key)
        mls[1][wave][l32] = l_tot;
    }
    float *stage = reinterpret_cast<float *>(&ring[0][0][0][0]);   // [wave][db][g][lane] f32x4
#pragma unroll
    for (int db = 0; db < G::DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g)
            *reinterpret_cast<f32x4_t *>(stage + (((wave * G::DB + db) * 4 + g) * 64 + lane) * 4) =
                f32x4_t{oacc[db][4 * g], oacc[db][4 * g + 1], oacc[db][4 * g + 2], oacc[db][4 * g + 3]};
    __syncthreads();
    float mw[NW], M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        mw[w] = mls[0][w][l32];
        M = fmaxf(M, mw[w]);
    }
    float fw[NW], L = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        fw[w] = M == -INFINITY ? 0.f : fast_exp2(mw[w] - M);   // a wave without keys of this row: mw = -inf, weight 0
        L = fmaf(fw[w], mls[1][w][l32], L);
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    if (qrow < Nq) {
        void *orow = lay.o_kind == FA_O_F32 ? (void *)(static_cast<float *>(O) + oe + qrow * lay.os[2])
                                            : (void *)(static_cast<uint16_t *>(O) + oe + qrow * lay.os[2]);
        // wave w merges and stores the (db, g) groups with (4 db + g) % NW == w
#pragma unroll
        for (int db = 0; db < G::DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                if ((4 * db + g) % NW != wave)
                    continue;
                f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int w = 0; w < NW; ++w)
                    acc += fw[w] * *reinterpret_cast<const f32x4_t *>(stage + (((w * G::DB + db) * 4 + g) * 64 + lane) * 4);
                const int dim0 = 32 * db + 8 * g + 4 * hh;
                if (dim0 < d)
                    store_o4(orow, dim0, lay.o_kind, acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
            }
        if (wave == 0 && hh == 0)
            LSE[(size_t)bhi * Nq + qrow] = L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY;
    }
}

int units_per_head(int Nq, bool causal)
{
    const int n_qtiles = (Nq + BM - 1) / BM;
    (void)causal;
    return n_qtiles;
}

// Kernel choice: the split-key kernel when the tiled kernel would launch
// fewer workgroups than the GPU has CUs (d = 96 excepted: its two-slot rings
// per wave would not fit in LDS), with 8 waves per 32-row block when even
// that grid (four blocks per query tile) fits one workgroup per CU at d <= 64
// (the rings of 8 waves take 128 KB of LDS).  Returns the split kernel's
// waves per workgroup, or 0 for the tiled kernel.  FA_FWD_SPLIT=0 / 1 / 8 in
// the environment forces the tiled kernel / 4 waves / 8 waves (4 above d = 64);
// the tests run every kernel on the same shapes.
int split_waves(const FwdArgs &a, int D)
{
    if (D == 96)
        return 0;
    const long long tiled = (long long)((a.Nq + BM - 1) / BM) * a.B * a.H;
    if (tiled >= (1 << 20))   // keep the split grid (4x) far inside the 32-bit grid limit
        return 0;
    const char *e = std::getenv("FA_FWD_SPLIT");
    if (e && e[0] == '0' && e[1] == 0)
        return 0;
    if (e && e[0] == '1' && e[1] == 0)
        return 4;
    if (e && e[0] == '8' && e[1] == 0)
        return D <= 64 ? 8 : 4;
    if (tiled <= 64 && D <= 64)
        return 8;
    return tiled < 256 ? 4 : 0;
}

template <int D, bool BF16, int NW>
hipError_t launch_split(const FwdArgs &a, hipStream_t stream)
{
    const int n_qblocks = (a.Nq + SPLIT_ROWS - 1) / SPLIT_ROWS;
    const long long grid = (long long)n_qblocks * a.B * a.H;
    hipLaunchKernelGGL((fwd_split_kernel<D, BF16, NW>), dim3((unsigned)grid), dim3(64 * NW), 0, stream,
                       (const uint16_t *)a.q, (const uint16_t *)a.k, (const uint16_t *)a.v, a.o, a.lse, a.lay,
                       a.H, a.Hkv, a.Nq, a.Nk, n_qblocks, a.scale * kLog2e, a.causal ? 1 : 0, a.kv_lens);
    return hipGetLastError();
}

template <int D, bool BF16>
hipError_t launch(const FwdArgs &a, hipStream_t stream)
{
    if constexpr (D != 96) {
        const int nw = split_waves(a, D);
        if constexpr (D <= 64) {
            if (nw == 8)
                return launch_split<D, BF16, 8>(a, stream);
        }
        if (nw != 0)
            return launch_split<D, BF16, 4>(a, stream);
    }
    const int n_qtiles = (a.Nq + BM - 1) / BM;
    const int n_units = units_per_head(a.Nq, a.causal);
    const long long grid = (long long)n_units * a.B * a.H;
    hipLaunchKernelGGL((fwd_kernel<D, BF16>), dim3((unsigned)grid), dim3(NTHREADS), 0, stream,
                       (const uint16_t *)a.q, (const uint16_t *)a.k, (const uint16_t *)a.v, a.o, a.lse, a.lay,
                       a.H, a.Hkv, a.Nq, a.Nk, n_qtiles, n_units, a.scale * kLog2e, a.causal ? 1 : 0,
                       a.kv_lens);
    return hipGetLastError();
}

}  // namespace

// upper bound of the tiled kernel's grid; the split-key kernel's grid is 4x
// this, and split_waves() keeps it for tiled grids below 2^20 only
long long fwd_grid_size(int B, int H, int Nq) { return (long long)((Nq + BM - 1) / BM) * B * H; }

hipError_t launch_fwd(const FwdArgs &a, hipStream_t stream)
{
    // LDS geometry of the smallest padded head dim that holds d
    const int d = a.lay.d;
    if (d <= 32)
        return a.bf16 ? launch<32, true>(a, stream) : launch<32, false>(a, stream);
    if (d <= 64)
        return a.bf16 ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
    if (d <= 96)
        return a.bf16 ? launch<96, true>(a, stream) : launch<96, false>(a, stream);
    return a.bf16 ? launch<128, true>(a, stream) : launch<128, false>(a, stream);
}

}  // namespace fa
