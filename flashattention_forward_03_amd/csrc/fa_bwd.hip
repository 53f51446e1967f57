// Exact attention backward for gfx950 (MI355X).
//
// Method (gpu-inference page, section 02): the probabilities are recomputed
// from the forward's saved log-sum-exp instead of being stored, and the work
// splits into a row term D_i = dO_i . O_i, a pass that owns a block of query
// rows and accumulates dQ over their keys, and a pass that owns a block of
// keys and accumulates dK and dV over the query rows that see them.  The row
// term is formed by the dQ pass, which holds each row's dO anyway, and
// written out for the dK/dV pass, which runs after it, together with the
// row's LSE in base-2 units (so that pass forms P with one FMA per element).  With P_ij = exp(scale q_i.k_j - LSE_i) (zero where masked):
//   dV_j = sum_i P_ij dO_i,  dP_ij = dO_i . v_j,  dS_ij = P_ij (dP_ij - D_i),
//   dK_j = scale sum_i dS_ij q_i,  dQ_i = scale sum_j dS_ij k_j.
// Every gradient is written once by the block that owns it (no atomics), so
// results are bitwise reproducible.  dK and dV of a K/V head sum over the
// query heads that share it (grouped-query attention).
//
// gfx950 mapping (a head dim d <= 64 runs on the d = 64 geometry, d <= 128 on the
// 128 one: columns past d read as zero and are not stored; rows are d wide in
// memory), both passes on the 32x32x16 MFMA with the same
// register chaining as the forward (an accumulator's registers are the next
// MFMA's B operand once the rows of the first product are permuted by sigma):
//   * dQ pass: a workgroup = 4 waves x 32 query rows; Q and dO rows are held
//     as B operands, and D_i = dO_i . O_i is formed from the dO operands and
//     the O row before the loop (-D_i, kept in 16 registers, is where each
//     tile's dP product starts); K and V tiles of 32 keys stream through a three-slot LDS
//     ring (buffer-to-LDS copies).  Per tile: S^T = K Q^T, dP^T = V dO^T,
//     P^T and dS^T lane-local (each lane owns a query row, so LSE_i and D_i
//     are per-lane scalars), then dQ^T += K^T dS^T with K^T read by the
//     transposing LDS read.
//   * dK/dV pass: a workgroup = 4 waves x 32 keys; K and V rows are held as B
//     operands, V negated; Q and dO tiles of 32 rows, and their LSE and D
//     values, stream through the ring.  Per tile: S = Q K^T and
//     D - dP = D + dO (-V)^T (the dP product starts from D, so dS needs one
//     multiply) with a lane owning a key column, P with the rows' LSE read
//     from LDS, then dV^T += dO^T P and (-dK)^T += Q^T (-dS) with dO^T, Q^T
//     read transposed; dK is stored with -scale.
#include <climits>

#include "fa_common.h"
#include "fa_internal.h"
#include "fa_tile.h"

namespace fa {
namespace {

constexpr int BQ = 128;        // query rows per dQ workgroup (32 per wave)
constexpr int BK = 128;        // keys per dK/dV workgroup (32 per wave)
constexpr int BT = 32;         // rows per streamed tile
constexpr int STAGES = 3;      // LDS ring depth (tiles)

// Head groups per XCD for a launch of `grid` workgroups over BHn heads: each
// XCD's heads are taken one group after the other, so that fewer heads'
// streamed rows compete for its L2, while every group keeps at least 2048
// workgroups (more than two rounds of the 768 resident slots at d = 64).
__device__ __forceinline__ int head_groups(int BHn, int grid)
{
    int ng = 1;
    while (ng < 8 && BHn % (16 * ng) == 0 && grid / (2 * ng) >= 2048)
        ng *= 2;
    return ng;
}

// ---------------------------------------------------------------- dQ pass ---

template <int D, bool BF16>
__global__ __launch_bounds__(NTHREADS, D == 64 ? 3 : 2) void bwd_dq_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
    const uint16_t *__restrict__ dO, const float *__restrict__ O, const float *__restrict__ LSE,
    float *__restrict__ delta, float *__restrict__ dQ, int H, int Hkv, int Nq, int Nk, int d, int n_qtiles,
    float c_log2, float scale, int causal_flag, const int32_t *__restrict__ kv_lens)
{
    using G = Geometry<D>;
    static_assert(G::BN == BT, "tile rows");
    constexpr int PER = 2 * G::PIECES_PER_WAVE;   // copies per lane per tile (K + V)
    const unsigned rb = (unsigned)d * 2u;          // bytes per K/V row in memory
    __shared__ __attribute__((aligned(1024))) unsigned char kring[STAGES][G::TILE];
    __shared__ __attribute__((aligned(1024))) unsigned char vring[STAGES][G::TILE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int hh = lane >> 5;
    const bool causal = causal_flag != 0;

    // heaviest query tiles first (as the forward), heads contiguous per XCD
    // and, on long or wide launches, taken in groups per XCD
    const int BHn = gridDim.x / n_qtiles;
    const int ng = head_groups(BHn, gridDim.x);
    const int per = gridDim.x / ng;
    const int hgi = blockIdx.x / per;   // head group
    const int rr = blockIdx.x - hgi * per;
    const int BHg = BHn / ng;
    const int slot = rr % BHg;
    const int bhi = (BHn & 7) ? slot : (slot & 7) * (BHn >> 3) + hgi * (BHg >> 3) + (slot >> 3);
    const int qt = causal ? n_qtiles - 1 - rr / BHg : rr / BHg;
    const int b = bhi / H, h = bhi - b * H;
    const int kvh = h / (H / Hkv);
    int kvlen = Nk;
    if (kv_lens) {
        kvlen = kv_lens[b];
        kvlen = kvlen < 0 ? 0 : (kvlen > Nk ? Nk : kvlen);
    }
    const size_t qbase = (size_t)bhi * Nq;
    const uint16_t *Kb = K + ((size_t)b * Hkv + kvh) * Nk * d;
    const uint16_t *Vb = V + ((size_t)b * Hkv + kvh) * Nk * d;

    const int q0 = qt * BQ;
    const int dq = Nk - Nq;
    const int wave_first_row = q0 + wave * 32;
    int key_end = kvlen, wave_key_end = kvlen;
    if (causal) {
        key_end = min(key_end, max(min(q0 + BQ, Nq) - 1 + dq + 1, 0));
        wave_key_end = min(wave_key_end, max(min(wave_first_row + 32, Nq) - 1 + dq + 1, 0));
    }
    const int n_tiles = __builtin_amdgcn_readfirstlane((key_end + BT - 1) / BT);
    const int wave_tiles = min(n_tiles, (wave_key_end + BT - 1) / BT);
    const int qrow = wave_first_row + l32;
    int lim = kvlen;
    if (causal)
        lim = min(lim, qrow + dq + 1);

    // ranges end at the last valid key: padded rows [kvlen, Nk) read as zero,
    // so their (masked) products add 0 * 0, never 0 * NaN from caller memory
    const u32x4s_t krs = make_rsrc(Kb, kvlen * rb), vrs = make_rsrc(Vb, kvlen * rb);
    unsigned koff[G::PIECES_PER_WAVE], voff[G::PIECES_PER_WAVE];
    dma_offsets<D, true>(wave, lane, d, rb, koff);   // both tiles are read by rows
    dma_offsets<D, true>(wave, lane, d, rb, voff);
    // copies of the next tile (in order) into ring slot st: resources at the
    // tile's first key, advanced by one tile per copy in scalar registers
    uint64_t kb_next = ((uint64_t)krs[1] << 32) | krs[0];
    uint64_t vb_next = ((uint64_t)vrs[1] << 32) | vrs[0];
    uint32_t range_next = krs[2];
    const uint32_t kTileBytes = (uint32_t)BT * rb;
    uint32_t klds[STAGES], vlds[STAGES];
#pragma unroll
    for (int i = 0; i < STAGES; ++i) {
        klds[i] = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void *)(kring[i] + wave * 1024));
        vlds[i] = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void *)(vring[i] + wave * 1024));
    }
    auto issue = [&](int st) {
        const u32x4s_t kr = {(uint32_t)kb_next, (uint32_t)(kb_next >> 32), range_next, krs[3]};
        const u32x4s_t vr = {(uint32_t)vb_next, (uint32_t)(vb_next >> 32), range_next, vrs[3]};
        dma_tile_lds<D>(kr, koff, klds[st]);
        dma_tile_lds<D>(vr, voff, vlds[st]);
        kb_next += kTileBytes;
        vb_next += kTileBytes;
        range_next -= kTileBytes;
    };
#pragma unroll
    for (int i = 0; i < STAGES - 1; ++i)
        if (i < n_tiles)
            issue(i);

    // Q and dO rows of this lane's query (B operands), its LSE, and
    // D = dO . O over the head dims this lane holds (8 per k-step), summed
    // with the other half of the row held by lane ^ 32
    u32x4_t qf[G::KSTEPS], gf[G::KSTEPS];
    float lse2 = INFINITY, Di = 0.f;   // lse2 = +inf makes P = 0 (rows past Nq, rows without keys)
    f32x16_t dneg;                     // -D in every register: the start of the dP product
    {
        const bool ok = qrow < Nq;
        const size_t r = qbase + (ok ? qrow : 0);
        const uint16_t *qp = Q + r * d + 8 * hh;
        const uint16_t *gp = dO + r * d + 8 * hh;
        const float *op = O + r * d + 8 * hh;
        f32x4_t of[G::KSTEPS][2];
#pragma unroll
        for (int c = 0; c < G::KSTEPS; ++c) {
            const bool in = ok && 16 * c + 8 * hh < d;   // 8 columns, all inside d or all past it
            qf[c] = in ? load16(qp + 16 * c) : u32x4_t{0, 0, 0, 0};
            gf[c] = in ? load16(gp + 16 * c) : u32x4_t{0, 0, 0, 0};
            of[c][0] = in ? *reinterpret_cast<const f32x4_t *>(op + 16 * c) : f32x4_t{};
            of[c][1] = in ? *reinterpret_cast<const f32x4_t *>(op + 16 * c + 4) : f32x4_t{};
        }
        float l = -INFINITY;
        if (ok) {
            l = LSE[r];
            if (l > -INFINITY)
                lse2 = l * kLog2e;
        }
        float dpart = 0.f;
#pragma unroll
        for (int c = 0; c < G::KSTEPS; ++c)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                dpart = fmaf(of[c][j >> 1][2 * (j & 1)], lo16<BF16>(gf[c][j]),
                             fmaf(of[c][j >> 1][2 * (j & 1) + 1], hi16<BF16>(gf[c][j]), dpart));
        Di = dpart + other_half(dpart);
#pragma unroll
        for (int r = 0; r < 16; ++r)
            dneg[r] = -Di;
        if (ok && hh == 0) {
            // delta[0] = D, delta[1] = LSE * log2(e) (-inf stays -inf) for the dK/dV pass
            delta[r] = Di;
            delta[(size_t)(gridDim.x / n_qtiles) * Nq + r] = l * kLog2e;
        }
#pragma unroll
        for (int c = 0; c < G::KSTEPS; ++c) {
            asm volatile("" : "+v"(qf[c]));
            asm volatile("" : "+v"(gf[c]));
        }
        asm volatile("" : "+v"(lse2), "+v"(Di));
    }

    f32x16_t acc[G::DB];
#pragma unroll
    for (int db = 0; db < G::DB; ++db)
        acc[db] = f32x16_t{};
    int ko[G::NBLK][G::KSTEPS];   // K (and V) operand read offsets inside a tile
    qk_offsets<D>(sigma(l32), hh, ko);
    // first tile that needs the mask (both conditions only grow with t)
    int mask_t = kvlen / BT;
    if (causal) {
        const int x1 = wave_first_row + dq + 1;
        mask_t = min(mask_t, x1 <= 0 ? 0 : x1 / BT);
    }

    // As the forward: the K and V operand reads go out before the next copy
    // is issued; with the fast tag the caller guarantees the wave computes
    // tile t unmasked and tile t+STAGES-1 exists, so no per-tile test runs.
    auto iter = [&](int t, int cur, int fill, auto fast_tag) {
        constexpr bool fast = decltype(fast_tag)::value;
        if (fast || t + STAGES - 2 < n_tiles)
            wait_vmcnt<(STAGES - 2) * PER>();
        else
            wait_vmcnt<0>();
        __syncthreads();
        const bool comp = fast || t < wave_tiles;
        u32x4_t ka0[G::NBLK][G::KSTEPS], va0[G::NBLK][G::KSTEPS];
        if (comp) {
            qk_read<D>(kring[cur], ko, ka0);
            qk_read<D>(vring[cur], ko, va0);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (fast || t + STAGES - 1 < n_tiles)
            issue(fill);
        __builtin_amdgcn_sched_barrier(0);
        if (comp) {
            const int kt0 = t * BT;
            f32x16_t s[1], dp[1];
            qk_mma<D, BF16>(ka0, qf, s);    // S^T = K Q^T
            qk_mma_from<D, BF16>(va0, gf, dp, dneg);   // (dP - D)^T = V dO^T - D
            __builtin_amdgcn_sched_barrier(0);
            if (!fast && t >= mask_t)
                mask_tile<D>(s, lim - (kt0 + 8 * hh));
            // P^T and dS^T, packed to 16 bits as the B operand of dQ^T += K^T dS^T
            u32x4_t dsf[2];
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int r = 8 * h2 + 2 * q;
                    const float p0 = fast_exp2(fmaf(s[0][r], c_log2, -lse2));
                    const float p1 = fast_exp2(fmaf(s[0][r + 1], c_log2, -lse2));
                    dsf[h2][q] = pack2<BF16>(p0 * dp[0][r], p1 * dp[0][r + 1]);
                }
            __builtin_amdgcn_sched_barrier(0);
            u32x4_t ka[G::DB][G::PCH];
            pv_operands<D, true>(kring[cur], lane, hh, ka);   // K^T
            pv_mfma<D, BF16>(ka, dsf, acc);
        }
    };
    const LoopTag<true> F;
    const LoopTag<false> C;
    const int fast_end = __builtin_amdgcn_readfirstlane(min(min(n_tiles - (STAGES - 1), wave_tiles), mask_t));
    int t = 0;
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
    __syncthreads();

    if (qrow < Nq) {
        float *op = dQ + (qbase + qrow) * d + 4 * hh;
#pragma unroll
        for (int db = 0; db < G::DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                if (32 * db + 8 * g < d)
                    *reinterpret_cast<f32x4_t *>(op + 32 * db + 8 * g) =
                        f32x4_t{acc[db][4 * g] * scale, acc[db][4 * g + 1] * scale, acc[db][4 * g + 2] * scale,
                                acc[db][4 * g + 3] * scale};
    }
}

// ------------------------------------------------------------- dK/dV pass ---

// Copy 32 consecutive fp32 values (a tile's LSE or D rows, from the
// resource's first row) into this wave's LDS slot at 32-bit address lds:
// lanes 0..31 load one dword each (voff = 4 * lane), lanes 32..63 read out
// of range (zero) into the slot's unused half.
__device__ __forceinline__ void dma_dword_lds(const u32x4s_t &rsrc, unsigned voff, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dword %0, %2, 0 offen lds"
                 :
                 : "v"(voff), "s"(lds), "s"(rsrc)
                 : "memory", "m0");
}

// pv_operands in two halves: the per-lane byte offsets of its transposing
// reads inside a tile (loop-invariant), then the reads at a tile's base.
template <int D, bool KSWZ = false>
__device__ __forceinline__ void pv_offsets(int lane, int hh, int (&to)[D / 32][kBN<D> / 16][2])
{
    using G = Geometry<D>;
    const int j16 = lane & 15;
    const int g16 = lane >> 4;
#pragma unroll
    for (int db = 0; db < G::DB; ++db) {
        const int col = 32 * db + 16 * (g16 & 1) + 4 * (j16 & 3);
        const int chunk = col >> 3;
        const int half = (col & 7) * 2;
#pragma unroll
        for (int c = 0; c < G::PCH; ++c) {
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int r = 16 * c + 8 * hh + (j16 >> 2) + 4 * e;
                const int sw = KSWZ ? swz_k(r) : swz_v(r);
                to[db][c][e] = r * G::ROWB + (swz_slot<G::DC>(chunk, sw) << 4) + half;
            }
        }
    }
}

template <int D>
__device__ __forceinline__ void pv_read(const unsigned char *vb, const int (&to)[D / 32][kBN<D> / 16][2],
                                        u32x4_t (&va)[D / 32][kBN<D> / 16])
{
    using G = Geometry<D>;
#pragma unroll
    for (int db = 0; db < G::DB; ++db)
#pragma unroll
        for (int c = 0; c < G::PCH; ++c) {
            const u32x2_t y0 = __builtin_bit_cast(
                u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(vb + to[db][c][0])));
            const u32x2_t y1 = __builtin_bit_cast(
                u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(vb + to[db][c][1])));
            va[db][c] = u32x4_t{y0[0], y0[1], y1[0], y1[1]};
        }
}

template <int D, bool BF16>
__global__ __launch_bounds__(NTHREADS, D == 64 ? 3 : 1) void bwd_dkdv_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
    const uint16_t *__restrict__ dO, const float *__restrict__ delta, float *__restrict__ dK,
    float *__restrict__ dV, int H, int Hkv, int Nq, int Nk, int d, int n_ktiles, float c_log2,
    float scale, int causal_flag, const int32_t *__restrict__ kv_lens)
{
    using G = Geometry<D>;
    const unsigned rb = (unsigned)d * 2u;   // bytes per Q/dO row in memory
    static_assert(G::BN == BT, "tile rows");
    constexpr int PER = 2 * G::PIECES_PER_WAVE + 2;   // Q, dO pieces + LSE, D rows
    // Q and dO tiles of one ring slot side by side, so that one lane offset
    // (plus a constant) addresses both
    __shared__ __attribute__((aligned(1024))) unsigned char qgring[STAGES][2][G::TILE];
    __shared__ __attribute__((aligned(256))) unsigned char sring[STAGES][4][2][256];   // per wave: LSE, D

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int hh = lane >> 5;
    const bool causal = causal_flag != 0;

    // lowest key tiles first (they have the most query rows when causal),
    // K/V heads contiguous per XCD and, on long or wide launches, in groups
    const int BHn = gridDim.x / n_ktiles;
    const int ng = head_groups(BHn, gridDim.x);
    const int per = gridDim.x / ng;
    const int hgi = blockIdx.x / per;   // head group
    const int rr = blockIdx.x - hgi * per;
    const int BHg = BHn / ng;
    const int slot = rr % BHg;
    const int g = (BHn & 7) ? slot : (slot & 7) * (BHn >> 3) + hgi * (BHg >> 3) + (slot >> 3);   // b * Hkv + kvh
    const int kt = rr / BHg;
    const int b = g / Hkv, kvh = g - b * Hkv;
    const int grp = H / Hkv;
    const size_t n_rows = (size_t)(BHn / Hkv) * H * Nq;   // B * H * Nq: delta[1] starts here
    int kvlen = Nk;
    if (kv_lens) {
        kvlen = kv_lens[b];
        kvlen = kvlen < 0 ? 0 : (kvlen > Nk ? Nk : kvlen);
    }
    const int dq = Nk - Nq;
    const int k0 = kt * BK;
    const int kw0 = k0 + wave * 32;   // this wave's first key
    const int key = kw0 + l32;        // this lane's key (accumulator column)

    // query tiles that see any key of the workgroup, per query head
    int qt_begin = 0;
    if (causal)
        qt_begin = max(0, k0 - dq) / BT;
    int n_qt = (Nq + BT - 1) / BT - qt_begin;
    if (k0 >= kvlen || (causal && k0 - dq > Nq - 1))
        n_qt = 0;
    const int n_tiles = n_qt > 0 ? n_qt * grp : 0;   // (query head, query tile) pairs

    // K and -V rows of this lane's key (B operands; the sign flip of a
    // 16-bit value is exact)
    u32x4_t kf[G::KSTEPS], vf[G::KSTEPS];
    {
        const bool ok = key < kvlen;   // padded keys: zero operands (their P and dS are masked)
        const size_t r = ((size_t)g * Nk + (ok ? key : 0)) * d + 8 * hh;
#pragma unroll
        for (int c = 0; c < G::KSTEPS; ++c) {
            const bool in = ok && 16 * c + 8 * hh < d;   // columns past d: zero operands
            kf[c] = in ? load16(K + r + 16 * c) : u32x4_t{0, 0, 0, 0};
            vf[c] = in ? load16(V + r + 16 * c) ^ 0x80008000u : u32x4_t{0, 0, 0, 0};
        }
    }

    // Copies stream the (query head, query tile) pairs in order: pair i is
    // head j = i / n_qt of the group and tile qi = i % n_qt.  The buffer
    // resources sit at the next pair's first row and advance by one tile per
    // copy in scalar registers (re-based when the head changes), so the lane
    // offsets are the tile-0 ones and no division runs per tile.
    unsigned qoff[G::PIECES_PER_WAVE];
    dma_offsets<D, true>(wave, lane, d, rb, qoff);   // Q and dO tiles: same row layout
    const unsigned roff = lane < 32 ? (unsigned)lane * 4u : kOutOfRange;
    uint32_t qlds[STAGES], glds[STAGES], llds[STAGES], dlds[STAGES];
#pragma unroll
    for (int i = 0; i < STAGES; ++i) {
        qlds[i] = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void *)(qgring[i][0] + wave * 1024));
        glds[i] = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void *)(qgring[i][1] + wave * 1024));
        llds[i] = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void *)sring[i][wave][0]);
        dlds[i] = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void *)sring[i][wave][1]);
    }
    u32x4s_t qr, gr, lr, dr;
    int nx_qi = 0, nx_j = 0;   // the next pair to copy
    auto set_head = [&](int j) {
        const size_t row0 = ((size_t)b * H + kvh * grp + j) * Nq + (size_t)qt_begin * BT;
        const int rows = Nq - qt_begin * BT;
        qr = make_rsrc(Q + row0 * d, rows * rb);
        gr = make_rsrc(dO + row0 * d, rows * rb);
        lr = make_rsrc(delta + n_rows + row0, rows * 4);   // LSE * log2(e)
        dr = make_rsrc(delta + row0, rows * 4);            // D
    };
    auto advance = [](u32x4s_t &r, uint32_t bytes) {
        const uint64_t base = (((uint64_t)r[1]) << 32 | r[0]) + bytes;
        r[0] = (uint32_t)base;
        r[1] = (uint32_t)(base >> 32);
        r[2] -= bytes;
    };
    if (n_tiles > 0)
        set_head(0);
    auto issue = [&](int st) {   // copy the next pair into ring slot st
        dma_tile_lds<D>(qr, qoff, qlds[st]);
        dma_tile_lds<D>(gr, qoff, glds[st]);
        dma_dword_lds(lr, roff, llds[st]);
        dma_dword_lds(dr, roff, dlds[st]);
        if (++nx_qi == n_qt) {
            nx_qi = 0;
            if (++nx_j < grp)
                set_head(nx_j);
        } else {
            advance(qr, BT * rb);
            advance(gr, BT * rb);
            advance(lr, BT * 4);
            advance(dr, BT * 4);
        }
    };
#pragma unroll
    for (int i = 0; i < STAGES - 1; ++i)
        if (i < n_tiles)
            issue(i);
#pragma unroll
    for (int c = 0; c < G::KSTEPS; ++c) {
        asm volatile("" : "+v"(kf[c]));
        asm volatile("" : "+v"(vf[c]));
    }

    f32x16_t dkacc[G::DB], dvacc[G::DB];
#pragma unroll
    for (int db = 0; db < G::DB; ++db) {
        dkacc[db] = f32x16_t{};
        dvacc[db] = f32x16_t{};
    }
    const int qrow_perm = sigma(l32);
    int ro[1][G::KSTEPS];   // row-read offsets of the Q / dO operands inside a tile
    qk_offsets<D>(qrow_perm, hh, ro);
    int to[G::DB][G::PCH][2];   // transposing-read offsets of Q^T / dO^T inside a tile
    pv_offsets<D, true>(lane, hh, to);
    const int lim_key = min(kvlen, Nk);
    // rows this lane's key is visible to: [row_lo, Nq), none past the key range
    const int row_lo = key >= lim_key ? INT_MAX : (causal ? key - dq : INT_MIN);

    int cur_qi = 0;   // tile index of the pair being computed
    auto iter = [&](int t, int cur, int fill) {
        if (t + STAGES - 2 < n_tiles)
            wait_vmcnt<(STAGES - 2) * PER>();
        else
            wait_vmcnt<0>();
        __syncthreads();
        if (t + STAGES - 1 < n_tiles)
            issue(fill);
        const int q0 = (qt_begin + cur_qi) * BT;
        if (++cur_qi == n_qt)
            cur_qi = 0;
        // wave-uniform: does any query of this tile see any key of this wave?
        const bool live = kw0 < lim_key && (!causal || kw0 <= q0 + BT - 1 + dq);
        if (live) {
            // this lane's rows: register r is query q0 + 16*(r/8) + 8*hh + r%8
            const float *ls = reinterpret_cast<const float *>(sring[cur][wave][0]);
            const float *ds = reinterpret_cast<const float *>(sring[cur][wave][1]);
            f32x16_t s[1], dp[1];
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                const f32x4_t da = *reinterpret_cast<const f32x4_t *>(ds + 16 * h2 + 8 * hh);
                const f32x4_t dbv = *reinterpret_cast<const f32x4_t *>(ds + 16 * h2 + 8 * hh + 4);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    dp[0][8 * h2 + e] = e < 4 ? da[e] : dbv[e - 4];
            }
            u32x4_t qa[1][G::KSTEPS], ga[1][G::KSTEPS];
            qk_read<D>(qgring[cur][0], ro, qa);
            qk_read<D>(qgring[cur][1], ro, ga);
            qk_mma<D, BF16>(qa, kf, s);                        // S = Q K^T
#pragma unroll
            for (int c = 0; c < G::KSTEPS; ++c)
                dp[0] = mma32<BF16>(ga[0][c], vf[c], dp[0]);   // D - dP = D + dO (-V)^T
            __builtin_amdgcn_sched_barrier(0);
            // P, and -dS = P (D - dP)
            float p[16], dsv[16];
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                const f32x4_t la = *reinterpret_cast<const f32x4_t *>(ls + 16 * h2 + 8 * hh);
                const f32x4_t lb = *reinterpret_cast<const f32x4_t *>(ls + 16 * h2 + 8 * hh + 4);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int r = 8 * h2 + e;
                    p[r] = fast_exp2(fmaf(s[0][r], c_log2, -(e < 4 ? la[e] : lb[e - 4])));
                    dsv[r] = p[r] * dp[0][r];
                }
            }
            // wave-uniform: may any element of this block be masked?  (p and
            // dS both zeroed: a row with no visible key has LSE = -inf)
            const bool edge = kw0 + 32 > lim_key || q0 + BT > Nq || (causal && kw0 + 31 > q0 + dq);
            if (edge) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int qi = q0 + 16 * (r >> 3) + 8 * hh + (r & 7);
                    const bool vis = qi >= row_lo && qi < Nq;
                    p[r] = vis ? p[r] : 0.f;
                    dsv[r] = vis ? dsv[r] : 0.f;
                }
            }
            u32x4_t pf[2], dsf[2];
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    pf[h2][q] = pack2<BF16>(p[8 * h2 + 2 * q], p[8 * h2 + 2 * q + 1]);
                    dsf[h2][q] = pack2<BF16>(dsv[8 * h2 + 2 * q], dsv[8 * h2 + 2 * q + 1]);
                }
            __builtin_amdgcn_sched_barrier(0);
            u32x4_t ta[G::DB][G::PCH];
            pv_read<D>(qgring[cur][1], to, ta);   // dO^T
            pv_mfma<D, BF16>(ta, pf, dvacc);      // dV^T += dO^T P
            __builtin_amdgcn_sched_barrier(0);
            pv_read<D>(qgring[cur][0], to, ta);   // Q^T
            pv_mfma<D, BF16>(ta, dsf, dkacc);     // (-dK)^T += Q^T (-dS)
        }
    };
    int t = 0;
    for (; t + 2 < n_tiles; t += 3) {
        iter(t, 0, 2);
        iter(t + 1, 1, 0);
        iter(t + 2, 2, 1);
    }
    if (t < n_tiles)
        iter(t, 0, 2);
    if (t + 1 < n_tiles)
        iter(t + 1, 1, 0);
    __syncthreads();

    if (key < Nk) {
        const size_t r = ((size_t)g * Nk + key) * d + 4 * hh;
        const float kscale = -scale;   // the accumulator holds -dK / scale
#pragma unroll
        for (int db = 0; db < G::DB; ++db)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (32 * db + 8 * q >= d)
                    continue;
                *reinterpret_cast<f32x4_t *>(dK + r + 32 * db + 8 * q) =
                    f32x4_t{dkacc[db][4 * q] * kscale, dkacc[db][4 * q + 1] * kscale,
                            dkacc[db][4 * q + 2] * kscale, dkacc[db][4 * q + 3] * kscale};
                *reinterpret_cast<f32x4_t *>(dV + r + 32 * db + 8 * q) =
                    f32x4_t{dvacc[db][4 * q], dvacc[db][4 * q + 1], dvacc[db][4 * q + 2], dvacc[db][4 * q + 3]};
            }
    }
}

template <int D, bool BF16>
hipError_t launch(const BwdArgs &a, hipStream_t stream)
{
    const float c_log2 = a.scale * kLog2e;
    // dQ first: it also writes the row term D and LSE * log2(e), which the
    // dK/dV pass reads
    const int n_qtiles = (a.Nq + BQ - 1) / BQ;
    hipError_t e = hipSuccess;
    if (n_qtiles > 0) {
        hipLaunchKernelGGL((bwd_dq_kernel<D, BF16>), dim3((unsigned)((long long)n_qtiles * a.B * a.H)),
                           dim3(NTHREADS), 0, stream, (const uint16_t *)a.q, (const uint16_t *)a.k,
                           (const uint16_t *)a.v, (const uint16_t *)a.dout, a.o, a.lse, a.delta, a.dq, a.H,
                           a.Hkv, a.Nq, a.Nk, a.d, n_qtiles, c_log2, a.scale, a.causal ? 1 : 0, a.kv_lens);
        e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    const int n_ktiles = (a.Nk + BK - 1) / BK;
    if (n_ktiles > 0) {
        hipLaunchKernelGGL((bwd_dkdv_kernel<D, BF16>), dim3((unsigned)((long long)n_ktiles * a.B * a.Hkv)),
                           dim3(NTHREADS), 0, stream, (const uint16_t *)a.q, (const uint16_t *)a.k,
                           (const uint16_t *)a.v, (const uint16_t *)a.dout, a.delta, a.dk, a.dv, a.H,
                           a.Hkv, a.Nq, a.Nk, a.d, n_ktiles, c_log2, a.scale, a.causal ? 1 : 0, a.kv_lens);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace

long long bwd_grid_size(int B, int H, int Nq, int Nk)
{
    const long long a = (long long)((Nq + BQ - 1) / BQ) * B * H;
    const long long c = (long long)((Nk + BK - 1) / BK) * B * H;
    return a > c ? a : c;
}

hipError_t launch_bwd(const BwdArgs &a, hipStream_t stream)
{
    // LDS geometry of the smaller padded head dim (64 or 128) that holds d
    if (a.d > 64)
        return a.bf16 ? launch<128, true>(a, stream) : launch<128, false>(a, stream);
    return a.bf16 ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
}

}  // namespace fa
