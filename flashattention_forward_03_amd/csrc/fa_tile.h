// Tile machinery shared by the forward and backward attention kernels
// (internal header): LDS geometry and swizzles, the buffer-to-LDS tile copy,
// the key-row permutation that chains two MFMAs, and the operand reads.
#pragma once

#include "fa_common.h"

namespace fa {
namespace {

// Key-tile rows per padded head dim: 32 where a 32-row tile still splits
// into 1 KB copy pieces over the 4 waves (d = 64, 128); the smaller tile
// frees the registers for one more wave per SIMD (measured faster: 4 waves
// at d = 64, 3 at d = 128); 64 for d = 32, 96.
template <int D>
constexpr int kBN = (D == 64 || D == 128) ? 32 : 64;
constexpr int NTHREADS = 256;

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;

// The key-row permutation used when loading the S^T A operand: A row rho is
// taken from key row sigma(rho) (bits 2 and 3 swapped).  With it, accumulator
// register r of block blk in lane l is key blk*32 + 16*(r/8) + 8*(l/32) + r%8,
// i.e. registers 8c'..8c'+7 are exactly the 8 keys the PV MFMA's B operand
// needs from this lane.
__device__ __forceinline__ int sigma(int rho) { return (rho & 0x13) | ((rho & 4) << 1) | ((rho & 8) >> 1); }

// LDS swizzles (16-byte chunk index XOR a row function) so that the MFMA
// operand reads hit distinct banks.
__device__ __forceinline__ int swz_k(int row)
{
    // bit1 | (bit0 ^ bit2) << 1 | bit3 << 2: distinct slots for the rows one
    // ds_read_b128 serves per cycle, whether 8 lanes (32 banks) or 16 lanes
    // (64 banks, split by row parity) are served together
    return ((row >> 1) & 1) | (((row ^ (row >> 2)) & 1) << 1) | (((row >> 3) & 1) << 2);
}
__device__ __forceinline__ int swz_v(int row) { return (row & 3) << 1; }

// LDS slot of 16-byte chunk c of a row with DC chunks under row key s (0..7):
// an XOR inside aligned groups of 8 chunks (4 for a short row or the last
// group of a 12-chunk row), so the slot stays inside the row; it is its own
// inverse.
template <int DC>
__device__ __forceinline__ int swz_slot(int c, int s)
{
    if constexpr (DC == 4)
        return c ^ (s & 3);
    else if constexpr (DC % 8 == 0)
        return c ^ s;
    else
        return c < 8 ? (c ^ s) : (8 | ((c & 3) ^ (s & 3)));
}

// LDS tile geometry for a padded head dim D in {32, 64, 96, 128}; the
// actual head dim d <= D (a multiple of 8) fills the first d columns and
// the rest read as zero.
template <int D>
struct Geometry {
    static constexpr int DC = D / 8;                 // 16-byte chunks per row
    static constexpr int KSTEPS = D / 16;            // MFMA k-steps over d
    static constexpr int BN = kBN<D>;                // key rows per tile
    static constexpr int NBLK = BN / 32;             // 32-key blocks per tile
    static constexpr int PCH = BN / 16;              // 16-key PV k-steps per tile
    static constexpr int DB = D / 32;                // 32-wide column blocks of O
    static constexpr int ROWB = D * 2;               // bytes per LDS row
    static constexpr int TILE = BN * ROWB;           // bytes per K (or V) tile
    static constexpr int PIECES = TILE / 1024;       // 1 KB DMA pieces per tile
    static constexpr int PIECES_PER_WAVE = PIECES / 4;
    static_assert(PIECES_PER_WAVE * 4 == PIECES, "tile must split over 4 waves");
};

// A tile of BN rows is copied into LDS with the buffer-to-LDS load (16
// bytes per lane) from a buffer resource whose base is the tile's first row
// (row stride rs bytes) and whose range ends at the last valid row: rows
// past it read as zero (those keys or rows are always masked).  off[u] is
// the lane's byte offset for its u-th 1 KB piece of the tile (chunk picked
// so that it lands in its swizzled LDS slot), the same for every tile; the
// padding columns past d get an offset beyond any buffer range, so they
// read as zero too.
constexpr unsigned kOutOfRange = 0x80000000u;   // beyond any buffer range (< 2^31 bytes)

template <int D, bool IS_K>
__device__ __forceinline__ void dma_offsets(int wave, int lane, int d, unsigned rs,
                                            unsigned (&off)[Geometry<D>::PIECES_PER_WAVE])
{
    using G = Geometry<D>;
#pragma unroll
    for (int u = 0; u < G::PIECES_PER_WAVE; ++u) {
        const int slot = (u * 4 + wave) * 64 + lane;   // 16-byte slot of the tile
        const int row = slot / G::DC;
        const int pc = slot - row * G::DC;
        const int lc = swz_slot<G::DC>(pc, IS_K ? swz_k(row) : swz_v(row));
        const bool valid = lc * 8 < d;
        off[u] = valid ? (unsigned)row * rs + (unsigned)lc * 16u : kOutOfRange;
    }
}

// The copy is issued with inline assembly on purpose: the compiler cannot
// tell which LDS bytes a direct-to-LDS load writes, so for the builtin it
// waits for the load (vmcnt(0)) before every later LDS read, which would
// drain the prefetch ring on each tile.  Here every wait is explicit: a
// tile is read only after wait_vmcnt for its own loads and a workgroup
// barrier for the other waves' loads.
typedef uint32_t u32x4s_t __attribute__((ext_vector_type(4)));

// Buffer resource for the K (or V) rows of one (b, h): base, no stride,
// nbytes in range (loads past it return zero), raw 32-bit dword format.
__device__ __forceinline__ u32x4s_t make_rsrc(const void *base, int nbytes)
{
    const uint64_t a = (uint64_t)base;
    u32x4s_t r;
    r[0] = __builtin_amdgcn_readfirstlane((uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xffffu);
    r[2] = __builtin_amdgcn_readfirstlane((uint32_t)nbytes);
    r[3] = 0x00020000u;
    return r;
}

// The same copy from a buffer resource that starts at the tile's first row:
// the lane offsets off[] are the tile-0 offsets and never change, so a tile
// costs no vector instruction; rows past the resource's range and the
// out-of-range padding columns read as zero.  lds is the 32-bit LDS address
// of this wave's piece 0 in the ring slot (piece u is 4 KB further), so no
// generic-pointer conversion runs per copy.  The caller moves the resource
// from tile to tile in scalar registers (base + tile bytes, range - tile
// bytes); device addresses stay below 2^48, so the high base word never
// carries into the stride field.
template <int D>
__device__ __forceinline__ void dma_tile_lds(const u32x4s_t &r, const unsigned *off, uint32_t lds)
{
    using G = Geometry<D>;
#pragma unroll
    for (int u = 0; u < G::PIECES_PER_WAVE; ++u)
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %2, 0 offen lds"
                     :
                     : "v"(off[u]), "s"(lds + (uint32_t)(u * 4 * 1024)), "s"(r)
                     : "memory", "m0");
}

// Per-lane byte offsets of the K operand reads of qk_tile inside a tile, one
// per (32-key block, k-step): loop-invariant, so that each read is one LDS
// instruction with the tile's base as its immediate offset.
template <int D>
__device__ __forceinline__ void qk_offsets(int krow_in_blk, int hh, int (&ko)[kBN<D> / 32][D / 16])
{
    using G = Geometry<D>;
#pragma unroll
    for (int blk = 0; blk < G::NBLK; ++blk) {
        const int row = blk * 32 + krow_in_blk;
        const int sw = swz_k(row);
#pragma unroll
        for (int c = 0; c < G::KSTEPS; ++c)
            ko[blk][c] = row * G::ROWB + (swz_slot<G::DC>(2 * c + hh, sw) << 4);
    }
}

// S = K Q^T of one tile with the offsets of qk_offsets, in two halves (the
// K operand reads, then the MFMAs) so that other work can sit between the
// reads and their first use.
template <int D>
__device__ __forceinline__ void qk_read(const unsigned char *kb, const int (&ko)[kBN<D> / 32][D / 16],
                                        u32x4_t (&ka)[kBN<D> / 32][D / 16])
{
    using G = Geometry<D>;
#pragma unroll
    for (int blk = 0; blk < G::NBLK; ++blk)
#pragma unroll
        for (int c = 0; c < G::KSTEPS; ++c)
            ka[blk][c] = *reinterpret_cast<const u32x4_t *>(kb + ko[blk][c]);
}

template <int D, bool BF16>
__device__ __forceinline__ void qk_mma(const u32x4_t (&ka)[kBN<D> / 32][D / 16], const u32x4_t (&qf)[D / 16],
                                       f32x16_t (&s)[kBN<D> / 32])
{
    using G = Geometry<D>;
#pragma unroll
    for (int c = 0; c < G::KSTEPS; ++c)
#pragma unroll
        for (int blk = 0; blk < G::NBLK; ++blk)
            s[blk] = c == 0 ? mma32<BF16>(ka[blk][c], qf[c], f32x16_t{}) : mma32<BF16>(ka[blk][c], qf[c], s[blk]);
}

// qk_mma starting from the accumulator values `from` (read, not changed).
template <int D, bool BF16>
__device__ __forceinline__ void qk_mma_from(const u32x4_t (&ka)[kBN<D> / 32][D / 16], const u32x4_t (&qf)[D / 16],
                                            f32x16_t (&s)[kBN<D> / 32], const f32x16_t &from)
{
    using G = Geometry<D>;
#pragma unroll
    for (int c = 0; c < G::KSTEPS; ++c)
#pragma unroll
        for (int blk = 0; blk < G::NBLK; ++blk)
            s[blk] = mma32<BF16>(ka[blk][c], qf[c], c == 0 ? from : s[blk]);
}

template <int D, bool BF16>
__device__ __forceinline__ void qk_tile(const unsigned char *kb, int krow_in_blk, int hh,
                                        const u32x4_t (&qf)[D / 16], f32x16_t (&s)[kBN<D> / 32])
{
    using G = Geometry<D>;
    u32x4_t ka[G::NBLK][G::KSTEPS];
#pragma unroll
    for (int blk = 0; blk < G::NBLK; ++blk) {
        const int row = blk * 32 + krow_in_blk;
        const unsigned char *rp = kb + row * G::ROWB;
        const int sw = swz_k(row);
#pragma unroll
        for (int c = 0; c < G::KSTEPS; ++c)
            ka[blk][c] = *reinterpret_cast<const u32x4_t *>(rp + (swz_slot<G::DC>(2 * c + hh, sw) << 4));
    }
#pragma unroll
    for (int c = 0; c < G::KSTEPS; ++c)
#pragma unroll
        for (int blk = 0; blk < G::NBLK; ++blk)
            s[blk] = c == 0 ? mma32<BF16>(ka[blk][c], qf[c], f32x16_t{}) : mma32<BF16>(ka[blk][c], qf[c], s[blk]);
}

// qk_tile accumulating onto the values already in s (the first product of
// the tile starts from them instead of zero).
template <int D, bool BF16>
__device__ __forceinline__ void qk_tile_acc(const unsigned char *kb, int krow_in_blk, int hh,
                                            const u32x4_t (&qf)[D / 16], f32x16_t (&s)[kBN<D> / 32])
{
    using G = Geometry<D>;
    u32x4_t ka[G::NBLK][G::KSTEPS];
#pragma unroll
    for (int blk = 0; blk < G::NBLK; ++blk) {
        const int row = blk * 32 + krow_in_blk;
        const unsigned char *rp = kb + row * G::ROWB;
        const int sw = swz_k(row);
#pragma unroll
        for (int c = 0; c < G::KSTEPS; ++c)
            ka[blk][c] = *reinterpret_cast<const u32x4_t *>(rp + (swz_slot<G::DC>(2 * c + hh, sw) << 4));
    }
#pragma unroll
    for (int c = 0; c < G::KSTEPS; ++c)
#pragma unroll
        for (int blk = 0; blk < G::NBLK; ++blk)
            s[blk] = mma32<BF16>(ka[blk][c], qf[c], s[blk]);
}

// V^T operands of the P V MFMAs of one tile (A operand: row = column of O,
// k = 8 consecutive tile keys), read with the transposing LDS read.  KSWZ:
// the tile was stored with the row-read swizzle swz_k (a tile that is also
// read by rows) instead of swz_v.
template <int D, bool KSWZ = false>
__device__ __forceinline__ void pv_operands(const unsigned char *vb, int lane, int hh,
                                            u32x4_t (&va)[D / 32][kBN<D> / 16])
{
    using G = Geometry<D>;
    const int j16 = lane & 15;
    const int g16 = lane >> 4;   // 16-lane group: bit0 = column half, bit1 = hh
#pragma unroll
    for (int db = 0; db < G::DB; ++db) {
        const int col = 32 * db + 16 * (g16 & 1) + 4 * (j16 & 3);
        const int chunk = col >> 3;
        const int half = (col & 7) * 2;
#pragma unroll
        for (int c = 0; c < G::PCH; ++c) {
            const int r0 = 16 * c + 8 * hh + (j16 >> 2);
            const int r1 = r0 + 4;
            const unsigned char *a0, *a1;
            if constexpr (KSWZ) {
                a0 = vb + r0 * G::ROWB + (swz_slot<G::DC>(chunk, swz_k(r0)) << 4) + half;
                a1 = vb + r1 * G::ROWB + (swz_slot<G::DC>(chunk, swz_k(r1)) << 4) + half;
            } else {
                a0 = vb + r0 * G::ROWB + (swz_slot<G::DC>(chunk, swz_v(r0)) << 4) + half;
                a1 = vb + r1 * G::ROWB + (swz_slot<G::DC>(chunk, swz_v(r1)) << 4) + half;
            }
            const u32x2_t y0 = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)a0));
            const u32x2_t y1 = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)a1));
            va[db][c] = u32x4_t{y0[0], y0[1], y1[0], y1[1]};
        }
    }
}

// O^T += V^T P^T for one tile; the two column blocks' MFMA chains alternate.
template <int D, bool BF16>
__device__ __forceinline__ void pv_mfma(const u32x4_t (&va)[D / 32][kBN<D> / 16], const u32x4_t (&pf)[kBN<D> / 16],
                                        f32x16_t (&oacc)[D / 32])
{
#pragma unroll
    for (int c = 0; c < kBN<D> / 16; ++c)
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
            oacc[db] = mma32<BF16>(va[db][c], pf[c], oacc[db]);
}

template <int D, bool BF16>
__device__ __forceinline__ void pv_tile(const unsigned char *vb, int lane, int hh,
                                        const u32x4_t (&pf)[kBN<D> / 16], f32x16_t (&oacc)[D / 32])
{
    u32x4_t va[D / 32][kBN<D> / 16];
    pv_operands<D>(vb, lane, hh, va);
    pv_mfma<D, BF16>(va, pf, oacc);
}

// Causal / padding mask: rel = number of valid keys counted from this lane's
// first tile key (kt0 + 8*hh).
template <int D>
__device__ __forceinline__ void mask_tile(f32x16_t (&s)[kBN<D> / 32], int rel)
{
#pragma unroll
    for (int blk = 0; blk < kBN<D> / 32; ++blk)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int koff = blk * 32 + 16 * (r >> 3) + (r & 7);
            s[blk][r] = koff < rel ? s[blk][r] : -INFINITY;
        }
}

// ---- online softmax of one 32-key tile (shared by the forward and the
// grouped-query decode)

// Bound on the probabilities formed against a stale running max, in
// exponent (log2) units: f16 P must stay below 65504, bf16 has fp32's range.
template <bool BF16>
constexpr float kRescaleLog2 = BF16 ? 32.0f : 15.0f;
// Per-lane online-softmax state.  The running max m is kept only in base-2
// units and negated, nmc = -m*c (c = scale*log2(e) > 0), which is what each
// probability p = exp2(s*c + nmc) adds; nmc is +inf until a key is seen.
struct RowState {
    float nmc;   // -m*c
    float l;     // running sum of exp2(s*c + nmc), fp32
};

// Probabilities of one tile against the row's current (possibly stale) max
// m: p = exp2(s*c + nmc) with nmc = -m*c, packed to 16 bits for the MFMA,
// summed in fp32 (4 independent partial sums).  Returns the row sum of this
// lane's 32 p.
template <int NB, bool BF16>
__device__ __forceinline__ float exp_tile(const f32x16_t (&s)[NB], float nmc, float c_log2, u32x4_t (&pf)[2 * NB])
{
    float ps[4];
#pragma unroll
    for (int blk = 0; blk < NB; ++blk)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int r = 8 * h2 + 2 * q;
                const float p0 = fast_exp2(fmaf(s[blk][r], c_log2, nmc));
                const float p1 = fast_exp2(fmaf(s[blk][r + 1], c_log2, nmc));
                pf[2 * blk + h2][q] = pack2<BF16>(p0, p1);
                // the first pair starts each partial sum (no 0 + x: x may be -0)
                ps[q] = (blk == 0 && h2 == 0) ? p0 + p1 : ps[q] + (p0 + p1);
            }
    return (ps[0] + ps[1]) + (ps[2] + ps[3]);
}

template <int D>
__device__ __forceinline__ void rescale_acc(f32x16_t (&oacc)[D / 32], float alpha)
{
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
        oacc[db] *= alpha;
}

// Online softmax step for one tile.  The running max m only has to keep
// p = exp2(s*c - m*c) below 2^tau (no overflow in the 16-bit P, fp32 sums),
// and the exact softmax does not depend on which m is used (m cancels in
// O = sum p v / sum p and LSE = m + ln l).  So the common path does not
// compute the tile max at all: it forms p against the current m and checks
// the row sum (sum >= max p); only when some row of the wave exceeds 2^tau,
// overflowed, or has no finite m yet (its first keys) does the wave take
// the exact path: tile max, new m = max(m, tile max), l and the O
// accumulators scaled by alpha = exp2((m_old - m_new) * c), p recomputed.
// The no-finite-m case needs no compare of its own: nmc is +inf then, which
// makes the row sum +inf or NaN.  Every scaling by alpha stays inside the
// exact path, so the common path carries no alpha at all: its l update is
// one add.
template <int D, bool BF16>
__device__ __forceinline__ void softmax_tile(const f32x16_t (&s)[kBN<D> / 32], RowState &st,
                                             u32x4_t (&pf)[kBN<D> / 16], float c_log2, float tau_log2,
                                             f32x16_t (&oacc)[D / 32])
{
    const float limit = exp2f(tau_log2);
    // While m is -inf, nmc is +inf, so p = exp2(s*c + inf) is +inf (or NaN
    // for a masked score) and the one compare below sends the row to the
    // exact path; the exact path is marked unlikely for the code layout.
    float psum = exp_tile<kBN<D> / 32, BF16>(s, st.nmc, c_log2, pf);
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(!(psum <= limit)) != 0, 0)) {
        // exact path: tile max (lane-local, then the other half of the wave),
        // then p again against the new max (p <= 1)
        float mx = s[0][0];
#pragma unroll
        for (int blk = 0; blk < kBN<D> / 32; ++blk)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                mx = fmaxf(mx, s[blk][r]);
        mx = fmaxf(mx, other_half(mx));
        // new max in the same units: nmc = -max(m, mx)*c (c > 0, so the max
        // commutes with the scaling), updated in place after the old value's
        // last use, and alpha = exp2((m_old - m_new)*c) = exp2(min(dx, 0))
        // with dx = -mx*c - nmc_old: 0 when m was -inf and is now finite; 1
        // when m is still -inf (O and l are 0)
        const float nx = -(mx * c_log2);
        const float dx = nx - st.nmc;
        st.nmc = fminf(st.nmc, nx);
        const float alpha = (st.nmc == INFINITY) ? 1.f : fast_exp2(fminf(dx, 0.f));
        st.l *= alpha;
        if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0)
            rescale_acc<D>(oacc, alpha);
        // (a row with no key yet: p = exp2(-inf + 0) = 0)
        psum = exp_tile<kBN<D> / 32, BF16>(s, st.nmc == INFINITY ? 0.f : st.nmc, c_log2, pf);
    }
    st.l += psum;
}

// Compile-time flag for a tile loop's iteration: true for the check-free
// iteration (the caller has shown that every per-tile test passes).
template <bool B>
struct LoopTag {
    static constexpr bool value = B;
};

// s_waitcnt for "at most N vector-memory operations outstanding" (other
// counters untouched).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt field is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

}  // namespace
}  // namespace fa
