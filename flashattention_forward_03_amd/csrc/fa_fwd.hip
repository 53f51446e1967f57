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
//   * workgroup = 4 waves = BM = 128 query rows (32 per wave), one (b, h);
//   * key tiles of BN = 64 rows, K and V double-buffered in LDS, loaded with
//     16-byte coalesced global reads one tile ahead;
//   * scores are formed transposed, S^T = K Q^T, with the 32x32x16 MFMA so
//     that each lane owns ONE query row (lane % 32) and 32 of its 64 scores:
//     the row max / sum are lane-local plus one permlane32 swap, and the
//     accumulator registers are directly the B operand of the second MFMA;
//   * O^T = V^T P^T with the same MFMA; V^T fragments come straight from the
//     row-major LDS tile through the gfx950 transposing read ds_read_b64_tr_b16;
//   * softmax in base 2: p = exp2(s * scale * log2(e) - m * scale * log2(e)),
//     one FMA + one v_exp_f32 per score; l accumulates p in fp32 before it is
//     rounded to 16 bits for the MFMA (a bf16-rounded sum would put up to
//     2^-9 of error into ln l);
//   * O is written in fp32 [B, H, Nq, d], LSE = m * scale + ln(l) in fp32.
#include "fa_common.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int BM = 128;
constexpr int BN = 64;
constexpr int NTHREADS = 256;

// The key-row permutation used when loading the S^T A operand: A row rho is
// taken from key row sigma(rho) (bits 2 and 3 swapped).  With it, accumulator
// register r of block blk in lane l is key blk*32 + 16*(r/8) + 8*(l/32) + r%8,
// i.e. registers 8c'..8c'+7 are exactly the 8 keys the PV MFMA's B operand
// needs from this lane.
__device__ __forceinline__ int sigma(int rho) { return (rho & 0x13) | ((rho & 4) << 1) | ((rho & 8) >> 1); }

// LDS swizzles (16-byte chunk index XOR a row function) so that the MFMA
// operand reads hit distinct banks.
__device__ __forceinline__ int swz_k(int row) { return (row & 3) | ((row >> 1) & 4); }
__device__ __forceinline__ int swz_v(int row) { return (row & 3) << 1; }

template <int D, bool BF16, bool CAUSAL>
__global__ __launch_bounds__(NTHREADS, 2) void fwd_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
    float *__restrict__ O, float *__restrict__ LSE, int H, int Nq, int Nk, int n_qtiles,
    float c_log2, float scale, const int32_t *__restrict__ kv_lens)
{
    constexpr int DC = D / 8;                          // 16-byte chunks per row
    constexpr int KSTEPS = D / 16;                     // MFMA k-steps over d
    constexpr int NBLK = BN / 32;                      // 32-key blocks per tile
    constexpr int PCH = BN / 16;                       // 16-key PV k-steps per tile
    constexpr int DB = D / 32;                         // 32-wide column blocks of O
    constexpr int ROWB = D * 2;                        // bytes per LDS row
    constexpr int TILE = BN * ROWB;                    // bytes per K (or V) tile
    constexpr int LOADS = BN * DC / NTHREADS;          // 16-byte loads per thread per tensor
    static_assert(LOADS * NTHREADS == BN * DC, "tile must split evenly");

    __shared__ __attribute__((aligned(16))) unsigned char smem[2 * 2 * TILE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int hh = lane >> 5;

    // ---- which (b, h, query tile)
    const int logical = xcd_contiguous_id(blockIdx.x, gridDim.x);
    const int bh = logical / n_qtiles;
    int qt = logical - bh * n_qtiles;
    if (CAUSAL)
        qt = n_qtiles - 1 - qt;   // longest rows first
    const int b = bh / H;
    const int q0 = qt * BM;

    int kvlen = Nk;
    if (kv_lens) {
        kvlen = kv_lens[b];
        kvlen = kvlen < 0 ? 0 : (kvlen > Nk ? Nk : kvlen);
    }
    const int dq = Nk - Nq;   // causal: row i sees keys j <= i + dq
    int key_end = kvlen;
    int wave_key_end = kvlen;
    if (CAUSAL) {
        const int last = min(q0 + BM, Nq) - 1;
        key_end = min(key_end, max(last + dq + 1, 0));
        const int wlast = min(q0 + wave * 32 + 32, Nq) - 1;
        wave_key_end = min(wave_key_end, max(wlast + dq + 1, 0));
    }
    const int n_tiles = (key_end + BN - 1) / BN;
    const int wave_first_row = q0 + wave * 32;

    // ---- this lane's query row and its Q fragments (B operand of S^T = K Q^T)
    const int qrow = wave_first_row + l32;
    u32x4_t qf[KSTEPS];
    {
        const uint16_t *qp = Q + ((size_t)bh * Nq + (qrow < Nq ? qrow : 0)) * D + 8 * hh;
#pragma unroll
        for (int c = 0; c < KSTEPS; ++c)
            qf[c] = qrow < Nq ? load16(qp + 16 * c) : u32x4_t{0, 0, 0, 0};
    }

    f32x16_t oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
        oacc[db] = f32x16_t{};
    float m_run = -INFINITY;
    float l_run = 0.f;

    const uint16_t *Kb = K + (size_t)bh * Nk * D;
    const uint16_t *Vb = V + (size_t)bh * Nk * D;
    u32x4_t kreg[LOADS], vreg[LOADS];

    auto gload = [&](int t) {
        const int kt0 = t * BN;
#pragma unroll
        for (int u = 0; u < LOADS; ++u) {
            const int id = tid + u * NTHREADS;
            const int row = id / DC, cc = id % DC;
            const int key = kt0 + row;
            if (key < Nk) {
                kreg[u] = load16(Kb + (size_t)key * D + cc * 8);
                vreg[u] = load16(Vb + (size_t)key * D + cc * 8);
            } else {
                kreg[u] = u32x4_t{0, 0, 0, 0};
                vreg[u] = u32x4_t{0, 0, 0, 0};
            }
        }
    };
    auto lstore = [&](int buf) {
        unsigned char *kb = smem + buf * 2 * TILE;
        unsigned char *vb = kb + TILE;
#pragma unroll
        for (int u = 0; u < LOADS; ++u) {
            const int id = tid + u * NTHREADS;
            const int row = id / DC, cc = id % DC;
            *reinterpret_cast<u32x4_t *>(kb + row * ROWB + ((cc ^ swz_k(row)) << 4)) = kreg[u];
            *reinterpret_cast<u32x4_t *>(vb + row * ROWB + ((cc ^ swz_v(row)) << 4)) = vreg[u];
        }
    };

    if (n_tiles > 0) {
        gload(0);
        lstore(0);
    }
    __syncthreads();

    // per-lane constants of the operand reads
    const int krow_in_blk = sigma(l32);
    const int j16 = lane & 15;
    const int g16 = lane >> 4;   // 16-lane group: bit0 = column half, bit1 = hh

    for (int t = 0; t < n_tiles; ++t) {
        const int buf = t & 1;
        if (t + 1 < n_tiles)
            gload(t + 1);
        const int kt0 = t * BN;
        if (kt0 < wave_key_end) {
            const unsigned char *kb = smem + buf * 2 * TILE;
            const unsigned char *vb = kb + TILE;

            // ---- S^T = K Q^T for the 64 keys of this tile (two 32-key blocks)
            f32x16_t s[NBLK];
#pragma unroll
            for (int blk = 0; blk < NBLK; ++blk) {
                s[blk] = f32x16_t{};
                const int row = blk * 32 + krow_in_blk;
                const unsigned char *rp = kb + row * ROWB;
                const int sw = swz_k(row);
#pragma unroll
                for (int c = 0; c < KSTEPS; ++c) {
                    const u32x4_t a = *reinterpret_cast<const u32x4_t *>(rp + (((2 * c + hh) ^ sw) << 4));
                    s[blk] = mma32<BF16>(a, qf[c], s[blk]);
                }
            }

            // ---- masks (only on tiles that cross the padded length or the diagonal)
            const bool need_mask = (kt0 + BN > kvlen) || (CAUSAL && kt0 + BN - 1 > wave_first_row + dq);
            if (need_mask) {
                int lim = kvlen;
                if (CAUSAL)
                    lim = min(lim, qrow + dq + 1);
                const int kbase = kt0 + 8 * hh;
#pragma unroll
                for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = kbase + blk * 32 + 16 * (r >> 3) + (r & 7);
                        if (key >= lim)
                            s[blk][r] = -INFINITY;
                    }
            }

            // ---- online softmax (raw-score units for m; base-2 exponent)
            float mx = s[0][0];
#pragma unroll
            for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    mx = fmaxf(mx, s[blk][r]);
            mx = fmaxf(mx, other_half(mx));
            const float m_new = fmaxf(m_run, mx);
            const float mc = (m_new == -INFINITY) ? 0.f : m_new * c_log2;
            const float alpha = fast_exp2(m_run * c_log2 - mc);
            m_run = m_new;

            u32x4_t pf[PCH];
            float psum = 0.f;
#pragma unroll
            for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int r = 8 * h2 + 2 * q;
                        const float p0 = fast_exp2(fmaf(s[blk][r], c_log2, -mc));
                        const float p1 = fast_exp2(fmaf(s[blk][r + 1], c_log2, -mc));
                        const uint32_t w = pack2<BF16>(p0, p1);
                        pf[2 * blk + h2][q] = w;
                        psum += p0 + p1;
                    }
            l_run = l_run * alpha + psum;
#pragma unroll
            for (int db = 0; db < DB; ++db)
                oacc[db] *= alpha;

            // ---- O^T += V^T P^T
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int col = 32 * db + 16 * (g16 & 1) + 4 * (j16 & 3);
                const int chunk = col >> 3;
                const int half = (col & 7) * 2;
#pragma unroll
                for (int c = 0; c < PCH; ++c) {
                    const int r0 = 16 * c + 8 * hh + (j16 >> 2);
                    const int r1 = r0 + 4;
                    typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
                    const unsigned char *a0 = vb + r0 * ROWB + ((chunk ^ swz_v(r0)) << 4) + half;
                    const unsigned char *a1 = vb + r1 * ROWB + ((chunk ^ swz_v(r1)) << 4) + half;
                    const i16x4_t x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(a0));
                    const i16x4_t x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(a1));
                    const u32x2_t y0 = __builtin_bit_cast(u32x2_t, x0);
                    const u32x2_t y1 = __builtin_bit_cast(u32x2_t, x1);
                    const u32x4_t a = {y0[0], y0[1], y1[0], y1[1]};
                    oacc[db] = mma32<BF16>(a, pf[c], oacc[db]);
                }
            }
        }
        if (t + 1 < n_tiles)
            lstore(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: O = O_acc / l, LSE = m * scale + ln(l)
    const float l_tot = l_run + other_half(l_run);
    if (qrow < Nq) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        float *op = O + ((size_t)bh * Nq + qrow) * D + 4 * hh;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                f32x4_t v = {oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv,
                             oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv};
                *reinterpret_cast<f32x4_t *>(op + 32 * db + 8 * g) = v;
            }
        if (hh == 0)
            LSE[(size_t)bh * Nq + qrow] = l_tot > 0.f ? m_run * scale + __log2f(l_tot) * kLn2 : -INFINITY;
    }
}

template <int D, bool BF16, bool CAUSAL>
hipError_t launch(const FwdArgs &a, hipStream_t stream)
{
    const int n_qtiles = (a.Nq + BM - 1) / BM;
    const long long grid = (long long)n_qtiles * a.B * a.H;
    hipLaunchKernelGGL((fwd_kernel<D, BF16, CAUSAL>), dim3((unsigned)grid), dim3(NTHREADS), 0, stream,
                       (const uint16_t *)a.q, (const uint16_t *)a.k, (const uint16_t *)a.v, a.o, a.lse,
                       a.H, a.Nq, a.Nk, n_qtiles, a.scale * kLog2e, a.scale, a.kv_lens);
    return hipGetLastError();
}

template <int D, bool BF16>
hipError_t launch_c(const FwdArgs &a, hipStream_t s)
{
    return a.causal ? launch<D, BF16, true>(a, s) : launch<D, BF16, false>(a, s);
}

}  // namespace

long long fwd_grid_size(int B, int H, int Nq) { return (long long)((Nq + BM - 1) / BM) * B * H; }

hipError_t launch_fwd(const FwdArgs &a, hipStream_t stream)
{
    if (a.d == 64)
        return a.bf16 ? launch_c<64, true>(a, stream) : launch_c<64, false>(a, stream);
    return a.bf16 ? launch_c<128, true>(a, stream) : launch_c<128, false>(a, stream);
}

}  // namespace fa
