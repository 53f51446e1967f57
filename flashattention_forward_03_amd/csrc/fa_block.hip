// Kernels of the pre-LayerNorm attention block (the encoder layer drawn on
// the Kernel-Inference-Engine page: LayerNorm, dense Q/K/V, attention, dense
// W_O, residual), around the attention forward of fa_fwd.hip:
//
//   ln_stats_kernel   per-row mean and 1/sqrt(var + eps), Welford's one-pass
//                     update (per 16-byte chunk, then merged across lanes);
//   ln_fold_kernel    once per weight set: W' = W diag(gamma) in the 16-bit
//                     dtype, b' = b + W beta and c = sum_k W'[n, k];
//   gemm_kernel       Y = A W^T on 32x32x16 MFMA (16-bit operands, fp32
//                     accumulate) with one of two epilogues:
//                       LN:   y = rstd_t (acc - mean_t c_n) + b'_n, which is
//                             LN(x) W^T + b with the normalisation folded in
//                             (no normalised activation is ever stored);
//                       BIAS: y = acc + b_n (+ residual[t, n]).
#include <climits>

#include "fa_internal.h"
#include "fa_tile.h"

namespace fa {
namespace {

template <bool BF16>
__device__ __forceinline__ float widen16(uint16_t h)
{
    if constexpr (BF16)
        return __uint_as_float((uint32_t)h << 16);
    else
        return (float)__builtin_bit_cast(_Float16, h);
}

template <bool BF16>
__device__ __forceinline__ uint16_t narrow16(float x)
{
    if constexpr (BF16)
        return __builtin_bit_cast(uint16_t, (__bf16)x);
    else
        return __builtin_bit_cast(uint16_t, (_Float16)x);
}

// ------------------------------------------------------------ row moments ---

// Count, mean and sum of squared deviations of a set of values; merging two
// sets is the parallel form of Welford's update.
struct Moments {
    float n, mean, m2;
};

__device__ __forceinline__ void merge_into(Moments &a, float nb, float mb, float m2b)
{
    const float n = a.n + nb;
    if (n > 0.f) {
        const float fb = nb / n;
        const float delta = mb - a.mean;
        a.m2 += m2b + delta * delta * a.n * fb;
        a.mean += delta * fb;
        a.n = n;
    }
}

// One wave per row; each lane folds its 16-byte chunks (8 values: their own
// mean and squared deviations first) into its running moments, then the 64
// lanes merge pairwise over a butterfly.
template <bool BF16>
__global__ __launch_bounds__(256) void ln_stats_kernel(const uint16_t *__restrict__ x, float *__restrict__ mean,
                                                       float *__restrict__ rstd, int T, int C, float eps)
{
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= T)
        return;
    const uint16_t *xr = x + (size_t)row * C;
    const int chunks = C >> 3;
    Moments m{0.f, 0.f, 0.f};
#pragma unroll 4
    for (int c = lane; c < chunks; c += 64) {
        const u32x4_t v = load16(xr + c * 8);
        float e[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            e[2 * i] = lo16<BF16>(v[i]);
            e[2 * i + 1] = hi16<BF16>(v[i]);
        }
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            s += e[i];
        const float mc = s * 0.125f;
        float q = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            q += (e[i] - mc) * (e[i] - mc);
        merge_into(m, 8.f, mc, q);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const float nb = __shfl_xor(m.n, off);
        const float mb = __shfl_xor(m.mean, off);
        const float qb = __shfl_xor(m.m2, off);
        merge_into(m, nb, mb, qb);
    }
    if (lane == 0) {
        mean[row] = m.mean;
        rstd[row] = 1.0f / __builtin_sqrtf(m.m2 / (float)C + eps);
    }
}

// ----------------------------------------------------------- weight fold ---

template <bool BF16>
__global__ __launch_bounds__(256) void ln_fold_kernel(const float *__restrict__ gamma, const float *__restrict__ beta,
                                                      const uint16_t *__restrict__ w, const float *__restrict__ bias,
                                                      uint16_t *__restrict__ wf, float *__restrict__ bias_f,
                                                      float *__restrict__ colsum, int C)
{
    __shared__ float red[2][4];
    const int n = blockIdx.x;
    const uint16_t *wr = w + (size_t)n * C;
    uint16_t *fr = wf + (size_t)n * C;
    float sc = 0.f, sb = 0.f;
    for (int k = threadIdx.x; k < C; k += 256) {
        const float wv = widen16<BF16>(wr[k]);
        const uint16_t p = narrow16<BF16>(gamma[k] * wv);
        fr[k] = p;
        sc += widen16<BF16>(p);
        sb += beta[k] * wv;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        sc += __shfl_xor(sc, off);
        sb += __shfl_xor(sb, off);
    }
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        red[0][wave] = sc;
        red[1][wave] = sb;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        colsum[n] = (red[0][0] + red[0][1]) + (red[0][2] + red[0][3]);
        bias_f[n] = (bias ? bias[n] : 0.f) + ((red[1][0] + red[1][1]) + (red[1][2] + red[1][3]));
    }
}

// ------------------------------------------------------------------ GEMM ---

// Workgroup tile: 256 rows of A (tokens) x 256 rows of W (output features),
// k in steps of 64 (one 128-byte LDS row per matrix row).  8 waves: wave w
// owns tokens 64 (w & 3) .. +63 and features 128 (w >> 2) .. +127, i.e. 2 x 4
// blocks of 32 x 32 (128 accumulator registers), so each k16 step reads 6
// operands from LDS for 8 MFMAs.  Two LDS stages of 64 KB: the copy of k-step
// j + 1 overlaps the MFMAs of k-step j.
constexpr int GM_TILE = 256;
constexpr int GM_BK = 64;
constexpr int GM_THREADS = 512;
constexpr int GM_OPB = GM_TILE * GM_BK * 2;   // bytes per operand tile (32 KB)

// 16-byte buffer-to-LDS copy (64 lanes fill 1 KB from LDS byte address
// lds_addr on) with the k-step's byte offset in soffset.
__device__ __forceinline__ void dma16(const u32x4s_t &rsrc, unsigned voff, unsigned soff, uint32_t lds_addr)
{
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %2, %3 offen lds"
                 :
                 : "v"(voff), "s"(lds_addr), "s"(rsrc), "s"(soff)
                 : "memory", "m0");
}

template <bool BF16, int EPI>
__global__ __launch_bounds__(GM_THREADS, 1) void gemm_kernel(GemmArgs g)
{
    // [operand: 0 = A, 1 = W][stage]; a tile row is 8 16-byte slots, slot =
    // chunk ^ swz_k(row) so that the MFMA operand reads are conflict-free
    __shared__ __attribute__((aligned(1024))) unsigned char lds[2][2][GM_OPB];
    __shared__ __attribute__((aligned(16))) float fv[512];   // epilogue: the tile's bias, then colsum

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int tiles_n = (g.N + GM_TILE - 1) / GM_TILE;
    const int L = xcd_contiguous_id(blockIdx.x, gridDim.x);
    const int mb = L / tiles_n, nb = L - mb * tiles_n;
    const int m0 = mb * GM_TILE, n0 = nb * GM_TILE;
    const int rows_a = min(GM_TILE, g.M - m0), rows_w = min(GM_TILE, g.N - n0);
    const unsigned lda_b = (unsigned)g.K * 2u;

    // rows past M (N) are outside the buffer range and read as zero
    const u32x4s_t ra = make_rsrc(static_cast<const uint16_t *>(g.a) + (size_t)m0 * g.K, rows_a * (int)lda_b);
    const u32x4s_t rw = make_rsrc(static_cast<const uint16_t *>(g.w) + (size_t)n0 * g.K, rows_w * (int)lda_b);

    // this wave copies 1 KB pieces 4 wave .. 4 wave + 3 of each operand tile:
    // piece p = tile rows 8p .. 8p + 7, lane -> row 8p + lane / 8, slot lane % 8
    unsigned voff[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int row = (wave * 4 + u) * 8 + (lane >> 3);
        const int chunk = (lane & 7) ^ swz_k(row);
        voff[u] = (unsigned)row * lda_b + (unsigned)chunk * 16u;
    }
    // LDS byte address of this wave's first piece (operand A, stage 0)
    const uint32_t lds_wave =
        __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void *)&lds[0][0][0]) + wave * 4 * 1024;
    auto issue = [&](int stage, int kt) {
        const unsigned soff = __builtin_amdgcn_readfirstlane((unsigned)kt * (GM_BK * 2));
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            dma16(ra, voff[u], soff, lds_wave + stage * GM_OPB + u * 1024);
            dma16(rw, voff[u], soff, lds_wave + 2 * GM_OPB + stage * GM_OPB + u * 1024);
        }
    };

    const int wt = wave & 3, wn = wave >> 2;
    const int r32 = lane & 31;
    const int sw = swz_k(r32);   // row bits 0..3 are lane bits 0..3 in every 32-row block
    const int hh = lane >> 5;
    int rd[4];                   // byte offset of this lane's operand in a 32-row block, per k16 step
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
        rd[ks] = r32 * 128 + (((2 * ks + hh) ^ sw) << 4);

    // the epilogue's per-token statistics, loaded while the k-loop runs
    int tok[2];
    float tm[2] = {0.f, 0.f}, tr[2] = {0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        tok[j] = m0 + wt * 64 + j * 32 + r32;
        if constexpr (EPI == GEMM_EPI_LN) {
            if (tok[j] < g.M) {
                tm[j] = g.mean[tok[j]];
                tr[j] = g.rstd[tok[j]];
            }
        }
    }
    f32x16_t acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
            acc[i][j] = f32x16_t{};

    // Operands of k16 step ks + 1 are read while the MFMAs of step ks run
    // (two register sets); the scheduling barriers keep the compiler from
    // sinking the reads next to their MFMAs.
    auto compute = [&](int stage) {
        const unsigned char *at = &lds[0][stage][wt * 64 * 128];
        const unsigned char *wtile = &lds[1][stage][wn * 128 * 128];
        u32x4_t wf[2][4], xf[2][2];
        auto read = [&](int ks, int buf) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                wf[buf][i] = *reinterpret_cast<const u32x4_t *>(wtile + i * 32 * 128 + rd[ks]);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                xf[buf][j] = *reinterpret_cast<const u32x4_t *>(at + j * 32 * 128 + rd[ks]);
        };
        read(0, 0);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int buf = ks & 1;
            if (ks + 1 < 4)
                read(ks + 1, buf ^ 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = mma32<BF16>(wf[buf][i], xf[buf][j], acc[i][j]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    const int KT = g.K / GM_BK;
    issue(0, 0);
    for (int kt = 0; kt < KT; kt += 2) {
        wait_vmcnt<0>();
        __syncthreads();
        if (kt + 1 < KT)
            issue(1, kt + 1);
        compute(0);
        if (kt + 1 < KT) {
            wait_vmcnt<0>();
            __syncthreads();
            if (kt + 2 < KT)
                issue(0, kt + 2);
            compute(1);
        }
    }

    // epilogue: block (i, j) register r of lane l is feature
    // n0 + 128 wn + 32 i + 8 (r / 4) + 4 (l / 32) + r % 4 and token
    // m0 + 64 wt + 32 j + l % 32.  Every load it needs is issued before its
    // first store (the output may not alias the inputs): the tile's
    // per-feature vectors go through LDS, the residual pieces straight into
    // registers.  The finished 16-bit tile is then staged in LDS (free after
    // the last k-step) and written out by rows: a store straight from the
    // accumulator layout would touch 32 output rows per instruction.
    const float *__restrict__ bias = g.bias;
    const float *__restrict__ colsum = g.colsum;
    const uint16_t *__restrict__ res = static_cast<const uint16_t *>(g.res);
    uint16_t *__restrict__ y = static_cast<uint16_t *>(g.y);
    {
        const int t = threadIdx.x;
        const int n = n0 + (t & 255);
        const float *src = t < 256 ? bias : colsum;
        fv[t] = (src && n < g.N) ? src[n] : 0.f;
    }
    u32x2_t rv[4][4][2];
    if constexpr (EPI == GEMM_EPI_BIAS) {
        if (res) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const int n = n0 + wn * 128 + i * 32 + q * 8 + hh * 4;
                        rv[i][q][j] = (tok[j] < g.M && n < g.N)
                                          ? *reinterpret_cast<const u32x2_t *>(res + (size_t)tok[j] * g.N + n)
                                          : u32x2_t{0u, 0u};
                    }
        }
    }
    __syncthreads();   // every wave is done with the operand tiles; fv is filled
    // the output tile: 256 rows of 512 bytes, 16-byte slot = chunk ^ (row % 32)
    unsigned char *ot = &lds[0][0][0];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int nl = wn * 128 + i * 32 + q * 8 + hh * 4;   // feature within the tile
            const f32x4_t bv = *reinterpret_cast<const f32x4_t *>(fv + nl);
            const f32x4_t cv = *reinterpret_cast<const f32x4_t *>(fv + 256 + nl);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float a = acc[i][j][q * 4 + e];
                    if constexpr (EPI == GEMM_EPI_LN)
                        v[e] = __builtin_fmaf(tr[j], __builtin_fmaf(-tm[j], cv[e], a), bv[e]);
                    else
                        v[e] = a + bv[e];
                }
                if constexpr (EPI == GEMM_EPI_BIAS) {
                    if (res) {
                        v[0] += lo16<BF16>(rv[i][q][j][0]);
                        v[1] += hi16<BF16>(rv[i][q][j][0]);
                        v[2] += lo16<BF16>(rv[i][q][j][1]);
                        v[3] += hi16<BF16>(rv[i][q][j][1]);
                    }
                }
                const int row = wt * 64 + j * 32 + r32;
                const int slot = (nl >> 3) ^ (row & 31);
                *reinterpret_cast<u32x2_t *>(ot + row * 512 + slot * 16 + hh * 8) =
                    u32x2_t{pack2<BF16>(v[0], v[1]), pack2<BF16>(v[2], v[3])};
            }
        }
    }
    __syncthreads();
    // rows out: wave w writes rows 32 w .. 32 w + 31, two per instruction
    {
        const int chunk = lane & 31;
        const int n = n0 + chunk * 8;
#pragma unroll 4
        for (int it = 0; it < 16; ++it) {
            const int row = wave * 32 + it * 2 + hh;
            const u32x4_t v = *reinterpret_cast<const u32x4_t *>(ot + row * 512 + ((chunk ^ (row & 31)) << 4));
            if (m0 + row < g.M && n < g.N)
                *reinterpret_cast<u32x4_t *>(y + (size_t)(m0 + row) * g.N + n) = v;
        }
    }
}

}  // namespace

hipError_t launch_ln_stats(const void *x, float *mean, float *rstd, int T, int C, float eps, bool bf16,
                           hipStream_t stream)
{
    const dim3 grid((unsigned)((T + 3) / 4)), block(256);
    const uint16_t *xp = static_cast<const uint16_t *>(x);
    if (bf16)
        hipLaunchKernelGGL(ln_stats_kernel<true>, grid, block, 0, stream, xp, mean, rstd, T, C, eps);
    else
        hipLaunchKernelGGL(ln_stats_kernel<false>, grid, block, 0, stream, xp, mean, rstd, T, C, eps);
    return hipGetLastError();
}

hipError_t launch_ln_fold(const float *gamma, const float *beta, const void *w, const float *bias, void *w_folded,
                          float *bias_folded, float *colsum, int N, int C, bool bf16, hipStream_t stream)
{
    const dim3 grid((unsigned)N), block(256);
    const uint16_t *wp = static_cast<const uint16_t *>(w);
    uint16_t *fp = static_cast<uint16_t *>(w_folded);
    if (bf16)
        hipLaunchKernelGGL(ln_fold_kernel<true>, grid, block, 0, stream, gamma, beta, wp, bias, fp, bias_folded,
                           colsum, C);
    else
        hipLaunchKernelGGL(ln_fold_kernel<false>, grid, block, 0, stream, gamma, beta, wp, bias, fp, bias_folded,
                           colsum, C);
    return hipGetLastError();
}

long long gemm_grid_size(int M, int N)
{
    return (long long)((M + GM_TILE - 1) / GM_TILE) * ((N + GM_TILE - 1) / GM_TILE);
}

hipError_t launch_gemm(const GemmArgs &g, int epi, bool bf16, hipStream_t stream)
{
    const dim3 grid((unsigned)gemm_grid_size(g.M, g.N)), block(GM_THREADS);
    if (epi == GEMM_EPI_LN) {
        if (bf16)
            hipLaunchKernelGGL((gemm_kernel<true, GEMM_EPI_LN>), grid, block, 0, stream, g);
        else
            hipLaunchKernelGGL((gemm_kernel<false, GEMM_EPI_LN>), grid, block, 0, stream, g);
    } else {
        if (bf16)
            hipLaunchKernelGGL((gemm_kernel<true, GEMM_EPI_BIAS>), grid, block, 0, stream, g);
        else
            hipLaunchKernelGGL((gemm_kernel<false, GEMM_EPI_BIAS>), grid, block, 0, stream, g);
    }
    return hipGetLastError();
}

}  // namespace fa
