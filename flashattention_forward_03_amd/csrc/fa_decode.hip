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
// The work is bandwidth bound (one FMA per byte of K/V), so there is no MFMA
// here: the kernel is laid out for HBM streaming.
//   * Split-KV: one workgroup per (sequence, group of 4 heads, chunk of 16
//     pages = 256 tokens) so that enough workgroups fill the 256 CUs even
//     when a batch mixes short and long sequences.  Chunk boundaries depend
//     only on logical token positions.
//   * One wave per head of the group.  The pool is [page, head, 16, d], so
//     the group's rows of one page are 4 * 16 * d * 2 bytes contiguous (16 KB
//     at d = 128): the four waves stream the same pages, and HBM sees
//     contiguous 16 KB reads instead of scattered 4 KB ones (measured on
//     MI355X: random 4 KB blocks read at ~5.2 TB/s, 16 KB blocks at ~6.1).
//   * Within a wave, token row r = lane / (d/8) with 8 consecutive head dims
//     per lane: each wave step is one fully coalesced 16-byte load per lane
//     for K and one for V; sixteen steps are loaded before any is used.
//   * q.k is reduced over the d/8 lanes of a row with DPP moves; every lane
//     keeps its own online-softmax state for its token stream; the streams
//     of a wave are merged through LDS at the end of the chunk with the
//     log-sum-exp rule.
//   * Chunks of one (sequence, head) are merged by a second small kernel with
//     the same rule; a sequence with a single chunk is finished directly.
#include "fa_common.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int PAGE = 16;
constexpr int NTHREADS = 256;
constexpr int STEPS_IN_FLIGHT = 16;  // wave steps loaded before any is used
constexpr int GROUP = NTHREADS / 64;  // heads per workgroup, one per wave

// Sum over the 16 lanes of a DPP row (lanes 16k .. 16k+15), result in all of them.
__device__ __forceinline__ float row16_sum(float x)
{
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));  // quad [1,0,3,2]
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));  // quad [2,3,0,1]
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false)); // row_half_mirror
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false)); // row_mirror
    return x;
}

// Sum over aligned groups of 8 lanes.
__device__ __forceinline__ float row8_sum(float x)
{
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));
    return x;
}

template <bool BF16>
__device__ __forceinline__ void widen8(const u32x4_t &w, float *f)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = lo16<BF16>(w[i]);
        f[2 * i + 1] = hi16<BF16>(w[i]);
    }
}

template <int D, bool BF16>
__global__ __launch_bounds__(NTHREADS) void decode_split_kernel(
    const uint16_t *__restrict__ Qp, const uint16_t *__restrict__ Kp, const uint16_t *__restrict__ Vp,
    const int32_t *__restrict__ page_table, const int32_t *__restrict__ kv_lens, float *__restrict__ O,
    float *__restrict__ LSE, float *__restrict__ part_o, float *__restrict__ part_ml, int H, int n_hgroups,
    int max_pages, int num_pages, int max_chunks, float c_log2)
{
    constexpr int TPR = D / 8;              // lanes per token row (8 head dims each)
    constexpr int RPW = 64 / TPR;           // token rows per wave step (4 or 8)
    constexpr int SPP = PAGE / RPW;         // wave steps per page (4 or 2)
    constexpr int CHUNK = kDecodeChunkPages;
    constexpr int DPL = D / 64;             // head dims per lane in the final merge

    __shared__ float sm_m[GROUP][RPW], sm_l[GROUP][RPW];
    __shared__ float sm_o[GROUP][RPW][D + 4];

    const int chunk = blockIdx.x % max_chunks;
    const int shg = blockIdx.x / max_chunks;
    const int s = shg / n_hgroups, hg = shg - s * n_hgroups;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int h = hg * GROUP + wave;
    const bool head_ok = h < H;

    int kvlen = kv_lens[s];
    kvlen = kvlen < 0 ? 0 : (kvlen > max_pages * PAGE ? max_pages * PAGE : kvlen);
    const int npages = (kvlen + PAGE - 1) / PAGE;
    const int nchunks = (npages + CHUNK - 1) / CHUNK;
    if (chunk >= nchunks)   // uniform over the workgroup (depends on s only)
        return;
    const int p_begin = chunk * CHUNK;
    const int p_end = min(p_begin + CHUNK, npages);
    const int nsteps = head_ok ? (p_end - p_begin) * SPP : 0;

    const int r = lane / TPR;      // token row within a wave step
    const int gd = lane - r * TPR; // which 8 head dims
    const size_t sh = (size_t)s * H + (head_ok ? h : 0);

    float qv[8];
    widen8<BF16>(load16(Qp + sh * D + 8 * gd), qv);
#pragma unroll
    for (int i = 0; i < 8; ++i)
        qv[i] *= c_log2;

    float m = -INFINITY, l = 0.f, acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        acc[i] = 0.f;

    // the chunk's physical page ids, one per lane (CHUNK <= 64), read once so
    // that the K/V loads of each step do not wait behind a page-table load
    static_assert(CHUNK <= 64, "one page id per lane");
    int phys_lane = 0;
    if (lane < p_end - p_begin) {
        phys_lane = page_table[(size_t)s * max_pages + p_begin + lane];
        phys_lane = phys_lane < 0 ? 0 : (phys_lane >= num_pages ? num_pages - 1 : phys_lane);
    }
    const size_t head_off = (size_t)(head_ok ? h : 0) * PAGE * D + 8 * gd;
    const size_t page_stride = (size_t)H * PAGE * D;

    for (int k0 = 0; k0 < nsteps; k0 += STEPS_IN_FLIGHT) {
        u32x4_t kr[STEPS_IN_FLIGHT], vr[STEPS_IN_FLIGHT];
        bool ok[STEPS_IN_FLIGHT];
#pragma unroll
        for (int u = 0; u < STEPS_IN_FLIGHT; ++u) {
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
        float t[STEPS_IN_FLIGHT];
        float mx = -INFINITY;
#pragma unroll
        for (int u = 0; u < STEPS_IN_FLIGHT; ++u) {
            float kf[8];
            widen8<BF16>(kr[u], kf);
            float dot = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                dot = fmaf(qv[i], kf[i], dot);
            dot = (TPR == 16) ? row16_sum(dot) : row8_sum(dot);
            t[u] = ok[u] ? dot : -INFINITY;
            mx = fmaxf(mx, t[u]);
        }
        const float m_new = fmaxf(m, mx);
        if (m_new == -INFINITY)
            continue;
        const float alpha = fast_exp2(m - m_new);
        l *= alpha;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            acc[i] *= alpha;
#pragma unroll
        for (int u = 0; u < STEPS_IN_FLIGHT; ++u) {
            const float p = fast_exp2(t[u] - m_new);
            l += p;
            float vf[8];
            widen8<BF16>(vr[u], vf);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                acc[i] = fmaf(p, vf[i], acc[i]);
        }
        m = m_new;
    }

    // ---- merge the RPW token streams of each wave's head (log-sum-exp rule)
    if (gd == 0) {
        sm_m[wave][r] = m;
        sm_l[wave][r] = l;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
        sm_o[wave][r][8 * gd + i] = acc[i];
    __syncthreads();
    if (!head_ok)
        return;
    float M = -INFINITY;
#pragma unroll
    for (int j = 0; j < RPW; ++j)
        M = fmaxf(M, sm_m[wave][j]);
    float w[RPW];
    float L = 0.f;
#pragma unroll
    for (int j = 0; j < RPW; ++j) {
        w[j] = sm_m[wave][j] == -INFINITY ? 0.f : fast_exp2(sm_m[wave][j] - M);
        L = fmaf(w[j], sm_l[wave][j], L);
    }
    const size_t slot = sh * max_chunks + chunk;
#pragma unroll
    for (int k = 0; k < DPL; ++k) {
        const int dim = lane + 64 * k;
        float num = 0.f;
#pragma unroll
        for (int j = 0; j < RPW; ++j)
            num = fmaf(w[j], sm_o[wave][j][dim], num);
        if (nchunks == 1)
            O[sh * D + dim] = num / L;
        else
            part_o[slot * D + dim] = num;
    }
    if (lane == 0) {
        if (nchunks == 1) {
            LSE[sh] = (M + __log2f(L)) * kLn2;
        } else {
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

template <int D, bool BF16>
hipError_t launch(const DecodeArgs &a, hipStream_t stream)
{
    const int max_chunks = decode_max_chunks(a.max_pages);
    const int n_hgroups = (a.H + GROUP - 1) / GROUP;
    const long long grid = (long long)a.S * n_hgroups * max_chunks;
    hipLaunchKernelGGL((decode_split_kernel<D, BF16>), dim3((unsigned)grid), dim3(NTHREADS), 0, stream,
                       (const uint16_t *)a.q, (const uint16_t *)a.k_pages, (const uint16_t *)a.v_pages,
                       a.page_table, a.kv_lens, a.o, a.lse, a.part_o, a.part_ml, a.H, n_hgroups, a.max_pages,
                       a.num_pages, max_chunks, a.scale * kLog2e);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL((decode_combine_kernel<D>), dim3((unsigned)(a.S * n_hgroups)), dim3(NTHREADS), 0, stream,
                       a.kv_lens, a.part_o, a.part_ml, a.o, a.lse, a.H, n_hgroups, a.max_pages, max_chunks);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream)
{
    if (a.d == 64)
        return a.bf16 ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
    return a.bf16 ? launch<128, true>(a, stream) : launch<128, false>(a, stream);
}

}  // namespace fa
