// Internal launcher interface between the C-ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

// Output element types of the forward's O.
constexpr int FA_O_F16 = 0;
constexpr int FA_O_BF16 = 1;
constexpr int FA_O_F32 = 2;

// Forward layout, passed to the kernel by value: element strides (batch,
// head, row) of Q, K, V and O (head dim contiguous), the head dim d and
// O's element type.
struct FwdLayout {
    long long qs[3], ks[3], vs[3], os[3];
    int d;
    int o_kind;
};

struct FwdArgs {
    const void *q, *k, *v;
    void *o;
    float *lse;
    int B, H, Hkv, Nq, Nk;   // query head h reads K/V head h / (H / Hkv)
    float scale;
    bool causal, bf16;
    const int32_t *kv_lens;
    FwdLayout lay;
};

struct DecodeArgs {
    const void *q, *k_pages, *v_pages;
    const int32_t *page_table, *kv_lens;
    float *o, *lse;
    int S, H, Hkv, d, page_size, max_pages, num_pages;   // query head h reads K/V head h / (H / Hkv)
    float scale;
    bool bf16;
    float *part_o, *part_ml;   // workspace views (NULL when one chunk covers every sequence)
};

// Forward: number of workgroups one call launches.
long long fwd_grid_size(int B, int H, int Nq);
hipError_t launch_fwd(const FwdArgs &a, hipStream_t stream);

// Backward (contiguous [B, heads, N, d] tensors, d = 8..128): dQ, with
// D = rowsum(dO * O) into delta, then dK/dV.
struct BwdArgs {
    const void *q, *k, *v, *dout;
    const float *o, *lse;
    float *dq, *dk, *dv, *delta;
    int B, H, Hkv, Nq, Nk, d;   // d = 8..128, a multiple of 8
    float scale;
    bool causal, bf16;
    const int32_t *kv_lens;
};
long long bwd_grid_size(int B, int H, int Nq, int Nk);
hipError_t launch_bwd(const BwdArgs &a, hipStream_t stream);

// Paged KV cache append: T new tokens' K/V rows [T, Hkv, d] into the pools.
struct KvAppendArgs {
    const void *k_new, *v_new;
    const int32_t *seq_ids, *positions;
    int T;
    void *k_pages, *v_pages;
    const int32_t *page_table;
    int S, Hkv, d, max_pages, num_pages;
};
hipError_t launch_kv_append(const KvAppendArgs &a, hipStream_t stream);

// Pre-LayerNorm block: row statistics, the LayerNorm fold of a dense layer's
// weights, and the dense-layer GEMM Y[M, N] = A[M, K] W[N, K]^T (row-major,
// 16-bit, contiguous) with the LayerNorm or the bias (+ residual) epilogue.
constexpr int GEMM_EPI_LN = 0;     // y = rstd[t] (acc - mean[t] colsum[n]) + bias[n]
constexpr int GEMM_EPI_BIAS = 1;   // y = acc + bias[n] (+ res[t, n])
struct GemmArgs {
    const void *a, *w;
    void *y;
    int M, N, K;                         // K a multiple of 64, N of 8
    const float *mean, *rstd, *colsum;   // LN epilogue
    const float *bias;                   // [N] or NULL
    const void *res;                     // [M, N] or NULL (bias epilogue)
};
hipError_t launch_ln_stats(const void *x, float *mean, float *rstd, int T, int C, float eps, bool bf16,
                           hipStream_t stream);
hipError_t launch_ln_fold(const float *gamma, const float *beta, const void *w, const float *bias, void *w_folded,
                          float *bias_folded, float *colsum, int N, int C, bool bf16, hipStream_t stream);
long long gemm_grid_size(int M, int N);
hipError_t launch_gemm(const GemmArgs &g, int epi, bool bf16, hipStream_t stream);

// Decode: pages per split-KV chunk that the workspace is sized for (the
// kernels use chunks of 8, 16 or 32 pages, never more partials than 8-page
// chunks give), and the launch.
constexpr int kDecodeChunkPages = 8;
inline int decode_max_chunks(int max_pages) { return (max_pages + kDecodeChunkPages - 1) / kDecodeChunkPages; }
hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);

}  // namespace fa
