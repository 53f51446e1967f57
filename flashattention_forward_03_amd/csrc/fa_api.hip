// C-ABI layer: argument checks (all before any HIP call), workspace sizing,
// dispatch to the kernel launchers, HIP error capture.  See include/fa.h.
#include <climits>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <mutex>

#include "fa.h"
#include "fa_internal.h"

namespace {

thread_local int g_last_hip_error = 0;

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool log_enabled()
{
    static const bool on = [] {
        const char *e = std::getenv("FA_LOG");
        return e && e[0] == '1';
    }();
    return on;
}

int hip_fail(hipError_t e, const char *what)
{
    g_last_hip_error = (int)e;
    if (log_enabled())
        std::fprintf(stderr, "fa: %s failed: %s\n", what, hipGetErrorString(e));
    return FA_ERR_HIP;
}

bool scale_ok(float s) { return std::isfinite(s) && s > 0.f; }
bool eps_ok(float e) { return std::isfinite(e) && e >= 0.f; }

// Dense-layer GEMM sizes: M rows, K inputs (a multiple of 64, 16-byte
// copies of 64-element k-steps, 32-bit offsets over 256 rows), N outputs (a
// multiple of 8: 4-element stores and 16-byte bias reads).
int gemm_check(int M, int K, int N, int dtype)
{
    if (M < 0 || K < 0 || N < 0)
        return FA_ERR_SHAPE;
    if (K < 64 || K % 64 != 0 || N % 8 != 0)
        return FA_ERR_UNSUPPORTED;
    if (dtype != FA_DTYPE_F16 && dtype != FA_DTYPE_BF16)
        return FA_ERR_UNSUPPORTED;
    if ((long long)K * 512 >= (1LL << 31) || fa::gemm_grid_size(M, N) > INT_MAX)
        return FA_ERR_SHAPE;
    return FA_OK;
}

// Byte offsets of the block's stages in its workspace (256-byte aligned).
struct BlockLayout {
    size_t mean, rstd, qkv, o, lse, total;
};

bool block_layout(int B, int N, int H, int H_kv, int d, BlockLayout &L)
{
    if (B < 0 || N < 0 || H < 0 || d < 0 || (H > 0 && (H_kv < 1 || H % H_kv != 0)))
        return false;
    auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
    const size_t T = (size_t)B * N, C = (size_t)H * d, R = ((size_t)H + 2 * (size_t)H_kv) * d;
    L.mean = 0;
    L.rstd = L.mean + up(T * 4);
    L.qkv = L.rstd + up(T * 4);
    L.o = L.qkv + up(T * R * 2);
    L.lse = L.o + up(T * C * 2);
    L.total = L.lse + up((size_t)B * H * N * 4);
    return true;
}

size_t decode_ws_bytes(long long S, long long H, long long d, int max_pages)
{
    const long long chunks = fa::decode_max_chunks(max_pages);
    if (chunks <= 1)
        return 0;
    return (size_t)(S * H * chunks * d * 4 + S * H * chunks * 2 * 4);
}

}  // namespace

extern "C" {

int fa_version(void) { return 1; }

const char *fa_status_str(int status)
{
    switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "invalid size (negative, or too large to index)";
    case FA_ERR_UNSUPPORTED: return "unsupported head dim, page size or dtype";
    case FA_ERR_ALIGN: return "pointer not aligned as required";
    case FA_ERR_WORKSPACE: return "workspace missing or too small";
    case FA_ERR_SCRATCH: return "problem needs more scratch than the no-allocation entry point's fixed buffer";
    case FA_ERR_HIP: return "HIP launch failed";
    case FA_ERR_ARG: return "invalid argument (scale must be finite and > 0; causal 0 or 1; eps finite and >= 0)";
    case FA_ERR_NOMEM: return "not enough free pages";
    default: return "unknown status";
    }
}

int fa_last_hip_error(void) { return g_last_hip_error; }

int fa_fwd_ex(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H, int H_kv, int Nq,
              int Nk, int d, const int64_t *q_strides, const int64_t *k_strides, const int64_t *v_strides,
              const int64_t *o_strides, float scale, int causal, const int32_t *kv_lens, int dtype, int o_dtype,
              void *stream)
{
    if (B < 0 || H < 0 || Nq < 0 || Nk < 0)
        return FA_ERR_SHAPE;
    if (H > 0 && (H_kv < 1 || H % H_kv != 0))
        return FA_ERR_SHAPE;
    if (d < 8 || d > 128 || d % 8 != 0)
        return FA_ERR_UNSUPPORTED;
    if (dtype != FA_DTYPE_F16 && dtype != FA_DTYPE_BF16)
        return FA_ERR_UNSUPPORTED;
    if (o_dtype != FA_DTYPE_F16 && o_dtype != FA_DTYPE_BF16 && o_dtype != FA_DTYPE_F32)
        return FA_ERR_UNSUPPORTED;
    if (causal != 0 && causal != 1)
        return FA_ERR_ARG;
    if (!scale_ok(scale))
        return FA_ERR_ARG;
    // strides: NULL = contiguous [B, heads, rows, d]
    fa::FwdLayout lay{};
    const int64_t *given[4] = {q_strides, k_strides, v_strides, o_strides};
    long long *dst[4] = {lay.qs, lay.ks, lay.vs, lay.os};
    const long long heads[4] = {H, H_kv, H_kv, H}, rows[4] = {Nq, Nk, Nk, Nq};
    for (int i = 0; i < 4; ++i) {
        for (int j = 0; j < 3; ++j) {
            const long long def = j == 0 ? heads[i] * rows[i] * d : (j == 1 ? rows[i] * d : d);
            dst[i][j] = given[i] ? given[i][j] : def;
            if (dst[i][j] < 0)
                return FA_ERR_SHAPE;
        }
        if (dst[i][2] < d)   // rows must not overlap
            return FA_ERR_SHAPE;
    }
    lay.d = d;
    lay.o_kind = o_dtype == FA_DTYPE_F32 ? fa::FA_O_F32 : (o_dtype == FA_DTYPE_BF16 ? fa::FA_O_BF16 : fa::FA_O_F16);
    if (B == 0 || H == 0 || Nq == 0)
        return FA_OK;
    if (fa::fwd_grid_size(B, H, Nq) > INT_MAX)
        return FA_ERR_SHAPE;
    // the keys of one (b, K/V head) are addressed with 32-bit byte offsets
    if (((long long)Nk + 64) * lay.ks[2] * 2 > INT_MAX || ((long long)Nk + 64) * lay.vs[2] * 2 > INT_MAX)
        return FA_ERR_SHAPE;
    if (!q || !o || !lse || (Nk > 0 && (!k || !v)))
        return FA_ERR_NULL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4) ||
        !aligned(kv_lens, 4))
        return FA_ERR_ALIGN;
    // 16-byte Q / K / V row pieces; 4-element O stores (16 or 8 bytes)
    for (int j = 0; j < 3; ++j)
        if (lay.qs[j] % 8 || lay.ks[j] % 8 || lay.vs[j] % 8 || lay.os[j] % 4)
            return FA_ERR_ALIGN;

    fa::FwdArgs a{q, k, v, o, lse, B, H, H_kv, Nq, Nk, scale, causal == 1, dtype == FA_DTYPE_BF16, kv_lens, lay};
    const hipError_t e = fa::launch_fwd(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return hip_fail(e, "fa_fwd launch");
    return FA_OK;
}

int fa_fwd_gqa(const void *q, const void *k, const void *v, float *o, float *lse, int B, int H, int H_kv,
               int Nq, int Nk, int d, float scale, int causal, const int32_t *kv_lens, int dtype, void *stream)
{
    return fa_fwd_ex(q, k, v, o, lse, B, H, H_kv, Nq, Nk, d, nullptr, nullptr, nullptr, nullptr, scale, causal,
                     kv_lens, dtype, FA_DTYPE_F32, stream);
}

int fa_fwd(const void *q, const void *k, const void *v, float *o, float *lse, int B, int H, int Nq,
           int Nk, int d, float scale, int causal, const int32_t *kv_lens, int dtype, void *stream)
{
    return fa_fwd_gqa(q, k, v, o, lse, B, H, H, Nq, Nk, d, scale, causal, kv_lens, dtype, stream);
}

int fa_bwd(const void *q, const void *k, const void *v, const float *o, const void *dout, const float *lse,
           float *dq, float *dk, float *dv, float *delta, int B, int H, int H_kv, int Nq, int Nk, int d,
           float scale, int causal, const int32_t *kv_lens, int dtype, void *stream)
{
    if (B < 0 || H < 0 || Nq < 0 || Nk < 0)
        return FA_ERR_SHAPE;
    if (H > 0 && (H_kv < 1 || H % H_kv != 0))
        return FA_ERR_SHAPE;
    if (d < 8 || d > 128 || d % 8 != 0)
        return FA_ERR_UNSUPPORTED;
    if (dtype != FA_DTYPE_F16 && dtype != FA_DTYPE_BF16)
        return FA_ERR_UNSUPPORTED;
    if (causal != 0 && causal != 1)
        return FA_ERR_ARG;
    if (!scale_ok(scale))
        return FA_ERR_ARG;
    if (B == 0 || H == 0 || (Nq == 0 && Nk == 0))
        return FA_OK;
    if (fa::bwd_grid_size(B, H, Nq, Nk) > INT_MAX)
        return FA_ERR_SHAPE;
    // rows of one (b, head) are addressed with 32-bit byte offsets
    if (((long long)(Nq > Nk ? Nq : Nk) + 64) * d * 2 > INT_MAX)
        return FA_ERR_SHAPE;
    if ((Nq > 0 && (!q || !o || !dout || !lse || !dq || !delta)) || (Nk > 0 && (!k || !v || !dk || !dv)))
        return FA_ERR_NULL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(dout, 16) ||
        !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(lse, 4) || !aligned(delta, 4) ||
        !aligned(kv_lens, 4))
        return FA_ERR_ALIGN;
    fa::BwdArgs a{q, k, v, dout, o, lse, dq, dk, dv, delta, B, H, H_kv, Nq, Nk, d, scale, causal == 1,
                  dtype == FA_DTYPE_BF16, kv_lens};
    const hipError_t e = fa::launch_bwd(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return hip_fail(e, "fa_bwd launch");
    return FA_OK;
}

int fa_kv_append(const void *k_new, const void *v_new, const int32_t *seq_ids, const int32_t *positions, int T,
                 void *k_pages, void *v_pages, const int32_t *page_table, int S, int H_kv, int d, int page_size,
                 int max_pages_per_seq, int num_pages, int dtype, void *stream)
{
    if (T < 0 || S < 0 || H_kv < 1 || max_pages_per_seq < 1 || num_pages < 1)
        return FA_ERR_SHAPE;
    if (d < 8 || d > 256 || d % 8 != 0 || page_size != 16)
        return FA_ERR_UNSUPPORTED;
    if (dtype != FA_DTYPE_F16 && dtype != FA_DTYPE_BF16)
        return FA_ERR_UNSUPPORTED;
    if ((long long)max_pages_per_seq * page_size > INT_MAX || (long long)S * max_pages_per_seq > INT_MAX)
        return FA_ERR_SHAPE;
    if (T == 0 || S == 0)
        return FA_OK;
    if (!k_new || !v_new || !seq_ids || !positions || !k_pages || !v_pages || !page_table)
        return FA_ERR_NULL;
    if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_pages, 16) || !aligned(v_pages, 16) ||
        !aligned(seq_ids, 4) || !aligned(positions, 4) || !aligned(page_table, 4))
        return FA_ERR_ALIGN;
    fa::KvAppendArgs a{k_new, v_new, seq_ids, positions, T, k_pages, v_pages, page_table, S, H_kv, d,
                       max_pages_per_seq, num_pages};
    const hipError_t e = fa::launch_kv_append(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return hip_fail(e, "fa_kv_append launch");
    return FA_OK;
}

size_t fa_decode_workspace_bytes(int S, int H, int d, int max_pages_per_seq, int page_size)
{
    if (S < 0 || H < 0 || (d != 64 && d != 128) || max_pages_per_seq < 1 || page_size != 16)
        return 0;
    return decode_ws_bytes(S, H, d, max_pages_per_seq);
}

}  // extern "C"

namespace {

// Fixed device scratch of the no-allocation decode entry point: the split-KV
// partials live here instead of in a caller workspace.  Every GPU the library
// runs on holds one copy until the process ends.  Host code never names the
// array directly (in host code the name is a stand-in, not a device address):
// it uses the address that hipGetSymbolAddress returned for the current
// device.
constexpr size_t kNoAllocScratchBytes = (size_t)40 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];   // device address of `scratch`, per device (set once)

// The scratch address on the current device: looked up on the first call
// per device (with that device current), cached afterwards.
hipError_t scratch_on_current_device(void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        if (!p)
            return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

// Paged decode behind fa_decode_paged{,_gqa,_noalloc}: argument checks, then
// the split-KV partials in the caller's workspace or (use_scratch) in the
// library's fixed device scratch.
int decode_impl(const void *q, const void *k_pages, const void *v_pages, const int32_t *page_table,
                const int32_t *kv_lens, float *o, float *lse, int S, int H, int H_kv, int d, int page_size,
                int max_pages_per_seq, int num_pages, float scale, int dtype, void *workspace,
                size_t workspace_bytes, bool use_scratch, void *stream)
{
    if (S < 0 || H < 0 || max_pages_per_seq < 1 || num_pages < 1)
        return FA_ERR_SHAPE;
    if (H > 0 && (H_kv < 1 || H % H_kv != 0))
        return FA_ERR_SHAPE;
    if (d != 64 && d != 128)
        return FA_ERR_UNSUPPORTED;
    if (page_size != 16)
        return FA_ERR_UNSUPPORTED;
    if (dtype != FA_DTYPE_F16 && dtype != FA_DTYPE_BF16)
        return FA_ERR_UNSUPPORTED;
    if (!scale_ok(scale))
        return FA_ERR_ARG;
    if ((long long)max_pages_per_seq * page_size > INT_MAX)
        return FA_ERR_SHAPE;
    if (S == 0 || H == 0)
        return FA_OK;
    if ((long long)S * H * fa::decode_max_chunks(max_pages_per_seq) > INT_MAX)
        return FA_ERR_SHAPE;
    if (!q || !k_pages || !v_pages || !page_table || !kv_lens || !o || !lse)
        return FA_ERR_NULL;
    if (!aligned(q, 16) || !aligned(k_pages, 16) || !aligned(v_pages, 16) || !aligned(o, 16) ||
        !aligned(page_table, 4) || !aligned(kv_lens, 4) || !aligned(lse, 4))
        return FA_ERR_ALIGN;
    const size_t need = decode_ws_bytes(S, H, d, max_pages_per_seq);
    if (use_scratch) {
        if (need > kNoAllocScratchBytes)
            return FA_ERR_SCRATCH;
    } else if (need > 0) {
        if (!workspace || workspace_bytes < need)
            return FA_ERR_WORKSPACE;
        if (!aligned(workspace, 16))
            return FA_ERR_ALIGN;
    }
    if (use_scratch && need > 0) {
        const hipError_t e = scratch_on_current_device(&workspace);
        if (e != hipSuccess)
            return hip_fail(e, "fa_decode_paged_noalloc scratch lookup");
    }
    const long long chunks = fa::decode_max_chunks(max_pages_per_seq);
    float *part_o = need ? static_cast<float *>(workspace) : nullptr;
    float *part_ml = need ? part_o + (size_t)S * H * chunks * d : nullptr;

    fa::DecodeArgs a{q, k_pages, v_pages, page_table, kv_lens, o, lse, S, H, H_kv, d, page_size,
                     max_pages_per_seq, num_pages, scale, dtype == FA_DTYPE_BF16, part_o, part_ml};
    const hipError_t e = fa::launch_decode(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return hip_fail(e, "fa_decode_paged launch");
    return FA_OK;
}

}  // namespace

extern "C" {

int fa_decode_paged_gqa(const void *q, const void *k_pages, const void *v_pages, const int32_t *page_table,
                        const int32_t *kv_lens, float *o, float *lse, int S, int H, int H_kv, int d, int page_size,
                        int max_pages_per_seq, int num_pages, float scale, int dtype, void *workspace,
                        size_t workspace_bytes, void *stream)
{
    return decode_impl(q, k_pages, v_pages, page_table, kv_lens, o, lse, S, H, H_kv, d, page_size,
                       max_pages_per_seq, num_pages, scale, dtype, workspace, workspace_bytes, false, stream);
}

int fa_decode_paged(const void *q, const void *k_pages, const void *v_pages, const int32_t *page_table,
                    const int32_t *kv_lens, float *o, float *lse, int S, int H, int d, int page_size,
                    int max_pages_per_seq, int num_pages, float scale, int dtype, void *workspace,
                    size_t workspace_bytes, void *stream)
{
    return fa_decode_paged_gqa(q, k_pages, v_pages, page_table, kv_lens, o, lse, S, H, H, d, page_size,
                               max_pages_per_seq, num_pages, scale, dtype, workspace, workspace_bytes, stream);
}

int fa_decode_paged_noalloc(const void *q, const void *k_pages, const void *v_pages, const int32_t *page_table,
                            const int32_t *kv_lens, float *o, float *lse, int S, int H, int H_kv, int d,
                            int page_size, int max_pages_per_seq, int num_pages, float scale, int dtype,
                            void *stream)
{
    return decode_impl(q, k_pages, v_pages, page_table, kv_lens, o, lse, S, H, H_kv, d, page_size,
                       max_pages_per_seq, num_pages, scale, dtype, nullptr, 0, true, stream);
}

// ------------------------------------------------------ pre-LN block ---

int fa_ln_stats(const void *x, float *mean, float *rstd, int T, int C, float eps, int dtype, void *stream)
{
    if (T < 0 || C < 0)
        return FA_ERR_SHAPE;
    if (C < 8 || C % 8 != 0)
        return FA_ERR_UNSUPPORTED;
    if (dtype != FA_DTYPE_F16 && dtype != FA_DTYPE_BF16)
        return FA_ERR_UNSUPPORTED;
    if (!eps_ok(eps))
        return FA_ERR_ARG;
    if (T == 0)
        return FA_OK;
    if (!x || !mean || !rstd)
        return FA_ERR_NULL;
    if (!aligned(x, 16) || !aligned(mean, 16) || !aligned(rstd, 16))
        return FA_ERR_ALIGN;
    const hipError_t e =
        fa::launch_ln_stats(x, mean, rstd, T, C, eps, dtype == FA_DTYPE_BF16, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return hip_fail(e, "fa_ln_stats launch");
    return FA_OK;
}

int fa_ln_fold_weights(const float *gamma, const float *beta, const void *w, const float *bias, void *w_folded,
                       float *bias_folded, float *colsum, int N, int C, int dtype, void *stream)
{
    if (N < 0 || C < 0)
        return FA_ERR_SHAPE;
    if (C < 8 || C % 8 != 0)
        return FA_ERR_UNSUPPORTED;
    if (dtype != FA_DTYPE_F16 && dtype != FA_DTYPE_BF16)
        return FA_ERR_UNSUPPORTED;
    if (N == 0)
        return FA_OK;
    if (!gamma || !beta || !w || !w_folded || !bias_folded || !colsum)
        return FA_ERR_NULL;
    if (!aligned(gamma, 16) || !aligned(beta, 16) || !aligned(w, 16) || !aligned(bias, 16) ||
        !aligned(w_folded, 16) || !aligned(bias_folded, 16) || !aligned(colsum, 16))
        return FA_ERR_ALIGN;
    const hipError_t e = fa::launch_ln_fold(gamma, beta, w, bias, w_folded, bias_folded, colsum, N, C,
                                            dtype == FA_DTYPE_BF16, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return hip_fail(e, "fa_ln_fold_weights launch");
    return FA_OK;
}

int fa_ln_linear(const void *x, const float *mean, const float *rstd, const void *w_folded, const float *bias_folded,
                 const float *colsum, void *y, int T, int C, int N, int dtype, void *stream)
{
    const int st = gemm_check(T, C, N, dtype);
    if (st != FA_OK || T == 0 || N == 0)
        return st;
    if (!x || !mean || !rstd || !w_folded || !bias_folded || !colsum || !y)
        return FA_ERR_NULL;
    if (!aligned(x, 16) || !aligned(mean, 16) || !aligned(rstd, 16) || !aligned(w_folded, 16) ||
        !aligned(bias_folded, 16) || !aligned(colsum, 16) || !aligned(y, 16))
        return FA_ERR_ALIGN;
    const fa::GemmArgs g{x, w_folded, y, T, N, C, mean, rstd, colsum, bias_folded, nullptr};
    const hipError_t e =
        fa::launch_gemm(g, fa::GEMM_EPI_LN, dtype == FA_DTYPE_BF16, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return hip_fail(e, "fa_ln_linear launch");
    return FA_OK;
}

int fa_linear(const void *a, const void *w, const float *bias, const void *residual, void *y, int M, int K, int N,
              int dtype, void *stream)
{
    const int st = gemm_check(M, K, N, dtype);
    if (st != FA_OK || M == 0 || N == 0)
        return st;
    if (!a || !w || !y)
        return FA_ERR_NULL;
    if (!aligned(a, 16) || !aligned(w, 16) || !aligned(bias, 16) || !aligned(residual, 16) || !aligned(y, 16))
        return FA_ERR_ALIGN;
    const fa::GemmArgs g{a, w, y, M, N, K, nullptr, nullptr, nullptr, bias, residual};
    const hipError_t e =
        fa::launch_gemm(g, fa::GEMM_EPI_BIAS, dtype == FA_DTYPE_BF16, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return hip_fail(e, "fa_linear launch");
    return FA_OK;
}

size_t fa_prenorm_attention_workspace_bytes(int B, int N, int H, int H_kv, int d)
{
    BlockLayout L;
    if (!block_layout(B, N, H, H_kv, d, L))
        return 0;
    return L.total;
}

int fa_prenorm_attention(const void *x, const void *w_qkv_folded, const float *b_qkv_folded, const float *colsum_qkv,
                         const void *w_o, const float *b_o, void *y, int B, int N, int H, int H_kv, int d,
                         float eps, float scale, int causal, const int32_t *kv_lens, int dtype, void *workspace,
                         size_t workspace_bytes, void *stream)
{
    if (B < 0 || N < 0 || H < 0)
        return FA_ERR_SHAPE;
    if (H > 0 && (H_kv < 1 || H % H_kv != 0))
        return FA_ERR_SHAPE;
    if (d < 8 || d > 128 || d % 8 != 0)
        return FA_ERR_UNSUPPORTED;
    const long long C = (long long)H * d, R = (long long)(H + 2 * (long long)H_kv) * d, T = (long long)B * N;
    if (H > 0 && C % 64 != 0)
        return FA_ERR_UNSUPPORTED;
    if (dtype != FA_DTYPE_F16 && dtype != FA_DTYPE_BF16)
        return FA_ERR_UNSUPPORTED;
    if (!eps_ok(eps) || !scale_ok(scale) || (causal != 0 && causal != 1))
        return FA_ERR_ARG;
    if (T == 0 || H == 0)
        return FA_OK;
    // every stage's limits, before anything is launched
    if (T > INT_MAX || C * 512 >= (1LL << 31) || R > INT_MAX || fa::gemm_grid_size((int)T, (int)R) > INT_MAX ||
        fa::fwd_grid_size(B, H, N) > INT_MAX || ((long long)N + 64) * R * 2 > INT_MAX)
        return FA_ERR_SHAPE;
    BlockLayout L;
    if (!block_layout(B, N, H, H_kv, d, L))
        return FA_ERR_SHAPE;
    if (!workspace || workspace_bytes < L.total)
        return FA_ERR_WORKSPACE;
    if (!x || !w_qkv_folded || !b_qkv_folded || !colsum_qkv || !w_o || !y)
        return FA_ERR_NULL;
    if (!aligned(workspace, 256))
        return FA_ERR_ALIGN;
    if (!aligned(x, 16) || !aligned(w_qkv_folded, 16) || !aligned(b_qkv_folded, 16) || !aligned(colsum_qkv, 16) ||
        !aligned(w_o, 16) || !aligned(b_o, 16) || !aligned(y, 16) || !aligned(kv_lens, 4))
        return FA_ERR_ALIGN;

    unsigned char *ws = static_cast<unsigned char *>(workspace);
    float *mean = reinterpret_cast<float *>(ws + L.mean);
    float *rstd = reinterpret_cast<float *>(ws + L.rstd);
    uint16_t *qkv = reinterpret_cast<uint16_t *>(ws + L.qkv);
    uint16_t *o = reinterpret_cast<uint16_t *>(ws + L.o);
    float *lse = reinterpret_cast<float *>(ws + L.lse);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const bool bf16 = dtype == FA_DTYPE_BF16;

    hipError_t e = fa::launch_ln_stats(x, mean, rstd, (int)T, (int)C, eps, bf16, s);
    if (e != hipSuccess)
        return hip_fail(e, "fa_prenorm_attention stats launch");
    const fa::GemmArgs gq{x, w_qkv_folded, qkv, (int)T, (int)R, (int)C, mean, rstd, colsum_qkv, b_qkv_folded, nullptr};
    e = fa::launch_gemm(gq, fa::GEMM_EPI_LN, bf16, s);
    if (e != hipSuccess)
        return hip_fail(e, "fa_prenorm_attention qkv launch");
    // q, k, v are column ranges of the qkv rows: [b, n, head, d]
    const int64_t qs[3] = {(int64_t)N * R, d, R};
    const int64_t os[3] = {(int64_t)N * C, d, C};
    const int st = fa_fwd_ex(qkv, qkv + (size_t)H * d, qkv + (size_t)(H + H_kv) * d, o, lse, B, H, H_kv, N, N, d, qs,
                             qs, qs, os, scale, causal, kv_lens, dtype, dtype, stream);
    if (st != FA_OK)
        return st;
    const fa::GemmArgs go{o, w_o, y, (int)T, (int)C, (int)C, nullptr, nullptr, nullptr, b_o, x};
    e = fa::launch_gemm(go, fa::GEMM_EPI_BIAS, bf16, s);
    if (e != hipSuccess)
        return hip_fail(e, "fa_prenorm_attention output launch");
    return FA_OK;
}

}  // extern "C"
