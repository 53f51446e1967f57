// Paged KV cache: append kernel (device) for gfx950 (MI355X).
//
// The cache of the inference kernel cookbook page (recipe 02 "KV Cache":
// K and V of past tokens are stored once and reused by every decode step;
// recipe 03 "Paged Attention": fixed-size pages found through a page
// table).  Appending writes the K and V rows of new tokens -- a prefill
// chunk, or the one token of a decode step -- into their pages: token at
// logical position t of sequence s goes to page page_table[s][t / 16],
// row t % 16, of the [num_pages, H_kv, 16, d] pools.
//
// Pure data movement (bandwidth bound): one wave per new token moves its
// H_kv * d * 2 bytes of K and of V in 16-byte pieces, lanes over the
// (head, 8-dim piece) pairs, so each wave's reads are contiguous and its
// writes are contiguous 16 * d * 2-byte-strided runs of d * 2 bytes.
#include "fa_common.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int KV_PAGE = 16;
constexpr int KV_THREADS = 256;   // 4 waves = 4 tokens per workgroup

__global__ __launch_bounds__(KV_THREADS) void kv_append_kernel(
    const uint16_t *__restrict__ k_new, const uint16_t *__restrict__ v_new, const int32_t *__restrict__ seq_ids,
    const int32_t *__restrict__ positions, int T, uint16_t *__restrict__ k_pages, uint16_t *__restrict__ v_pages,
    const int32_t *__restrict__ page_table, int S, int Hkv, int d, int max_pages, int num_pages)
{
    const int tok = blockIdx.x * (KV_THREADS / 64) + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (tok >= T)
        return;
    const int s = seq_ids[tok];
    const int t = positions[tok];
    if (s < 0 || s >= S || t < 0 || t >= max_pages * KV_PAGE)
        return;   // out of contract: skipped
    const int page = page_table[(size_t)s * max_pages + t / KV_PAGE];
    if (page < 0 || page >= num_pages)
        return;
    const int row = t % KV_PAGE;
    const int per_head = d / 8;            // 16-byte pieces per head row
    const int pieces = Hkv * per_head;     // per token
    const size_t src = (size_t)tok * Hkv * d;
    const size_t page_base = (size_t)page * Hkv * KV_PAGE * d;
    for (int p = lane; p < pieces; p += 64) {
        const int h = p / per_head, c = p - h * per_head;
        const size_t dst = page_base + ((size_t)h * KV_PAGE + row) * d + 8 * c;
        *reinterpret_cast<u32x4_t *>(k_pages + dst) = load16(k_new + src + 8 * p);
        *reinterpret_cast<u32x4_t *>(v_pages + dst) = load16(v_new + src + 8 * p);
    }
}

}  // namespace

hipError_t launch_kv_append(const KvAppendArgs &a, hipStream_t stream)
{
    const int per_wg = KV_THREADS / 64;
    hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)((a.T + per_wg - 1) / per_wg)), dim3(KV_THREADS), 0, stream,
                       (const uint16_t *)a.k_new, (const uint16_t *)a.v_new, a.seq_ids, a.positions, a.T,
                       (uint16_t *)a.k_pages, (uint16_t *)a.v_pages, a.page_table, a.S, a.Hkv, a.d, a.max_pages,
                       a.num_pages);
    return hipGetLastError();
}

}  // namespace fa
