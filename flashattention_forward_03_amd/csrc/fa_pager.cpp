// Paged KV cache: host-side page allocator.
//
// The allocation policy of the paged cache (inference kernel cookbook page,
// recipe 03: fixed-size pages and a page table instead of one contiguous
// buffer per sequence, so memory is used in page-sized pieces; NanoInfer
// page, paged KV-cache allocator).  A sequence grows one page at a time
// from a free list and returns all its pages when it ends.  The free list
// is a stack: the most recently freed page is handed out first.
//
// The page table lives in host memory here ([max_seqs, max_pages_per_seq]
// int32, -1 where unused); the caller copies it to the device array the
// decode and append kernels read.
#include <cstdint>
#include <mutex>
#include <new>
#include <vector>

#include "fa.h"

struct fa_pager {
    int num_pages, max_seqs, max_pages;
    std::vector<int32_t> table;     // [max_seqs * max_pages]
    std::vector<int32_t> npages;    // pages held per sequence
    std::vector<int32_t> length;    // tokens reserved per sequence
    std::vector<int32_t> free_list; // stack of free page ids
    mutable std::mutex mu;
};

namespace {
constexpr int kPage = 16;
}

extern "C" {

fa_pager *fa_pager_create(int num_pages, int max_seqs, int max_pages_per_seq)
{
    if (num_pages < 1 || max_seqs < 1 || max_pages_per_seq < 1 ||
        (long long)max_seqs * max_pages_per_seq > (1LL << 31) - 1 ||
        (long long)max_pages_per_seq * kPage > (1LL << 31) - 1)
        return nullptr;
    fa_pager *p = new (std::nothrow) fa_pager;
    if (!p)
        return nullptr;
    try {
        p->num_pages = num_pages;
        p->max_seqs = max_seqs;
        p->max_pages = max_pages_per_seq;
        p->table.assign((size_t)max_seqs * max_pages_per_seq, -1);
        p->npages.assign(max_seqs, 0);
        p->length.assign(max_seqs, 0);
        p->free_list.resize(num_pages);
        // page 0 on top of the stack, so a fresh pager hands out 0, 1, 2, ...
        for (int i = 0; i < num_pages; ++i)
            p->free_list[i] = num_pages - 1 - i;
    } catch (...) {
        delete p;
        return nullptr;
    }
    return p;
}

void fa_pager_destroy(fa_pager *p) { delete p; }

int fa_pager_reserve(fa_pager *p, int seq, int len)
{
    if (!p)
        return FA_ERR_NULL;
    std::lock_guard<std::mutex> g(p->mu);
    if (seq < 0 || seq >= p->max_seqs || len < 0 || (long long)len > (long long)p->max_pages * kPage)
        return FA_ERR_SHAPE;
    const int need = (len + kPage - 1) / kPage;
    const int have = p->npages[seq];
    if (need > have) {
        if ((size_t)(need - have) > p->free_list.size())
            return FA_ERR_NOMEM;   // nothing changed
        int32_t *row = p->table.data() + (size_t)seq * p->max_pages;
        for (int i = have; i < need; ++i) {
            row[i] = p->free_list.back();
            p->free_list.pop_back();
        }
        p->npages[seq] = need;
    }
    if (len > p->length[seq])
        p->length[seq] = len;
    return FA_OK;
}

int fa_pager_release(fa_pager *p, int seq)
{
    if (!p)
        return FA_ERR_NULL;
    std::lock_guard<std::mutex> g(p->mu);
    if (seq < 0 || seq >= p->max_seqs)
        return FA_ERR_SHAPE;
    int32_t *row = p->table.data() + (size_t)seq * p->max_pages;
    for (int i = p->npages[seq] - 1; i >= 0; --i) {   // last page of the sequence ends on top
        p->free_list.push_back(row[i]);
        row[i] = -1;
    }
    p->npages[seq] = 0;
    p->length[seq] = 0;
    return FA_OK;
}

int fa_pager_length(const fa_pager *p, int seq)
{
    if (!p || seq < 0 || seq >= p->max_seqs)
        return -1;
    std::lock_guard<std::mutex> g(p->mu);
    return p->length[seq];
}

int fa_pager_free_pages(const fa_pager *p)
{
    if (!p)
        return -1;
    std::lock_guard<std::mutex> g(p->mu);
    return (int)p->free_list.size();
}

int fa_pager_copy_table(const fa_pager *p, int32_t *dst, size_t dst_entries)
{
    if (!p || !dst)
        return FA_ERR_NULL;
    std::lock_guard<std::mutex> g(p->mu);
    if (dst_entries < p->table.size())
        return FA_ERR_SHAPE;
    for (size_t i = 0; i < p->table.size(); ++i)
        dst[i] = p->table[i];
    return FA_OK;
}

}  // extern "C"
