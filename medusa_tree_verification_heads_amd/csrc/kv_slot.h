// Cache slot addressing shared by the compaction kernels: slot s of sequence b is
// row b*capacity + s of a contiguous cache, or row page*page_size + s%page_size of
// the page pool when the cache is paged.  An out-of-range slot, page index or page
// yields -1.
#pragma once

#include "common.h"

struct KvSlots {
    void* k;
    void* v;
    const int32_t* table;
    int layout, capacity, page_size, max_pages, num_pages;
};

__device__ __forceinline__ long slot_row(const KvSlots& c, int b, int slot) {
    if (slot < 0 || slot >= c.capacity) return -1;
    if (c.layout == MDT_KV_CONTIG) return (long)b * c.capacity + slot;
    const int pg = slot / c.page_size;
    if (pg >= c.max_pages) return -1;
    const int page = c.table[(long)b * c.max_pages + pg];
    if (page < 0 || page >= c.num_pages) return -1;
    return (long)page * c.page_size + slot % c.page_size;
}

// Host-side checks of the compaction arguments (shared by mdt_kv_compact and
// mdt_accept_compact); fills *slots and *row_vec (16-byte vectors per row) on success.
mdt_status mdt_check_compact_args(mdt_dtype dt, int B, int T, int H, int Dh, int path_stride, const void* k_rot,
                                  const void* v, const mdt_kv_cache* cache, const int32_t* prefix_len,
                                  const int32_t* new_prefix_len, KvSlots* slots, int* row_vec);
