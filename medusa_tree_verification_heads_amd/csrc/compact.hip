// mdt_kv_compact: append the accepted path's keys/values after the prefix.
//
// "MEDUSA 精读", section 3 (after selecting the accepted path, the KV cache keeps
// only that path) and section 6 (implementation checklist: compact the KV cache).
// The key rows come from k_rot, already rotated at prefix_len + depth; node
// path[j] has depth j, so slot prefix_len + j gets exactly the position it was
// rotated for.
//
// Grid (B, path_stride, layers): workgroup (b, j, l) copies one row of H*Dh keys and
// values of layer l with 16-byte vector moves.  Every workgroup of a sequence first validates the
// whole sequence (path nodes, length, destination slots, pages), so either the
// full path is written or nothing of it.
//
// mdt_next_state: the node output of a sequence's deepest accepted node becomes the
// hidden state the next step starts from (summary page, section 3.2: the next
// iteration continues from the last accepted token).  One workgroup per sequence
// copies that row with 16-byte moves.  mdt_next_logits copies the same node's verifier
// logits row into the next step's LM-head slot (that row is the LM head applied to the
// next hidden state), spread over many workgroups.
#include "kv_slot.h"

namespace {

// blockIdx.z is the layer: layer l reads k_rot + l*k_stride, v + l*v_stride and writes
// the cache rows at an offset of l*c_stride (all in 16-byte vectors).
__global__ __launch_bounds__(256) void compact_kernel(KvSlots cache, const int32_t* __restrict__ path, int path_stride,
                                                      const int32_t* __restrict__ n_acc, const uint4* __restrict__ k_rot,
                                                      const uint4* __restrict__ v, int T, int row_vec,
                                                      const int32_t* __restrict__ prefix_len,
                                                      int32_t* __restrict__ new_len, long k_stride, long v_stride,
                                                      long c_stride) {
    const int b = blockIdx.x, j = blockIdx.y, l = blockIdx.z;
    const int n = n_acc[b];
    const int L = prefix_len[b];
    bool ok = n >= 1 && n <= path_stride && L >= 0;
    for (int q = 0; q < path_stride && ok; ++q) {
        if (q >= n) break;
        const int node = path[(long)b * path_stride + q];
        ok = node >= 0 && node < T && slot_row(cache, b, L + q) >= 0;
    }
    if (j == 0 && l == 0 && threadIdx.x == 0) new_len[b] = ok ? L + n : -1;
    if (!ok || j >= n) return;
    const int node = path[(long)b * path_stride + j];
    const long dst = slot_row(cache, b, L + j) * row_vec;
    const long src = ((long)b * T + node) * row_vec;
    uint4* K = (uint4*)cache.k + l * c_stride;
    uint4* Vv = (uint4*)cache.v + l * c_stride;
    k_rot += l * k_stride;
    v += l * v_stride;
    for (int e = threadIdx.x; e < row_vec; e += blockDim.x) {
        K[dst + e] = k_rot[src + e];
        Vv[dst + e] = v[src + e];
    }
}

__global__ __launch_bounds__(256) void next_state_kernel(const uint4* __restrict__ x, const int32_t* __restrict__ path,
                                                           int path_stride, const int32_t* __restrict__ n_acc, int T,
                                                           int row_vec, uint4* __restrict__ h_next) {
    const int b = blockIdx.x;
    const int n = n_acc[b];
    const int node = path[(long)b * path_stride + min(max(n - 1, 0), path_stride - 1)];
    const bool ok = n >= 1 && n <= path_stride && node >= 0 && node < T;
    const long src = ((long)b * T + (ok ? node : 0)) * row_vec;
    uint4* dst = h_next + (long)b * row_vec;
    for (int e = threadIdx.x; e < row_vec; e += blockDim.x) dst[e] = ok ? x[src + e] : make_uint4(0, 0, 0, 0);
}

// grid (ceil(V / kNextLogitsPerWg), B): each thread moves four elements, all four loads
// issued before the stores.
constexpr int kNextLogitsPerWg = 4 * 256;

__global__ __launch_bounds__(256) void next_logits_kernel(const float* __restrict__ z, const int32_t* __restrict__ path,
                                                            int path_stride, const int32_t* __restrict__ n_acc, int T,
                                                            int V, long out_stride, float* __restrict__ out) {
    const int b = blockIdx.y;
    const int n = n_acc[b];
    const int node = path[(long)b * path_stride + min(max(n - 1, 0), path_stride - 1)];
    const bool ok = n >= 1 && n <= path_stride && node >= 0 && node < T;
    const float* src = z + ((long)b * T + (ok ? node : 0)) * V;
    float* dst = out + (long)b * out_stride;
    const int e0 = blockIdx.x * kNextLogitsPerWg + threadIdx.x;
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = ok && e0 + 256 * j < V ? src[e0 + 256 * j] : 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        if (e0 + 256 * j < V) dst[e0 + 256 * j] = v[j];
}

}  // namespace

mdt_status mdt_check_compact_args(mdt_dtype dt, int B, int T, int H, int Dh, int path_stride, const void* k_rot,
                                  const void* v, const mdt_kv_cache* cache, const int32_t* prefix_len,
                                  const int32_t* new_prefix_len, KvSlots* slots, int* row_vec) {
    MDT_REQUIRE(dt == MDT_F32 || dt == MDT_BF16, MDT_ERR_DTYPE, "dtype %d not supported", (int)dt);
    MDT_REQUIRE(B >= 1 && B <= 65535 && T >= 1 && T <= MDT_MAX_NODES && H >= 1 && Dh >= 1, MDT_ERR_SHAPE,
                "bad shape B=%d T=%d H=%d Dh=%d", B, T, H, Dh);
    MDT_REQUIRE(path_stride >= 1 && path_stride <= MDT_MAX_NODES, MDT_ERR_SHAPE, "path_stride out of range");
    const size_t row_bytes = (size_t)H * Dh * (dt == MDT_BF16 ? 2 : 4);
    MDT_REQUIRE(row_bytes % 16 == 0, MDT_ERR_SHAPE, "H*Dh*element size must be a multiple of 16 bytes");
    MDT_REQUIRE(cache, MDT_ERR_NULL, "cache is NULL");
    MDT_REQUIRE(k_rot && v && prefix_len && new_prefix_len && cache->k && cache->v, MDT_ERR_NULL,
                "a tensor pointer is NULL");
    MDT_REQUIRE(mdt_aligned16(k_rot) && mdt_aligned16(v) && mdt_aligned16(cache->k) && mdt_aligned16(cache->v),
                MDT_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
    if (cache->layout == MDT_KV_PAGED) {
        MDT_REQUIRE(cache->page_table, MDT_ERR_NULL, "page_table is NULL");
        MDT_REQUIRE(cache->page_size >= 1 && cache->max_pages >= 1 && cache->num_pages >= 1 &&
                        (long)cache->max_pages * cache->page_size == cache->capacity,
                    MDT_ERR_SHAPE, "bad paged-cache geometry");
    } else {
        MDT_REQUIRE(cache->layout == MDT_KV_CONTIG, MDT_ERR_VALUE, "unknown cache layout %d", cache->layout);
        MDT_REQUIRE(cache->capacity >= 0, MDT_ERR_SHAPE, "capacity must be >= 0");
    }
    *slots = KvSlots{cache->k, cache->v, cache->page_table, cache->layout, cache->capacity, cache->page_size,
                     cache->max_pages, cache->num_pages};
    *row_vec = (int)(row_bytes / 16);
    return MDT_OK;
}

extern "C" mdt_status mdt_kv_compact(void* stream, mdt_dtype dt, int B, int T, int H, int Dh, const int32_t* path,
                                     int path_stride, const int32_t* n_acc, const void* k_rot, const void* v,
                                     const mdt_kv_cache* cache, const int32_t* prefix_len,
                                     int32_t* new_prefix_len) {
    KvSlots c;
    int row_vec = 0;
    mdt_status st = mdt_check_compact_args(dt, B, T, H, Dh, path_stride, k_rot, v, cache, prefix_len,
                                           new_prefix_len, &c, &row_vec);
    if (st != MDT_OK) return st;
    MDT_REQUIRE(path && n_acc, MDT_ERR_NULL, "a tensor pointer is NULL");
    MDT_LAUNCH("compact_kernel", compact_kernel, dim3(B, path_stride), dim3(256), 0, (hipStream_t)stream, c, path,
               path_stride, n_acc, (const uint4*)k_rot, (const uint4*)v, T, row_vec, prefix_len, new_prefix_len, 0L,
               0L, 0L);
    return mdt_launched("compact_kernel");
}

extern "C" mdt_status mdt_kv_compact_layers(void* stream, mdt_dtype dt, int n_layers, int B, int T, int H, int Dh,
                                            const int32_t* path, int path_stride, const int32_t* n_acc,
                                            const void* k_rot, long long k_rot_layer_stride, const void* v,
                                            long long v_layer_stride, const mdt_kv_cache* cache,
                                            long long cache_layer_stride, const int32_t* prefix_len,
                                            int32_t* new_prefix_len) {
    KvSlots c;
    int row_vec = 0;
    mdt_status st = mdt_check_compact_args(dt, B, T, H, Dh, path_stride, k_rot, v, cache, prefix_len,
                                           new_prefix_len, &c, &row_vec);
    if (st != MDT_OK) return st;
    MDT_REQUIRE(path && n_acc, MDT_ERR_NULL, "a tensor pointer is NULL");
    MDT_REQUIRE(n_layers >= 1 && n_layers <= 65535, MDT_ERR_SHAPE, "n_layers=%d out of range 1..65535", n_layers);
    const long long elt = dt == MDT_BF16 ? 2 : 4;
    const long long rows_in = (long long)B * T * row_vec * 16 / elt;  // elements of one layer's k_rot / v
    const long long rows_c = cache->layout == MDT_KV_PAGED ? (long long)cache->num_pages * cache->page_size
                                                           : (long long)B * cache->capacity;
    MDT_REQUIRE(k_rot_layer_stride >= 0 && v_layer_stride >= 0 && cache_layer_stride >= 0 &&
                    (k_rot_layer_stride * elt) % 16 == 0 && (v_layer_stride * elt) % 16 == 0 &&
                    (cache_layer_stride * elt) % 16 == 0,
                MDT_ERR_ALIGN, "layer strides must be non-negative multiples of 16 bytes");
    MDT_REQUIRE(n_layers == 1 || (k_rot_layer_stride >= rows_in && v_layer_stride >= rows_in &&
                                  cache_layer_stride >= rows_c * row_vec * 16 / elt),
                MDT_ERR_SHAPE, "layer strides smaller than one layer");
    MDT_LAUNCH("compact_kernel", compact_kernel, dim3(B, path_stride, n_layers), dim3(256), 0, (hipStream_t)stream, c,
               path, path_stride, n_acc, (const uint4*)k_rot, (const uint4*)v, T, row_vec, prefix_len,
               new_prefix_len, (long)(k_rot_layer_stride * elt / 16), (long)(v_layer_stride * elt / 16),
               (long)(cache_layer_stride * elt / 16));
    return mdt_launched("compact_kernel");
}

extern "C" mdt_status mdt_next_state(void* stream, mdt_dtype dt, int B, int T, int d, const void* x,
                                     const int32_t* path, int path_stride, const int32_t* n_acc, void* h_next) {
    MDT_REQUIRE(dt == MDT_F32 || dt == MDT_BF16, MDT_ERR_DTYPE, "dtype %d not supported", (int)dt);
    MDT_REQUIRE(B >= 1 && B <= 65535 && T >= 1 && T <= MDT_MAX_NODES && d >= 1, MDT_ERR_SHAPE,
                "bad shape B=%d T=%d d=%d", B, T, d);
    MDT_REQUIRE(path_stride >= 1 && path_stride <= MDT_MAX_NODES, MDT_ERR_SHAPE, "path_stride out of range");
    const size_t row_bytes = (size_t)d * (dt == MDT_BF16 ? 2 : 4);
    MDT_REQUIRE(row_bytes % 16 == 0, MDT_ERR_SHAPE, "d*element size must be a multiple of 16 bytes");
    MDT_REQUIRE(x && path && n_acc && h_next, MDT_ERR_NULL, "a tensor pointer is NULL");
    MDT_REQUIRE(mdt_aligned16(x) && mdt_aligned16(h_next), MDT_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
    MDT_LAUNCH("next_state_kernel", next_state_kernel, dim3(B), dim3(256), 0, (hipStream_t)stream, (const uint4*)x,
               path, path_stride, n_acc, T, (int)(row_bytes / 16), (uint4*)h_next);
    return mdt_launched("next_state_kernel");
}

extern "C" mdt_status mdt_next_logits(void* stream, int B, int T, int V, int K, const float* vlogits,
                                      const int32_t* path, int path_stride, const int32_t* n_acc,
                                      float* head_logits) {
    MDT_REQUIRE(B >= 1 && B <= 65535 && T >= 1 && T <= MDT_MAX_NODES && V >= 1 && V <= (1 << 30) && K >= 1 &&
                    K <= MDT_MAX_HEADS,
                MDT_ERR_SHAPE, "bad shape B=%d T=%d V=%d K=%d", B, T, V, K);
    MDT_REQUIRE(path_stride >= 1 && path_stride <= MDT_MAX_NODES, MDT_ERR_SHAPE, "path_stride out of range");
    MDT_REQUIRE(vlogits && path && n_acc && head_logits, MDT_ERR_NULL, "a tensor pointer is NULL");
    MDT_REQUIRE(head_logits + (size_t)B * (K + 1) * V <= vlogits || vlogits + (size_t)B * T * V <= head_logits,
                MDT_ERR_VALUE, "head_logits must not overlap vlogits");
    MDT_LAUNCH("next_logits_kernel", next_logits_kernel, dim3((V + kNextLogitsPerWg - 1) / kNextLogitsPerWg, B),
               dim3(256), 0, (hipStream_t)stream, vlogits, path, path_stride, n_acc, T, V, (long)(K + 1) * V,
               head_logits);
    return mdt_launched("next_logits_kernel");
}
