// mdt_accept_path and mdt_accept_compact: greedy or typical acceptance over the candidate
// tree (the selection is accept_wave in accept_core.h; the summary page's "Typical
// Acceptance Scheme" and "Notes on Medusa", section 3, are cited there).
//
// mdt_accept_path: one wave per sequence.  mdt_accept_compact runs the same selection in
// wave 0 of a 1024-thread workgroup per sequence and then lets the whole workgroup copy
// the accepted rows into the cache, with the checks and effects of mdt_kv_compact.
#include "accept_core.h"

namespace {

template <int NW>
__global__ __launch_bounds__(64) void accept_kernel(AcceptArgs A) {
    accept_wave<NW>(A, blockIdx.x, threadIdx.x, A.stats + (long)blockIdx.x * A.T, nullptr);
}

template <int NW>
__global__ __launch_bounds__(kCopyThreads) void accept_compact_kernel(AcceptArgs A, KvSlots cache,
                                                                      const uint4* __restrict__ k_rot,
                                                                      const uint4* __restrict__ v, int row_vec,
                                                                      const int32_t* __restrict__ prefix_len,
                                                                      int32_t* __restrict__ new_len) {
    __shared__ int32_t s_path[MDT_MAX_NODES];
    __shared__ long s_dst[MDT_MAX_NODES];
    __shared__ int s_n, s_ok;
    const int b = blockIdx.x, tid = threadIdx.x;
    if (tid < 64) {
        const int n = accept_wave<NW>(A, b, tid, A.stats + (long)b * A.T, s_path);
        if (tid == 0) s_n = n;
    }
    const int L = prefix_len[b];
    __syncthreads();
    compact_path_block(cache, k_rot, v, row_vec, A.T, b, s_n, s_path, s_dst, &s_ok, L, new_len);
}

}  // namespace

mdt_status mdt_check_accept(int B, const mdt_tree_dev* tree, const mdt_row_stats* stats, const float* edge_logit,
                        const int32_t* tree_tokens, int mode, float eps, float delta, float temperature,
                        int32_t* path, int path_stride, int32_t* n_acc, AcceptArgs* A) {
    MDT_REQUIRE(B >= 1 && B <= 65535, MDT_ERR_SHAPE, "B=%d out of range", B);
    mdt_status st = mdt_check_tree(tree);
    if (st != MDT_OK) return st;
    MDT_REQUIRE(mode == MDT_ACCEPT_GREEDY || mode == MDT_ACCEPT_TYPICAL, MDT_ERR_VALUE, "unknown mode %d", mode);
    MDT_REQUIRE(temperature >= 0.f && temperature == temperature, MDT_ERR_VALUE, "temperature must be >= 0");
    if (mode == MDT_ACCEPT_TYPICAL)
        MDT_REQUIRE(eps > 0.f && delta > 0.f, MDT_ERR_VALUE, "eps and delta must be > 0");
    MDT_REQUIRE(path_stride >= tree->max_depth + 1, MDT_ERR_SHAPE, "path_stride %d < max_depth + 1", path_stride);
    MDT_REQUIRE(stats && edge_logit && tree_tokens && path && n_acc, MDT_ERR_NULL, "a tensor pointer is NULL");
    const bool typ = mode == MDT_ACCEPT_TYPICAL;
    *A = AcceptArgs{stats, edge_logit, tree_tokens, tree->parent, tree->depth, tree->anc, tree->T, tree->anc_words,
                    mode, typ ? eps : 1.f, typ ? delta : 1.f, temperature, path, path_stride, n_acc, 0};
    return MDT_OK;
}


extern "C" mdt_status mdt_accept_path(void* stream, int B, const mdt_tree_dev* tree, const mdt_row_stats* stats,
                                      const float* edge_logit, const int32_t* tree_tokens, int mode, float eps,
                                      float delta, float temperature, int32_t* path, int path_stride,
                                      int32_t* n_acc) {
    AcceptArgs A;
    mdt_status st = mdt_check_accept(B, tree, stats, edge_logit, tree_tokens, mode, eps, delta, temperature, path,
                                 path_stride, n_acc, &A);
    if (st != MDT_OK) return st;
    auto kern = A.W == 1 ? accept_kernel<1> : A.W == 2 ? accept_kernel<2> : A.W == 3 ? accept_kernel<3>
                                                                                 : accept_kernel<4>;
    MDT_LAUNCH("accept_kernel", kern, dim3(B), dim3(64), 0, (hipStream_t)stream, A);
    return mdt_launched("accept_kernel");
}

extern "C" mdt_status mdt_accept_compact(void* stream, mdt_dtype dt, int B, int H, int Dh, const mdt_tree_dev* tree,
                                         const mdt_row_stats* stats, const float* edge_logit,
                                         const int32_t* tree_tokens, int mode, float eps, float delta,
                                         float temperature, int32_t* path, int path_stride, int32_t* n_acc,
                                         const void* k_rot, const void* v, const mdt_kv_cache* cache,
                                         const int32_t* prefix_len, int32_t* new_prefix_len) {
    AcceptArgs A;
    mdt_status st = mdt_check_accept(B, tree, stats, edge_logit, tree_tokens, mode, eps, delta, temperature, path,
                                 path_stride, n_acc, &A);
    if (st != MDT_OK) return st;
    KvSlots c;
    int row_vec = 0;
    st = mdt_check_compact_args(dt, B, tree->T, H, Dh, path_stride, k_rot, v, cache, prefix_len, new_prefix_len, &c,
                                &row_vec);
    if (st != MDT_OK) return st;
    auto kern = A.W == 1 ? accept_compact_kernel<1>
              : A.W == 2 ? accept_compact_kernel<2>
              : A.W == 3 ? accept_compact_kernel<3> : accept_compact_kernel<4>;
    MDT_LAUNCH("accept_compact_kernel", kern, dim3(B), dim3(kCopyThreads), 0, (hipStream_t)stream,
               A, c, (const uint4*)k_rot, (const uint4*)v, row_vec, prefix_len, new_prefix_len);
    return mdt_launched("accept_compact_kernel");
}
