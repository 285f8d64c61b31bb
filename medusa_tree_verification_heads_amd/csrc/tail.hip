// mdt_verify_accept_compact: the end of a step in two launches -- the verifier's tile
// kernel (LM head on every node, per-tile row partials, edge logits), then one workgroup
// per sequence that merges its rows' partials into the row statistics, selects the
// accepted path and appends its keys and values to the cache.
//
// Summary page "Medusa: Simple LLM Inference Acceleration Framework with Multiple
// Decoding Heads", section 3.2 (verification, acceptance and the cache update end one
// iteration) and "Tree Attention" steps 5-6; the statistics, the acceptance rule and the
// cache update are those of verify_core.h and accept_core.h, computed in the same order,
// so every output equals what mdt_verify_logits, mdt_accept_path and mdt_kv_compact write.
#include "accept_core.h"
#include "verify_core.h"

namespace {

// grid B, block 1024: 16-lane groups merge the sequence's rows (64 at a time), wave 0
// selects from the statistics in LDS, the workgroup copies the path's rows.
template <int NW>
__global__ __launch_bounds__(kCopyThreads) void merge_accept_compact_kernel(
    const Part* __restrict__ part, int nblk_n, int V, AcceptArgs A, mdt_row_stats* __restrict__ stats,
    float* __restrict__ edge, KvSlots cache, const uint4* __restrict__ k_rot, const uint4* __restrict__ v,
    int row_vec, const int32_t* __restrict__ prefix_len, int32_t* __restrict__ new_len) {
    __shared__ mdt_row_stats s_stats[MDT_MAX_NODES];
    __shared__ int32_t s_path[MDT_MAX_NODES];
    __shared__ long s_dst[MDT_MAX_NODES];
    __shared__ int s_n, s_ok;
    const int b = blockIdx.x, tid = threadIdx.x;
    const int T = A.T;
    const float inv_tau = A.tau > 0.f ? 1.f / A.tau : 0.f;
    // the selection's node data and the prefix length do not depend on the merge: their
    // loads go out together with the partials'
    NodeData<NW> nd;
    if (tid < 64) load_nodes<NW>(A, b, tid, nd);
    const int L = prefix_len[b];
    // 16 lanes per row: the workgroup merges 64 rows at a time
    for (int i0 = 0; i0 < T; i0 += kCopyThreads / kMergeLanes) {
        const int i = i0 + tid / kMergeLanes, sub = tid % kMergeLanes;
        const int row = b * T + min(i, T - 1);
        const Part p = merge_row(part + (long)row * nblk_n, nblk_n, inv_tau, sub);
        if (sub == 0 && i < T) {
            const mdt_row_stats st = row_stats_of(p, A.tau);
            stats[row] = st;
            s_stats[i] = st;
            edge_defaults(row, T, V, A.tokens, A.parent, edge);
        }
    }
    __syncthreads();
    if (tid < 64) {
        // A.V = V: tokens outside the vocabulary fail without reading their edge entry
        const int n = select_path<NW>(A, b, tid, nd, s_stats, s_path);
        if (tid == 0) s_n = n;
    }
    __syncthreads();
    compact_path_block(cache, k_rot, v, row_vec, T, b, s_n, s_path, s_dst, &s_ok, L, new_len);
}

}  // namespace

extern "C" mdt_status mdt_verify_accept_compact(void* stream, mdt_dtype dt, int B, int T, int d, int V, int H, int Dh,
                                                const void* x, const void* Wlm, const mdt_tree_dev* tree,
                                                const int32_t* tree_tokens, float temperature, int mode, float eps,
                                                float delta, mdt_row_stats* stats, float* edge_logit,
                                                float* logits_opt, int32_t* path, int path_stride, int32_t* n_acc,
                                                const void* k_rot, const void* v, const mdt_kv_cache* cache,
                                                const int32_t* prefix_len, int32_t* new_prefix_len, void* ws,
                                                size_t ws_bytes) {
    // every check of the three calls before the first launch
    AcceptArgs A;
    mdt_status st = mdt_check_accept(B, tree, stats, edge_logit, tree_tokens, mode, eps, delta, temperature, path,
                                     path_stride, n_acc, &A);
    if (st != MDT_OK) return st;
    MDT_REQUIRE(T == tree->T, MDT_ERR_SHAPE, "T=%d differs from the tree's %d nodes", T, tree->T);
    KvSlots c;
    int row_vec = 0;
    st = mdt_check_compact_args(dt, B, T, H, Dh, path_stride, k_rot, v, cache, prefix_len, new_prefix_len, &c,
                                &row_vec);
    if (st != MDT_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    int nblk_n = 0;
    st = mdt_verify_tiles(s, dt, B, T, d, V, x, Wlm, tree, tree_tokens, temperature, stats, edge_logit, logits_opt, ws,
                          ws_bytes, &nblk_n);
    if (st != MDT_OK) return st;
    A.V = V;
    auto kern = A.W == 1 ? merge_accept_compact_kernel<1>
              : A.W == 2 ? merge_accept_compact_kernel<2>
              : A.W == 3 ? merge_accept_compact_kernel<3> : merge_accept_compact_kernel<4>;
    MDT_LAUNCH("merge_accept_compact", kern, dim3(B), dim3(kCopyThreads), 0, s, (const Part*)ws, nblk_n, V, A, stats,
               edge_logit, c, (const uint4*)k_rot, (const uint4*)v, row_vec, prefix_len, new_prefix_len);
    return mdt_launched("merge_accept_compact");
}
