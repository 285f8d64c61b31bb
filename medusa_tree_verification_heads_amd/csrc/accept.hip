// mdt_accept_path: greedy or typical acceptance over the candidate tree.
//
// Summary page "Medusa: Simple LLM Inference Acceleration Framework with Multiple
// Decoding Heads", section "Typical Acceptance Scheme": a candidate passes if the
// verifier gives it probability > min(eps, delta * exp(-H)), H the entropy in
// nats of the verifier distribution at its parent; at temperature 0 only the
// most probable token has non-zero probability (greedy); the first token is
// accepted unconditionally; the step keeps the longest accepted prefix among all
// branches.  "Notes on Medusa", section 3: greedy verification descends into the
// child that carries the verifier's token.
//
// One wave per sequence.  Lanes test the edges of nodes lane, lane+64, ...; a
// ballot turns the results into a bitmask P of passing nodes.  A node is accepted
// iff its ancestor-or-self row has no bit outside P.  A max-reduction over
// (depth, -index) of the accepted nodes picks the deepest, leftmost one, and its
// ancestor row gives the path directly (node j sits at position depth(j)).
// mdt_accept_compact runs the same selection in wave 0 of a 256-thread workgroup
// per sequence and then lets the whole workgroup copy the accepted rows into the
// cache, with the checks and effects of mdt_kv_compact.
#include <math.h>

#include "kv_slot.h"

namespace {


struct AcceptArgs {
    const mdt_row_stats* stats;
    const float* edge;
    const int32_t* tokens;
    const int32_t* parent;
    const int32_t* depth;
    const uint64_t* anc;
    int T, W, mode;
    float eps, delta, tau;
    int32_t* path;
    int path_stride;
    int32_t* n_acc;
};

// One wave: acceptance of sequence b, for trees of NW = ceil(T/64) mask words.  Writes
// path[b][*] and n_acc[b]; returns the accepted node count (uniform over the wave) and, if
// lds_path is non-null, leaves the path there as well.  Two rounds of global loads: every
// per-node value (parent, token, edge logit, depth, mask row) is requested at once, then
// the parents' statistics; the chosen node's depth and mask row come from other lanes'
// registers.
template <int NW>
__device__ int accept_wave(const AcceptArgs& A, int b, int lane, int32_t* lds_path) {
    const int T = A.T;
    const float ln_eps = logf(A.eps), ln_delta = logf(A.delta);
    const bool onehot_passes = 1.f > fminf(A.eps, A.delta);  // typical at tau = 0, candidate is the argmax
    if (lds_path)
        for (int j = lane; j < A.path_stride; j += 64) lds_path[j] = -1;
    int par[NW], tok[NW], dep[NW];
    float edg[NW];
    uint64_t an[NW][NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const int c = min(w * 64 + lane, T - 1);  // clamped: lanes past T are ignored below
        par[w] = A.parent[c];
        tok[w] = A.tokens[(long)b * T + c];
        edg[w] = A.edge[(long)b * T + c];
        dep[w] = A.depth[c];
#pragma unroll
        for (int x = 0; x < NW; ++x) an[w][x] = A.anc[(long)c * NW + x];
    }
    mdt_row_stats st[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) st[w] = A.stats[(long)b * T + min(max(par[w], 0), T - 1)];
    uint64_t P[NW];  // passing nodes; the ballot is uniform, so every lane holds the mask
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const int c = w * 64 + lane;
        bool pass = false;
        if (c == 0) {
            pass = true;
        } else if (c < T && par[w] >= 0 && par[w] < c) {
            if (A.mode == MDT_ACCEPT_GREEDY) {
                pass = tok[w] == st[w].argmax;
            } else if (A.tau == 0.f) {
                pass = tok[w] == st[w].argmax && onehot_passes;
            } else {
                const float lp = edg[w] / A.tau - st[w].logZ;
                pass = lp > fminf(ln_eps, ln_delta - st[w].entropy);
            }
        }
        P[w] = __ballot(pass);
    }
    // deepest accepted node, smallest index among equals
    int key = -1;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const int c = w * 64 + lane;
        bool ok = c < T;
#pragma unroll
        for (int x = 0; x < NW; ++x) ok = ok && ((an[w][x] & ~P[x]) == 0);
        if (ok && dep[w] >= 0 && dep[w] < 256) key = max(key, (dep[w] << 16) | (0xffff - c));
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) key = max(key, __shfl_xor(key, off, 64));
    const int best = 0xffff - (key & 0xffff);  // the root is always accepted, so key >= 0
    const int bw = best >> 6, bl = best & 63;
    int best_dep = 0;
    uint64_t abest[NW];
#pragma unroll
    for (int x = 0; x < NW; ++x) abest[x] = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {  // the chosen node's depth and mask row, from lane bl
        const int dw = __shfl(dep[w], bl, 64);
#pragma unroll
        for (int x = 0; x < NW; ++x) {
            const uint64_t a = __shfl(an[w][x], bl, 64);
            if (w == bw) abest[x] = a;
        }
        if (w == bw) best_dep = dw;
    }
    const int nb = best_dep + 1;
    int32_t* pb = A.path + (long)b * A.path_stride;
    for (int j = lane; j < A.path_stride; j += 64)
        if (j >= nb) pb[j] = -1;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const int c = w * 64 + lane;
        if (c < T && ((abest[w] >> lane) & 1ull)) {
            const int dc = dep[w];
            if (dc >= 0 && dc < A.path_stride) {
                pb[dc] = c;
                if (lds_path) lds_path[dc] = c;
            }
        }
    }
    const int n = min(nb, A.path_stride);
    if (lane == 0) A.n_acc[b] = n;
    return n;
}

template <int NW>
__global__ __launch_bounds__(64) void accept_kernel(AcceptArgs A) {
    accept_wave<NW>(A, blockIdx.x, threadIdx.x, nullptr);
}

constexpr int kCopyThreads = 1024;
constexpr int kCopyBatch = 4;  // 16-byte vectors of k and of v a thread loads before it stores

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
        const int n = accept_wave<NW>(A, b, tid, s_path);
        if (tid == 0) s_n = n;
    }
    __syncthreads();
    const int n = s_n, L = prefix_len[b];
    if (tid == 0) s_ok = 1;
    __syncthreads();
    if (!(n >= 1 && L >= 0)) {
        if (tid == 0) new_len[b] = -1;
        return;
    }
    for (int j = tid; j < n; j += kCopyThreads) {
        const int node = s_path[j];
        const long row = slot_row(cache, b, L + j);
        s_dst[j] = row;
        if (!(node >= 0 && node < A.T && row >= 0)) s_ok = 0;
    }
    __syncthreads();
    if (tid == 0) new_len[b] = s_ok ? L + n : -1;
    if (!s_ok) return;
    uint4* K = (uint4*)cache.k;
    uint4* Vv = (uint4*)cache.v;
    const int total = n * row_vec;
    for (int e0 = tid; e0 < total; e0 += kCopyThreads * kCopyBatch) {
        uint4 kk[kCopyBatch], vv[kCopyBatch];
#pragma unroll
        for (int u = 0; u < kCopyBatch; ++u) {  // loads first (clamped to the last item), stores after
            const int e = min(e0 + u * kCopyThreads, total - 1);
            const int j = e / row_vec;
            const long src = ((long)b * A.T + s_path[j]) * row_vec + (e - j * row_vec);
            kk[u] = k_rot[src];
            vv[u] = v[src];
        }
#pragma unroll
        for (int u = 0; u < kCopyBatch; ++u) {
            const int e = e0 + u * kCopyThreads;
            if (e < total) {
                const int j = e / row_vec;
                const long dst = s_dst[j] * row_vec + (e - j * row_vec);
                K[dst] = kk[u];
                Vv[dst] = vv[u];
            }
        }
    }
}

mdt_status check_accept(int B, const mdt_tree_dev* tree, const mdt_row_stats* stats, const float* edge_logit,
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
                    mode, typ ? eps : 1.f, typ ? delta : 1.f, temperature, path, path_stride, n_acc};
    return MDT_OK;
}

}  // namespace

extern "C" mdt_status mdt_accept_path(void* stream, int B, const mdt_tree_dev* tree, const mdt_row_stats* stats,
                                      const float* edge_logit, const int32_t* tree_tokens, int mode, float eps,
                                      float delta, float temperature, int32_t* path, int path_stride,
                                      int32_t* n_acc) {
    AcceptArgs A;
    mdt_status st = check_accept(B, tree, stats, edge_logit, tree_tokens, mode, eps, delta, temperature, path,
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
    mdt_status st = check_accept(B, tree, stats, edge_logit, tree_tokens, mode, eps, delta, temperature, path,
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
