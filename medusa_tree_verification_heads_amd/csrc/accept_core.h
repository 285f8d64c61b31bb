// Acceptance and compaction pieces shared by mdt_accept_path, mdt_accept_compact and
// mdt_verify_accept_compact.
//
// Summary page "Medusa: Simple LLM Inference Acceleration Framework with Multiple
// Decoding Heads", section "Typical Acceptance Scheme": a candidate passes if the
// verifier gives it probability > min(eps, delta * exp(-H)), H the entropy in nats of
// the verifier distribution at its parent; at temperature 0 only the most probable
// token has non-zero probability (greedy); the first token is accepted
// unconditionally; the step keeps the longest accepted prefix among all branches.
// "Notes on Medusa", section 3: greedy verification descends into the child that
// carries the verifier's token.  "MEDUSA 精读", section 3: only the accepted path's
// keys and values stay in the cache.
//
// One wave selects: lanes test the edges of nodes lane, lane+64, ...; a ballot turns
// the results into a bitmask P of passing nodes.  A node is accepted iff its
// ancestor-or-self row has no bit outside P.  A max-reduction over (depth, -index) of
// the accepted nodes picks the deepest, leftmost one, and its ancestor row gives the
// path directly (node j sits at position depth(j)).
#pragma once

#include <math.h>

#include "kv_slot.h"

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
    int V;  // > 0: a token outside [0, V) fails its edge (its edge logit is not read)
};

// Per-node inputs of one sequence's selection, as one lane holds them (nodes lane, lane+64, ...).
template <int NW>
struct NodeData {
    int par[NW], tok[NW], dep[NW];
    float edg[NW];
    uint64_t an[NW][NW];
};

// Request every per-node value of sequence b at once (parent, token, edge logit, depth,
// mask row); lanes past T read the last node and are ignored by the selection.
template <int NW>
__device__ __forceinline__ void load_nodes(const AcceptArgs& A, int b, int lane, NodeData<NW>& nd) {
    const int T = A.T;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const int c = min(w * 64 + lane, T - 1);
        nd.par[w] = A.parent[c];
        nd.tok[w] = A.tokens[(long)b * T + c];
        nd.edg[w] = A.edge[(long)b * T + c];
        nd.dep[w] = A.depth[c];
#pragma unroll
        for (int x = 0; x < NW; ++x) nd.an[w][x] = A.anc[(long)c * NW + x];
    }
}

// One wave: the selection of sequence b from its node data and `stb`, the sequence's T
// rows of statistics (global memory or LDS).  Writes path[b][*] and n_acc[b]; returns the
// accepted node count (uniform over the wave) and, if lds_path is non-null, leaves the
// path there as well.  The parents' statistics are the only loads; the chosen node's
// depth and mask row come from other lanes' registers.
template <int NW>
__device__ int select_path(const AcceptArgs& A, int b, int lane, const NodeData<NW>& nd, const mdt_row_stats* stb,
                           int32_t* lds_path) {
    const int T = A.T;
    const float ln_eps = logf(A.eps), ln_delta = logf(A.delta);
    const bool onehot_passes = 1.f > fminf(A.eps, A.delta);  // typical at tau = 0, candidate is the argmax
    if (lds_path)
        for (int j = lane; j < A.path_stride; j += 64) lds_path[j] = -1;
    const int(&par)[NW] = nd.par;
    const int(&tok)[NW] = nd.tok;
    const int(&dep)[NW] = nd.dep;
    const float(&edg)[NW] = nd.edg;
    const uint64_t(&an)[NW][NW] = nd.an;
    mdt_row_stats st[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) st[w] = stb[min(max(par[w], 0), T - 1)];
    uint64_t P[NW];  // passing nodes; the ballot is uniform, so every lane holds the mask
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const int c = w * 64 + lane;
        bool pass = false;
        if (c == 0) {
            pass = true;
        } else if (c < T && par[w] >= 0 && par[w] < c && (A.V <= 0 || (tok[w] >= 0 && tok[w] < A.V))) {
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

// One wave: load the node data, then select (two rounds of loads).
template <int NW>
__device__ int accept_wave(const AcceptArgs& A, int b, int lane, const mdt_row_stats* stb, int32_t* lds_path) {
    NodeData<NW> nd;
    load_nodes<NW>(A, b, lane, nd);
    return select_path<NW>(A, b, lane, nd, stb, lds_path);
}

constexpr int kCopyThreads = 1024;
constexpr int kCopyBatch = 4;  // 16-byte vectors of k and of v a thread loads before it stores

// After the selection (path in s_path, n nodes, written by wave 0 before a barrier), the
// whole 1024-thread workgroup appends the path's rotated keys and values of sequence b at
// slots L .. L + n - 1 (L = prefix_len[b], read by the caller), with the checks and effects
// of mdt_kv_compact: new_len[b] is L + n, or -1 (and nothing written) if a node, the length
// or a destination slot is out of range.  s_dst holds MDT_MAX_NODES rows.
__device__ __forceinline__ void compact_path_block(const KvSlots& cache, const uint4* __restrict__ k_rot,
                                                   const uint4* __restrict__ v, int row_vec, int T, int b, int n,
                                                   const int32_t* s_path, long* s_dst, int* s_ok, int L,
                                                   int32_t* __restrict__ new_len) {
    const int tid = threadIdx.x;
    if (tid == 0) *s_ok = 1;
    __syncthreads();
    if (!(n >= 1 && L >= 0)) {
        if (tid == 0) new_len[b] = -1;
        return;
    }
    for (int j = tid; j < n; j += kCopyThreads) {
        const int node = s_path[j];
        const long row = slot_row(cache, b, L + j);
        s_dst[j] = row;
        if (!(node >= 0 && node < T && row >= 0)) *s_ok = 0;
    }
    __syncthreads();
    if (tid == 0) new_len[b] = *s_ok ? L + n : -1;
    if (!*s_ok) return;
    uint4* K = (uint4*)cache.k;
    uint4* Vv = (uint4*)cache.v;
    const int total = n * row_vec;
    for (int e0 = tid; e0 < total; e0 += kCopyThreads * kCopyBatch) {
        uint4 kk[kCopyBatch], vv[kCopyBatch];
#pragma unroll
        for (int u = 0; u < kCopyBatch; ++u) {  // loads first (clamped to the last item), stores after
            const int e = min(e0 + u * kCopyThreads, total - 1);
            const int j = e / row_vec;
            const long src = ((long)b * T + s_path[j]) * row_vec + (e - j * row_vec);
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

// Host-side checks of the acceptance arguments (shared by the three entry points); fills *A.
mdt_status mdt_check_accept(int B, const mdt_tree_dev* tree, const mdt_row_stats* stats, const float* edge_logit,
                            const int32_t* tree_tokens, int mode, float eps, float delta, float temperature,
                            int32_t* path, int path_stride, int32_t* n_acc, AcceptArgs* A);
