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
#include <math.h>

#include "common.h"

namespace {

__global__ __launch_bounds__(64) void accept_kernel(const mdt_row_stats* __restrict__ stats,
                                                    const float* __restrict__ edge, const int32_t* __restrict__ tokens,
                                                    const int32_t* __restrict__ parent, const int32_t* __restrict__ depth,
                                                    const uint64_t* __restrict__ anc, int T, int W, int mode, float eps,
                                                    float delta, float tau, int32_t* __restrict__ path,
                                                    int path_stride, int32_t* __restrict__ n_acc) {
    const int b = blockIdx.x;
    const int lane = threadIdx.x;
    const float ln_eps = logf(eps), ln_delta = logf(delta);
    const bool onehot_passes = 1.f > fminf(eps, delta);  // typical at tau = 0, candidate is the argmax
    __shared__ uint64_t P[MDT_MAX_NODES / 64];
    for (int w = 0; w < W; ++w) {
        const int c = w * 64 + lane;
        bool pass = false;
        if (c == 0) {
            pass = true;
        } else if (c < T) {
            const int p = parent[c];
            if (p >= 0 && p < c) {
                const mdt_row_stats st = stats[(long)b * T + p];
                const int tok = tokens[(long)b * T + c];
                if (mode == MDT_ACCEPT_GREEDY) {
                    pass = tok == st.argmax;
                } else if (tau == 0.f) {
                    pass = tok == st.argmax && onehot_passes;
                } else {
                    const float lp = edge[(long)b * T + c] / tau - st.logZ;
                    pass = lp > fminf(ln_eps, ln_delta - st.entropy);
                }
            }
        }
        const uint64_t bal = __ballot(pass);
        if (lane == 0) P[w] = bal;
    }
    __syncthreads();
    // deepest accepted node, smallest index among equals
    int key = -1;
    for (int w = 0; w < W; ++w) {
        const int c = w * 64 + lane;
        if (c >= T) break;
        bool ok = true;
        for (int x = 0; x < W; ++x) ok = ok && ((anc[(long)c * W + x] & ~P[x]) == 0);
        const int dep = depth[c];
        if (ok && dep >= 0 && dep < 256) key = max(key, (dep << 16) | (0xffff - c));
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) key = max(key, __shfl_xor(key, off, 64));
    const int best = 0xffff - (key & 0xffff);  // the root is always accepted, so key >= 0
    const int nb = depth[best] + 1;
    int32_t* pb = path + (long)b * path_stride;
    for (int j = lane; j < path_stride; j += 64)
        if (j >= nb) pb[j] = -1;
    for (int w = 0; w < W; ++w) {
        const int c = w * 64 + lane;
        if (c < T && ((anc[(long)best * W + w] >> lane) & 1ull)) {
            const int dc = depth[c];
            if (dc >= 0 && dc < path_stride) pb[dc] = c;
        }
    }
    if (lane == 0) n_acc[b] = min(nb, path_stride);
}

}  // namespace

extern "C" mdt_status mdt_accept_path(void* stream, int B, const mdt_tree_dev* tree, const mdt_row_stats* stats,
                                      const float* edge_logit, const int32_t* tree_tokens, int mode, float eps,
                                      float delta, float temperature, int32_t* path, int path_stride,
                                      int32_t* n_acc) {
    MDT_REQUIRE(B >= 1 && B <= 65535, MDT_ERR_SHAPE, "B=%d out of range", B);
    mdt_status st = mdt_check_tree(tree);
    if (st != MDT_OK) return st;
    MDT_REQUIRE(mode == MDT_ACCEPT_GREEDY || mode == MDT_ACCEPT_TYPICAL, MDT_ERR_VALUE, "unknown mode %d", mode);
    MDT_REQUIRE(temperature >= 0.f && temperature == temperature, MDT_ERR_VALUE, "temperature must be >= 0");
    if (mode == MDT_ACCEPT_TYPICAL)
        MDT_REQUIRE(eps > 0.f && delta > 0.f, MDT_ERR_VALUE, "eps and delta must be > 0");
    MDT_REQUIRE(path_stride >= tree->max_depth + 1, MDT_ERR_SHAPE, "path_stride %d < max_depth + 1", path_stride);
    MDT_REQUIRE(stats && edge_logit && tree_tokens && path && n_acc, MDT_ERR_NULL, "a tensor pointer is NULL");
    MDT_LAUNCH("accept_kernel", accept_kernel, dim3(B), dim3(64), 0, (hipStream_t)stream, stats, edge_logit,
               tree_tokens, tree->parent, tree->depth, tree->anc, tree->T, tree->anc_words, mode,
               mode == MDT_ACCEPT_TYPICAL ? eps : 1.f, mode == MDT_ACCEPT_TYPICAL ? delta : 1.f, temperature, path,
               path_stride, n_acc);
    return mdt_launched("accept_kernel");
}
