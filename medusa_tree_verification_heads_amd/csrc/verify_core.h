// Row statistics of the verifier logits, shared by mdt_verify_logits and
// mdt_verify_accept_compact.
//
// Summary page "Medusa: Simple LLM Inference Acceleration Framework with Multiple
// Decoding Heads", section "Typical Acceptance Scheme": the verifier's probability of a
// candidate and the entropy in nats of its distribution.  The tile kernels reduce each
// row of a vocabulary tile to a partial (max m, argmax a, s = sum e^{(z-m)/tau},
// u = sum e^{(z-m)/tau} (z-m)/tau); merging the partials of a row gives
// logZ = M/tau + ln S and H = ln S - U/S.
#pragma once

#include <climits>
#include <math.h>

#include "common.h"

struct Part {
    float m;
    int a;
    float s;
    float u;
};

// Merge two partials.  The one with the larger maximum keeps its sums; the other's are
// scaled by e^{(m_small - m_big)/tau} (one exponential) and its u shifted to the common
// reference: u' = f (u + s d), d = (m_small - m_big)/tau.  inv_tau = 1/tau (0 at tau = 0,
// where only the maximum and argmax are kept).
__device__ __forceinline__ Part part_merge(Part p, Part q, float inv_tau) {
    if (q.m == -INFINITY) return p;
    if (p.m == -INFINITY) return q;
    const bool pb = better(p.m, p.a, q.m, q.a);
    const Part& hi = pb ? p : q;
    const Part& lo = pb ? q : p;
    Part r;
    r.m = hi.m;
    r.a = hi.a;
    if (inv_tau > 0.f) {
        const float dl = (lo.m - hi.m) * inv_tau;  // <= 0
        const float f = __expf(dl);
        r.s = fmaf(f, lo.s, hi.s);
        r.u = fmaf(f, fmaf(lo.s, dl, lo.u), hi.u);
    } else {
        r.s = r.u = 0.f;
    }
    return r;
}

__device__ __forceinline__ Part shfl_xor_part(Part p, int off) {
    Part q;
    q.m = __shfl_xor(p.m, off, 64);
    q.a = __shfl_xor(p.a, off, 64);
    q.s = __shfl_xor(p.s, off, 64);
    q.u = __shfl_xor(p.u, off, 64);
    return q;
}

#ifndef MDT_MERGE_LANES
#define MDT_MERGE_LANES 16
#endif
#ifndef MDT_MERGE_BATCH
#define MDT_MERGE_BATCH 8
#endif
constexpr int kMergeLanes = MDT_MERGE_LANES;  // lanes that merge one row (a wave merges 4 rows at once)

// The merged partial of one row on a 16-lane group (sub = lane % 16), uniform over the
// group.  Lane sub merges partials sub, sub + 16, ..., in that order (the loads of 256
// partials issued before their merges), then the group combines in a fixed xor tree: the
// result does not depend on scheduling, and every caller gets the same bits.
__device__ __forceinline__ Part merge_row(const Part* __restrict__ pr, int nblk_n, float inv_tau, int sub) {
    constexpr int kBatch = MDT_MERGE_BATCH;
    Part p{-INFINITY, INT_MAX, 0.f, 0.f};
    for (int j0 = 0; j0 < nblk_n; j0 += kMergeLanes * kBatch) {
        Part q[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) q[u] = pr[min(j0 + sub + kMergeLanes * u, nblk_n - 1)];
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
            if (j0 + sub + kMergeLanes * u < nblk_n) p = part_merge(p, q[u], inv_tau);
    }
#pragma unroll
    for (int off = 1; off < kMergeLanes; off <<= 1) p = part_merge(p, shfl_xor_part(p, off), inv_tau);
    return p;
}

__device__ __forceinline__ mdt_row_stats row_stats_of(const Part& p, float tau) {
    mdt_row_stats st;
    st.max = p.m;
    st.argmax = p.a;
    if (tau > 0.f) {
        const float lnS = logf(p.s);
        st.logZ = p.m / tau + lnS;
        st.entropy = lnS - p.u / p.s;
    } else {
        st.logZ = 0.f;
        st.entropy = 0.f;
    }
    return st;
}

// The edge entries of row `row` = b*T + c that no tile writes: 0 for the root, -inf for a
// token outside [0, V) or a node without a valid parent.
__device__ __forceinline__ void edge_defaults(int row, int T, int V, const int32_t* __restrict__ tokens,
                                              const int32_t* __restrict__ parent, float* __restrict__ edge) {
    const int c = row % T;
    const int tok = tokens[row];
    const int pr = parent[c];
    if (c == 0)
        edge[row] = 0.f;
    else if (tok < 0 || tok >= V || pr < 0 || pr >= T)
        edge[row] = -INFINITY;
}

// Host: validate the verifier's arguments and launch its tile kernel (partials into ws,
// edge logits owned by tiles, optional full logits); *nblk_n receives the partials per row.
mdt_status mdt_verify_tiles(hipStream_t s, mdt_dtype dt, int B, int T, int d, int V, const void* x, const void* Wlm,
                            const mdt_tree_dev* tree, const int32_t* tree_tokens, float temperature,
                            mdt_row_stats* stats, float* edge_logit, float* logits_opt, void* ws, size_t ws_bytes,
                            int* nblk_n);
