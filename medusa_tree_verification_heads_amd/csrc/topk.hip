// mdt_topk_tree_expand: per-head top-k over the vocabulary and the tree's tokens/positions.
//
// Summary page "Medusa: Simple LLM Inference Acceleration Framework with Multiple
// Decoding Heads", section "Tree Attention", steps 1-2 (top-s_k of every head,
// the candidates fill the tree level by level; the root is the LM head's top
// token) and step 4 (position id = prefix length + depth).
//
// Selection is a total order: larger value first, equal values by smaller index.
// A wave selects its k best elements in k rounds; each round every lane offers
// its best element that comes after the previous winner, and a DPP row-op
// reduction picks the winner.
//
// Stage A: every workgroup reduces a 2048-element slice of one row to k
// candidates.  Rounds over all 2048 elements would cost k full scans, so a
// threshold first discards almost everything: in each wave the k-th largest of
// the 64 lane maxima (counted with multiplicity) is a value that at least k of the
// wave's elements reach, so the slice's k best all lie at or above the largest of
// the four wave thresholds.  The elements that reach it (typically little more
// than k) are packed into LDS and one wave selects among them.  If more than
// kCap elements reach it (many equal values), the workgroup falls back to rounds
// over every element.  Stage B: one workgroup per sequence, one wave per head row
// merges the slices' candidates and then all threads fill the tree tokens and
// positions.
#include <climits>

#include "common.h"

namespace {

constexpr int kSlice = 2048;          // elements per stage-A workgroup
constexpr int kPerLaneA = kSlice / 256;
constexpr int kCap = 256;             // threshold survivors a stage-A workgroup keeps
constexpr int kMaxPerLaneB = 8;       // stage-B candidates per lane

struct Cand {
    float v;
    int i;
};

// k rounds of wave-wide selection over E elements per lane; winners go to out[0..k).
template <int E>
__device__ void wave_select(const float (&v)[E], const int (&idx)[E], int k, Cand* out) {
    float lv = INFINITY;
    int li = -1;
    for (int r = 0; r < k; ++r) {
        float bv = -INFINITY;
        int bi = INT_MAX;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const bool after = better(lv, li, v[e], idx[e]);
            if (after && better(v[e], idx[e], bv, bi)) {
                bv = v[e];
                bi = idx[e];
            }
        }
        wave_argmax_dpp(bv, bi);
        if ((threadIdx.x & 63) == 0) out[r] = Cand{bv, bi};
        lv = bv;
        li = bi;
    }
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_max_step(float v) {
    const int vb = __builtin_bit_cast(int, v);
    return fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(vb, vb, CTRL, ROW_MASK, 0xf, false)));
}

// Maximum over the wave, uniform (same DPP sequence as wave_argmax_dpp).
__device__ __forceinline__ float wave_max_dpp(float v) {
    v = dpp_max_step<0xB1, 0xf>(v);
    v = dpp_max_step<0x4E, 0xf>(v);
    v = dpp_max_step<0x141, 0xf>(v);
    v = dpp_max_step<0x140, 0xf>(v);
    v = dpp_max_step<0x142, 0xa>(v);
    v = dpp_max_step<0x143, 0xc>(v);
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// k-th largest of the lanes' m, equal values counted separately (-inf if the wave
// holds fewer than k finite values).
__device__ float wave_kth_largest(float m, int k) {
    float t = -INFINITY;
    int cnt = 0;
    for (int r = 0; r < k; ++r) {
        const float mx = wave_max_dpp(m);
        t = mx;
        cnt += __popcll(__ballot(m == mx));
        if (cnt >= k || mx == -INFINITY) break;
        if (m == mx) m = -INFINITY;
    }
    return t;
}

__device__ __forceinline__ int lanes_below(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
}

__global__ __launch_bounds__(256) void topk_slices(const float* __restrict__ logits, int V, int k, int nslice,
                                                   Cand* __restrict__ cand) {
    __shared__ Cand surv[kCap];
    __shared__ Cand wave_best[4 * MDT_MAX_TOPK];
    __shared__ float wave_t[4];
    __shared__ int n_surv;
    const int row = blockIdx.y;
    const int slice = blockIdx.x;
    const float* x = logits + (size_t)row * V;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // wave w owns elements base + w*512 + [0, 512): coalesced 256-byte rows
    const int base = slice * kSlice + wave * (kSlice / 4) + lane;
    float v[kPerLaneA];
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < kPerLaneA; ++j) {
        const int e = base + 64 * j;
        v[j] = e < V ? x[e] : -INFINITY;
        m = fmaxf(m, v[j]);
    }
    const float tw = wave_kth_largest(m, k);
    if (lane == 0) wave_t[wave] = tw;
    if (threadIdx.x == 0) n_surv = 0;
    __syncthreads();
    const float thr = fmaxf(fmaxf(wave_t[0], wave_t[1]), fmaxf(wave_t[2], wave_t[3]));
    int nw = 0;
#pragma unroll
    for (int j = 0; j < kPerLaneA; ++j) nw += __popcll(__ballot(base + 64 * j < V && v[j] >= thr));
    int at = 0;
    if (lane == 0 && nw > 0) at = atomicAdd(&n_surv, nw);
    at = __shfl(at, 0, 64);
#pragma unroll
    for (int j = 0; j < kPerLaneA; ++j) {
        const int e = base + 64 * j;
        const bool keep = e < V && v[j] >= thr;
        const uint64_t bal = __ballot(keep);
        const int slot = at + lanes_below(bal);
        if (keep && slot < kCap) surv[slot] = Cand{v[j], e};
        at += __popcll(bal);
    }
    __syncthreads();
    const int n = n_surv;  // uniform over the workgroup
    Cand* out = cand + ((size_t)row * nslice + slice) * k;
    if (n <= kCap) {
        if (wave == 0) {
            float cv[kCap / 64];
            int ci[kCap / 64];
#pragma unroll
            for (int j = 0; j < kCap / 64; ++j) {
                const int c = lane + 64 * j;
                cv[j] = c < n ? surv[c].v : -INFINITY;
                ci[j] = c < n ? surv[c].i : INT_MAX;
            }
            wave_select<kCap / 64>(cv, ci, k, out);
        }
        return;
    }
    // many equal values at the threshold: rounds over every element
    int idx[kPerLaneA];
#pragma unroll
    for (int j = 0; j < kPerLaneA; ++j) idx[j] = base + 64 * j < V ? base + 64 * j : INT_MAX;
    wave_select<kPerLaneA>(v, idx, k, wave_best + wave * k);
    __syncthreads();
    if (wave == 0) {
        float mv[2];
        int mi[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int c = lane + 64 * j;
            mv[j] = c < 4 * k ? wave_best[c].v : -INFINITY;
            mi[j] = c < 4 * k ? wave_best[c].i : INT_MAX;
        }
        wave_select<2>(mv, mi, k, out);
    }
}

template <int E>
__global__ void topk_merge_expand(const Cand* __restrict__ cand, int K1, int k, int nslice,
                                  const int32_t* __restrict__ parent, const int32_t* __restrict__ depth,
                                  const int32_t* __restrict__ rank, int T, const int32_t* __restrict__ prefix_len,
                                  int32_t* __restrict__ topk_idx, float* __restrict__ topk_val,
                                  int32_t* __restrict__ tokens, int32_t* __restrict__ pos) {
    __shared__ Cand best[(MDT_MAX_HEADS + 1) * MDT_MAX_TOPK];
    const int b = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // the tree-fill inputs of this thread's first node are requested with the candidates
    const int i0 = min((int)threadIdx.x, T - 1);
    const int dep0 = depth[i0], rk0 = rank[i0], par0 = parent[i0];
    const int L = prefix_len[b];
    {  // the block has exactly K1 waves: wave w merges head row w
        const int row = b * K1 + wave;
        const Cand* c = cand + (size_t)row * nslice * k;
        const int n = nslice * k;
        float v[E];
        int idx[E];
#pragma unroll
        for (int j = 0; j < E; ++j) {  // unconditional loads (clamped), out-of-range entries replaced
            const Cand q = c[min(lane + 64 * j, n - 1)];
            const bool in = lane + 64 * j < n;
            v[j] = in ? q.v : -INFINITY;
            idx[j] = in ? q.i : INT_MAX;
        }
        wave_select<E>(v, idx, k, best + wave * k);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < K1 * k; e += blockDim.x) {
        topk_idx[(size_t)b * K1 * k + e] = best[e].i;
        topk_val[(size_t)b * K1 * k + e] = best[e].v;
    }
    for (int i = threadIdx.x; i < T; i += blockDim.x) {
        const bool first = i == (int)threadIdx.x;
        const int dep = first ? dep0 : depth[i], rk = first ? rk0 : rank[i];
        const int par = first ? par0 : parent[i];
        const bool ok = dep >= 0 && dep < K1 && rk >= 0 && rk < k && (i == 0 ? dep == 0 : par < i);
        tokens[(size_t)b * T + i] = ok ? best[dep * k + rk].i : -1;
        pos[(size_t)b * T + i] = L + dep;
    }
}

int num_slices(int V) { return (V + kSlice - 1) / kSlice; }

}  // namespace

extern "C" size_t mdt_topk_workspace(int B, int K, int V, int k_cfg) {
    if (B < 1 || K < 0 || V < 1 || k_cfg < 1) return 0;
    return (size_t)B * (K + 1) * num_slices(V) * k_cfg * sizeof(Cand);
}

extern "C" mdt_status mdt_topk_tree_expand(void* stream, int B, int K, int V, int k_cfg, const float* logits,
                                           const mdt_tree_dev* tree, const int32_t* prefix_len, int32_t* topk_idx,
                                           float* topk_val, int32_t* tree_tokens, int32_t* pos_ids, void* ws,
                                           size_t ws_bytes) {
    MDT_REQUIRE(B >= 1 && B <= 65535, MDT_ERR_SHAPE, "B=%d out of range", B);
    MDT_REQUIRE(K >= 1 && K <= MDT_MAX_HEADS, MDT_ERR_SHAPE, "K=%d out of range 1..%d", K, MDT_MAX_HEADS);
    MDT_REQUIRE(k_cfg >= 1 && k_cfg <= MDT_MAX_TOPK && k_cfg <= V, MDT_ERR_SHAPE, "k_cfg=%d out of range 1..%d",
                k_cfg, MDT_MAX_TOPK);
    MDT_REQUIRE(V >= 1, MDT_ERR_SHAPE, "V=%d out of range", V);
    MDT_REQUIRE((long)num_slices(V) * k_cfg <= 64L * kMaxPerLaneB, MDT_ERR_UNSUPPORTED,
                "V=%d with k=%d exceeds the merge capacity", V, k_cfg);
    mdt_status st = mdt_check_tree(tree);
    if (st != MDT_OK) return st;
    MDT_REQUIRE(tree->max_depth <= K, MDT_ERR_TREE, "tree depth %d exceeds K=%d", tree->max_depth, K);
    MDT_REQUIRE(tree->max_rank < k_cfg, MDT_ERR_TREE, "tree rank %d needs top-k > k_cfg=%d", tree->max_rank, k_cfg);
    MDT_REQUIRE(logits && prefix_len && topk_idx && topk_val && tree_tokens && pos_ids, MDT_ERR_NULL,
                "a tensor pointer is NULL");
    MDT_REQUIRE(ws, MDT_ERR_WORKSPACE, "workspace is NULL");
    MDT_REQUIRE(ws_bytes >= mdt_topk_workspace(B, K, V, k_cfg), MDT_ERR_WORKSPACE, "workspace too small");
    MDT_REQUIRE(mdt_aligned16(ws), MDT_ERR_ALIGN, "workspace must be 16-byte aligned");
    hipStream_t s = (hipStream_t)stream;
    const int K1 = K + 1;
    const int ns = num_slices(V);
    Cand* cand = (Cand*)ws;
    MDT_LAUNCH("topk_slices", topk_slices, dim3(ns, B * K1), dim3(256), 0, s, logits, V, k_cfg, ns, cand);
    st = mdt_launched("topk_slices");
    if (st != MDT_OK) return st;
    // candidates per lane in the merge: 1, 2, 4 or 8
    const int per_lane = (ns * k_cfg + 63) / 64;
    auto kern = per_lane <= 1 ? topk_merge_expand<1>
              : per_lane <= 2 ? topk_merge_expand<2>
              : per_lane <= 4 ? topk_merge_expand<4> : topk_merge_expand<kMaxPerLaneB>;
    MDT_LAUNCH("topk_merge_expand", kern, dim3(B), dim3(64 * K1), 0, s, cand, K1, k_cfg, ns, tree->parent,
               tree->depth, tree->rank, tree->T, prefix_len, topk_idx, topk_val, tree_tokens, pos_ids);
    return mdt_launched("topk_merge_expand");
}
