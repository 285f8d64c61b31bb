// mdt_topk_tree_expand: per-head top-k over the vocabulary and the tree's tokens/positions.
//
// Summary page "Medusa: Simple LLM Inference Acceleration Framework with Multiple
// Decoding Heads", section "Tree Attention", steps 1-2 (top-s_k of every head,
// the candidates fill the tree level by level; the root is the LM head's top
// token) and step 4 (position id = prefix length + depth).
//
// Selection is a total order: larger value first, equal values by smaller index.
//
// Rows of up to 32768 logits (every vocabulary of the workloads): one launch,
// topk_rows, one workgroup per (sequence, head row) with the whole row in
// registers.  A radix search over the thread maxima gives a threshold that at
// least k elements reach; the few elements at or above it are ranked directly.
// The workgroup then writes the tree tokens of the nodes at its own depth, since a
// node's token depends on its depth's row only.  Heavy ties (more than 1024
// elements at the threshold) fall back to k selection rounds per wave.
//
// Longer rows: two launches.  A wave selects its k best elements in k rounds;
// each round every lane offers its best element that comes after the previous
// winner, and a DPP row-op reduction picks the winner.  Stage A: every workgroup
// reduces a 2048-element slice of one row to k candidates.  Rounds over all 2048
// elements would cost k full scans, so a threshold first discards almost
// everything: in each wave the k-th largest of the 64 lane maxima (counted with
// multiplicity) is a value that at least k of the wave's elements reach, so the
// slice's k best all lie at or above the largest of the four wave thresholds.
// The elements that reach it (typically little more than k) are packed into LDS
// and one wave selects among them.  If more than kCap elements reach it (many
// equal values), the workgroup falls back to rounds over every element.  Stage
// B: one workgroup per sequence, one wave per head row merges the slices'
// candidates and then all threads fill the tree tokens and positions.
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

// One workgroup per (sequence, head row) when the whole row fits in registers: 1024
// threads hold 32 logits each (elements tid + 1024 j, so every wave load reads 256
// contiguous bytes).  A threshold that at least k elements reach comes from the
// thread maxima: two 8-bit radix passes over their order-preserving keys (LDS
// histograms, one wave scanning the 256 bins from the top) locate the k-th largest
// maximum to 16 key bits, and every element at or above that bin's lower bound is a
// candidate (typically a few more than k).  Each candidate's rank is the number of
// candidates ahead of it in the total order, so the k best land in place without
// sequential rounds.  The workgroup then writes the tree tokens of the nodes at its
// depth (a node's token depends on its own depth's row only) and their positions, so
// no second launch is needed.  Heavy ties (more than 1024 candidates) fall back to
// per-wave selection rounds over every element.
constexpr int kRowThreads = 1024;
constexpr int kRowPer = 32;
constexpr int kRowMaxV = kRowThreads * kRowPer;
constexpr int kRowWaves = kRowThreads / 64;

// Order-preserving map of a float onto uint32 (larger float, larger key); -0 is first
// made +0 so that equal values get equal keys.
__device__ __forceinline__ uint32_t order_key(float f) {
    const uint32_t u = __float_as_uint(f + 0.f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// 64-bit key of (value, index): larger key = earlier in (value desc, index asc).
__device__ __forceinline__ uint64_t cand_key(float v, int i) {
    return ((uint64_t)order_key(v) << 32) | (uint32_t)(~(uint32_t)i);
}

// Exclusive prefix sum over the wave of a count below 2^11: bit b of every lane's count
// contributes 2^b for each lower lane that has it (one ballot and one mbcnt per bit).
__device__ __forceinline__ int wave_excl_prefix11(int x) {
    int r = 0;
#pragma unroll
    for (int bit = 0; bit < 11; ++bit) r += lanes_below(__ballot((x >> bit) & 1)) << bit;
    return r;
}

// Wave 0: scan 256 bins from the top; the bin where the running count reaches `need`,
// and how many of the counted items lie strictly above it.
__device__ __forceinline__ void radix_pick(const int* hist, int need, int lane, int* out_bin, int* out_above) {
    int c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) c[j] = hist[255 - 4 * lane - j];
    const int sl = c[0] + c[1] + c[2] + c[3];
    int run = wave_excl_prefix11(sl);  // items in bins above this lane's
    if (run < need && run + sl >= need) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (run + c[j] >= need) {
                *out_bin = 255 - 4 * lane - j;
                *out_above = run;
                break;
            }
            run += c[j];
        }
    }
}

// Largest 64-bit value over the wave, uniform (same DPP sequence as wave_argmax_dpp).
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
#define MDT_MAX64_STEP(CTRL, ROWS)                                                                   \
    {                                                                                               \
        const int hi = (int)(x >> 32), lo = (int)(uint32_t)x;                                        \
        const uint64_t o = ((uint64_t)(uint32_t)__builtin_amdgcn_update_dpp(hi, hi, CTRL, ROWS, 0xf, false) << 32) | \
                           (uint32_t)__builtin_amdgcn_update_dpp(lo, lo, CTRL, ROWS, 0xf, false);    \
        x = o > x ? o : x;                                                                          \
    }
    MDT_MAX64_STEP(0xB1, 0xf)
    MDT_MAX64_STEP(0x4E, 0xf)
    MDT_MAX64_STEP(0x141, 0xf)
    MDT_MAX64_STEP(0x140, 0xf)
    MDT_MAX64_STEP(0x142, 0xa)
    MDT_MAX64_STEP(0x143, 0xc)
#undef MDT_MAX64_STEP
    const uint32_t hi = __builtin_amdgcn_readlane((int)(x >> 32), 63);
    const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)x, 63);
    return ((uint64_t)hi << 32) | lo;
}

// Index of a thread's element j: with 16-byte loads (VEC4) the thread holds runs of four
// (elements 4(tid + 1024 q) + c, j = 4q + c), otherwise single elements tid + 1024 j.
// Either way a thread's indices increase with j.
template <bool VEC4>
__device__ __forceinline__ int row_elem(int tid, int j) {
    return VEC4 ? 4 * (tid + kRowThreads * (j >> 2)) + (j & 3) : tid + kRowThreads * j;
}

// Inverse of order_key.
__device__ __forceinline__ float key_value(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// k rounds over a thread's kRowPer elements (element j has index row_elem(tid, j), valid
// below V; kk holds their order keys): each round every lane offers its best element
// after the previous winner, and a 64-bit (key, ~index) wave maximum picks the winner.
// Values come back from the keys (a -0 element reads as +0).
template <bool VEC4>
__device__ void wave_select_row(const uint32_t (&kk)[kRowPer], int tid, int V, int k, Cand* out) {
    uint32_t lk = 0xffffffffu;
    int li = -1;  // previous winner (key, index); the first round admits everything
    for (int r = 0; r < k; ++r) {
        uint32_t bk = 0;
        int bi = INT_MAX;
        bool any = false;
#pragma unroll
        for (int j = 0; j < kRowPer; ++j) {
            const int e = row_elem<VEC4>(tid, j);
            const bool after = (kk[j] < lk) | ((kk[j] == lk) & (e > li)) | (r == 0);
            const bool take = (e < V) & after & (!any | (kk[j] > bk));  // same key: smaller j came first
            bk = take ? kk[j] : bk;
            bi = take ? e : bi;
            any = any | take;
        }
        const uint64_t mine = any ? (((uint64_t)bk << 32) | (uint32_t)~(uint32_t)bi) : 0ull;
        const uint64_t w = wave_max_u64(mine);
        lk = (uint32_t)(w >> 32);
        li = (int)~(uint32_t)w;
        if ((threadIdx.x & 63) == 0) out[r] = Cand{w ? key_value(lk) : -INFINITY, w ? li : INT_MAX};
    }
}

template <bool VEC4>
__global__ __launch_bounds__(kRowThreads) void topk_rows(const float* __restrict__ logits, int V, int k, int K1,
                                                         const int32_t* __restrict__ parent,
                                                         const int32_t* __restrict__ depth,
                                                         const int32_t* __restrict__ rank, int T,
                                                         const int32_t* __restrict__ prefix_len,
                                                         int32_t* __restrict__ topk_idx, float* __restrict__ topk_val,
                                                         int32_t* __restrict__ tokens, int32_t* __restrict__ pos) {
    __shared__ Cand surv[kRowThreads + 64];  // candidates, then one discard slot per lane
    __shared__ Cand wave_best[kRowWaves * MDT_MAX_TOPK];
    __shared__ Cand best[MDT_MAX_TOPK];
    __shared__ int hist[2][256];
    __shared__ int pick[5];  // bin 1, count above it, bin 2, count above it, candidates
    __shared__ int node[3][MDT_MAX_NODES];  // depth, rank, parent
    __shared__ int node_L;
    const int row = blockIdx.x, b = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // The output pointers are held in vector registers from here on: left to itself the
    // compiler reloads kernel arguments late to free scalar registers, and such a reload
    // waits on memory in the middle of the selection.
    asm volatile("" : "+v"(topk_idx), "+v"(topk_val), "+v"(tokens), "+v"(pos));
    // The tree inputs of this thread's node (T <= MDT_MAX_NODES) and the prefix length,
    // used at the end, are requested first and parked in LDS once the logits are in
    // flight.  The prefix length is read with a vector load through a register offset
    // (a scalar load would share the counter that every later wait for an LDS result
    // waits on).
    int vzero;
    asm volatile("v_mov_b32 %0, 0" : "=v"(vzero));
    const int L = prefix_len[b + vzero];
    const int i0 = min(tid, T - 1);
    const int dep0 = depth[i0], rk0 = rank[i0], par0 = parent[i0];
    // the row through a buffer resource: one 32-bit offset register per load
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(logits + ((size_t)b * K1 + row) * V), (short)0, V * 4, 0x00020000);
    float v[kRowPer];
    if constexpr (VEC4) {
#pragma unroll
        for (int q = 0; q < kRowPer / 4; ++q) {
            // four adjacent dword loads, which the compiler merges into one 16-byte load
            const int off = 4 * min(row_elem<true>(tid, 4 * q), V - 4);
#pragma unroll
            for (int c = 0; c < 4; ++c)
                v[4 * q + c] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, off + 4 * c, 0, 0));
        }
    } else {
#pragma unroll
        for (int j = 0; j < kRowPer; ++j)
            v[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, 4 * min(row_elem<false>(tid, j), V - 1), 0, 0));
    }
    __builtin_amdgcn_sched_barrier(0);
    // unconditional (threads past T rewrite node T-1 with its own values): a store under
    // a branch would let the compiler sink the loads behind the logits
    node[0][i0] = dep0;
    node[1][i0] = rk0;
    node[2][i0] = par0;
    node_L = L;
    if (tid < 512) hist[tid >> 8][tid & 255] = 0;
    if (tid == 0) pick[4] = 0;
    // elements past the row become NaN: no comparison selects them and fmaxf skips them
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < kRowPer; ++j) {
        v[j] = row_elem<VEC4>(tid, j) < V ? v[j] : __builtin_nanf("");
        m = fmaxf(m, v[j]);
    }
    const uint32_t km = order_key(m);
    __syncthreads();
    atomicAdd(&hist[0][km >> 24], 1);
    __syncthreads();
    if (wave == 0) radix_pick(hist[0], k, lane, &pick[0], &pick[1]);
    __syncthreads();
    const int b1 = pick[0];
    if ((int)(km >> 24) == b1) atomicAdd(&hist[1][(km >> 16) & 255], 1);
    __syncthreads();
    if (wave == 0) radix_pick(hist[1], k - pick[1], lane, &pick[2], &pick[3]);
    __syncthreads();
    const uint32_t thr = ((uint32_t)b1 << 24) | ((uint32_t)pick[2] << 16);

    // the same test as a float comparison: v >= tf exactly when order_key(v) >= thr
    // (keys at or below that of -inf mean every element)
    const float tf = (thr & 0x80000000u) ? __uint_as_float(thr & 0x7fffffffu)
                   : thr <= order_key(-INFINITY) ? -INFINITY : __uint_as_float(~thr);
    // candidates: only a thread whose maximum passes holds any; it counts them, takes
    // its slots with one LDS atomic and writes every element (the ones that fail go to
    // a slot of its own past the list, so no write sits under a branch)
    if (m >= tf) {
        uint32_t mask = 0;  // bit j: element j passes (a bit mask keeps the tests in VGPRs)
#pragma unroll
        for (int j = 0; j < kRowPer; ++j) mask |= (v[j] >= tf ? 1u : 0u) << j;
        int at = atomicAdd(&pick[4], (int)__popc(mask));
        if ((mask & (mask - 1u)) == 0u) {
            // the usual case, one candidate (the thread's maximum itself), or none (a thread
            // past the row end when the threshold is -inf)
            if (mask != 0u && at < kRowThreads) surv[at] = Cand{m, row_elem<VEC4>(tid, __builtin_ctz(mask))};
        } else {
            const int trash = kRowThreads + lane;
#pragma unroll
            for (int j = 0; j < kRowPer; ++j) {
                const int in = (int)((mask >> j) & 1u);
                surv[in && at < kRowThreads ? at : trash] = Cand{v[j], row_elem<VEC4>(tid, j)};
                at += in;
            }
        }
    }
    __syncthreads();
    const int n = pick[4];  // uniform over the workgroup
    if (n <= 64) {
        // one wave: lane c holds candidate c; its rank counts the candidates ahead of it
        if (wave == 0) {
            const Cand c = surv[min(lane, max(n - 1, 0))];
            const uint64_t key = lane < n ? cand_key(c.v, c.i) : 0ull;
            const uint32_t khi = (uint32_t)(key >> 32), klo = (uint32_t)key;
            int r = 0;
            for (int s2 = 0; s2 < n; ++s2) {
                const uint64_t o = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(khi, s2) << 32) |
                                   (uint32_t)__builtin_amdgcn_readlane(klo, s2);
                r += o > key ? 1 : 0;
            }
            if (lane < n && r < k) best[r] = c;
        }
    } else if (n <= kRowThreads) {
        if (tid < n) {
            const Cand c = surv[tid];
            const uint64_t key = cand_key(c.v, c.i);
            int r = 0;
            for (int s2 = 0; s2 < n; ++s2) {
                const Cand o = surv[s2];
                r += cand_key(o.v, o.i) > key ? 1 : 0;
            }
            if (r < k) best[r] = c;
        }
    } else {
        // many equal values at the threshold: every wave selects among its own elements,
        // then one wave among the waves' winners
        uint32_t kk[kRowPer];
#pragma unroll
        for (int j = 0; j < kRowPer; ++j) kk[j] = order_key(v[j]);
        wave_select_row<VEC4>(kk, tid, V, k, wave_best + wave * k);
        __syncthreads();
        if (wave == 0) {
            constexpr int E = kRowWaves * MDT_MAX_TOPK / 64;
            float mv[E];
            int mi[E];
#pragma unroll
            for (int j = 0; j < E; ++j) {
                const int c = lane + 64 * j;
                mv[j] = c < kRowWaves * k ? wave_best[c].v : -INFINITY;
                mi[j] = c < kRowWaves * k ? wave_best[c].i : INT_MAX;
            }
            wave_select<E>(mv, mi, k, best);
        }
    }
    __syncthreads();
    const size_t o = ((size_t)b * K1 + row) * k;
    if (tid < k) {
        const Cand c = best[tid];
        topk_idx[o + tid] = c.i;
        // the heavy-tie path selected on keys, which read -0 as +0: take the value itself
        topk_val[o + tid] = n > kRowThreads ? logits[((size_t)b * K1 + row) * V + c.i] : c.v;
    }
    // nodes at this row's depth; row 0 also writes the nodes whose depth is out of range
    if (tid < T) {
        const int i = tid;
        const int dep = node[0][i], rk = node[1][i], par = node[2][i];
        const bool in_range = dep >= 0 && dep < K1;
        if (in_range ? dep == row : row == 0) {
            const bool ok = in_range && rk >= 0 && rk < k && (i == 0 ? dep == 0 : par < i);
            tokens[(size_t)b * T + i] = ok ? best[rk].i : -1;
            pos[(size_t)b * T + i] = node_L + dep;
        }
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
    if (V <= kRowMaxV) {
        auto kern = V % 4 == 0 ? topk_rows<true> : topk_rows<false>;
        MDT_LAUNCH("topk_rows", kern, dim3(K1, B), dim3(kRowThreads), 0, s, logits, V, k_cfg, K1, tree->parent,
                   tree->depth, tree->rank, tree->T, prefix_len, topk_idx, topk_val, tree_tokens, pos_ids);
        return mdt_launched("topk_rows");
    }
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
