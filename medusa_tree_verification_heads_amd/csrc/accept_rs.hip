// mdt_accept_rejection: rejection-sampling acceptance on the candidate tree.
//
// "Accelerating LLM Inference with Speculative Decoding: Notes on Medusa", section 2,
// and the summary page "Medusa: Simple LLM Inference Acceleration Framework with
// Multiple Decoding Heads", section "Typical Acceptance Scheme" (first paragraph): a
// candidate x drafted with probability q(x) is accepted with probability
// min(1, p(x)/q(x)); after a rejection the token comes from norm(max(0, p - q)).
// On the tree the walk starts at the root; the children of the current node (one
// head's candidates) are tried in rank order against the current residual r (the
// verifier distribution p at the node at first, norm(max(0, r - q)) after each
// rejection); an accepted child becomes the current node.  When no child is accepted
// the next token is drawn from r by its inverse CDF.  The random numbers are inputs.
//
// One 1024-thread workgroup per sequence; thread t holds vocabulary entries
// [32t, 32t + 32) of r in registers; q is recomputed from the head row (its maximum
// and normaliser are kept) wherever it is needed, with the same expression every
// time.  Row softmaxes, residual updates and the final running sum are register work
// plus fixed-order block reductions (the results do not depend on scheduling).
#include <math.h>

#include "common.h"

namespace {

constexpr int kRsThreads = 1024;
constexpr int kRsPer = 32;
constexpr int kRsMaxV = kRsThreads * kRsPer;
constexpr int kRsWaves = kRsThreads / 64;

struct RsArgs {
    const float* z;        // [B*T][V] verifier logits
    const float* head;     // [B][K1][V] head logits (row 0 = LM head)
    const int32_t* tokens; // [B][T]
    const int32_t* parent;
    const int32_t* depth;
    const float* u_acc;    // [B][T]
    const float* u_res;    // [B]
    int T, V, K1;
    float tau;
    int32_t* path;
    int path_stride;
    int32_t* n_acc;
    int32_t* next_token;
};

// Sum / maximum over the workgroup, identical on every thread: wave trees of xor shuffles,
// then the 16 wave results in wave order.  `red` is reused after the trailing barrier.
__device__ float block_sum(float v, float* red) {
    v = wave_sum(v);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < kRsWaves; ++w) s += red[w];
    __syncthreads();
    return s;
}

__device__ float block_max(float v, float* red) {
    v = wave_max(v);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    float s = -INFINITY;
#pragma unroll
    for (int w = 0; w < kRsWaves; ++w) s = fmaxf(s, red[w]);
    __syncthreads();
    return s;
}

// The thread's 32 entries of a row of V floats, through a buffer resource whose range is
// the row (one offset register for all 32 loads; the hardware returns 0 past the range),
// with the entries past V set to -inf so that every later use needs no index test.
__device__ __forceinline__ void load_row(const float* row, int V, float (&out)[kRsPer]) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)row, (short)0, V * 4, 0x00020000);
    const int voff = (int)threadIdx.x * (kRsPer * 4);
    const int nv = V - (int)threadIdx.x * kRsPer;  // entries of this thread inside the row
#pragma unroll
    for (int j = 0; j < kRsPer; ++j) {
        const float x = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, voff + 4 * j, 0, 0));
        out[j] = j < nv ? x : -INFINITY;
    }
}

// out = softmax(row / tau) over the thread's entries (0 past V); exponentials in base 2.
__device__ void row_softmax(const float* __restrict__ row, int V, float tau, float (&out)[kRsPer], float* red) {
    const float kl = 1.4426950408889634f / tau;  // exp(y / tau) = exp2(y * log2(e) / tau)
    float m = -INFINITY;
    load_row(row, V, out);
#pragma unroll
    for (int j = 0; j < kRsPer; ++j) m = fmaxf(m, out[j]);
    m = block_max(m, red);
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < kRsPer; ++j) {
        out[j] = exp2f((out[j] - m) * kl);  // -inf past V gives 0
        s += out[j];
    }
    s = block_sum(s, red);
#pragma unroll
    for (int j = 0; j < kRsPer; ++j) out[j] = out[j] / s;
}

// Maximum and normaliser of softmax(row / tau): q(v) = exp2f((row[v] - m) * log2(e) / tau) / s.
__device__ void row_norm(const float* __restrict__ row, int V, float tau, float* red, float& m, float& s) {
    float x[kRsPer];
    float mm = -INFINITY;
    load_row(row, V, x);
#pragma unroll
    for (int j = 0; j < kRsPer; ++j) mm = fmaxf(mm, x[j]);
    m = block_max(mm, red);
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < kRsPer; ++j) ss += exp2f((x[j] - m) * (1.4426950408889634f / tau));
    s = block_sum(ss, red);
}

__global__ __launch_bounds__(kRsThreads) void accept_rs_kernel(RsArgs A) {
    __shared__ int par_s[MDT_MAX_NODES], dep_s[MDT_MAX_NODES], tok_s[MDT_MAX_NODES];
    __shared__ int first_child[MDT_MAX_NODES], next_sib[MDT_MAX_NODES], path_s[MDT_MAX_NODES];
    __shared__ float uacc_s[MDT_MAX_NODES];
    __shared__ float red[kRsWaves];
    __shared__ float bx[2];
    __shared__ int pick;
    const int b = blockIdx.x, tid = threadIdx.x;
    const int T = A.T, V = A.V;
    if (tid < T) {
        par_s[tid] = A.parent[tid];
        dep_s[tid] = A.depth[tid];
        tok_s[tid] = A.tokens[(size_t)b * T + tid];
        uacc_s[tid] = A.u_acc[(size_t)b * T + tid];
    }
    if (tid == 0) pick = -1;
    __syncthreads();
    if (tid < T) {
        // children have larger packed indices than their parent, siblings in rank order
        int fc = -1, ns = -1;
        for (int c = tid + 1; c < T; ++c)
            if (par_s[c] == tid) { fc = c; break; }
        for (int c = tid + 1; c < T; ++c)
            if (par_s[c] == par_s[tid]) { ns = c; break; }
        first_child[tid] = fc;
        next_sib[tid] = ns;
    }
    __syncthreads();

    const int v0 = tid * kRsPer;
    float r[kRsPer];
    row_softmax(A.z + (size_t)b * T * V, V, A.tau, r, red);
    int cur = 0, n = 1, qdepth = -1;
    float qm = 0.f, qs = 1.f;
    const float* hrow = A.head;
    bool none = false;
    if (tid == 0) path_s[0] = 0;
    while (true) {
        const int d = dep_s[cur];
        int acc = -1;
        for (int c = first_child[cur]; c >= 0; c = next_sib[c]) {
            if (d + 1 >= A.K1) break;  // no head for that depth (the host check prevents it)
            if (qdepth != d + 1) {
                hrow = A.head + ((size_t)b * A.K1 + d + 1) * V;
                row_norm(hrow, V, A.tau, red, qm, qs);
                qdepth = d + 1;
            }
            const int x = tok_s[c];
            if (x >= 0 && x < V && x / kRsPer == tid) {
                const int xl = x - v0;
                float rx = 0.f;
#pragma unroll
                for (int j = 0; j < kRsPer; ++j) rx = j == xl ? r[j] : rx;
                bx[0] = rx;
                bx[1] = exp2f((hrow[x] - qm) * (1.4426950408889634f / A.tau)) / qs;
            }
            __syncthreads();
            const float rx = bx[0], qx = bx[1];
            __syncthreads();
            const bool valid = x >= 0 && x < V;
            const float a = qx > 0.f ? fminf(1.f, rx / qx) : 1.f;
            if (valid && uacc_s[c] < a) {
                acc = c;
                break;
            }
            float s = 0.f;
            float hv[kRsPer];
            load_row(hrow, V, hv);
#pragma unroll
            for (int j = 0; j < kRsPer; ++j) {
                const float qv = exp2f((hv[j] - qm) * (1.4426950408889634f / A.tau)) / qs;  // 0 past V
                r[j] = fmaxf(r[j] - qv, 0.f);
                s += r[j];
            }
            s = block_sum(s, red);
            if (!(s > 0.f)) {
                none = true;
                break;
            }
#pragma unroll
            for (int j = 0; j < kRsPer; ++j) r[j] = r[j] / s;
        }
        if (acc < 0) break;
        cur = acc;
        if (tid == 0) path_s[n] = cur;
        ++n;
        row_softmax(A.z + ((size_t)b * T + cur) * V, V, A.tau, r, red);
    }
    if (!none) {
        // inverse CDF: the entry where the running sum first exceeds u * total, running sums
        // in vocabulary order (thread sums, then a scan over threads).  Thread t covers
        // [lo_t, hi_t) with hi_t = base + its inclusive sum and lo_t taken from thread t-1's
        // hi (the wave's base for lane 0, which equals the previous wave's last hi bit for
        // bit), so adjacent ranges share their bound exactly; the smallest claiming thread
        // wins (an LDS atomic minimum), so the pick is the same on every run.
        float own = 0.f;
#pragma unroll
        for (int j = 0; j < kRsPer; ++j) own += r[j];
        const int lane = tid & 63, wave = tid >> 6;
        float incl = own;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float t = __shfl_up(incl, off, 64);
            if (lane >= off) incl += t;
        }
        if (lane == 63) red[wave] = incl;
        if (tid == 0) pick = 0x7fffffff;
        __syncthreads();
        float base = 0.f, total = 0.f;
#pragma unroll
        for (int w = 0; w < kRsWaves; ++w) {
            base += w < wave ? red[w] : 0.f;
            total += red[w];
        }
        const float target = A.u_res[b] * total;
        const float prev = __shfl_up(incl, 1, 64);
        const float hi = base + incl;
        const float lo = lane == 0 ? base : base + prev;
        if (own > 0.f && lo <= target && target < hi) {
            float run = lo;
            int y = -1, last = -1;
#pragma unroll
            for (int j = 0; j < kRsPer; ++j) {
                run += r[j];
                last = r[j] > 0.f ? j : last;
                y = (y < 0 && run > target) ? j : y;
            }
            atomicMin(&pick, v0 + (y >= 0 ? y : last));  // a rounding shortfall keeps the range's last entry
        }
        __syncthreads();
        if (pick == 0x7fffffff) {
            // target at or past the total by rounding: the last entry with mass
            int last = -1;
#pragma unroll
            for (int j = 0; j < kRsPer; ++j) last = r[j] > 0.f ? j : last;
            const float lm = block_max(last >= 0 ? (float)(v0 + last) : -1.f, red);
            if (tid == 0) pick = (int)lm;
            __syncthreads();
        }
    }
    if (tid < A.path_stride) A.path[(size_t)b * A.path_stride + tid] = tid < n ? path_s[tid] : -1;
    if (tid == 0) {
        A.n_acc[b] = n;
        A.next_token[b] = none ? -1 : pick;
    }
}

}  // namespace

extern "C" mdt_status mdt_accept_rejection(void* stream, int B, int V, int K, const mdt_tree_dev* tree,
                                           const float* vlogits, const float* head_logits,
                                           const int32_t* tree_tokens, float temperature, const float* u_accept,
                                           const float* u_resample, int32_t* path, int path_stride, int32_t* n_acc,
                                           int32_t* next_token) {
    MDT_REQUIRE(B >= 1 && B <= 65535, MDT_ERR_SHAPE, "B=%d out of range", B);
    mdt_status st = mdt_check_tree(tree);
    if (st != MDT_OK) return st;
    MDT_REQUIRE(V >= 1, MDT_ERR_SHAPE, "V=%d out of range", V);
    MDT_REQUIRE(V <= kRsMaxV, MDT_ERR_UNSUPPORTED, "rejection sampling supports V <= %d (got %d)", kRsMaxV, V);
    MDT_REQUIRE(K >= 1 && K <= MDT_MAX_HEADS, MDT_ERR_SHAPE, "K=%d out of range", K);
    MDT_REQUIRE(tree->max_depth <= K, MDT_ERR_TREE, "tree depth %d exceeds K=%d", tree->max_depth, K);
    MDT_REQUIRE(temperature > 0.f && temperature == temperature, MDT_ERR_VALUE,
                "rejection sampling needs temperature > 0");
    MDT_REQUIRE(path_stride >= tree->max_depth + 1 && path_stride <= kRsThreads, MDT_ERR_SHAPE,
                "path_stride %d out of range", path_stride);
    MDT_REQUIRE(vlogits && head_logits && tree_tokens && u_accept && u_resample && path && n_acc && next_token,
                MDT_ERR_NULL, "a tensor pointer is NULL");
    RsArgs A{vlogits, head_logits, tree_tokens, tree->parent, tree->depth, u_accept, u_resample, tree->T, V,
             K + 1, temperature, path, path_stride, n_acc, next_token};
    MDT_LAUNCH("accept_rs_kernel", accept_rs_kernel, dim3(B), dim3(kRsThreads), 0, (hipStream_t)stream, A);
    return mdt_launched("accept_rs_kernel");
}
