// Host layer of libmdt: error reporting, device properties and the static tree builders.
//
// The tree builders follow the Medusa pages: the Cartesian-product tree of the
// summary page ("Tree Attention", steps 1-2) and the sparse tree of section
// "Optimized Tree Construction" (steps 2-4: path accuracy = product of per-node
// accuracies, nodes added greedily from the frontier), also "Notes on Medusa",
// sections 3-4.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <queue>
#include <vector>

#include "common.h"

namespace {
thread_local char g_last_error[512] = "";

constexpr int kMaxProfiled = 4096;
thread_local void** g_prof_events = nullptr;
thread_local int g_prof_capacity = 0;
thread_local int g_prof_count = 0;
thread_local const char* g_prof_names[kMaxProfiled];

struct Node {
    std::vector<int> path;  // rank path r_1..r_l
};

bool path_less(const std::vector<int>& a, const std::vector<int>& b) {
    if (a.size() != b.size()) return a.size() < b.size();
    return a < b;
}

// Fill a host tree from a set of rank paths (root included), packed breadth-first.
mdt_status pack_tree(std::vector<std::vector<int>> paths, mdt_tree_host* out) {
    std::sort(paths.begin(), paths.end(), path_less);
    const int T = (int)paths.size();
    if (T < 1 || T > MDT_MAX_NODES || !paths[0].empty())
        return mdt_fail(MDT_ERR_SHAPE, "tree must hold the root and 1..%d nodes (got %d)", MDT_MAX_NODES, T);
    const int W = (T + 63) / 64;
    mdt_tree_host t;
    std::memset(&t, 0, sizeof(t));
    t.T = T;
    t.anc_words = W;
    t.parent = (int32_t*)std::calloc(T, sizeof(int32_t));
    t.depth = (int32_t*)std::calloc(T, sizeof(int32_t));
    t.rank = (int32_t*)std::calloc(T, sizeof(int32_t));
    t.anc = (uint64_t*)std::calloc((size_t)T * W, sizeof(uint64_t));
    if (!t.parent || !t.depth || !t.rank || !t.anc) {
        mdt_tree_free(&t);
        return mdt_fail(MDT_ERR_ALLOC, "tree allocation failed");
    }
    for (int i = 0; i < T; ++i) {
        const std::vector<int>& p = paths[i];
        t.depth[i] = (int)p.size();
        t.rank[i] = p.empty() ? 0 : p.back();
        t.max_depth = std::max(t.max_depth, t.depth[i]);
        t.max_rank = std::max(t.max_rank, t.rank[i]);
        if (i == 0) {
            t.parent[i] = -1;
        } else {
            std::vector<int> pp(p.begin(), p.end() - 1);
            auto it = std::lower_bound(paths.begin(), paths.begin() + i, pp, path_less);
            if (it == paths.begin() + i || *it != pp) {
                mdt_tree_free(&t);
                return mdt_fail(MDT_ERR_TREE, "node %d has no parent in the tree", i);
            }
            t.parent[i] = (int)(it - paths.begin());
        }
        // ancestor-or-self bits: parent precedes i, so its row is complete
        uint64_t* row = t.anc + (size_t)i * W;
        if (i > 0) std::memcpy(row, t.anc + (size_t)t.parent[i] * W, W * sizeof(uint64_t));
        row[i >> 6] |= 1ull << (i & 63);
    }
    *out = t;
    return MDT_OK;
}

struct Cand {
    double logscore;
    std::vector<int> path;
};

// Priority: larger score first; then smaller depth; then lexicographically smaller path.
struct CandWorse {
    bool operator()(const Cand& a, const Cand& b) const {
        if (a.logscore != b.logscore) return a.logscore < b.logscore;
        if (a.path.size() != b.path.size()) return a.path.size() > b.path.size();
        return a.path > b.path;
    }
};
}  // namespace

// ---------------------------------------------------------------------------
// errors
// ---------------------------------------------------------------------------

mdt_status mdt_fail(mdt_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return st;
}

mdt_status mdt_launched(const char* kernel) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return mdt_fail(MDT_ERR_HIP, "%s: %s", kernel, hipGetErrorString(e));
    return MDT_OK;
}

void mdt_profile_slot(const char* kernel, hipEvent_t* start, hipEvent_t* stop) {
    *start = *stop = nullptr;
    if (!g_prof_events) return;
    const int i = g_prof_count++;
    if (i < kMaxProfiled) g_prof_names[i] = kernel;
    if (2 * i + 1 < g_prof_capacity) {
        *start = (hipEvent_t)g_prof_events[2 * i];
        *stop = (hipEvent_t)g_prof_events[2 * i + 1];
    }
}

int mdt_num_cus() {
    static std::mutex mu;
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    std::lock_guard<std::mutex> lock(mu);
    if (cache[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev] = n;
    }
    return cache[dev];
}

extern "C" {

int mdt_abi_version(void) { return MDT_ABI_VERSION; }

mdt_status mdt_profile_attach(void** events, int capacity) {
    MDT_REQUIRE(capacity >= 0, MDT_ERR_SHAPE, "capacity must be >= 0");
    MDT_REQUIRE(events || capacity == 0, MDT_ERR_NULL, "events is NULL");
    g_prof_events = capacity > 0 ? events : nullptr;
    g_prof_capacity = capacity;
    g_prof_count = 0;
    return MDT_OK;
}

int mdt_profile_detach(void) {
    g_prof_events = nullptr;
    g_prof_capacity = 0;
    return g_prof_count;
}

const char* mdt_profile_kernel(int i) {
    if (i < 0 || i >= g_prof_count || i >= kMaxProfiled) return "";
    return g_prof_names[i];
}

const char* mdt_last_error(void) { return g_last_error; }

const char* mdt_status_string(int st) {
    switch (st) {
        case MDT_OK: return "ok";
        case MDT_ERR_NULL: return "null pointer";
        case MDT_ERR_SHAPE: return "bad shape";
        case MDT_ERR_DTYPE: return "bad dtype";
        case MDT_ERR_ALIGN: return "misaligned pointer";
        case MDT_ERR_TREE: return "bad tree";
        case MDT_ERR_VALUE: return "bad parameter value";
        case MDT_ERR_WORKSPACE: return "workspace too small";
        case MDT_ERR_HIP: return "HIP error";
        case MDT_ERR_UNSUPPORTED: return "unsupported";
        case MDT_ERR_ALLOC: return "host allocation failed";
        default: return "unknown status";
    }
}

// ---------------------------------------------------------------------------
// trees
// ---------------------------------------------------------------------------

mdt_status mdt_tree_build_cartesian(int K, const int* s, mdt_tree_host* out) {
    MDT_REQUIRE(out, MDT_ERR_NULL, "out is NULL");
    MDT_REQUIRE(K >= 0 && K <= MDT_MAX_HEADS, MDT_ERR_SHAPE, "K=%d out of range 0..%d", K, MDT_MAX_HEADS);
    MDT_REQUIRE(K == 0 || s, MDT_ERR_NULL, "s is NULL");
    long total = 1, level = 1;
    for (int j = 0; j < K; ++j) {
        MDT_REQUIRE(s[j] >= 1 && s[j] <= MDT_MAX_TOPK, MDT_ERR_SHAPE, "s[%d]=%d out of range 1..%d", j, s[j],
                    MDT_MAX_TOPK);
        level *= s[j];
        total += level;
        MDT_REQUIRE(total <= MDT_MAX_NODES, MDT_ERR_SHAPE, "Cartesian tree exceeds %d nodes", MDT_MAX_NODES);
    }
    std::vector<std::vector<int>> paths(1);
    std::vector<std::vector<int>> frontier(1);
    for (int j = 0; j < K; ++j) {
        std::vector<std::vector<int>> next;
        for (const auto& p : frontier)
            for (int r = 0; r < s[j]; ++r) {
                std::vector<int> c = p;
                c.push_back(r);
                next.push_back(c);
            }
        paths.insert(paths.end(), next.begin(), next.end());
        frontier.swap(next);
    }
    return pack_tree(paths, out);
}

mdt_status mdt_tree_build_scored(int K, int k_cfg, int T, double a0, double rho, double gamma, int rank_base,
                                 int depth_base, mdt_tree_host* out) {
    MDT_REQUIRE(out, MDT_ERR_NULL, "out is NULL");
    MDT_REQUIRE(K >= 1 && K <= MDT_MAX_HEADS, MDT_ERR_SHAPE, "K=%d out of range 1..%d", K, MDT_MAX_HEADS);
    MDT_REQUIRE(k_cfg >= 1 && k_cfg <= MDT_MAX_TOPK, MDT_ERR_SHAPE, "k_cfg=%d out of range", k_cfg);
    MDT_REQUIRE(T >= 1 && T <= MDT_MAX_NODES, MDT_ERR_SHAPE, "T=%d out of range 1..%d", T, MDT_MAX_NODES);
    MDT_REQUIRE(a0 > 0 && a0 <= 1 && rho > 0 && rho <= 1 && gamma > 0 && gamma <= 1, MDT_ERR_VALUE,
                "a0, rho, gamma must lie in (0, 1]");
    MDT_REQUIRE(rank_base >= 0 && depth_base >= 0, MDT_ERR_VALUE, "rank_base/depth_base must be >= 0");
    double cands = 0, lvl = 1;
    for (int j = 0; j < K; ++j) {
        lvl *= k_cfg;
        cands += lvl;
    }
    MDT_REQUIRE(T - 1 <= cands, MDT_ERR_SHAPE, "T=%d exceeds the %g candidate nodes", T, cands);
    const double la = std::log(a0), lr = std::log(rho), lg = std::log(gamma);
    // log score of a path: l*ln(a0) + R*ln(rho) + D*ln(gamma), R = sum(r_j + rank_base),
    // D = sum(j - 1 + depth_base); equal (l, R, D) give bitwise equal values.
    auto logscore = [&](const std::vector<int>& p) {
        long R = 0, D = 0;
        for (size_t j = 0; j < p.size(); ++j) {
            R += p[j] + rank_base;
            D += (long)j + depth_base;
        }
        return (double)p.size() * la + (double)R * lr + (double)D * lg;
    };
    std::priority_queue<Cand, std::vector<Cand>, CandWorse> frontier;
    for (int r = 0; r < k_cfg; ++r) {
        std::vector<int> p{r};
        frontier.push(Cand{logscore(p), p});
    }
    std::vector<std::vector<int>> chosen(1);
    while ((int)chosen.size() < T) {
        Cand best = frontier.top();
        frontier.pop();
        chosen.push_back(best.path);
        if ((int)best.path.size() < K)
            for (int r = 0; r < k_cfg; ++r) {
                std::vector<int> c = best.path;
                c.push_back(r);
                frontier.push(Cand{logscore(c), c});
            }
    }
    return pack_tree(chosen, out);
}

// Path score from an accuracy table: the product of acc[j][r_j] over the path, multiplied
// in path order in double precision (equal paths give bitwise equal products).
static double table_score(const std::vector<int>& p, const double* acc, int k_cfg) {
    double s = 1.0;
    for (size_t j = 0; j < p.size(); ++j) s *= acc[j * k_cfg + p[j]];
    return s;
}

mdt_status mdt_tree_build_table(int K, int k_cfg, int T, const double* acc, mdt_tree_host* out) {
    MDT_REQUIRE(out && acc, MDT_ERR_NULL, "out or acc is NULL");
    MDT_REQUIRE(K >= 1 && K <= MDT_MAX_HEADS, MDT_ERR_SHAPE, "K=%d out of range 1..%d", K, MDT_MAX_HEADS);
    MDT_REQUIRE(k_cfg >= 1 && k_cfg <= MDT_MAX_TOPK, MDT_ERR_SHAPE, "k_cfg=%d out of range", k_cfg);
    MDT_REQUIRE(T >= 1 && T <= MDT_MAX_NODES, MDT_ERR_SHAPE, "T=%d out of range 1..%d", T, MDT_MAX_NODES);
    for (int i = 0; i < K * k_cfg; ++i)
        MDT_REQUIRE(acc[i] >= 0.0 && acc[i] <= 1.0, MDT_ERR_VALUE, "accuracy %d is not in [0, 1]", i);
    double cands = 0, lvl = 1;
    for (int j = 0; j < K; ++j) {
        lvl *= k_cfg;
        cands += lvl;
    }
    MDT_REQUIRE(T - 1 <= cands, MDT_ERR_SHAPE, "T=%d exceeds the %g candidate nodes", T, cands);
    // A child's product never exceeds its parent's (accuracies <= 1) and ties go to the
    // smaller depth, so the greedy frontier takes the T-1 best paths and stays closed
    // under prefixes.
    std::priority_queue<Cand, std::vector<Cand>, CandWorse> frontier;
    for (int r = 0; r < k_cfg; ++r) {
        std::vector<int> p{r};
        frontier.push(Cand{table_score(p, acc, k_cfg), p});
    }
    std::vector<std::vector<int>> chosen(1);
    while ((int)chosen.size() < T) {
        Cand best = frontier.top();
        frontier.pop();
        chosen.push_back(best.path);
        if ((int)best.path.size() < K)
            for (int r = 0; r < k_cfg; ++r) {
                std::vector<int> c = best.path;
                c.push_back(r);
                frontier.push(Cand{table_score(c, acc, k_cfg), c});
            }
    }
    return pack_tree(chosen, out);
}

mdt_status mdt_tree_expected_length(const mdt_tree_host* t, int K, int k_cfg, const double* acc, double* out) {
    MDT_REQUIRE(t && acc && out, MDT_ERR_NULL, "tree, acc or out is NULL");
    MDT_REQUIRE(t->T >= 1 && t->T <= MDT_MAX_NODES && t->parent && t->depth && t->rank, MDT_ERR_TREE,
                "invalid host tree");
    MDT_REQUIRE(K >= 1 && K <= MDT_MAX_HEADS && k_cfg >= 1 && k_cfg <= MDT_MAX_TOPK, MDT_ERR_SHAPE,
                "K or k_cfg out of range");
    MDT_REQUIRE(t->max_depth <= K && t->max_rank < k_cfg, MDT_ERR_SHAPE, "the table does not cover the tree");
    // E[L] = sum over the non-root nodes of their path products ("Notes on Medusa",
    // section 4); each node's product is its parent's times its own accuracy.
    std::vector<double> prod(t->T, 1.0);
    double e = 0.0;
    for (int i = 1; i < t->T; ++i) {
        const int p = t->parent[i], d = t->depth[i], r = t->rank[i];
        MDT_REQUIRE(p >= 0 && p < i && d >= 1 && d <= K && r >= 0 && r < k_cfg, MDT_ERR_TREE, "invalid node %d", i);
        prod[i] = prod[p] * acc[(d - 1) * k_cfg + r];
        e += prod[i];
    }
    *out = e;
    return MDT_OK;
}

void mdt_tree_free(mdt_tree_host* t) {
    if (!t) return;
    std::free(t->parent);
    std::free(t->depth);
    std::free(t->rank);
    std::free(t->anc);
    std::memset(t, 0, sizeof(*t));
}

static size_t anc_offset(int T) { return ((size_t)3 * T * sizeof(int32_t) + 15) & ~(size_t)15; }

size_t mdt_tree_image_bytes(int T) {
    if (T < 1) return 0;
    return anc_offset(T) + (size_t)T * ((T + 63) / 64) * sizeof(uint64_t);
}

mdt_status mdt_tree_pack(const mdt_tree_host* t, void* dst, size_t bytes) {
    MDT_REQUIRE(t && dst, MDT_ERR_NULL, "tree or dst is NULL");
    MDT_REQUIRE(t->T >= 1 && t->T <= MDT_MAX_NODES && t->parent && t->depth && t->rank && t->anc, MDT_ERR_TREE,
                "invalid host tree");
    MDT_REQUIRE(bytes >= mdt_tree_image_bytes(t->T), MDT_ERR_SHAPE, "image buffer too small");
    const int T = t->T;
    char* d = (char*)dst;
    std::memset(d, 0, mdt_tree_image_bytes(T));
    std::memcpy(d, t->parent, T * sizeof(int32_t));
    std::memcpy(d + T * sizeof(int32_t), t->depth, T * sizeof(int32_t));
    std::memcpy(d + 2 * T * sizeof(int32_t), t->rank, T * sizeof(int32_t));
    std::memcpy(d + anc_offset(T), t->anc, (size_t)T * t->anc_words * sizeof(uint64_t));
    return MDT_OK;
}

mdt_status mdt_tree_dev_init(const mdt_tree_host* t, const void* dev_image, mdt_tree_dev* out) {
    MDT_REQUIRE(t && dev_image && out, MDT_ERR_NULL, "tree, image or out is NULL");
    MDT_REQUIRE(mdt_aligned16(dev_image), MDT_ERR_ALIGN, "tree image must be 16-byte aligned");
    MDT_REQUIRE(t->T >= 1 && t->T <= MDT_MAX_NODES && t->anc_words == (t->T + 63) / 64, MDT_ERR_TREE,
                "invalid host tree");
    const int T = t->T;
    const char* d = (const char*)dev_image;
    out->T = T;
    out->max_depth = t->max_depth;
    out->max_rank = t->max_rank;
    out->anc_words = t->anc_words;
    out->parent = (const int32_t*)d;
    out->depth = (const int32_t*)(d + T * sizeof(int32_t));
    out->rank = (const int32_t*)(d + 2 * T * sizeof(int32_t));
    out->anc = (const uint64_t*)(d + anc_offset(T));
    return MDT_OK;
}

}  // extern "C"

// Validation shared by the calls that take a device tree.
mdt_status mdt_check_tree(const mdt_tree_dev* t) {
    MDT_REQUIRE(t, MDT_ERR_NULL, "tree is NULL");
    MDT_REQUIRE(t->parent && t->depth && t->rank && t->anc, MDT_ERR_NULL, "tree arrays are NULL");
    MDT_REQUIRE(t->T >= 1 && t->T <= MDT_MAX_NODES, MDT_ERR_TREE, "tree T=%d out of range", t->T);
    MDT_REQUIRE(t->anc_words == (t->T + 63) / 64, MDT_ERR_TREE, "tree anc_words inconsistent with T");
    MDT_REQUIRE(t->max_depth >= 0 && t->max_depth < t->T && t->max_depth <= MDT_MAX_HEADS, MDT_ERR_TREE,
                "tree max_depth=%d out of range", t->max_depth);
    MDT_REQUIRE(t->max_rank >= 0 && t->max_rank < MDT_MAX_TOPK, MDT_ERR_TREE, "tree max_rank out of range");
    return MDT_OK;
}
