/*
 * mdt.h -- C ABI of the Medusa draft-and-verify step for AMD Instinct MI355X (gfx950).
 *
 * One verify step is six calls, in this order on one HIP stream:
 *
 *   mdt_medusa_heads      K Medusa heads + LM head on the last hidden state -> logits
 *   mdt_topk_tree_expand  per-head top-k, candidate tokens and position ids of the static tree
 *   mdt_tree_attention    tree-masked attention of the packed tree over the prefix KV cache
 *   mdt_verify_logits     LM head on every tree node -> per-row argmax / log-partition / entropy
 *   mdt_accept_path       greedy or typical acceptance -> longest accepted path
 *   mdt_kv_compact        append the accepted path's keys/values to the cache
 *   mdt_accept_compact    the last two in one launch (same results)
 *   mdt_verify_accept_compact  the last three in two launches (same results)
 *   mdt_next_state        hidden state the next step starts from (multi-step decoding)
 *   mdt_next_logits       the next step's LM-head row, taken from the verifier
 *   mdt_accept_rejection  rejection-sampling acceptance on the tree (a third acceptance rule)
 *   mdt_kv_compact_layers mdt_kv_compact for every layer of a model in one launch
 *   mdt_embed, mdt_rmsnorm, mdt_add_rmsnorm, mdt_linear, mdt_linear_split
 *                         the decoder-layer pieces of the full verify forward
 *
 * The pages this follows are the Medusa pages: "Medusa: Simple LLM Inference
 * Acceleration Framework with Multiple Decoding Heads" (summary page, section 3.2
 * information flow and section 3.4), "Accelerating LLM Inference with Speculative
 * Decoding: Notes on Medusa" and "MEDUSA 精读".  Each call below cites its passage.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Pointers marked "device" are device memory owned by the caller; the library
 *    never frees or retains them past the call.  Pointers marked "host" are read
 *    during the call only.
 *  - Arrays are row-major, shapes written outermost first.  "bf16" is the 16-bit
 *    bfloat16 pattern; accumulation is always fp32.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *    enqueues work and returns; it performs no device->host copy and no
 *    synchronisation.  Launch errors are reported as MDT_ERR_HIP.
 *  - Every call validates its arguments before launching anything; on any error
 *    nothing is launched and nothing is written.  The message of the last error
 *    of the calling thread is returned by mdt_last_error().
 *  - bf16/f32 tensor base pointers must be 16-byte aligned (MDT_ERR_ALIGN).
 *  - Values that only the device knows (prefix lengths, page-table entries, tree
 *    arrays) are bounds-checked in the kernels: an out-of-range value never leads
 *    to an out-of-bounds access; its effect is stated per call.
 *  - Workspace: calls that need scratch take `ws`/`ws_bytes`, at least the size
 *    returned by the matching mdt_*_workspace() query.  Contents need not be
 *    initialised and are undefined afterwards.  Two calls in flight at the same
 *    time must not share a workspace.
 *  - The library allocates no device memory and keeps no global mutable state
 *    apart from thread-local state (the error message and an optional profiling
 *    attachment, see mdt_profile_attach) and a per-device cache of the
 *    compute-unit count, so calls are thread-safe.
 */
#ifndef MDT_H
#define MDT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MDT_ABI_VERSION 1

/* Limits of this implementation. */
#define MDT_MAX_NODES 256   /* tree nodes including the root */
#define MDT_MAX_HEADS 8     /* Medusa heads K */
#define MDT_MAX_TOPK 32     /* per-head top-k */

/* Every enum below is a 32-bit int on both sides of the ABI.  C++ sees each with a fixed
 * underlying type, so that any int32 a C caller passes (an unknown dtype, say) is a valid
 * value of the type, which the argument checks then reject with an error code. */
#ifdef __cplusplus
#define MDT_ENUM(name) enum name : int32_t
#else
#define MDT_ENUM(name) enum name
#endif

typedef MDT_ENUM(mdt_status) {
    MDT_OK = 0,
    MDT_ERR_NULL = -1,        /* a required pointer is NULL */
    MDT_ERR_SHAPE = -2,       /* a size is out of range or sizes are inconsistent */
    MDT_ERR_DTYPE = -3,       /* unknown dtype */
    MDT_ERR_ALIGN = -4,       /* a tensor base pointer is not 16-byte aligned */
    MDT_ERR_TREE = -5,        /* invalid tree description */
    MDT_ERR_VALUE = -6,       /* a scalar parameter is out of range */
    MDT_ERR_WORKSPACE = -7,   /* workspace NULL or too small */
    MDT_ERR_HIP = -8,         /* the HIP runtime reported an error */
    MDT_ERR_UNSUPPORTED = -9, /* valid request the library does not implement */
    MDT_ERR_ALLOC = -10       /* host allocation failed */
} mdt_status;

typedef MDT_ENUM(mdt_dtype) {
    MDT_F32 = 0,   /* float32 storage */
    MDT_BF16 = 1   /* bfloat16 storage */
} mdt_dtype;

typedef MDT_ENUM(mdt_accept_mode) {
    MDT_ACCEPT_GREEDY = 0,
    MDT_ACCEPT_TYPICAL = 1
} mdt_accept_mode;

typedef MDT_ENUM(mdt_act) {
    MDT_ACT_NONE = 0,   /* mdt_linear: plain product */
    MDT_ACT_SWIGLU = 1  /* mdt_linear: SwiGLU of an interleaved gate/up product */
} mdt_act;

typedef MDT_ENUM(mdt_kv_layout) {
    MDT_KV_CONTIG = 0,  /* k,v: [B][capacity][H][Dh] */
    MDT_KV_PAGED = 1    /* k,v: [num_pages][page_size][H][Dh] + page_table [B][max_pages] */
} mdt_kv_layout;

/* ------------------------------------------------------------------------- */
/* Static candidate tree                                                      */
/* ------------------------------------------------------------------------- */

/*
 * A tree node is a rank path (r_1..r_l): the depth-l node carries the rank-r_l
 * candidate of Medusa head l and extends the node (r_1..r_{l-1}).  The root
 * (depth 0) carries the LM head's top token.  Nodes are packed breadth-first:
 * root, then by depth, then by rank path, so parent[i] < i.
 *
 * Host form, owned by the library from a successful mdt_tree_build_* until
 * mdt_tree_free().
 */
typedef struct mdt_tree_host {
    int32_t T;          /* nodes including the root, 1..MDT_MAX_NODES */
    int32_t max_depth;  /* depth of the deepest node */
    int32_t max_rank;   /* largest rank used at any depth (top-k must exceed it) */
    int32_t anc_words;  /* 64-bit words per ancestor-mask row: ceil(T/64) */
    int32_t* parent;    /* [T]; parent[0] = -1 */
    int32_t* depth;     /* [T] */
    int32_t* rank;      /* [T]; 0 for the root */
    uint64_t* anc;      /* [T][anc_words]: bit j of row i set iff node j is i or an ancestor of i */
} mdt_tree_host;

/*
 * Device form: the arrays of a packed image (see mdt_tree_image_bytes) in device
 * memory, plus host-side scalars used for validation and launch sizes.
 */
typedef struct mdt_tree_dev {
    int32_t T;
    int32_t max_depth;
    int32_t max_rank;
    int32_t anc_words;
    const int32_t* parent;  /* device [T] */
    const int32_t* depth;   /* device [T] */
    const int32_t* rank;    /* device [T] */
    const uint64_t* anc;    /* device [T][anc_words] */
} mdt_tree_dev;

/*
 * Cartesian-product tree: every rank path with r_j < s[j-1], depth <= K.
 * Summary page, section "Tree Attention", steps 1-2 (level k holds prod_{i<=k} s_i
 * nodes); "Notes on Medusa", section 3 (node count).  Host-only.
 * Errors: MDT_ERR_NULL (s or out), MDT_ERR_SHAPE (K < 0 or > MDT_MAX_HEADS, s[j] < 1
 * or > MDT_MAX_TOPK, total nodes > MDT_MAX_NODES), MDT_ERR_ALLOC.
 */
mdt_status mdt_tree_build_cartesian(int K, const int* s, mdt_tree_host* out);

/*
 * Sparse tree: the T-1 best rank paths (depth <= K, ranks < k_cfg) by path score
 * prod_j a0 * rho^(r_j + rank_base) * gamma^(j - 1 + depth_base), found by the
 * greedy frontier construction of the summary page, section "Optimized Tree
 * Construction", steps 2-4, and "Notes on Medusa", section 4.  Scores are compared
 * as j-sums of logarithms in double precision; ties go to the smaller depth, then
 * to the lexicographically smaller rank path.  Host-only.
 * Errors: MDT_ERR_NULL, MDT_ERR_SHAPE (T < 1 or > MDT_MAX_NODES or more than the
 * candidate count, K or k_cfg out of range), MDT_ERR_VALUE (a0, rho, gamma not in
 * (0, 1]), MDT_ERR_ALLOC.
 */
mdt_status mdt_tree_build_scored(int K, int k_cfg, int T, double a0, double rho, double gamma,
                                 int rank_base, int depth_base, mdt_tree_host* out);

/*
 * Sparse tree from a calibrated accuracy table: acc[j][r] (host, [K][k_cfg], values in
 * [0, 1]) is the accuracy of the rank-r candidate of head j+1 -- the top-(r+1) accuracy
 * minus the top-r accuracy (summary page, section "Optimized Tree Construction", step
 * 1).  Under the pages' independence assumption (step 2) a path's score is the product
 * of its nodes' accuracies; the tree keeps the T-1 best rank paths by the greedy frontier
 * of steps 3-4 ("Notes on Medusa", section 4), which maximises the expected acceptance
 * length among trees of T nodes.  Products are formed in path order in double precision;
 * ties go to the smaller depth, then to the lexicographically smaller rank path.
 * Host-only.  Errors: MDT_ERR_NULL, MDT_ERR_SHAPE (as mdt_tree_build_scored),
 * MDT_ERR_VALUE (an accuracy outside [0, 1]), MDT_ERR_ALLOC.
 */
mdt_status mdt_tree_build_table(int K, int k_cfg, int T, const double* acc, mdt_tree_host* out);

/*
 * Expected acceptance length of a tree under an accuracy table (as above): the sum over
 * the non-root nodes of the product of the accuracies on their root paths ("Notes on
 * Medusa", section 4: E[L] = sum_m P(L >= m)).  Host-only; *out in double precision.
 * Errors: MDT_ERR_NULL, MDT_ERR_TREE (an inconsistent tree), MDT_ERR_SHAPE (K, k_cfg out
 * of range or not covering the tree's depth and ranks).
 */
mdt_status mdt_tree_expected_length(const mdt_tree_host* tree, int K, int k_cfg, const double* acc, double* out);

/* Release the arrays of a host tree (safe on a zeroed struct). */
void mdt_tree_free(mdt_tree_host* tree);

/* Bytes of the packed image of a host tree: parent, depth, rank (int32) then anc (uint64, 8-aligned). */
size_t mdt_tree_image_bytes(int T);

/*
 * Write the packed image of `tree` into host buffer `dst` (>= mdt_tree_image_bytes(T)).
 * The caller copies it to device memory and calls mdt_tree_dev_init on that copy.
 * Errors: MDT_ERR_NULL, MDT_ERR_SHAPE (bytes too small).
 */
mdt_status mdt_tree_pack(const mdt_tree_host* tree, void* dst, size_t bytes);

/*
 * Fill `out` with pointers into a device copy `dev_image` of a packed image and
 * the scalars of `tree`.  Errors: MDT_ERR_NULL, MDT_ERR_ALIGN (dev_image not
 * 16-byte aligned), MDT_ERR_TREE.
 */
mdt_status mdt_tree_dev_init(const mdt_tree_host* tree, const void* dev_image, mdt_tree_dev* out);

/* ------------------------------------------------------------------------- */
/* 1. Heads                                                                   */
/* ------------------------------------------------------------------------- */

/*
 * logits[b][0][:] = Wlm h_b  and  logits[b][k][:] = W2_k (SiLU(W1_k h_b) + h_b), k = 1..K.
 * Summary page, section "MEDUSA Heads" (head equation; the residual is inside W2;
 * no biases) and section 3.2 (the LM head gives the next token, head k the token
 * k+1 further).  Softmax is omitted: it is monotone and the verifier recomputes
 * probabilities where needed.
 *
 *  dt      MDT_F32 or MDT_BF16: storage of h and all weights
 *  B,d,V,K sequences (1..1024), hidden size (multiple of 8), vocabulary (>= 1), heads (1..MDT_MAX_HEADS)
 *  h       device [B][d]
 *  W1      device [K][d][d]   W1[k][out][in]
 *  W2      device [K][V][d]   row v of head k
 *  Wlm     device [V][d], or NULL: slot 0 is then not written (a chained step whose slot 0
 *          already holds the LM-head row of its hidden state, see mdt_next_logits)
 *  logits  device f32 [B][K+1][V]  (output; slot 0 = LM head)
 *  ws      device workspace >= mdt_medusa_heads_workspace(B, d, K) bytes; holds the fp32
 *          head activations a[B][K][d] between the two kernels
 */
size_t mdt_medusa_heads_workspace(int B, int d, int K);
mdt_status mdt_medusa_heads(void* stream, mdt_dtype dt, int B, int d, int V, int K,
                            const void* h, const void* W1, const void* W2, const void* Wlm,
                            float* logits, void* ws, size_t ws_bytes);

/*
 * mdt_medusa_heads without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  It allocates nothing; the head activations live in a fixed array
 * of MDT_HEADS_NOALLOC_MAX_BYTES in device memory that the library holds on every GPU it
 * runs on until the process ends (its address is looked up once per device, on the
 * first call made with that device current).  Every call on one GPU shares that array
 * and leaves its last contents there: calls that overlap on one GPU (two streams, two
 * threads) race and must be ordered by the caller.  Nothing in it needs clearing (the
 * first kernel writes every activation the second reads).  Arguments, layouts and
 * results as mdt_medusa_heads.
 * Errors: as mdt_medusa_heads; MDT_ERR_WORKSPACE when B*K*d*4 bytes exceed
 * MDT_HEADS_NOALLOC_MAX_BYTES (checked first, before any HIP call); MDT_ERR_HIP when the
 * array's device address cannot be obtained.
 */
#define MDT_HEADS_NOALLOC_MAX_BYTES (4u << 20)
mdt_status mdt_medusa_heads_noalloc(void* stream, mdt_dtype dt, int B, int d, int V, int K,
                                    const void* h, const void* W1, const void* W2, const void* Wlm,
                                    float* logits);

/* ------------------------------------------------------------------------- */
/* 2. Top-k and tree expansion                                                */
/* ------------------------------------------------------------------------- */

/*
 * For every (b, head row r = 0..K): the k_cfg largest logits, value descending,
 * equal values by smaller index (summary page, "Tree Attention", step 1).  Then
 * for every node i of the tree: tree_tokens[b][i] = topk_idx[b][depth(i)][rank(i)]
 * (the root takes the LM head's top token, step 2 and section 3.2) and
 * pos_ids[b][i] = prefix_len[b] + depth(i) (step 4; positions 0-based, prefix at
 * 0..L-1).
 *
 *  logits       device f32 [B][K+1][V]
 *  tree         device tree; tree->max_depth <= K and tree->max_rank < k_cfg
 *  prefix_len   device int32 [B]
 *  topk_idx     device int32 [B][K+1][k_cfg] (output)
 *  topk_val     device f32   [B][K+1][k_cfg] (output)
 *  tree_tokens  device int32 [B][T] (output)
 *  pos_ids      device int32 [B][T] (output)
 *  ws           >= mdt_topk_workspace(B, K, V, k_cfg) bytes
 * k_cfg in 1..MDT_MAX_TOPK and <= V.  NaN logits are not supported.
 */
size_t mdt_topk_workspace(int B, int K, int V, int k_cfg);
mdt_status mdt_topk_tree_expand(void* stream, int B, int K, int V, int k_cfg,
                                const float* logits, const mdt_tree_dev* tree, const int32_t* prefix_len,
                                int32_t* topk_idx, float* topk_val, int32_t* tree_tokens, int32_t* pos_ids,
                                void* ws, size_t ws_bytes);

/* ------------------------------------------------------------------------- */
/* 3. Tree attention                                                          */
/* ------------------------------------------------------------------------- */

typedef struct mdt_kv_cache {
    int32_t layout;      /* mdt_kv_layout */
    int32_t capacity;    /* CONTIG: slots per sequence; PAGED: must equal max_pages * page_size */
    int32_t page_size;   /* PAGED: tokens per page (1..1024) */
    int32_t max_pages;   /* PAGED: columns of page_table */
    int32_t num_pages;   /* PAGED: physical pages in the pool */
    int32_t reserved;
    void* k;             /* device, see mdt_kv_layout; same dtype as the call */
    void* v;             /* device */
    const int32_t* page_table;  /* PAGED: device int32 [B][max_pages]; entries < 0 = unmapped */
} mdt_kv_cache;

/*
 * For every sequence b, head h and tree node i:
 *   o[b][i][h] = sum_j softmax_j(q'_i . k_j / sqrt(Dh)) v_j
 * over the prefix keys j < prefix_len[b] (already rotated when cached) and the
 * tree nodes j that are i or an ancestor of i (summary page, "Tree Attention",
 * step 3: the mask allows ancestors only; "Notes on Medusa", section 3).  q' and
 * the tree keys are rotated (RoPE, half-split pairs, angle pos * theta^(-2m/Dh))
 * at pos = prefix_len[b] + depth(i) (step 4).
 *
 *  dt         storage of q, k, v, cache, out, k_rot
 *  H, Dh      heads (>= 1), head dim (MDT_F32: 2..256 even; MDT_BF16: 128)
 *  q, k, v    device [B][T][H][Dh], tree queries/keys/values before rotation
 *  cache      host struct describing the device prefix cache
 *  prefix_len device int32 [B]; values outside [0, capacity] make the kernel use
 *             min(max(L, 0), capacity)
 *  rope_theta > 0
 *  out        device [B][T][H][Dh] (output) == [B*T][H*Dh], the verifier input
 *  k_rot      device [B][T][H][Dh] (output) rotated tree keys, as stored in the cache
 *  ws         >= mdt_tree_attention_workspace(dt, B, T, H, Dh, cache->capacity) bytes
 * Unmapped or out-of-pool pages read as zeros.
 */
size_t mdt_tree_attention_workspace(mdt_dtype dt, int B, int T, int H, int Dh, int capacity);
mdt_status mdt_tree_attention(void* stream, mdt_dtype dt, int B, int H, int Dh, const mdt_tree_dev* tree,
                              const void* q, const void* k, const void* v, const mdt_kv_cache* cache,
                              const int32_t* prefix_len, float rope_theta, void* out, void* k_rot,
                              void* ws, size_t ws_bytes);

/* ------------------------------------------------------------------------- */
/* 4. Verifier logits                                                         */
/* ------------------------------------------------------------------------- */

typedef struct mdt_row_stats {
    float max;       /* largest logit */
    int32_t argmax;  /* its index (smallest index among equal maxima) */
    float logZ;      /* log sum_v exp(z_v / tau); 0 when tau == 0 */
    float entropy;   /* entropy (nats) of softmax(z / tau); 0 when tau == 0 */
} mdt_row_stats;

/*
 * z_r = Wlm x_r for every row r = b*T + i of x (the node outputs, heads
 * concatenated), then per row the statistics above, and for every non-root node
 * c the edge logit edge_logit[b][c] = z_{b*T+parent(c)}[tree_tokens[b][c]]
 * (edge_logit[b][0] = 0).  Summary page, "Tree Attention", steps 5-6; "Notes on
 * Medusa", section 3 (node outputs pass through the LM head); "Typical
 * Acceptance Scheme" (entropy in nats).
 *
 *  dt           storage of x and Wlm
 *  B, T, d, V   rows = B*T
 *  x            device [B*T][d]
 *  Wlm          device [V][d]
 *  tree         device tree (T nodes)
 *  tree_tokens  device int32 [B][T]; tokens outside [0, V) give edge logit -inf
 *  temperature  tau >= 0
 *  stats        device [B*T] (output)
 *  edge_logit   device f32 [B][T] (output)
 *  logits_opt   device f32 [B*T][V] or NULL: full verifier logits (output)
 *  ws           >= mdt_verify_logits_workspace(dt, B, T, d, V) bytes
 */
size_t mdt_verify_logits_workspace(mdt_dtype dt, int B, int T, int d, int V);
mdt_status mdt_verify_logits(void* stream, mdt_dtype dt, int B, int T, int d, int V,
                             const void* x, const void* Wlm, const mdt_tree_dev* tree,
                             const int32_t* tree_tokens, float temperature, mdt_row_stats* stats,
                             float* edge_logit, float* logits_opt, void* ws, size_t ws_bytes);

/* ------------------------------------------------------------------------- */
/* 5. Acceptance                                                              */
/* ------------------------------------------------------------------------- */

/*
 * Per sequence: a non-root node c with parent p passes if
 *   GREEDY:  tree_tokens[c] == argmax of row p;
 *   TYPICAL: p_tau(token c | p) > min(eps, delta * exp(-H_p)), tested as
 *            edge/tau - logZ_p > min(ln eps, ln delta - H_p); at tau == 0 the
 *            verifier distribution is one-hot at the argmax.
 * (Summary page, "Typical Acceptance Scheme": criterion, entropy in nats,
 * temperature-0 behaviour, first token accepted unconditionally, longest accepted
 * prefix among all branches; "Notes on Medusa", section 3 for greedy.)
 * The root always passes; a node is accepted iff every node on its root path
 * passes.  The chosen node is the deepest accepted node (equal depth: smaller
 * packed index).  path[b][0..n-1] is its root path, n_acc[b] = n (>= 1);
 * path[b][n..path_stride-1] = -1.
 *
 *  stats, edge_logit, tree_tokens  device outputs of the previous calls
 *  mode         mdt_accept_mode
 *  eps, delta   > 0 (TYPICAL)
 *  temperature  >= 0
 *  path         device int32 [B][path_stride] (output), path_stride >= tree->max_depth + 1
 *  n_acc        device int32 [B] (output)
 */
mdt_status mdt_accept_path(void* stream, int B, const mdt_tree_dev* tree, const mdt_row_stats* stats,
                           const float* edge_logit, const int32_t* tree_tokens, int mode, float eps,
                           float delta, float temperature, int32_t* path, int path_stride, int32_t* n_acc);

/* ------------------------------------------------------------------------- */
/* 6. KV compaction                                                           */
/* ------------------------------------------------------------------------- */

/*
 * For every sequence b and j < n_acc[b]: cache slot prefix_len[b] + j receives
 * k_rot[b][path[b][j]] and v[b][path[b][j]]; new_prefix_len[b] = prefix_len[b] + n_acc[b].
 * Only the accepted path's keys/values are kept ("MEDUSA 精读", section 3 and the
 * implementation checklist of section 6).  The stored key already carries
 * position prefix_len + j because node path[j] has depth j.
 *
 *  k_rot, v        device [B][T][H][Dh] (outputs / inputs of mdt_tree_attention)
 *  path, n_acc     device, from mdt_accept_path (path_stride as there)
 *  cache           host struct of the device cache (written)
 *  prefix_len      device int32 [B]
 *  new_prefix_len  device int32 [B] (output); -1 for a sequence whose path, length
 *                  or destination slots are out of range, in which case nothing of
 *                  that sequence is written
 */
mdt_status mdt_kv_compact(void* stream, mdt_dtype dt, int B, int T, int H, int Dh, const int32_t* path,
                          int path_stride, const int32_t* n_acc, const void* k_rot, const void* v,
                          const mdt_kv_cache* cache, const int32_t* prefix_len, int32_t* new_prefix_len);

/*
 * mdt_accept_path followed by mdt_kv_compact in one launch: one workgroup per
 * sequence selects the path and appends its keys/values to the cache (the end of
 * a step on the summary page, section 3.2, and "MEDUSA 精读", section 3).  Every
 * output -- path, n_acc, the cache rows, new_prefix_len -- is exactly what the two
 * calls write in sequence with the same arguments; the arguments are those of the
 * two calls (T is tree->T), with the same checks and error codes.
 */
mdt_status mdt_accept_compact(void* stream, mdt_dtype dt, int B, int H, int Dh, const mdt_tree_dev* tree,
                              const mdt_row_stats* stats, const float* edge_logit, const int32_t* tree_tokens,
                              int mode, float eps, float delta, float temperature, int32_t* path, int path_stride,
                              int32_t* n_acc, const void* k_rot, const void* v, const mdt_kv_cache* cache,
                              const int32_t* prefix_len, int32_t* new_prefix_len);

/*
 * mdt_verify_logits, mdt_accept_path and mdt_kv_compact in two launches: the verifier's
 * tile kernel, then one workgroup per sequence that merges its rows' statistics, selects
 * the accepted path and appends its keys and values to the cache (the end of one
 * iteration: summary page, section 3.2, and "Tree Attention" steps 5-6).  Every output --
 * stats, edge_logit, logits_opt, path, n_acc, the cache rows, new_prefix_len -- is exactly
 * what the three calls write in sequence with the same arguments (one temperature serves
 * the verifier and the acceptance).  Arguments as in those calls, with x [B*T][d] the node
 * outputs and k_rot, v [B][T][H][Dh]; ws >= mdt_verify_logits_workspace(dt, B, T, d, V).
 * Every check of the three calls runs before the first launch, with the same error codes.
 */
mdt_status mdt_verify_accept_compact(void* stream, mdt_dtype dt, int B, int T, int d, int V, int H, int Dh,
                                     const void* x, const void* Wlm, const mdt_tree_dev* tree,
                                     const int32_t* tree_tokens, float temperature, int mode, float eps, float delta,
                                     mdt_row_stats* stats, float* edge_logit, float* logits_opt, int32_t* path,
                                     int path_stride, int32_t* n_acc, const void* k_rot, const void* v,
                                     const mdt_kv_cache* cache, const int32_t* prefix_len, int32_t* new_prefix_len,
                                     void* ws, size_t ws_bytes);

/*
 * Rejection-sampling acceptance on the tree.  "Accelerating LLM Inference with
 * Speculative Decoding: Notes on Medusa", section 2, and the summary page, section
 * "Typical Acceptance Scheme" (first paragraph): a candidate x drafted with
 * probability q(x) is accepted with probability min(1, p(x)/q(x)); after a rejection
 * the token is drawn from norm(max(0, p - q)).  On the tree: starting at the root
 * (always accepted), the children of the current node are tried in rank order; p is
 * the verifier distribution softmax(z/temperature) of the current node, q the
 * softmax(logits/temperature) of the head whose candidates they are (row depth+1 of
 * head_logits); child c is accepted iff u_accept[b][c] < min(1, r(x_c)/q(x_c)), r the
 * current residual (p at first; each rejection replaces r by norm(max(0, r - q))).
 * An accepted child becomes the current node.  When no child is accepted (or the node
 * is a leaf) the next token is the first vocabulary entry whose running sum of r
 * exceeds u_resample[b] times the total; it is -1 if a rejection left r without mass.
 * The random numbers are inputs, so the call is deterministic.
 *  B, V, K       sequences, vocabulary (1..32768, else MDT_ERR_UNSUPPORTED), heads
 *  tree          device tree; tree->max_depth <= K
 *  vlogits       device f32 [B*T][V]: verifier logits of every node (the logits_opt
 *                output of mdt_verify_logits)
 *  head_logits   device f32 [B][K+1][V]: the output of mdt_medusa_heads
 *  tree_tokens   device int32 [B][T]; a token outside 0..V-1 is never accepted
 *  temperature   > 0
 *  u_accept      device f32 [B][T], values in [0, 1) (entry c is used when child c is tried)
 *  u_resample    device f32 [B], values in [0, 1)
 *  path          device int32 [B][path_stride] (output), max_depth + 1 <= path_stride <= 1024;
 *                root..last accepted node, then -1
 *  n_acc         device int32 [B] (output): accepted node count (>= 1)
 *  next_token    device int32 [B] (output): the token drawn after the accepted path
 * The accepted path feeds mdt_kv_compact unchanged.
 * Errors: MDT_ERR_SHAPE, MDT_ERR_TREE, MDT_ERR_VALUE (temperature), MDT_ERR_NULL,
 * MDT_ERR_UNSUPPORTED (V > 32768).
 */
mdt_status mdt_accept_rejection(void* stream, int B, int V, int K, const mdt_tree_dev* tree, const float* vlogits,
                                const float* head_logits, const int32_t* tree_tokens, float temperature,
                                const float* u_accept, const float* u_resample, int32_t* path, int path_stride,
                                int32_t* n_acc, int32_t* next_token);

/*
 * Hidden state of the next step: h_next[b] = x[b][path[b][n_acc[b] - 1]], the node
 * output of sequence b's deepest accepted node.  The summary page, section 3.2, has the
 * next iteration continue from the last accepted token, whose hidden state feeds the
 * heads and whose LM-head row gives the next root; with x the node outputs that
 * mdt_verify_logits consumed, this row is exactly that hidden state.
 *  dt           MDT_BF16 or MDT_F32: storage type of x and h_next
 *  B, T, d      sequences, tree nodes (1..MDT_MAX_NODES), hidden size; d * element size
 *               must be a multiple of 16 bytes
 *  x            device [B][T][d] node outputs (the tree-attention output viewed as rows)
 *  path, path_stride, n_acc
 *               device, as written by mdt_accept_path / mdt_accept_compact
 *  h_next       device [B][d] (output; must not overlap x)
 * A sequence whose n_acc is outside 1..path_stride or whose last path node is outside
 * 0..T-1 gets a row of zeros.
 * Errors: MDT_ERR_DTYPE, MDT_ERR_SHAPE, MDT_ERR_NULL, MDT_ERR_ALIGN.
 */
mdt_status mdt_next_state(void* stream, mdt_dtype dt, int B, int T, int d, const void* x, const int32_t* path,
                          int path_stride, const int32_t* n_acc, void* h_next);

/*
 * LM-head slot of the next step: head_logits[b][0][:] = vlogits[b*T + path[b][n_acc[b] - 1]][:].
 * The next step's hidden state is that node's output (mdt_next_state), and its LM-head
 * row W_lm h_next is the verifier row mdt_verify_logits already computed for the node
 * (summary page, section 3.2: the next root is the original model's prediction at the
 * last accepted token).  A chained step can then call mdt_medusa_heads with Wlm = NULL
 * and skip one stream of W_lm.
 *  B, T, V, K   sequences, tree nodes (1..MDT_MAX_NODES), vocabulary, heads
 *  vlogits      device f32 [B*T][V]: the full logits output of mdt_verify_logits
 *  path, path_stride, n_acc
 *               device, as written by mdt_accept_path / mdt_accept_compact
 *  head_logits  device f32 [B][K+1][V]; only slot 0 of each sequence is written; must not
 *               overlap vlogits
 * A sequence whose n_acc is outside 1..path_stride or whose last path node is outside
 * 0..T-1 gets a row of zeros.
 * Errors: MDT_ERR_SHAPE, MDT_ERR_NULL, MDT_ERR_VALUE (overlap).
 */
mdt_status mdt_next_logits(void* stream, int B, int T, int V, int K, const float* vlogits, const int32_t* path,
                           int path_stride, const int32_t* n_acc, float* head_logits);

/*
 * mdt_kv_compact for a model of n_layers layers in one launch: layer l reads
 * k_rot + l*k_rot_layer_stride and v + l*v_layer_stride and writes the cache whose
 * k and v pointers are offset by l*cache_layer_stride (strides in elements, each a
 * multiple of 16 bytes, and at least one layer when n_layers > 1).  Every layer keeps
 * the same accepted path (the verify forward of the "Tree Attention" steps runs the
 * whole backbone on the tree, so each layer holds keys/values for every node).
 * Layer l's writes are exactly those of mdt_kv_compact on layer l's pointers.
 * Errors: as mdt_kv_compact, plus MDT_ERR_SHAPE (n_layers outside 1..65535, strides
 * smaller than one layer) and MDT_ERR_ALIGN (strides).
 */
mdt_status mdt_kv_compact_layers(void* stream, mdt_dtype dt, int n_layers, int B, int T, int H, int Dh,
                                 const int32_t* path, int path_stride, const int32_t* n_acc, const void* k_rot,
                                 long long k_rot_layer_stride, const void* v, long long v_layer_stride,
                                 const mdt_kv_cache* cache, long long cache_layer_stride,
                                 const int32_t* prefix_len, int32_t* new_prefix_len);

/* ------------------------------------------------------------------------- */
/* 7. Decoder layers of the verify forward (bf16 only)                        */
/* ------------------------------------------------------------------------- */

/*
 * The summary page (section 3.2 step 4; "Tree Attention" steps 3-5) runs the packed
 * tree through the whole backbone in one forward pass before the LM head, and
 * "Notes on Medusa", section 3, feeds the node outputs of that pass to the LM head.
 * The pages name the backbone (Vicuna, a Llama model) without giving its layer.  These
 * calls are the pieces of the Llama decoder layer: with M = B*T tree rows,
 *   x    = embed(tree_tokens)
 *   per layer:  h = rmsnorm(x, g_attn); q|k|v = h Wqkv^T (three segments);
 *               o = mdt_tree_attention(q, k, v); x = x + o Wo^T;
 *               h = rmsnorm(x, g_mlp); a = silu(h Wg^T) * (h Wu^T); x = x + a Wd^T
 * (the products with few output columns as mdt_linear_split, their residual add fused
 * into the next RMSNorm by mdt_add_rmsnorm)
 *   xf   = rmsnorm(x, g_final) -> mdt_verify_logits
 * Every matrix is bf16 and every product accumulates in fp32; each call rounds its
 * output to bf16 once.
 */

/*
 * y[m][:] = E[tokens[m]][:] for m < M (a token outside 0..V-1 gives a zero row).
 *  tokens  device int32 [M]; E device bf16 [V][d]; y device bf16 [M][d]; d % 8 == 0.
 * Errors: MDT_ERR_SHAPE, MDT_ERR_NULL, MDT_ERR_ALIGN (E, y).
 */
mdt_status mdt_embed(void* stream, int M, int d, int V, const int32_t* tokens, const void* E, void* y);

/*
 * y[m][j] = bf16(x[m][j] * r_m * g[j]), r_m = 1/sqrt(mean_j x[m][j]^2 + eps) (fp32).
 *  x device bf16 [M][d]; g device bf16 [d]; y device bf16 [M][d] (may equal x); d % 8 == 0.
 * Errors: MDT_ERR_SHAPE, MDT_ERR_VALUE (eps < 0), MDT_ERR_NULL, MDT_ERR_ALIGN.
 */
mdt_status mdt_rmsnorm(void* stream, int M, int d, const void* x, const void* g, float eps, void* y);

/*
 * The residual add that closes a split product, then the next RMSNorm:
 *   x[m][j] = bf16(x[m][j] + part[0][m][j] + ... + part[nparts-1][m][j])  (fp32 sum, in order)
 *   y[m][j] = bf16(x[m][j] * r_m * g[j])  with r_m of the updated row, as mdt_rmsnorm.
 *  part  device f32 [nparts][M][d] (1 <= nparts <= 64), e.g. from mdt_linear_split; must
 *        not overlap x
 *  x     device bf16 [M][d], read and written; y device bf16 [M][d], not x.
 * Errors: as mdt_rmsnorm, plus MDT_ERR_VALUE (nparts, overlap).
 */
mdt_status mdt_add_rmsnorm(void* stream, int M, int d, int nparts, const float* part, void* x, const void* g,
                           float eps, void* y);

/*
 * z = x W^T with x device bf16 [M][K] and W device bf16 [N][K] (fp32 accumulation), then
 *  act == MDT_ACT_NONE:   y[q][m][j] = bf16(z[m][q*N/nseg + j] (+ residual[m][q*N/nseg + j]))
 *                         for the nseg column segments q (y is nseg matrices [M][N/nseg]
 *                         back to back; with nseg == 1 simply [M][N]).  residual is
 *                         device bf16 [M][N] or NULL (then nseg may be > 1); y may be
 *                         the residual buffer itself, never x.
 *  act == MDT_ACT_SWIGLU: W holds gate and up rows interleaved in groups of 16: rows
 *                         32i..32i+15 are gate rows 16i.., rows 32i+16..32i+31 the up
 *                         rows 16i..; y device bf16 [M][N/2] with
 *                         y[m][16i + c] = bf16(silu(z[m][32i + c]) * z[m][32i + 16 + c]),
 *                         silu(u) = u / (1 + e^-u).  N % 32 == 0, no residual, nseg == 1.
 *  K % 32 == 0, N % 8 == 0, N/nseg % 8 == 0.
 * Errors: MDT_ERR_SHAPE, MDT_ERR_VALUE (act, residual with nseg > 1 or with SwiGLU),
 * MDT_ERR_NULL, MDT_ERR_ALIGN.
 */
mdt_status mdt_linear(void* stream, int M, int N, int K, const void* x, const void* W, const void* residual,
                      int nseg, int act, void* y);

/*
 * The inner dimension cut into nsplit slices of ks = ceil(K/nsplit) rounded up to a
 * multiple of 32 (the last slice shorter): part[s][m][n] = sum over k in slice s of
 * x[m][k] W[n][k], fp32, no rounding.  A product whose output has too few 64 x 64
 * tiles to fill the GPU runs on nsplit times as many workgroups this way; the slices
 * are added by mdt_add_rmsnorm.
 *  x, W as mdt_linear; part device f32 [nsplit][M][N]; 1 <= nsplit <= 64, nsplit*32 <= K
 *  and the rounding of ks must leave exactly nsplit slices.
 * Errors: MDT_ERR_SHAPE, MDT_ERR_VALUE (nsplit), MDT_ERR_NULL, MDT_ERR_ALIGN.
 */
mdt_status mdt_linear_split(void* stream, int M, int N, int K, const void* x, const void* W, int nsplit,
                            float* part);

/* ------------------------------------------------------------------------- */
/* Misc                                                                       */
/* ------------------------------------------------------------------------- */

int mdt_abi_version(void);

/*
 * Kernel timing hook (instrumentation, not part of the step).  While attached on
 * the calling thread, launch i of the library (counting from 0) is made with
 * hipExtLaunchKernelGGL and the start/stop events events[2i], events[2i+1], which
 * the runtime stamps when that kernel starts and ends on its stream; launches whose
 * pair lies beyond `capacity` events record nothing.  The caller creates the
 * events (hipEvent_t, timing enabled), reads hipEventElapsedTime(start, stop) of
 * each pair after synchronising, and names launch i with mdt_profile_kernel(i).
 * Errors: MDT_ERR_NULL (events NULL with capacity > 0), MDT_ERR_SHAPE (capacity < 0).
 */
mdt_status mdt_profile_attach(void** events, int capacity);
/* Stop recording; returns the number of launches seen since attach. */
int mdt_profile_detach(void);
/* Name of the kernel of launch i since the last attach ("" if out of range). */
const char* mdt_profile_kernel(int i);
const char* mdt_status_string(int status);
/* Message of the last failed call on this thread ("" if none). */
const char* mdt_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MDT_H */
