// mdt_tree_attention: tree-masked attention of the packed candidate tree.
//
// Summary page "Medusa: Simple LLM Inference Acceleration Framework with Multiple
// Decoding Heads", section "Tree Attention": step 3 (a node attends to the prefix
// and to its ancestors only; the node itself is included), step 4 (position id
// = prefix length + depth, rotary embedding as in Llama) and step 5 (one pass
// over all nodes).  "Notes on Medusa", section 3: the tree is flattened into
// one sequence and masked.
//
// bf16 path (Dh = 128), two kernels:
//  1. attn_stream: split-KV flash pass.  A workgroup owns one (sequence, head, prefix
//     key range); its waves own 16 or 32 tree queries each, rotated in registers (angles
//     from a per-depth cos/sin table in LDS).  64-key K and V tiles stream into an LDS
//     ring by direct global-to-LDS loads and both products run on MFMA 16x16x32 bf16:
//     S^T = K Q^T, then O^T = V^T P^T, so the probabilities stay in registers between the
//     two.  Online softmax keeps (max, sum) per query, the max in log2 units (scores scaled
//     by log2 e, exponentials by exp2).  The workgroup of the first key range then rotates
//     the tree keys at their depth positions (writing k_rot, which is what gets cached) and
//     attends to them under the ancestor-or-self bitmask.  Partial (m, l, O) go to the
//     workspace.
//  2. attn_combine: per (sequence, head, node) merge the partials, write o (bf16).
// fp32 path: one wave per (sequence, head, node) walks all allowed keys on VALU.
#include <math.h>

#include <cmath>

#include "common.h"
#include "dma_tile.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kTile = 64;          // keys per LDS tile
constexpr int kDh = 128;           // head dim of the MFMA path
constexpr int kMaxTilesPerSplit = (2048 - 2) / kTile;  // page-table entries of a split fit kStreamPages
                                                            // (page_size >= 1)

struct KV {
    const void* k;
    const void* v;
    const int32_t* table;
    int layout, capacity, page_size, max_pages, num_pages;
};

// Element offset of key slot j of sequence b, head h (or -1 if unmapped).
__device__ __forceinline__ long kv_offset(const KV& c, int b, int j, int h, int H, int Dh) {
    if (c.layout == MDT_KV_CONTIG) return (((long)b * c.capacity + j) * H + h) * Dh;
    const int pg = j / c.page_size;
    const int page = (pg < c.max_pages) ? c.table[(long)b * c.max_pages + pg] : -1;
    if (page < 0 || page >= c.num_pages) return -1;
    return (((long)page * c.page_size + (j % c.page_size)) * H + h) * Dh;
}

__device__ __forceinline__ int clamp_len(const int32_t* prefix_len, int b, int capacity) {
    const int L = prefix_len[b];
    return L < 0 ? 0 : (L > capacity ? capacity : L);
}

// Rotation angle of pair m at position pos (double precision).
__device__ __forceinline__ void rope_cs(int pos, int m, int Dh, double theta, double& c, double& s) {
    const double ang = (double)pos * pow(theta, -2.0 * (double)m / (double)Dh);
    sincos(ang, &s, &c);
}

// ---------------------------------------------------------------------------
// fp32 / generic VALU kernel: one wave per (b, h, node)
// ---------------------------------------------------------------------------

template <typename ST>
__global__ __launch_bounds__(64) void attn_valu(KV cache, const ST* __restrict__ q, const ST* __restrict__ k,
                                                const ST* __restrict__ v, const int32_t* __restrict__ prefix_len,
                                                const int32_t* __restrict__ depth, const uint64_t* __restrict__ anc,
                                                int T, int H, int Dh, int W, double theta, ST* __restrict__ out,
                                                ST* __restrict__ k_rot) {
    const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x;
    const int half = Dh / 2;
    const int L = clamp_len(prefix_len, b, cache.capacity);
    const float scale = 1.f / sqrtf((float)Dh);
    const long node = (((long)b * T + i) * H + h) * Dh;
    float q1[2] = {0, 0}, q2[2] = {0, 0};
    const int pos_i = L + depth[i];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int m = lane + 64 * p;
        if (m < half) {
            double c, s;
            rope_cs(pos_i, m, Dh, theta, c, s);
            const double x1 = Elt<ST>::ld(q + node + m), x2 = Elt<ST>::ld(q + node + m + half);
            q1[p] = (float)(x1 * c - x2 * s);
            q2[p] = (float)(x2 * c + x1 * s);
            const double y1 = Elt<ST>::ld(k + node + m), y2 = Elt<ST>::ld(k + node + m + half);
            Elt<ST>::st64(k_rot + node + m, y1 * c - y2 * s);
            Elt<ST>::st64(k_rot + node + m + half, y2 * c + y1 * s);
        }
    }
    float mx = -INFINITY, l = 0.f, o1[2] = {0, 0}, o2[2] = {0, 0};
    auto visit = [&](float s, const float* v1, const float* v2) {
        const float mn = fmaxf(mx, s);
        const float corr = expf(mx - mn);
        const float p = expf(s - mn);
        l = l * corr + p;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            o1[t] = o1[t] * corr + p * v1[t];
            o2[t] = o2[t] * corr + p * v2[t];
        }
        mx = mn;
    };
    const ST* K = (const ST*)cache.k;
    const ST* Vc = (const ST*)cache.v;
    for (int j = 0; j < L; ++j) {
        const long off = kv_offset(cache, b, j, h, H, Dh);
        float part = 0.f, v1[2] = {0, 0}, v2[2] = {0, 0};
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int m = lane + 64 * p;
            if (m < half && off >= 0) {
                part += q1[p] * Elt<ST>::ld(K + off + m) + q2[p] * Elt<ST>::ld(K + off + m + half);
                v1[p] = Elt<ST>::ld(Vc + off + m);
                v2[p] = Elt<ST>::ld(Vc + off + m + half);
            }
        }
        visit(wave_sum(part) * scale, v1, v2);
    }
    // tree keys: ancestors-or-self of i, packed order
    for (int w = 0; w < W; ++w) {
        uint64_t bits = anc[(long)i * W + w];
        while (bits) {
            const int j = w * 64 + __builtin_ctzll(bits);
            bits &= bits - 1;
            if (j >= T) break;
            const long nj = (((long)b * T + j) * H + h) * Dh;
            const int pos_j = L + depth[j];
            float part = 0.f, v1[2] = {0, 0}, v2[2] = {0, 0};
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                const int m = lane + 64 * p;
                if (m < half) {
                    double c, s;
                    rope_cs(pos_j, m, Dh, theta, c, s);
                    const double y1 = Elt<ST>::ld(k + nj + m), y2 = Elt<ST>::ld(k + nj + m + half);
                    ST r1, r2;  // the key exactly as stored in k_rot
                    Elt<ST>::st64(&r1, y1 * c - y2 * s);
                    Elt<ST>::st64(&r2, y2 * c + y1 * s);
                    part += q1[p] * Elt<ST>::ld(&r1) + q2[p] * Elt<ST>::ld(&r2);
                    v1[p] = Elt<ST>::ld(v + nj + m);
                    v2[p] = Elt<ST>::ld(v + nj + m + half);
                }
            }
            visit(wave_sum(part) * scale, v1, v2);
        }
    }
    const float inv = 1.f / l;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int m = lane + 64 * p;
        if (m < half) {
            Elt<ST>::st(out + node + m, o1[p] * inv);
            Elt<ST>::st(out + node + m + half, o2[p] * inv);
        }
    }
}

// ---------------------------------------------------------------------------
// bf16 MFMA path
// ---------------------------------------------------------------------------

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two floats to bf16 (round to nearest even, one v_cvt_pk_bf16_f32), lo in bits 0..15.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

__device__ __forceinline__ float elt(const u32x4& v, int t) {
    const uint32_t w = v[t >> 1];
    return __uint_as_float((t & 1) ? (w & 0xffff0000u) : (w << 16));
}

// cos/sin of pos * inv_freq: the angle is formed and reduced to [-pi, pi] in double
// precision, then evaluated in single precision.
__device__ __forceinline__ float2 rope_cs_table_entry(int pos, double inv_freq) {
    const double a = (double)pos * inv_freq;
    const double r = a - 6.283185307179586 * rint(a * 0.15915494309189535);
    float s, c;
    sincosf((float)r, &s, &c);
    return make_float2(c, s);
}

// Rotate the 8 pairs (lo[t], hi[t]) = (x_m, x_{m+64}), m = m0 + t, with cos/sin row cs, and
// multiply the rotated values by sc before they are rounded to bf16.
__device__ __forceinline__ void rotate8(u32x4& lo, u32x4& hi, const float2* cs, int m0, float sc = 1.f) {
    u32x4 a, b;
#pragma unroll
    for (int t = 0; t < 8; t += 2) {
        const float2 r0 = cs[m0 + t], r1 = cs[m0 + t + 1];
        const float x0 = elt(lo, t), y0 = elt(hi, t), x1 = elt(lo, t + 1), y1 = elt(hi, t + 1);
        a[t >> 1] = pack_bf16((x0 * r0.x - y0 * r0.y) * sc, (x1 * r1.x - y1 * r1.y) * sc);
        b[t >> 1] = pack_bf16((y0 * r0.x + x0 * r0.y) * sc, (y1 * r1.x + x1 * r1.y) * sc);
    }
    lo = a;
    hi = b;
}

struct AttnArgs {
    KV cache;
    const bf16_t* q;
    const bf16_t* k;
    const bf16_t* v;
    const int32_t* prefix_len;
    const int32_t* depth;
    const uint64_t* anc;
    bf16_t* k_rot;
    bf16_t* part_o;            // per partial state: O / l, bf16 (normalised: its scale is l's)
    float* part_ml;
    double theta;
    int T, Tpad, H, W, nsplit, tiles_per_split, max_depth;
    int page_shift;            // log2 of a paged cache's page size, -1 if not a power of two
    int nparts;                // partial states per (sequence, head): nsplit ranges, then the tree
    int tree_first;            // the tree workgroups take grid z = 0 (else z = nsplit)
    double inv_freq[kDh / 2];  // theta^(-2m/Dh), computed once on the host
};

// ---------------------------------------------------------------------------
// bf16 kernels: prefix keys streamed by direct global-to-LDS loads
// ---------------------------------------------------------------------------
//
// A workgroup of NWB waves works on one (sequence, head) at a time; wave w owns the QT query
// tiles 16 (QT w + t) .. +15 (with QT = 2 every K and V fragment a wave reads from LDS feeds
// both of its tiles, and 8 waves cover a 256-node tree).  Per 64-key tile: S^T = K Q^T, then
// O^T = V^T P^T on MFMA 16x16x32 bf16, so the probabilities stay in registers; online
// softmax in log2 units.  Prefix tiles stream through a two-stage LDS ring filled by
// global_load_lds_dwordx4: while a tile is multiplied the next one is in flight and no
// register holds it; its loads go out in parts between the blocks of S.  Both tiles stay
// row-major (one 256-byte row per key) with their 16-byte pieces swizzled per row: K row r
// keeps piece p in slot p ^ (r mod 16) (its MFMA fragments read 16 rows at once), V row r in
// slot p ^ (2 r mod 16); V^T fragments come from the LDS transpose read ds_read_b64_tr_b16 --
// in each 16-lane group, lane i receives element i mod 4 of the 8 bytes read by lane
// 4 e + i / 4 as its element e -- so 4 key rows x 16 dims land as 16 lanes x 4 keys.  The
// swizzles keep the fragment and transpose reads free of bank conflicts.  The tree keys
// are rotated at their depth positions (writing k_rot), staged in the ring by ordinary
// stores and attended to under the ancestor-or-self bitmask.
//
// One workgroup per (sequence, head, key range) plus one per (sequence, head) for the tree.
// (A persistent schedule -- a fixed grid walking equal shares of all prefix tiles with the
// ring running across (sequence, head) boundaries -- was no faster: at 7b-B16 its tiles
// took longer, at 33B the gain came from fewer partial states, which the split choice
// below now gives directly.)
//
// Waiting: the loops' only waits for the ring are their barriers (ring_barrier).  All LDS of
// a kernel is one array: with separate arrays the compiler tags each access with its array
// and then makes every read of the ring wait for all direct-to-LDS loads in flight (vmcnt(0)
// before each tile's first fragment read), which serialises the ring.  The transpose reads
// are issued as inline assembly for the same reason (the compiler's own form of that read
// always waits), with an explicit lgkmcnt wait that the MFMAs depend on.
// Cache policy of the K and V loads: non-temporal (streamed, read once) when the caches of
// the call hold more than the last-level cache (256 MiB), the default policy otherwise (a
// smaller cache stays resident from one decoding step to the next).
constexpr long kStreamedKvBytes = 256l << 20;
constexpr int kAuxStreamed = 2, kAuxDefault = 0;
#ifndef MDT_ATTN_S4
#define MDT_ATTN_S4 2
#endif
#ifndef MDT_ATTN_S8
#define MDT_ATTN_S8 2
#endif
constexpr int kStreamPages = 2048;               // page-table entries a workgroup stages
constexpr int kTileBytes = kTile * kDh * 2;      // one K (or V) tile: 16 KiB
constexpr int kStageBytes = 2 * kTileBytes;      // K then V
constexpr int kCsBytes = (MDT_MAX_HEADS + 1) * (kDh / 2) * (int)sizeof(float2);
constexpr int kInstr = kTile * (kDh / 8) / 64;   // load instructions per tile (K or V): 16

__device__ __forceinline__ int kslot(int p, int r) { return p ^ (r & 15); }
__device__ __forceinline__ int vslot(int p, int r) { return p ^ ((2 * r) & 14); }

// ds_read_b64_tr_b16 of the 8 bytes at LDS byte address a + OFF (see above on why it is
// assembly; the offset rides in the instruction's immediate field).
template <int OFF>
__device__ __forceinline__ u32x2 ds_read_tr16(uint32_t a) {
    static_assert(OFF >= 0 && OFF < 65536, "16-bit LDS offset");
    u32x2 r;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(a), "i"(OFF));
    return r;
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// Wait for this wave's LDS reads; the 16 values count as written by the wait, so nothing
// that uses them can be scheduled before it.
__device__ __forceinline__ void lds_wait16(u32x2 (&v)[8][2]) {
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(v[0][0]), "+v"(v[0][1]), "+v"(v[1][0]), "+v"(v[1][1]), "+v"(v[2][0]), "+v"(v[2][1]),
                   "+v"(v[3][0]), "+v"(v[3][1]), "+v"(v[4][0]), "+v"(v[4][1]), "+v"(v[5][0]), "+v"(v[5][1]),
                   "+v"(v[6][0]), "+v"(v[6][1]), "+v"(v[7][0]), "+v"(v[7][1]));
}

// Per-wave query state: in tile t the lane holds query qi(t) = 16 (QT wave + t) + lane % 16,
// dims 32 s + 8 g .. +8 of the rotated query (s = 0, 1: x_m; s = 2, 3: x_{m+64}), its
// running maximum m (replicated over g), the running sum l of the weights of the keys this
// lane holds (the query's sum is that of its four lanes l, l ^ 16, l ^ 32, l ^ 48, formed
// once when the state is written) and O^T accumulators (lane: dims 16 db + 4 g + e).
template <int QT>
struct QueryState {
    u32x4 bq[QT][4];
    f32x4 oacc[QT][8];
    float m_run[QT], l_run[QT];
};

__device__ __forceinline__ int query_of(int QT_, int t) {
    return (((int)threadIdx.x >> 6) * QT_ + t) * 16 + ((int)threadIdx.x & 15);
}

// Request the raw queries of (b, h) (rows past T read node 0 and are zeroed when rotated).
template <int QT>
__device__ __forceinline__ void load_queries(const AttnArgs& A, int b, int h, u32x4 (&bq)[QT][4]) {
    const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
    for (int t = 0; t < QT; ++t) {
        const int qi = query_of(QT, t);
        const long node = (((long)b * A.T + (qi < A.T ? qi : 0)) * A.H + h) * kDh;
#pragma unroll
        for (int s = 0; s < 4; ++s) bq[t][s] = *(const u32x4*)(A.q + node + 32 * s + 8 * g);
    }
}

// cos/sin of every (depth, pair) at positions L .. L + max_depth, by the workgroup's threads
// (published by the caller's barrier).
__device__ __forceinline__ void fill_rope_table(const AttnArgs& A, int L, float2* cs, int nthreads) {
    for (int e = threadIdx.x; e < (A.max_depth + 1) * (kDh / 2); e += nthreads)
        cs[e] = rope_cs_table_entry(L + e / (kDh / 2), A.inv_freq[e % (kDh / 2)]);
}

// Rotate raw queries into st.bq, scaled by log2(e) / sqrt(Dh) so that their products with the
// keys are the scores in log2 units of the softmax, and reset the running state.
template <int QT>
__device__ __forceinline__ void start_queries(const AttnArgs& A, const u32x4 (&raw)[QT][4], const int (&dq)[QT],
                                              const float2* cs, QueryState<QT>& st) {
    const float sl2 = (1.f / sqrtf((float)kDh)) * 1.4426950408889634f;
    const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
    for (int t = 0; t < QT; ++t) {
        const bool ok = query_of(QT, t) < A.T;
#pragma unroll
        for (int s = 0; s < 4; ++s) st.bq[t][s] = ok ? raw[t][s] : u32x4{0, 0, 0, 0};
        const float2* row = cs + dq[t] * (kDh / 2);
        rotate8(st.bq[t][0], st.bq[t][2], row, 8 * g, sl2);
        rotate8(st.bq[t][1], st.bq[t][3], row, 32 + 8 * g, sl2);
#pragma unroll
        for (int db = 0; db < 8; ++db) st.oacc[t][db] = f32x4{0.f, 0.f, 0.f, 0.f};
        st.m_run[t] = -INFINITY;
        st.l_run[t] = 0.f;
    }
}

// Partial state of the wave's queries into partial slot `slot` (rows of Tpad per slot): (m, l)
// in fp32 and the normalised output O / l in bf16 (a convex combination of value rows, so
// bf16 keeps its relative error at 2^-9 whatever the scale; it halves the partials' traffic).
template <int QT>
__device__ __forceinline__ void write_partial(const AttnArgs& A, long slot, const QueryState<QT>& st) {
    const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
    for (int t = 0; t < QT; ++t) {
        const int qi = query_of(QT, t);
        if (qi < A.Tpad) {
            const long base = slot * A.Tpad + qi;
            bf16_t* po = A.part_o + base * kDh;
            const float l = xor_sum_16_32(st.l_run[t]);
            const float inv_l = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
            for (int db = 0; db < 8; ++db) {
                u32x2 w;
                w[0] = pack_bf16(st.oacc[t][db][0] * inv_l, st.oacc[t][db][1] * inv_l);
                w[1] = pack_bf16(st.oacc[t][db][2] * inv_l, st.oacc[t][db][3] * inv_l);
                *(u32x2*)(po + db * 16 + 4 * g) = w;
            }
            if (g == 0) {
                A.part_ml[base * 2 + 0] = st.m_run[t];
                A.part_ml[base * 2 + 1] = l;
            }
        }
    }
}

// The scores S^T of one tile, as the 16x16 MFMA output blocks of its 16-key blocks, each less
// the reference its query's running maximum had when the tile was multiplied (0 before the
// first key): the accumulators start from minus that reference.
template <int QT>
struct QkAcc {
    f32x4 s[QT][kTile / 16];
};

template <int QT>
__device__ __forceinline__ float score_base(const QueryState<QT>& st, int t) {
    return st.m_run[t] == -INFINITY ? 0.f : st.m_run[t];
}

// S^T = K Q^T for one 64-key tile (K tile at `kst`); hook(kb) runs after each 16-key block.
template <int QT, typename Hook>
__device__ __forceinline__ void qk_tile(const char* kst, const QueryState<QT>& st, QkAcc<QT>& sa, Hook&& hook) {
    const int lane = threadIdx.x & 63, g = lane >> 4, c16 = lane & 15;
    const bf16_t* Ks = (const bf16_t*)kst;
    constexpr int KB = kTile / 16;
    float a0[QT];
#pragma unroll
    for (int t = 0; t < QT; ++t) a0[t] = -score_base(st, t);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        f32x4 acc[QT];
#pragma unroll
        for (int t = 0; t < QT; ++t) acc[t] = f32x4{a0[t], a0[t], a0[t], a0[t]};
        const int r = kb * 16 + c16;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const u32x4 kf = *(const u32x4*)(Ks + (r * 16 + kslot(4 * s + g, r)) * 8);
#pragma unroll
            for (int t = 0; t < QT; ++t) acc[t] = mfma16(kf, st.bq[t][s], acc[t]);
        }
#pragma unroll
        for (int t = 0; t < QT; ++t) sa.s[t][kb] = acc[t];
        hook(kb);
    }
}

// The online-softmax step of one tile of scores (nvalid of its keys real): update (m, l),
// rescale the O^T accumulators and leave the probabilities as bf16 MFMA operands in bp.
// Masked tiles also keep only the keys whose bit is set in qw[t] (bit j: key j of the tile;
// all ones for prefix keys, the ancestor-or-self bits for tree keys).  (The mask words come
// in as values: selecting one of a query's four words here would index a register array
// with a run-time index, which puts the whole state in scratch.)
template <int QT>
__device__ __forceinline__ void softmax_tile(QkAcc<QT>& sa, int nvalid, bool masked, const uint64_t (&qw)[QT],
                                             QueryState<QT>& st, u32x4 (&bp)[QT][kTile / 32]) {
    const int g = (threadIdx.x & 63) >> 4;
    constexpr int KB = kTile / 16, KS = kTile / 32;
    auto& sacc = sa.s;
#pragma unroll
    for (int t = 0; t < QT; ++t) {
        float tmax = -INFINITY;
        if (masked) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int jj = kb * 16 + 4 * g + e;
                    if (!(jj < nvalid && ((qw[t] >> jj) & 1ull))) sacc[t][kb][e] = -INFINITY;
                    tmax = fmaxf(tmax, sacc[t][kb][e]);
                }
        } else {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int e = 0; e < 4; ++e) tmax = fmaxf(tmax, sacc[t][kb][e]);
        }
        const float m_base = score_base(st, t);
        tmax = xor_max_16_32(tmax) + m_base;  // the tile's largest score
        // The reference maximum moves only when a score exceeds it by more than 2^8, so that
        // the accumulators are rarely rescaled; weights stay below 256 (fine for the bf16
        // probabilities and the fp32 sums).  A row with no key yet keeps -inf and a
        // reference of 0 (its weights are exp2(-inf) = 0).  While the reference stays, the
        // accumulated scores are already relative to it.
        const float m_new = tmax > st.m_run[t] + 8.f ? tmax : st.m_run[t];
        const float m_ref = m_new == -INFINITY ? 0.f : m_new;
        const float corr = __builtin_amdgcn_exp2f(st.m_run[t] - m_ref);
        const float delta = m_ref - m_base;
        float ts[4] = {0.f, 0.f, 0.f, 0.f};  // four independent sums, not one serial chain
        if (__all(delta == 0.f)) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float p = __builtin_amdgcn_exp2f(sacc[t][kb][e]);
                    sacc[t][kb][e] = p;
                    ts[e] += p;
                }
        } else {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float p = __builtin_amdgcn_exp2f(sacc[t][kb][e] - delta);
                    sacc[t][kb][e] = p;
                    ts[e] += p;
                }
        }
        // this lane's keys only: the four lanes of a query share m and so the rescaling
        st.l_run[t] = st.l_run[t] * corr + ((ts[0] + ts[1]) + (ts[2] + ts[3]));
        st.m_run[t] = m_new;
        if (__any(corr != 1.f))
#pragma unroll
            for (int db = 0; db < 8; ++db) st.oacc[t][db] *= corr;
        // within a 32-key step the key order is 4g+e (e<4), then 16+4g+(e-4)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            bp[t][ks][0] = pack_bf16(sacc[t][2 * ks][0], sacc[t][2 * ks][1]);
            bp[t][ks][1] = pack_bf16(sacc[t][2 * ks][2], sacc[t][2 * ks][3]);
            bp[t][ks][2] = pack_bf16(sacc[t][2 * ks + 1][0], sacc[t][2 * ks + 1][1]);
            bp[t][ks][3] = pack_bf16(sacc[t][2 * ks + 1][2], sacc[t][2 * ks + 1][3]);
        }
    }
}

// Scores and softmax of one 64-key tile (see qk_tile and softmax_tile).
template <int QT, typename Hook>
__device__ __forceinline__ void scores_tile(const char* kst, int nvalid, bool masked, const uint64_t (&qw)[QT],
                                            QueryState<QT>& st, u32x4 (&bp)[QT][kTile / 32], Hook&& hook) {
    QkAcc<QT> sa;
    qk_tile<QT>(kst, st, sa, hook);
    softmax_tile<QT>(sa, nvalid, masked, qw, st, bp);
}

// Per-lane byte offsets of the V^T fragment reads within a V tile: lane (dim 16 db + c16,
// group g) takes keys 32 ks + 4 g + e and 32 ks + 16 + 4 g + e (e < 4) by two transpose
// reads; as a source lane it reads the 8 bytes of key row 32 ks + 16 hf + 4 g + c16 / 4,
// dims 16 db + 4 (c16 mod 4) ..  The rows 32 ks + 16 hf add a multiple of 16 to the row, which
// leaves its swizzle alone: that part is the reads' immediate offset.
struct VOffsets {
    uint32_t o[8];
};
__device__ __forceinline__ VOffsets v_offsets() {
    const int lane = threadIdx.x & 63, g = lane >> 4, c16 = lane & 15;
    const int r0 = 4 * g + (c16 >> 2);
    VOffsets v;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
        const int p = 2 * db + ((c16 & 3) >> 1);
        v.o[db] = (uint32_t)((r0 * 16 + vslot(p, r0)) * 16 + 8 * (c16 & 1));
    }
    return v;
}

template <int KS>
__device__ __forceinline__ void read_v_step(uint32_t vbase, const VOffsets& vo, u32x2 (&vh)[8][2]) {
#pragma unroll
    for (int db = 0; db < 8; ++db) {
        vh[db][0] = ds_read_tr16<KS * 32 * kDh * 2>(vbase + vo.o[db]);
        vh[db][1] = ds_read_tr16<(KS * 32 + 16) * kDh * 2>(vbase + vo.o[db]);
    }
}

// O^T += V^T P^T for one 64-key tile (V tile at `vst`, probabilities from scores_tile).
template <int QT>
__device__ __forceinline__ void values_tile(const char* vst, const VOffsets& vo, const u32x4 (&bp)[QT][kTile / 32],
                                            QueryState<QT>& st) {
    const uint32_t vbase = lds_addr(vst);
    u32x2 vh[2][8][2];
    auto pv = [&](int ks) __attribute__((always_inline)) {
#pragma unroll
        for (int db = 0; db < 8; ++db) {
            const u32x4 av = {vh[ks][db][0][0], vh[ks][db][0][1], vh[ks][db][1][0], vh[ks][db][1][1]};
#pragma unroll
            for (int t = 0; t < QT; ++t) st.oacc[t][db] = mfma16(av, bp[t][ks], st.oacc[t][db]);
        }
    };
    read_v_step<0>(vbase, vo, vh[0]);
    lds_wait16(vh[0]);
    if constexpr (QT > 1) {  // registers: one step of V fragments at a time
        pv(0);
        read_v_step<1>(vbase, vo, vh[1]);
        lds_wait16(vh[1]);
        pv(1);
    } else {  // the reads of step 1 go out while the MFMAs of step 0 run
        read_v_step<1>(vbase, vo, vh[1]);
        __builtin_amdgcn_sched_barrier(0);
        pv(0);
        __builtin_amdgcn_sched_barrier(0);
        lds_wait16(vh[1]);
        pv(1);
    }
}

// One whole 64-key tile of the LDS stage `stage` (K, then V).
template <int QT, typename Hook>
__device__ __forceinline__ void attend_tile(const char* stage, const VOffsets& vo, int nvalid, bool masked,
                                            const uint64_t (&qw)[QT], QueryState<QT>& st, Hook&& hook) {
    u32x4 bp[QT][kTile / 32];
    scores_tile<QT>(stage, nvalid, masked, qw, st, bp, hook);
    values_tile<QT>(stage + kTileBytes, vo, bp, st);
}

// The tree keys of (b, h): rotate k at L + depth, store k_rot, stage 64 keys at a time into
// the ring's first stage (ordinary stores) and attend under the ancestor-or-self bitmask.
// The ring must be idle; cs holds the table of sequence b.
template <int QT, int NT>
__device__ __forceinline__ void tree_pass(const AttnArgs& A, int b, int h, char* ring, const float2* cs,
                                          const VOffsets& vo, bool busy, QueryState<QT>& st) {
    const int T = A.T, H = A.H, tid = threadIdx.x;
    bf16_t* Ks = (bf16_t*)ring;
    bf16_t* Vs = (bf16_t*)(ring + kTileBytes);
    for (int tb = 0; tb < T; tb += kTile) {
        __syncthreads();
        for (int c = tid; c < kTile * 8; c += NT) {
            const int key = c >> 3, dc = c & 7, j = tb + key;
            u32x4 klo = {0, 0, 0, 0}, khi = {0, 0, 0, 0};
            if (j < T) {
                const long node = (((long)b * T + j) * H + h) * kDh;
                klo = *(const u32x4*)(A.k + node + 8 * dc);
                khi = *(const u32x4*)(A.k + node + 64 + 8 * dc);
                rotate8(klo, khi, cs + min(max(A.depth[j], 0), A.max_depth) * (kDh / 2), 8 * dc);
                *(u32x4*)(A.k_rot + node + 8 * dc) = klo;
                *(u32x4*)(A.k_rot + node + 64 + 8 * dc) = khi;
            }
            *(u32x4*)(Ks + (key * 16 + kslot(dc, key)) * 8) = klo;
            *(u32x4*)(Ks + (key * 16 + kslot(dc + 8, key)) * 8) = khi;
        }
        for (int c = tid; c < kTile * 16; c += NT) {
            const int key = c >> 4, p = c & 15, j = tb + key;
            u32x4 vv = {0, 0, 0, 0};
            if (j < T) vv = *(const u32x4*)(A.v + (((long)b * T + j) * H + h) * kDh + 8 * p);
            *(u32x4*)(Vs + (key * 16 + vslot(p, key)) * 8) = vv;
        }
        uint64_t qw[QT];  // the ancestor-or-self bits of the tile's keys tb .. tb + 63
#pragma unroll
        for (int t = 0; t < QT; ++t) {
            const int qi = query_of(QT, t);
            qw[t] = qi < T && (tb >> 6) < A.W ? A.anc[(long)qi * A.W + (tb >> 6)] : 0ull;
        }
        __syncthreads();
        if (busy) attend_tile<QT>(ring, vo, min(kTile, T - tb), true, qw, st, [](int) {});
    }
}

// Load instruction j of a wave (of 2 kInstr per tile): which cache (k or v), its row of the
// tile, its piece and its 1-KiB block of the stage.
template <int NWB>
struct LoadSlot {
    static constexpr int kIPW = 2 * kInstr / NWB;
    __device__ __forceinline__ static bool isv(int j) { return ((int)threadIdx.x >> 6) * kIPW + j >= kInstr; }
    __device__ __forceinline__ static int block(int j) {
        const int i = ((int)threadIdx.x >> 6) * kIPW + j;
        return i >= kInstr ? i - kInstr : i;
    }
    __device__ __forceinline__ static int row(int j) { return (64 * block(j) + ((int)threadIdx.x & 63)) >> 4; }
    __device__ __forceinline__ static int piece(int j) {
        const int q = 64 * block(j) + ((int)threadIdx.x & 63), r = q >> 4, sl = q & 15;
        return isv(j) ? vslot(sl, r) : kslot(sl, r);  // the swizzles are involutions
    }
    __device__ __forceinline__ static int lds_offset(int j) { return (isv(j) ? kTileBytes : 0) + 1024 * block(j); }
};

// One (sequence, head, key range) per workgroup, or the tree of one (sequence, head).
// Grid (H, B, nsplit + 1), the z index outermost: the key ranges in order (the ranges that
// start past a short prefix exit at once) and the trees.  Small trees come last, where their
// short workgroups fill the CUs that the last key ranges leave idle; trees of more than 128
// nodes come first (a tree workgroup then does several masked tiles and would lengthen the
// tail).
template <int NWB, bool PAGED, int QT, int S, int AUX>
__global__ __launch_bounds__(64 * NWB, 8 / NWB) void attn_stream(AttnArgs A) {  // two waves per SIMD
    constexpr int NT = 64 * NWB;
    using LS = LoadSlot<NWB>;
    constexpr int kIPW = LS::kIPW;
    static_assert(2 * kInstr % NWB == 0, "loads divide among the waves");
    static_assert(S >= 2 && S <= 4 && (S - 2) * kIPW < 64, "ring stages / vmcnt range");
    constexpr int kRingBytes = S * kStageBytes;
    constexpr int kPageBytes = PAGED ? kStreamPages * 4 : 0;
    __shared__ __attribute__((aligned(1024))) char lds[kRingBytes + kCsBytes + kPageBytes];
    char* const ring = lds;
    float2* const cs = (float2*)(lds + kRingBytes);                  // cos/sin per (depth, pair)
    int* const pages = (int*)(lds + kRingBytes + kCsBytes);          // physical page of each page of the range
    // z < nsplit: prefix key range z; z = nsplit: the tree keys
    // grid z: the key ranges in order and the tree (first or last); z = nsplit below means the tree
    const int h = blockIdx.x, b = blockIdx.y;
    const int z = A.tree_first ? ((int)blockIdx.z == 0 ? A.nsplit : (int)blockIdx.z - 1) : (int)blockIdx.z;
    const bool tree_split = z == A.nsplit;
    const int wave = threadIdx.x >> 6;
    const int H = A.H;
    const int L = clamp_len(A.prefix_len, b, A.cache.capacity);
    const int j_begin = tree_split ? 0 : z * A.tiles_per_split * kTile;
    const int j_end = tree_split ? 0 : min(L, j_begin + A.tiles_per_split * kTile);
    const int ntiles = j_end > j_begin ? (j_end - j_begin + kTile - 1) / kTile : 0;
    const long slot = ((long)b * H + h) * A.nparts + z;
    QueryState<QT> st;
    if (!tree_split && ntiles == 0) {
        // a key range past this sequence's prefix: an empty partial (attn_combine skips it)
#pragma unroll
        for (int t = 0; t < QT; ++t) {
            st.m_run[t] = -INFINITY;
            st.l_run[t] = 0.f;
            const int qi = query_of(QT, t);
            if (qi < A.Tpad && (threadIdx.x & 63) < 16) {
                A.part_ml[(slot * A.Tpad + qi) * 2 + 0] = -INFINITY;
                A.part_ml[(slot * A.Tpad + qi) * 2 + 1] = 0.f;
            }
        }
        return;
    }
    const bf16_t* Kg = (const bf16_t*)A.cache.k;
    const bf16_t* Vg = (const bf16_t*)A.cache.v;
    const int psz = PAGED ? A.cache.page_size : 1;
    const int psh = PAGED ? A.page_shift : 0;  // log2 of the page size, or -1
    const int pg0 = j_begin / psz;

    u32x4 raw[QT][4];
    load_queries<QT>(A, b, h, raw);
    int dq[QT];
#pragma unroll
    for (int t = 0; t < QT; ++t) {
        const int qi = query_of(QT, t);
        dq[t] = qi < A.T ? min(max(A.depth[qi], 0), A.max_depth) : 0;
    }
    if (PAGED) {
        const int np = j_end > j_begin ? (j_end - 1) / psz - pg0 + 1 : 0;  // <= kStreamPages (host plan)
        for (int e = threadIdx.x; e < np; e += NT) {
            const int pg = pg0 + e;
            const int page = pg < A.cache.max_pages ? A.cache.table[(long)b * A.cache.max_pages + pg] : -1;
            pages[e] = (page >= 0 && page < A.cache.num_pages) ? page : -1;
        }
        __syncthreads();
    }
    // Per load instruction j the lane's row, piece and cache (k or v) are fixed, so its
    // source is src0[j] + (cache row of key t0 + row) * H * Dh; keys past the range's end
    // repeat its last key (they are masked).  An unmapped page reads the pool's first row (a
    // caller error: the value is meaningless but the access stays inside).
    const bf16_t* src0[kIPW];
#pragma unroll
    for (int j = 0; j < kIPW; ++j)
        src0[j] = (LS::isv(j) ? Vg : Kg) + (PAGED ? 0 : (size_t)b * A.cache.capacity * H * kDh) + h * kDh +
                  8 * LS::piece(j);
    const unsigned HK = (unsigned)(H * kDh);
    // sources of the tile of keys t0 .. (formed together: the page lookups are LDS reads)
    auto sources_with = [&](int t0, const bf16_t* (&src)[kIPW], bool pow2) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < kIPW; ++j) {
            const int key = min(t0 + LS::row(j), j_end - 1);
            unsigned row = (unsigned)key;
            if (PAGED) {
                const int pq = pow2 ? key >> psh : key / psz;
                const int page = pages[pq - pg0];
                row = page < 0 ? 0u : (unsigned)(page * psz + (key - pq * psz));
            }
            src[j] = src0[j] + (size_t)row * HK;
        }
    };
    auto sources = [&](int t0, const bf16_t* (&src)[kIPW]) __attribute__((always_inline)) {
        if (!PAGED || psh >= 0)
            sources_with(t0, src, true);
        else
            sources_with(t0, src, false);
    };
    // load instructions j0 .. j1 - 1 of a tile into ring stage `stage`
    auto issue_part = [&](const bf16_t* const (&src)[kIPW], int stage, int j0, int j1) __attribute__((always_inline)) {
        char* kst = ring + stage * kStageBytes;
#pragma unroll
        for (int j = 0; j < kIPW; ++j) {
            if (j < j0 || j >= j1) continue;
            __builtin_amdgcn_global_load_lds((const void*)src[j], (lds_void_t*)(kst + LS::lds_offset(j)), 16, 0,
                                             AUX);
        }
    };
    // tiles 0 .. S - 2 into stages 0 .. S - 2
#pragma unroll
    for (int t = 0; t < S - 1; ++t)
        if (t < ntiles) {
            const bf16_t* src[kIPW];
            sources(j_begin + t * kTile, src);
            issue_part(src, t, 0, kIPW);
        }
    fill_rope_table(A, L, cs, NT);
    // cos/sin table ready; the tiles already requested stay in flight (a plain
    // __syncthreads would wait for them)
    ring_barrier<63>();
    start_queries<QT>(A, raw, dq, cs, st);

    const VOffsets vo = v_offsets();
    // a wave whose query tiles are all padding only loads and meets the barriers
    const bool busy = wave * 16 * QT < A.Tpad;
    uint64_t all_keys[QT];
#pragma unroll
    for (int t = 0; t < QT; ++t) all_keys[t] = ~0ull;
    for (int t = 0; t < ntiles; ++t) {
        // tile t has landed once at most the loads of the later tiles already requested
        // (t + 1 .. t + S - 2) are outstanding; every wave is done with tile t - 1, whose
        // stage now takes tile t + S - 1
        const int later = min(S - 2, ntiles - 1 - t);
        if (S > 3 && later >= 2)
            ring_barrier<(S > 3 ? 2 : 0) * kIPW>();
        else if (S > 2 && later == 1)
            ring_barrier<(S > 2 ? 1 : 0) * kIPW>();
        else
            ring_barrier<0>();
        const bool ahead = t + S - 1 < ntiles;
        const bf16_t* src[kIPW];
        if (ahead) sources(j_begin + (t + S - 1) * kTile, src);
        const int nstage = (t + S - 1) % S;
        auto hook = [&](int kb) __attribute__((always_inline)) {
            if (ahead) {
                __builtin_amdgcn_sched_barrier(0);
                issue_part(src, nstage, kb * kIPW / 4, (kb + 1) * kIPW / 4);
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        const int base = j_begin + t * kTile;
        if (busy)
            attend_tile<QT>(ring + (t % S) * kStageBytes, vo, min(kTile, j_end - base), j_end - base < kTile,
                            all_keys, st, hook);
        else if (ahead)
            issue_part(src, nstage, 0, kIPW);
    }
    if (tree_split) tree_pass<QT, NT>(A, b, h, ring, cs, vo, busy, st);
    write_partial<QT>(A, slot, st);
}

// Merge the partial states of every (sequence, head, node): nparts consecutive slots per
// (sequence, head).  grid (T, H, B), block 64.
__device__ __forceinline__ void merge_partials(const bf16_t* __restrict__ part_o, const float* __restrict__ part_ml,
                                               int Tpad, int i, long s0, int n, long tree_slot, float& M,
                                               float& den, float& na, float& nb) {
    const int lane = threadIdx.x;
    // partial slots s0 .. s0 + n - 1 and tree_slot (if >= 0), in batches of 8, all loads of a
    // batch first; running max and sums rescale between batches (maxima in log2 units)
    const int total = n + (tree_slot >= 0 ? 1 : 0);
    M = -INFINITY;
    den = na = nb = 0.f;
    for (int u0 = 0; u0 < total; u0 += 8) {
        float ms[8], ls[8], oa[8], ob[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int k = min(u0 + u, total - 1);
            const long slot = k < n ? s0 + k : tree_slot;
            const long pidx = slot * Tpad + i;
            ms[u] = part_ml[pidx * 2];
            ls[u] = part_ml[pidx * 2 + 1];
            oa[u] = bf16_to_f32(part_o[pidx * kDh + lane]);
            ob[u] = bf16_to_f32(part_o[pidx * kDh + lane + 64]);
        }
        float bm = M;
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (u0 + u < total) bm = fmaxf(bm, ms[u]);
        if (bm == -INFINITY) continue;
        const float r = exp2f(M - bm);  // 0 while M is -inf
        den *= r;
        na *= r;
        nb *= r;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (u0 + u >= total || ms[u] == -INFINITY) continue;
            const float wgt = exp2f(ms[u] - bm) * ls[u];  // the partial's O is o * l
            den += wgt;
            na += oa[u] * wgt;
            nb += ob[u] * wgt;
        }
        M = bm;
    }
}

__global__ __launch_bounds__(64) void attn_combine(const bf16_t* __restrict__ part_o, const float* __restrict__ part_ml,
                                                   int T, int Tpad, int H, int nparts, bf16_t* __restrict__ out) {
    const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x;
    float M, den, na, nb;
    merge_partials(part_o, part_ml, Tpad, i, ((long)b * H + h) * nparts, nparts, -1, M, den, na, nb);
    bf16_t* o = out + (((long)b * T + i) * H + h) * kDh;
    o[lane] = f32_to_bf16(na / den);
    o[lane + 64] = f32_to_bf16(nb / den);
}

struct Plan {
    int Tpad, nsplit, tiles_per_split, nwb, nparts;
    size_t po_bytes, pml_bytes;
};

// Key ranges per (sequence, head): five or six (measured best at every workload shape: more
// ranges add per-workgroup set-up and partial states for the combine, about 2 us per range
// at 7b-B16 and 6 us at 33B; fewer leave a long tail), six when all workgroups fit one round
// of the CUs, and at least enough for 128 workgroups.  A paged cache's range stages its page
// numbers in LDS, at most kMaxTilesPerSplit tiles' worth.  The plan depends only on the
// shape, so the workspace size does too.
constexpr int kPlanCUs = 256;

Plan plan(int B, int T, int H, int capacity, bool paged) {
    Plan p;
    p.Tpad = (T + 15) / 16 * 16;
    const int waves = p.Tpad / 16;
    p.nwb = waves <= 4 ? 4 : (waves <= 8 ? 8 : 16);
    const int tiles = capacity > 0 ? (capacity + kTile - 1) / kTile : 1;
    const long bh = (long)B * H;
    int ns = bh <= kPlanCUs ? 6 : 5;
    ns = max(ns, (int)((128 + bh - 1) / bh));
    int tps = (tiles + ns - 1) / ns;
    if (paged) tps = min(tps, kMaxTilesPerSplit);
#ifdef MDT_ATTN_TPS
    tps = MDT_ATTN_TPS;
#endif
    p.tiles_per_split = max(1, min(tps, tiles));
    p.nsplit = (tiles + p.tiles_per_split - 1) / p.tiles_per_split;
    p.nparts = p.nsplit + 1;  // the key ranges, then the tree
    const size_t slots = (size_t)B * H * p.nparts;
    p.po_bytes = (slots * p.Tpad * kDh * sizeof(bf16_t) + 255) & ~(size_t)255;
    p.pml_bytes = slots * p.Tpad * 2 * sizeof(float);
    return p;
}

}  // namespace

extern "C" size_t mdt_tree_attention_workspace(mdt_dtype dt, int B, int T, int H, int Dh, int capacity) {
    if (dt != MDT_BF16 || B < 1 || T < 1 || H < 1) return 0;
    (void)Dh;
    // either cache layout (a paged cache may need more, shorter key ranges)
    const Plan pc = plan(B, T, H, capacity, false), pp = plan(B, T, H, capacity, true);
    return max(pc.po_bytes + pc.pml_bytes, pp.po_bytes + pp.pml_bytes);
}

extern "C" mdt_status mdt_tree_attention(void* stream, mdt_dtype dt, int B, int H, int Dh, const mdt_tree_dev* tree,
                                         const void* q, const void* k, const void* v, const mdt_kv_cache* cache,
                                         const int32_t* prefix_len, float rope_theta, void* out, void* k_rot,
                                         void* ws, size_t ws_bytes) {
    MDT_REQUIRE(dt == MDT_F32 || dt == MDT_BF16, MDT_ERR_DTYPE, "dtype %d not supported", (int)dt);
    MDT_REQUIRE(B >= 1 && B <= 65535 && H >= 1 && H <= 65535, MDT_ERR_SHAPE, "B=%d H=%d out of range", B, H);
    if (dt == MDT_BF16)
        MDT_REQUIRE(Dh == kDh, MDT_ERR_UNSUPPORTED, "bf16 tree attention supports Dh=128 (got %d)", Dh);
    else
        MDT_REQUIRE(Dh >= 2 && Dh <= 256 && Dh % 2 == 0, MDT_ERR_SHAPE, "Dh=%d must be even in 2..256", Dh);
    mdt_status st = mdt_check_tree(tree);
    if (st != MDT_OK) return st;
    MDT_REQUIRE(cache, MDT_ERR_NULL, "cache is NULL");
    MDT_REQUIRE(q && k && v && out && k_rot && prefix_len && cache->k && cache->v, MDT_ERR_NULL,
                "a tensor pointer is NULL");
    MDT_REQUIRE(mdt_aligned16(q) && mdt_aligned16(k) && mdt_aligned16(v) && mdt_aligned16(out) &&
                    mdt_aligned16(k_rot) && mdt_aligned16(cache->k) && mdt_aligned16(cache->v),
                MDT_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
    MDT_REQUIRE(rope_theta > 0.f, MDT_ERR_VALUE, "rope_theta must be > 0");
    if (cache->layout == MDT_KV_PAGED) {
        MDT_REQUIRE(cache->page_table, MDT_ERR_NULL, "page_table is NULL");
        MDT_REQUIRE(cache->page_size >= 1 && cache->page_size <= 1024 && cache->max_pages >= 1 &&
                        cache->num_pages >= 1,
                    MDT_ERR_SHAPE, "bad paged-cache geometry");
        MDT_REQUIRE((long)cache->max_pages * cache->page_size == cache->capacity, MDT_ERR_SHAPE,
                    "capacity must equal max_pages * page_size");
    } else {
        MDT_REQUIRE(cache->layout == MDT_KV_CONTIG, MDT_ERR_VALUE, "unknown cache layout %d", cache->layout);
        MDT_REQUIRE(cache->capacity >= 0, MDT_ERR_SHAPE, "capacity must be >= 0");
    }
    const int T = tree->T;
    KV kv{cache->k, cache->v, cache->page_table, cache->layout, cache->capacity, cache->page_size,
          cache->max_pages, cache->num_pages};
    hipStream_t s = (hipStream_t)stream;
    const double theta = (double)rope_theta;
    if (dt == MDT_F32) {
        MDT_LAUNCH("attn_valu", attn_valu<float>, dim3(T, H, B), dim3(64), 0, s, kv, (const float*)q,
                   (const float*)k, (const float*)v, prefix_len, tree->depth, tree->anc, T, H, Dh, tree->anc_words,
                   theta, (float*)out, (float*)k_rot);
        return mdt_launched("attn_valu");
    }
    const Plan p = plan(B, T, H, cache->capacity, cache->layout == MDT_KV_PAGED);
    MDT_REQUIRE(ws, MDT_ERR_WORKSPACE, "workspace is NULL");
    MDT_REQUIRE(mdt_aligned16(ws), MDT_ERR_ALIGN, "workspace must be 16-byte aligned");
    MDT_REQUIRE(ws_bytes >= p.po_bytes + p.pml_bytes, MDT_ERR_WORKSPACE, "workspace too small");
    int page_shift = -1;
    if (cache->layout == MDT_KV_PAGED && (cache->page_size & (cache->page_size - 1)) == 0)
        for (page_shift = 0; (1 << page_shift) < cache->page_size; ++page_shift) {
        }
    AttnArgs A{kv, (const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v, prefix_len, tree->depth, tree->anc,
               (bf16_t*)k_rot, (bf16_t*)ws, (float*)((char*)ws + p.po_bytes), theta, T, p.Tpad, H,
               tree->anc_words, p.nsplit, p.tiles_per_split, tree->max_depth, page_shift, p.nparts,
               p.Tpad > 128 ? 1 : 0, {}};
    for (int m = 0; m < kDh / 2; ++m) A.inv_freq[m] = std::pow(theta, -2.0 * (double)m / (double)kDh);
    const bool paged = cache->layout == MDT_KV_PAGED;
    // up to 8 query tiles: one per wave (4 or 8 waves); up to 16: two per wave on 8 waves
    const int threads = 64 * (p.nwb == 16 ? 8 : p.nwb);
    constexpr int S4 = MDT_ATTN_S4, S8 = MDT_ATTN_S8;
    const bool streamed = (long)B * cache->capacity * H * kDh * 2 * (long)sizeof(bf16_t) > kStreamedKvBytes;
    auto pick = [&](auto k_def, auto k_nt) { return streamed ? k_nt : k_def; };
    auto kern = p.nwb == 4
                    ? (paged ? pick(attn_stream<4, true, 1, S4, kAuxDefault>, attn_stream<4, true, 1, S4, kAuxStreamed>)
                             : pick(attn_stream<4, false, 1, S4, kAuxDefault>, attn_stream<4, false, 1, S4, kAuxStreamed>))
              : p.nwb == 8
                    ? (paged ? pick(attn_stream<8, true, 1, S8, kAuxDefault>, attn_stream<8, true, 1, S8, kAuxStreamed>)
                             : pick(attn_stream<8, false, 1, S8, kAuxDefault>, attn_stream<8, false, 1, S8, kAuxStreamed>))
                    : (paged ? pick(attn_stream<8, true, 2, S8, kAuxDefault>, attn_stream<8, true, 2, S8, kAuxStreamed>)
                             : pick(attn_stream<8, false, 2, S8, kAuxDefault>, attn_stream<8, false, 2, S8, kAuxStreamed>));
    MDT_LAUNCH("attn_stream", kern, dim3(H, B, p.nparts), dim3(threads), 0, s, A);
    st = mdt_launched("attn_stream");
    if (st != MDT_OK) return st;
    MDT_LAUNCH("attn_combine", attn_combine, dim3(T, H, B), dim3(64), 0, s, A.part_o, A.part_ml, T, p.Tpad, H,
               p.nparts, (bf16_t*)out);
    return mdt_launched("attn_combine");
}
