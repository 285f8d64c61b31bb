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
//  1. attn_tree_mfma: split-KV flash pass.  A workgroup owns one (sequence, head,
//     prefix key range); its waves each own 16 tree queries, rotated in registers.
//     64-key K and V tiles are staged in LDS (V transposed), the next tile already
//     in flight in registers, and both products run on MFMA 16x16x32 bf16:
//     S^T = K Q^T, then O^T = V^T P^T, so the probabilities stay in registers
//     between the two.  Online softmax keeps (max, sum) per query, the max in
//     log2 units (scores scaled by log2 e, exponentials by exp2).  One extra
//     workgroup per (sequence, head) rotates the tree keys at their depth
//     positions (writing k_rot, which is what gets cached) and attends to them
//     under the ancestor-or-self bitmask.  Rotation angles come from a per-depth
//     cos/sin table built in LDS.  Partial (m, l, O) go to the workspace.
//     Trees of up to 128 nodes use attn_stream, the same pass with the prefix tiles
//     streamed by direct global-to-LDS loads through a ring (see there).
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
constexpr int kKStride = kDh + 8;  // LDS row stride of K tile (elements)
constexpr int kVStride = kTile + 4;  // LDS row stride of transposed V tile (elements)
constexpr int kMaxSplitPages = 4096;  // page-table entries a workgroup stages in LDS
constexpr int kMaxTilesPerSplit = (2048 - 2) * 1 / kTile;  // page-table entries of a split fit both kernels' LDS
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

// Rotate the 8 pairs (lo[t], hi[t]) = (x_m, x_{m+64}), m = m0 + t, with cos/sin row cs.
__device__ __forceinline__ void rotate8(u32x4& lo, u32x4& hi, const float2* cs, int m0) {
    u32x4 a, b;
#pragma unroll
    for (int t = 0; t < 8; t += 2) {
        const float2 r0 = cs[m0 + t], r1 = cs[m0 + t + 1];
        const float x0 = elt(lo, t), y0 = elt(hi, t), x1 = elt(lo, t + 1), y1 = elt(hi, t + 1);
        a[t >> 1] = pack_bf16(x0 * r0.x - y0 * r0.y, x1 * r1.x - y1 * r1.y);
        b[t >> 1] = pack_bf16(y0 * r0.x + x0 * r0.y, y1 * r1.x + x1 * r1.y);
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
    float* part_o;
    float* part_ml;
    double theta;
    int T, Tpad, H, W, nsplit, tiles_per_split, max_depth;
    double inv_freq[kDh / 2];  // theta^(-2m/Dh), computed once on the host
};

// One (sequence, head, key split) per workgroup; NWB waves, wave w owns the QT query tiles
// 16 (QT w + t) .. +15, t < QT.  With QT = 2 every K and V fragment a wave reads from LDS
// feeds both of its tiles, and 8 waves cover a 256-node tree with registers to spare.
// Workgroups 0..nsplit-1 attend to prefix key ranges; workgroup nsplit rotates the tree
// keys (writing k_rot) and attends to them, masked by the ancestor-or-self bitmask.
// Grid (nsplit + 1, H, B); all partials are merged by attn_combine.
//
// Global loads are never issued under a branch and a loaded register is not touched
// before it is needed: the compiler's load counter is in-order, so either would make
// a wave wait for every load in flight.  Prefix pieces outside the split or on an
// unmapped page read the first 16 bytes of q instead (always present) and are zeroed
// when stored (a validity bit per piece); the pages of a paged cache are looked up in LDS.
template <int NWB, bool PAGED, int QT = 1>
__global__ __launch_bounds__(64 * NWB) void attn_tree_mfma(AttnArgs A) {
    constexpr int NT = 64 * NWB;
    constexpr int PPT = kTile * (kDh / 8) / NT;  // 16-byte K pieces per thread per tile
    constexpr int kVItems = (kTile / 2) * (kDh / 8);  // V items: (key pair, 8 dims)
    constexpr int VPT = kVItems / NT > 0 ? kVItems / NT : 1;
    static_assert(PPT + 2 * VPT <= 32, "validity bits per slot");
    __shared__ __attribute__((aligned(16))) bf16_t Ks[kTile * kKStride];
    __shared__ __attribute__((aligned(16))) bf16_t Vt[kDh * kVStride];
    __shared__ float2 cs[(MDT_MAX_HEADS + 1) * (kDh / 2)];  // cos/sin per (depth, pair)
    __shared__ int pages[PAGED ? kMaxSplitPages : 1];        // physical page of each page of the split
    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const bool tree_split = split == A.nsplit;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, c16 = lane & 15;
    const int H = A.H, T = A.T;
    const int L = clamp_len(A.prefix_len, b, A.cache.capacity);
    const int j_begin = tree_split ? 0 : split * A.tiles_per_split * kTile;
    const int j_end = tree_split ? 0 : min(L, j_begin + A.tiles_per_split * kTile);
    const float scale = 1.f / sqrtf((float)kDh);
    const bf16_t* Kg = (const bf16_t*)A.cache.k;
    const bf16_t* Vg = (const bf16_t*)A.cache.v;
    const int psz = PAGED ? A.cache.page_size : 1;
    const int pg0 = j_begin / psz;

    // this wave's queries (loaded first, so that waiting for them waits for nothing else):
    // in tile t the lane holds query qi[t], dims 32s + 8g .. +8; s = 0,1 hold x_m and
    // s = 2,3 hold x_{m+64}
    int qi[QT], dq_raw[QT];
    bool q_ok[QT];
    u32x4 bq[QT][4];
    uint64_t qa[QT][MDT_MAX_NODES / 64];
#pragma unroll
    for (int t = 0; t < QT; ++t) {
        qi[t] = (wave * QT + t) * 16 + c16;
        q_ok[t] = qi[t] < T;
        const int qc = q_ok[t] ? qi[t] : 0;
        const long node = (((long)b * T + qc) * H + h) * kDh;
#pragma unroll
        for (int s = 0; s < 4; ++s) bq[t][s] = *(const u32x4*)(A.q + node + 32 * s + 8 * g);
#pragma unroll
        for (int w = 0; w < MDT_MAX_NODES / 64; ++w) qa[t][w] = A.anc[(long)qc * A.W + min(w, A.W - 1)];
        dq_raw[t] = A.depth[qc];
    }

    if (PAGED) {
        const int np = j_end > j_begin ? (j_end - 1) / psz - pg0 + 1 : 0;  // <= kMaxSplitPages (host plan)
        for (int e = tid; e < np; e += NT) {
            const int pg = pg0 + e;
            const int page = pg < A.cache.max_pages ? A.cache.table[(long)b * A.cache.max_pages + pg] : -1;
            pages[e] = (page >= 0 && page < A.cache.num_pages) ? page : -1;
        }
        __syncthreads();
    }
    // element offset of prefix key j of this split, or -1 (outside the split, unmapped)
    auto key_off = [&](int j) -> long {
        if (j >= j_end) return -1;
        if (!PAGED) return (((long)b * A.cache.capacity + j) * H + h) * kDh;
        const int page = pages[j / psz - pg0];
        return page < 0 ? -1 : (((long)page * psz + j % psz) * H + h) * kDh;
    };

    // prefix tile staging through registers.  K: piece c = tid + NT*p is (key c/16, dims
    // 8*(c%16)..), stored row-major.  V: item c is (key pair c%32, dims 8*(c/32)..); the two
    // keys' values are packed per dimension into one dword, so the transposed LDS writes of
    // a wave hit consecutive dwords.  PF register slots: the PF tiles after the current
    // one are in flight while it runs.
    constexpr int PF = 1;
    u32x4 kr[PF][PPT], va[PF][VPT], vb[PF][VPT];
    uint32_t valid[PF];
    const int row_elems = H * kDh;  // elements between consecutive keys of a contiguous cache
    auto load_prefix = [&](int t0, int slot) {
        uint32_t m = 0;
        // contiguous cache: the tile's keys are consecutive rows from this base
        const long tile_base = (((long)b * A.cache.capacity + t0) * H + h) * kDh;
#pragma unroll
        for (int p = 0; p < PPT; ++p) {
            const int c = tid + NT * p;
            const int key = c >> 4;
            const long off = PAGED ? key_off(t0 + key) : (t0 + key < j_end ? tile_base + key * row_elems : -1);
            m |= (off >= 0 ? 1u : 0u) << p;
            kr[slot][p] = *(const u32x4*)(off >= 0 ? Kg + off + 8 * (c & 15) : A.q);
        }
#pragma unroll
        for (int p = 0; p < VPT; ++p) {
            const int c = tid + NT * p;
            const int key = 2 * (c & 31), dc = c >> 5;
            const bool item = c < kVItems;
            long oa, ob;
            if (PAGED) {
                oa = item ? key_off(t0 + key) : -1;
                ob = item ? key_off(t0 + key + 1) : -1;
            } else {
                oa = item && t0 + key < j_end ? tile_base + key * row_elems : -1;
                ob = item && t0 + key + 1 < j_end ? tile_base + (key + 1) * row_elems : -1;
            }
            m |= (oa >= 0 ? 1u : 0u) << (PPT + 2 * p);
            m |= (ob >= 0 ? 1u : 0u) << (PPT + 2 * p + 1);
            va[slot][p] = *(const u32x4*)(oa >= 0 ? Vg + oa + 8 * dc : A.q);
            vb[slot][p] = *(const u32x4*)(ob >= 0 ? Vg + ob + 8 * dc : A.q);
        }
        valid[slot] = m;
    };
    auto store_k = [&](int key, int dc, const u32x4& kv) { *(u32x4*)(Ks + key * kKStride + 8 * dc) = kv; };
    // keys 2*kp, 2*kp+1, dims 8*dc .. 8*dc+7 into the transposed V tile
    auto store_v_pair = [&](int kp, int dc, const u32x4& v0, const u32x4& v1) {
        // dim t of the pair: low halves (t even) or high halves (t odd) of word t/2,
        // key 2kp in the low 16 bits (one byte permute each)
#pragma unroll
        for (int t = 0; t < 8; ++t)
            ((uint32_t*)(Vt + (8 * dc + t) * kVStride))[kp] =
                __builtin_amdgcn_perm(v1[t >> 1], v0[t >> 1], (t & 1) ? 0x07060302u : 0x05040100u);
    };
    auto store_prefix = [&](int slot) {
        const u32x4 z{0, 0, 0, 0};
        const uint32_t m = valid[slot];
#pragma unroll
        for (int p = 0; p < PPT; ++p) {
            const int c = tid + NT * p;
            store_k(c >> 4, c & 15, ((m >> p) & 1u) ? kr[slot][p] : z);
        }
#pragma unroll
        for (int p = 0; p < VPT; ++p) {
            const int c = tid + NT * p;
            if (c < kVItems)
                store_v_pair(c & 31, c >> 5, ((m >> (PPT + 2 * p)) & 1u) ? va[slot][p] : z,
                             ((m >> (PPT + 2 * p + 1)) & 1u) ? vb[slot][p] : z);
        }
    };
#pragma unroll
    for (int s = 0; s < PF; ++s) load_prefix(j_begin + s * kTile, s);

    for (int e = tid; e < (A.max_depth + 1) * (kDh / 2); e += NT)
        cs[e] = rope_cs_table_entry(L + e / (kDh / 2), A.inv_freq[e % (kDh / 2)]);
    __syncthreads();  // cos/sin table ready
#pragma unroll
    for (int t = 0; t < QT; ++t) {
        if (!q_ok[t])
#pragma unroll
            for (int s = 0; s < 4; ++s) bq[t][s] = u32x4{0, 0, 0, 0};
        const int dq = q_ok[t] ? min(max(dq_raw[t], 0), A.max_depth) : 0;
        const float2* row = cs + dq * (kDh / 2);
        rotate8(bq[t][0], bq[t][2], row, 8 * g);
        rotate8(bq[t][1], bq[t][3], row, 32 + 8 * g);
#pragma unroll
        for (int w = 0; w < MDT_MAX_NODES / 64; ++w)
            if (!(tree_split && q_ok[t] && w < A.W)) qa[t][w] = 0;
    }

    f32x4 oacc[QT][8];
    float m_run[QT], l_run[QT];  // of query qi[t], replicated over g
#pragma unroll
    for (int t = 0; t < QT; ++t) {
#pragma unroll
        for (int db = 0; db < 8; ++db) oacc[t][db] = f32x4{0.f, 0.f, 0.f, 0.f};
        m_run[t] = -INFINITY;
        l_run[t] = 0.f;
    }

    // One staged tile: keys base..base+63, nvalid of them real.  The softmax runs in log2
    // units (scale * log2 e folded into the fma that forms each exponent), so it uses exp2.
    // Full prefix tiles skip the masking; the last prefix tile and tree tiles (bitmask) do not.
    const float sl2 = scale * 1.4426950408889634f;
    auto attend_tile = [&](int base, int nvalid, bool masked) {
        f32x4 sacc[QT][4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            f32x4 acc[QT];
#pragma unroll
            for (int t = 0; t < QT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
            const bf16_t* krow = Ks + (kb * 16 + c16) * kKStride + 8 * g;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const u32x4 kf = *(const u32x4*)(krow + 32 * s);
#pragma unroll
                for (int t = 0; t < QT; ++t) acc[t] = mfma16(kf, bq[t][s], acc[t]);
            }
#pragma unroll
            for (int t = 0; t < QT; ++t) sacc[t][kb] = acc[t];
        }
        u32x4 bp[QT][2];
#pragma unroll
        for (int t = 0; t < QT; ++t) {
            float tmax = -INFINITY;
            if (masked) {
                // tiles start at multiples of 64, so a tree tile reads one word of the query's
                // mask row; a prefix tile is only cut at nvalid
                const int wi = base >> 6;
                const uint64_t qw = !tree_split ? ~0ull
                                  : wi == 0     ? qa[t][0]
                                  : wi == 1     ? qa[t][1]
                                  : wi == 2     ? qa[t][2]
                                                : qa[t][3];
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int jj = kb * 16 + 4 * g + e;
                        const bool ok = jj < nvalid && ((qw >> jj) & 1ull);
                        const float sv = ok ? sacc[t][kb][e] : -INFINITY;
                        sacc[t][kb][e] = sv;
                        tmax = fmaxf(tmax, sv);
                    }
            } else {
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                    for (int e = 0; e < 4; ++e) tmax = fmaxf(tmax, sacc[t][kb][e]);
            }
            tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
            // the raw scores' maximum scaled once: rounding is monotone, so this is the maximum
            // of the scaled scores, and each score is scaled inside its exponent's fma
            tmax *= sl2;
            const float m_new = fmaxf(m_run[t], tmax);
            const bool live = m_new != -INFINITY;
            // v_exp_f32 itself: exp2f adds a rescaling around it for results below 2^-126,
            // which cannot matter next to the row maximum's weight of 1 and cost five more
            // VALU operations per score
            const float corr = live ? __builtin_amdgcn_exp2f(m_run[t] - m_new) : 1.f;
            float tsum = 0.f;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float p = live ? __builtin_amdgcn_exp2f(fmaf(sacc[t][kb][e], sl2, -m_new)) : 0.f;
                    sacc[t][kb][e] = p;
                    tsum += p;
                }
            tsum += __shfl_xor(tsum, 16, 64);
            tsum += __shfl_xor(tsum, 32, 64);
            l_run[t] = l_run[t] * corr + tsum;
            m_run[t] = m_new;
            // corr is exactly 1 unless the running maximum grew, which over a long prefix is
            // rare: the wave skips the 32 multiplies when no lane needs them
            if (__any(corr != 1.f))
#pragma unroll
                for (int db = 0; db < 8; ++db) oacc[t][db] *= corr;
            // within a 32-key step the key order is 4g+e (e<4), then 16+4g+(e-4)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                bp[t][ks][0] = pack_bf16(sacc[t][2 * ks][0], sacc[t][2 * ks][1]);
                bp[t][ks][1] = pack_bf16(sacc[t][2 * ks][2], sacc[t][2 * ks][3]);
                bp[t][ks][2] = pack_bf16(sacc[t][2 * ks + 1][0], sacc[t][2 * ks + 1][1]);
                bp[t][ks][3] = pack_bf16(sacc[t][2 * ks + 1][2], sacc[t][2 * ks + 1][3]);
            }
        }
        // O^T += V^T P^T, every V fragment feeding each of the wave's query tiles
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
            for (int db = 0; db < 8; ++db) {
                const bf16_t* vrow = Vt + (db * 16 + c16) * kVStride + 32 * ks + 4 * g;
                const u32x2 lo = *(const u32x2*)vrow;
                const u32x2 hi = *(const u32x2*)(vrow + 16);
                const u32x4 av = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
                for (int t = 0; t < QT; ++t) oacc[t][db] = mfma16(av, bp[t][ks], oacc[t][db]);
            }
        }
    };

    // prefix keys of this split, PF tiles per iteration; a tile past the end is staged as
    // zeros and not attended, and the tile PF ahead is always requested (a dummy past the end)
    for (int t0 = j_begin; t0 < j_end; t0 += PF * kTile) {
#pragma unroll
        for (int half = 0; half < PF; ++half) {
            const int tt = t0 + half * kTile;
            __syncthreads();
            store_prefix(half);
            __syncthreads();
            load_prefix(tt + PF * kTile, half);
            if (tt < j_end) attend_tile(tt, j_end - tt, j_end - tt < kTile);
        }
    }

    // tree keys: rotate k at L + depth, store k_rot, attend under the bitmask
    if (tree_split) {
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
                store_k(key, dc, klo);
                store_k(key, dc + 8, khi);
            }
            for (int c = tid; c < (kTile / 2) * (kDh / 8); c += NT) {
                const int kp = c & 31, dc = c >> 5, j = tb + 2 * kp;
                u32x4 v0 = {0, 0, 0, 0}, v1 = {0, 0, 0, 0};
                if (j < T) v0 = *(const u32x4*)(A.v + (((long)b * T + j) * H + h) * kDh + 8 * dc);
                if (j + 1 < T) v1 = *(const u32x4*)(A.v + (((long)b * T + j + 1) * H + h) * kDh + 8 * dc);
                store_v_pair(kp, dc, v0, v1);
            }
            __syncthreads();
            attend_tile(tb, min(kTile, T - tb), true);
        }
    }

#pragma unroll
    for (int t = 0; t < QT; ++t) {
        if (qi[t] < A.Tpad) {
            const long base = (((long)b * H + h) * (A.nsplit + 1) + split) * A.Tpad + qi[t];
            float* po = A.part_o + base * kDh;
#pragma unroll
            for (int db = 0; db < 8; ++db)
#pragma unroll
                for (int e = 0; e < 4; ++e) po[db * 16 + 4 * g + e] = oacc[t][db][e];
            if (g == 0) {
                A.part_ml[base * 2 + 0] = m_run[t];
                A.part_ml[base * 2 + 1] = l_run[t];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Streaming variant: K and V tiles by direct global-to-LDS loads
// ---------------------------------------------------------------------------
//
// The same split-KV flash pass (one (sequence, head, key split) per workgroup, waves owning
// query tiles, S^T = K Q^T then O^T = V^T P^T on MFMA, online softmax in log2 units, the
// last workgroup of each (sequence, head) attending to the rotated tree keys under the
// ancestor bitmask), with the prefix tiles streamed through a kRing-stage LDS ring filled
// by global_load_lds_dwordx4: while a tile is multiplied, the next kRing - 1 tiles are in
// flight and no register holds them.  Both tiles stay row-major (one 256-byte row per key)
// with their 16-byte pieces swizzled per row: K row r keeps piece p in slot p ^ (r mod 16)
// (its MFMA fragments read 16 rows at once), V row r in slot p ^ (2 r mod 16); V^T
// fragments come from the LDS transpose read ds_read_b64_tr_b16 -- in each 16-lane group,
// lane i receives element i mod 4 of the 8 bytes read by lane 4 e + i / 4 as its element
// e -- so 4 key rows x 16 dims land as 16 lanes x 4 keys.  The swizzles keep the fragment
// and transpose reads free of bank conflicts.
#ifndef MDT_ATTN_RING
#define MDT_ATTN_RING 2
#endif
constexpr int kRing = MDT_ATTN_RING;
constexpr int kStreamPages = 2048;              // page-table entries a streaming workgroup stages
constexpr int kTileBytes = kTile * kDh * 2;     // one K (or V) tile: 16 KiB
constexpr int kStageBytes = 2 * kTileBytes;     // K then V

__device__ __forceinline__ int kslot(int p, int r) { return p ^ (r & 15); }
__device__ __forceinline__ int vslot(int p, int r) { return p ^ ((2 * r) & 14); }

typedef short v4s_t __attribute__((ext_vector_type(4)));

template <int NWB, bool PAGED, int QT = 1>
__global__ __launch_bounds__(64 * NWB) void attn_stream(AttnArgs A) {
    constexpr int NT = 64 * NWB;
    constexpr int kInstr = kTile * (kDh / 8) / 64;  // load instructions per tile (K or V): 16
    constexpr int kIPW = 2 * kInstr / NWB;          // per wave per tile, K and V together
    static_assert(2 * kInstr % NWB == 0 && kIPW * (kRing - 2) < 64, "loads divide among the waves");
    __shared__ __attribute__((aligned(1024))) char ring[kRing * kStageBytes];
    __shared__ float2 cs[(MDT_MAX_HEADS + 1) * (kDh / 2)];  // cos/sin per (depth, pair)
    __shared__ int pages[PAGED ? kStreamPages : 1];          // physical page of each page of the split
    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const bool tree_split = split == A.nsplit;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, c16 = lane & 15;
    const int H = A.H, T = A.T;
    const int L = clamp_len(A.prefix_len, b, A.cache.capacity);
    const int j_begin = tree_split ? 0 : split * A.tiles_per_split * kTile;
    const int j_end = tree_split ? 0 : min(L, j_begin + A.tiles_per_split * kTile);
    const int ntiles = j_end > j_begin ? (j_end - j_begin + kTile - 1) / kTile : 0;
    const float scale = 1.f / sqrtf((float)kDh);
    const bf16_t* Kg = (const bf16_t*)A.cache.k;
    const bf16_t* Vg = (const bf16_t*)A.cache.v;
    const int psz = PAGED ? A.cache.page_size : 1;
    const int pg0 = j_begin / psz;

    // this wave's queries, loaded first: in tile t the lane holds query qi[t], dims
    // 32s + 8g .. +8; s = 0,1 hold x_m and s = 2,3 hold x_{m+64}
    int qi[QT], dq_raw[QT];
    bool q_ok[QT];
    u32x4 bq[QT][4];
    uint64_t qa[QT][MDT_MAX_NODES / 64];
#pragma unroll
    for (int t = 0; t < QT; ++t) {
        qi[t] = (wave * QT + t) * 16 + c16;
        q_ok[t] = qi[t] < T;
        const int qc = q_ok[t] ? qi[t] : 0;
        const long node = (((long)b * T + qc) * H + h) * kDh;
#pragma unroll
        for (int s = 0; s < 4; ++s) bq[t][s] = *(const u32x4*)(A.q + node + 32 * s + 8 * g);
#pragma unroll
        for (int w = 0; w < MDT_MAX_NODES / 64; ++w) qa[t][w] = A.anc[(long)qc * A.W + min(w, A.W - 1)];
        dq_raw[t] = A.depth[qc];
    }
    if (PAGED) {
        const int np = j_end > j_begin ? (j_end - 1) / psz - pg0 + 1 : 0;  // <= kStreamPages (host plan)
        for (int e = tid; e < np; e += NT) {
            const int pg = pg0 + e;
            const int page = pg < A.cache.max_pages ? A.cache.table[(long)b * A.cache.max_pages + pg] : -1;
            pages[e] = (page >= 0 && page < A.cache.num_pages) ? page : -1;
        }
        __syncthreads();
    }
    // element offset of prefix key j (j_begin <= j < j_end); an unmapped page reads the
    // pool's first row (a caller error: the value is meaningless but the access stays inside)
    auto key_off = [&](int j) -> long {
        if (!PAGED) return (((long)b * A.cache.capacity + j) * H + h) * kDh;
        const int page = pages[j / psz - pg0];
        return page < 0 ? 0 : (((long)page * psz + j % psz) * H + h) * kDh;
    };
    // the tile of keys t0 .. t0 + 63 into ring slot `slot`; keys past the split's end repeat
    // its last key (they are masked)
    auto issue = [&](int t0, int slot) {
        char* kst = ring + slot * kStageBytes;
#pragma unroll
        for (int j = 0; j < kIPW; ++j) {
            const int i = wave * kIPW + j;
            const bool isv = i >= kInstr;
            const int ii = isv ? i - kInstr : i;
            const int q = 64 * ii + lane;
            const int r = q >> 4, sl = q & 15;
            const int p = isv ? vslot(sl, r) : kslot(sl, r);  // the swizzles are involutions
            const long off = key_off(min(t0 + r, j_end - 1));
            const bf16_t* src = (isv ? Vg : Kg) + off + 8 * p;
            __builtin_amdgcn_global_load_lds((const void*)src, (lds_void_t*)(kst + (isv ? kTileBytes : 0) + 1024 * ii),
                                             16, 0, 0);
        }
    };
#pragma unroll
    for (int s = 0; s < kRing - 1; ++s)
        if (s < ntiles) issue(j_begin + s * kTile, s);

    for (int e = tid; e < (A.max_depth + 1) * (kDh / 2); e += NT)
        cs[e] = rope_cs_table_entry(L + e / (kDh / 2), A.inv_freq[e % (kDh / 2)]);
    __syncthreads();  // cos/sin table ready
#pragma unroll
    for (int t = 0; t < QT; ++t) {
        if (!q_ok[t])
#pragma unroll
            for (int s = 0; s < 4; ++s) bq[t][s] = u32x4{0, 0, 0, 0};
        const int dq = q_ok[t] ? min(max(dq_raw[t], 0), A.max_depth) : 0;
        const float2* row = cs + dq * (kDh / 2);
        rotate8(bq[t][0], bq[t][2], row, 8 * g);
        rotate8(bq[t][1], bq[t][3], row, 32 + 8 * g);
#pragma unroll
        for (int w = 0; w < MDT_MAX_NODES / 64; ++w)
            if (!(tree_split && q_ok[t] && w < A.W)) qa[t][w] = 0;
    }

    f32x4 oacc[QT][8];
    float m_run[QT], l_run[QT];  // of query qi[t], replicated over g
#pragma unroll
    for (int t = 0; t < QT; ++t) {
#pragma unroll
        for (int db = 0; db < 8; ++db) oacc[t][db] = f32x4{0.f, 0.f, 0.f, 0.f};
        m_run[t] = -INFINITY;
        l_run[t] = 0.f;
    }

    const float sl2 = scale * 1.4426950408889634f;
    // One tile in ring slot `slot`: keys base..base+63, nvalid of them real.
    auto attend_tile = [&](int slot, int base, int nvalid, bool masked) {
        const bf16_t* Ks = (const bf16_t*)(ring + slot * kStageBytes);
        const bf16_t* Vs = (const bf16_t*)(ring + slot * kStageBytes + kTileBytes);
        f32x4 sacc[QT][4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            f32x4 acc[QT];
#pragma unroll
            for (int t = 0; t < QT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
            const int r = kb * 16 + c16;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const u32x4 kf = *(const u32x4*)(Ks + (r * 16 + kslot(4 * s + g, r)) * 8);
#pragma unroll
                for (int t = 0; t < QT; ++t) acc[t] = mfma16(kf, bq[t][s], acc[t]);
            }
#pragma unroll
            for (int t = 0; t < QT; ++t) sacc[t][kb] = acc[t];
        }
        u32x4 bp[QT][2];
#pragma unroll
        for (int t = 0; t < QT; ++t) {
            float tmax = -INFINITY;
            if (masked) {
                const int wi = base >> 6;
                const uint64_t qw = !tree_split ? ~0ull
                                  : wi == 0     ? qa[t][0]
                                  : wi == 1     ? qa[t][1]
                                  : wi == 2     ? qa[t][2]
                                                : qa[t][3];
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int jj = kb * 16 + 4 * g + e;
                        const bool ok = jj < nvalid && ((qw >> jj) & 1ull);
                        const float sv = ok ? sacc[t][kb][e] : -INFINITY;
                        sacc[t][kb][e] = sv;
                        tmax = fmaxf(tmax, sv);
                    }
            } else {
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                    for (int e = 0; e < 4; ++e) tmax = fmaxf(tmax, sacc[t][kb][e]);
            }
            tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
            tmax *= sl2;
            const float m_new = fmaxf(m_run[t], tmax);
            const bool live = m_new != -INFINITY;
            const float corr = live ? __builtin_amdgcn_exp2f(m_run[t] - m_new) : 1.f;
            float tsum = 0.f;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float p = live ? __builtin_amdgcn_exp2f(fmaf(sacc[t][kb][e], sl2, -m_new)) : 0.f;
                    sacc[t][kb][e] = p;
                    tsum += p;
                }
            tsum += __shfl_xor(tsum, 16, 64);
            tsum += __shfl_xor(tsum, 32, 64);
            l_run[t] = l_run[t] * corr + tsum;
            m_run[t] = m_new;
            if (__any(corr != 1.f))
#pragma unroll
                for (int db = 0; db < 8; ++db) oacc[t][db] *= corr;
            // within a 32-key step the key order is 4g+e (e<4), then 16+4g+(e-4)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                bp[t][ks][0] = pack_bf16(sacc[t][2 * ks][0], sacc[t][2 * ks][1]);
                bp[t][ks][1] = pack_bf16(sacc[t][2 * ks][2], sacc[t][2 * ks][3]);
                bp[t][ks][2] = pack_bf16(sacc[t][2 * ks + 1][0], sacc[t][2 * ks + 1][1]);
                bp[t][ks][3] = pack_bf16(sacc[t][2 * ks + 1][2], sacc[t][2 * ks + 1][3]);
            }
        }
        // O^T += V^T P^T: lane (dim 16 db + c16, group g) takes keys 32 ks + 4 g + e and
        // 32 ks + 16 + 4 g + e (e < 4) by two transpose reads; as a source lane it reads the 8
        // bytes of key row 32 ks + 16 hf + 4 g + c16 / 4, dims 16 db + 4 (c16 mod 4) ..
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
            for (int db = 0; db < 8; ++db) {
                u32x2 half[2];
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const int r = 32 * ks + 16 * hf + 4 * g + (c16 >> 2);
                    const int p = 2 * db + ((c16 & 3) >> 1);
                    const bf16_t* src = Vs + (r * 16 + vslot(p, r)) * 8 + 4 * (c16 & 1);
                    const v4s_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) v4s_t*)(src));
                    half[hf] = __builtin_bit_cast(u32x2, v);
                }
                const u32x4 av = {half[0][0], half[0][1], half[1][0], half[1][1]};
#pragma unroll
                for (int t = 0; t < QT; ++t) oacc[t][db] = mfma16(av, bp[t][ks], oacc[t][db]);
            }
        }
    };

    // prefix tiles of this split: the tile kRing - 1 ahead is requested once a slot frees up
    for (int t = 0; t < ntiles; ++t) {
        const int later = min(kRing - 2, ntiles - 1 - t);
        if (later >= 2)
            ring_barrier<2 * kIPW>();
        else if (later == 1)
            ring_barrier<kIPW>();
        else
            ring_barrier<0>();
        if (t + kRing - 1 < ntiles) issue(j_begin + (t + kRing - 1) * kTile, (t + kRing - 1) % kRing);
        const int base = j_begin + t * kTile;
        attend_tile(t % kRing, base, min(kTile, j_end - base), j_end - base < kTile);
    }

    // tree keys: rotate k at L + depth, store k_rot, stage into slot 0, attend under the bitmask
    if (tree_split) {
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
            __syncthreads();
            attend_tile(0, tb, min(kTile, T - tb), true);
        }
    }

#pragma unroll
    for (int t = 0; t < QT; ++t) {
        if (qi[t] < A.Tpad) {
            const long base = (((long)b * H + h) * (A.nsplit + 1) + split) * A.Tpad + qi[t];
            float* po = A.part_o + base * kDh;
#pragma unroll
            for (int db = 0; db < 8; ++db)
#pragma unroll
                for (int e = 0; e < 4; ++e) po[db * 16 + 4 * g + e] = oacc[t][db][e];
            if (g == 0) {
                A.part_ml[base * 2 + 0] = m_run[t];
                A.part_ml[base * 2 + 1] = l_run[t];
            }
        }
    }
}

// Merge the split partials of every (sequence, head, node). grid (T, H, B), block 64.
__global__ __launch_bounds__(64) void attn_combine(const float* __restrict__ part_o, const float* __restrict__ part_ml,
                                                   int T, int Tpad, int H, int nsplit, bf16_t* __restrict__ out) {
    const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x;
    const long pbase = ((long)b * H + h) * nsplit * Tpad + i;
    // splits in batches of 8, all loads of a batch first; running max and sums rescale
    // between batches (maxima are in log2 units)
    float M = -INFINITY, den = 0.f, na = 0.f, nb = 0.f;
    for (int s0 = 0; s0 < nsplit; s0 += 8) {
        float ms[8], ls[8], oa[8], ob[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const long pidx = pbase + (long)min(s0 + u, nsplit - 1) * Tpad;
            ms[u] = part_ml[pidx * 2];
            ls[u] = part_ml[pidx * 2 + 1];
            oa[u] = part_o[pidx * kDh + lane];
            ob[u] = part_o[pidx * kDh + lane + 64];
        }
        float bm = M;
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (s0 + u < nsplit) bm = fmaxf(bm, ms[u]);
        if (bm == -INFINITY) continue;
        const float r = exp2f(M - bm);  // 0 while M is -inf
        den *= r;
        na *= r;
        nb *= r;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (s0 + u >= nsplit || ms[u] == -INFINITY) continue;
            const float wgt = exp2f(ms[u] - bm);
            den += ls[u] * wgt;
            na += oa[u] * wgt;
            nb += ob[u] * wgt;
        }
        M = bm;
    }
    bf16_t* o = out + (((long)b * T + i) * H + h) * kDh;
    o[lane] = f32_to_bf16(na / den);
    o[lane + 64] = f32_to_bf16(nb / den);
}

struct Plan {
    int Tpad, nsplit, tiles_per_split, nwb;
    size_t po_bytes, pml_bytes;
};

// Split choice by a cost model in units of one 64-key tile: a workgroup costs a fixed
// setup plus its tiles (the tree workgroup about three), and the workgroups run one per
// CU in rounds of kPlanCUs (the MFMA kernel holds one workgroup per CU).  More splits
// shorten every workgroup but add rounds and partial-state traffic for the combine.
// A fixed CU count (MI355X) keeps the plan, and so the workspace size, device-independent.
constexpr int kPlanCUs = 256;
constexpr double kSetupTiles = 1.2, kTreeTiles = 3.0, kCombineTilesPerSplit = 0.1;

Plan plan(int B, int T, int H, int capacity) {
    Plan p;
    p.Tpad = (T + 15) / 16 * 16;
    const int waves = p.Tpad / 16;
    p.nwb = waves <= 4 ? 4 : (waves <= 8 ? 8 : 16);
    const int tiles = capacity > 0 ? (capacity + kTile - 1) / kTile : 1;
    const long bh = (long)B * H;
    double best = 1e300;
    int best_tps = tiles < kMaxTilesPerSplit ? tiles : kMaxTilesPerSplit;
    for (int tps = 1; tps <= tiles && tps <= kMaxTilesPerSplit; ++tps) {
        const int ns = (tiles + tps - 1) / tps;
        const long wgs = bh * (ns + 1);
        const long rounds = (wgs + kPlanCUs - 1) / kPlanCUs;
        const double per_wg = kSetupTiles + (tps > kTreeTiles ? tps : kTreeTiles);
        const double cost = rounds * per_wg + kCombineTilesPerSplit * ns * ((bh + kPlanCUs - 1) / kPlanCUs);
        if (cost < best - 1e-9) {
            best = cost;
            best_tps = tps;
        }
    }
#ifdef MDT_ATTN_TPS
    best_tps = MDT_ATTN_TPS < tiles ? MDT_ATTN_TPS : tiles;
#endif
    p.tiles_per_split = best_tps;
    p.nsplit = (tiles + best_tps - 1) / best_tps;
    // prefix splits plus one tree split
    p.po_bytes = ((size_t)B * H * (p.nsplit + 1) * p.Tpad * kDh * sizeof(float) + 255) & ~(size_t)255;
    p.pml_bytes = (size_t)B * H * (p.nsplit + 1) * p.Tpad * 2 * sizeof(float);
    return p;
}

}  // namespace

extern "C" size_t mdt_tree_attention_workspace(mdt_dtype dt, int B, int T, int H, int Dh, int capacity) {
    if (dt != MDT_BF16 || B < 1 || T < 1 || H < 1) return 0;
    (void)Dh;
    const Plan p = plan(B, T, H, capacity);
    return p.po_bytes + p.pml_bytes;
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
    const Plan p = plan(B, T, H, cache->capacity);
    MDT_REQUIRE(ws, MDT_ERR_WORKSPACE, "workspace is NULL");
    MDT_REQUIRE(mdt_aligned16(ws), MDT_ERR_ALIGN, "workspace must be 16-byte aligned");
    MDT_REQUIRE(ws_bytes >= p.po_bytes + p.pml_bytes, MDT_ERR_WORKSPACE, "workspace too small");
    AttnArgs A{kv, (const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v, prefix_len, tree->depth, tree->anc,
               (bf16_t*)k_rot, (float*)ws, (float*)((char*)ws + p.po_bytes), theta, T, p.Tpad, H,
               tree->anc_words, p.nsplit, p.tiles_per_split, tree->max_depth, {}};
    for (int m = 0; m < kDh / 2; ++m) A.inv_freq[m] = std::pow(theta, -2.0 * (double)m / (double)kDh);
    const dim3 grid(p.nsplit + 1, H, B);
    const bool paged = cache->layout == MDT_KV_PAGED;
    // up to 8 query tiles: one per wave; up to 16: two per wave on 8 waves
    // trees of up to 128 nodes (one query tile per wave) stream their tiles through the LDS
    // ring; 256-node trees (two query tiles per wave, the softmax between the products
    // dominating) keep the register-staged kernel, which measured faster there (767 against
    // 855 us at the 33B shape) while the stream is faster or equal on the smaller trees
    auto kern = p.nwb == 4 ? (paged ? attn_stream<4, true> : attn_stream<4, false>)
              : p.nwb == 8 ? (paged ? attn_stream<8, true> : attn_stream<8, false>)
                           : (paged ? attn_tree_mfma<8, true, 2> : attn_tree_mfma<8, false, 2>);
    MDT_LAUNCH("attn_tree_mfma", kern, grid, dim3(64 * (p.nwb == 16 ? 8 : p.nwb)), 0, s, A);
    st = mdt_launched("attn_tree_mfma");
    if (st != MDT_OK) return st;
    MDT_LAUNCH("attn_combine", attn_combine, dim3(T, H, B), dim3(64), 0, s, A.part_o, A.part_ml, T, p.Tpad, H,
               p.nsplit + 1, (bf16_t*)out);
    return mdt_launched("attn_combine");
}
