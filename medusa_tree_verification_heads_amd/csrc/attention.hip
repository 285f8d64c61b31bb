// mdt_tree_attention: tree-masked attention of the packed candidate tree.
//
// Summary page "Medusa: Simple LLM Inference Acceleration Framework with Multiple
// Decoding Heads", section "Tree Attention": step 3 (a node attends to the prefix
// and to its ancestors only; the node itself is included), step 4 (position id
// = prefix length + depth, rotary embedding as in Llama) and step 5 (one pass
// over all nodes).  "Notes on Medusa", section 3: the tree is flattened into
// one sequence and masked.
//
// bf16 path (Dh = 128), three kernels:
//  1. rope:    rotate the tree's q and k at their depth positions; k_rot is an
//              output (it is what gets cached), q_rot (bf16) goes to the workspace.
//  2. prefix:  split-KV flash pass over the prefix cache.  A workgroup owns one
//              (sequence, head, key range); its waves each own 16 tree queries.
//              64-key K and V tiles are staged in LDS (V transposed), and both
//              products run on MFMA 16x16x32 bf16: S^T = K Q^T, then O^T = V^T P^T,
//              so the probabilities stay in registers between the two.  Online
//              softmax keeps (max, sum) per query; partial (m, l, O) go to the
//              workspace.
//  3. combine: per (sequence, head, node) merge the partials with the node's
//              tree keys (ancestor-or-self bitmask row) and write o (bf16).
// fp32 path: one wave per (sequence, head, node) walks all allowed keys on VALU.
#include <math.h>

#include "common.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kTile = 64;          // keys per LDS tile
constexpr int kDh = 128;           // head dim of the MFMA path
constexpr int kKStride = kDh + 8;  // LDS row stride of K tile (elements)
constexpr int kVStride = kTile + 4;  // LDS row stride of transposed V tile (elements)
constexpr int kMinTilesPerSplit = 4;

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

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// q_rot [B][H][Tpad][Dh] (bf16, rows >= T zero) and k_rot [B][T][H][Dh].
__global__ __launch_bounds__(256) void attn_rope(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                                                 const int32_t* __restrict__ prefix_len,
                                                 const int32_t* __restrict__ depth, int capacity, int T, int Tpad,
                                                 int H, double theta, bf16_t* __restrict__ q_rot,
                                                 bf16_t* __restrict__ k_rot) {
    const int i = blockIdx.x, b = blockIdx.y;
    const int half = kDh / 2;
    const int L = clamp_len(prefix_len, b, capacity);
    for (int e = threadIdx.x; e < H * half; e += blockDim.x) {
        const int h = e / half, m = e % half;
        bf16_t* qo = q_rot + (((long)b * H + h) * Tpad + i) * kDh;
        if (i >= T) {
            qo[m] = 0;
            qo[m + half] = 0;
            continue;
        }
        double c, s;
        rope_cs(L + depth[i], m, kDh, theta, c, s);
        const long node = (((long)b * T + i) * H + h) * kDh;
        const double x1 = bf16_to_f32(q[node + m]), x2 = bf16_to_f32(q[node + m + half]);
        qo[m] = f64_to_bf16(x1 * c - x2 * s);
        qo[m + half] = f64_to_bf16(x2 * c + x1 * s);
        const double y1 = bf16_to_f32(k[node + m]), y2 = bf16_to_f32(k[node + m + half]);
        k_rot[node + m] = f64_to_bf16(y1 * c - y2 * s);
        k_rot[node + m + half] = f64_to_bf16(y2 * c + y1 * s);
    }
}

// Prefix pass: grid (nsplit, H, B), block 64 * nw (nw = Tpad / 16 waves).
__global__ __launch_bounds__(1024) void attn_prefix_mfma(KV cache, const bf16_t* __restrict__ q_rot,
                                                         const int32_t* __restrict__ prefix_len, int H, int Tpad,
                                                         int tiles_per_split, int nsplit, float* __restrict__ part_o,
                                                         float* __restrict__ part_ml) {
    __shared__ __attribute__((aligned(16))) bf16_t Ks[kTile * kKStride];
    __shared__ __attribute__((aligned(16))) bf16_t Vt[kDh * kVStride];
    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, c16 = lane & 15;
    const int nthreads = blockDim.x;
    const int L = clamp_len(prefix_len, b, cache.capacity);
    const int j_begin = split * tiles_per_split * kTile;
    const int j_end = min(L, j_begin + tiles_per_split * kTile);
    const float scale = 1.f / sqrtf((float)kDh);

    // this wave's 16 queries as the B operand of S^T = K Q^T: lane holds query c16, dims 32s + 8g .. +8
    const int q0 = wave * 16;
    u32x4 bq[4];
    const bf16_t* qrow = q_rot + (((long)b * H + h) * Tpad + q0 + c16) * kDh;
#pragma unroll
    for (int s = 0; s < 4; ++s) bq[s] = *(const u32x4*)(qrow + 32 * s + 8 * g);

    f32x4 oacc[8];
#pragma unroll
    for (int db = 0; db < 8; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;  // for query c16 (replicated over g)

    const bf16_t* Kg = (const bf16_t*)cache.k;
    const bf16_t* Vg = (const bf16_t*)cache.v;
    for (int t0 = j_begin; t0 < j_end; t0 += kTile) {
        // stage the tile: 64 keys x 128 dims of K (row-major) and V (transposed)
        __syncthreads();
        for (int c = threadIdx.x; c < kTile * (kDh / 8); c += nthreads) {
            const int key = c >> 4, dc = c & 15;
            const int j = t0 + key;
            u32x4 kv = {0, 0, 0, 0}, vv = {0, 0, 0, 0};
            if (j < j_end) {
                const long off = kv_offset(cache, b, j, h, H, kDh);
                if (off >= 0) {
                    kv = *(const u32x4*)(Kg + off + 8 * dc);
                    vv = *(const u32x4*)(Vg + off + 8 * dc);
                }
            }
            *(u32x4*)(Ks + key * kKStride + 8 * dc) = kv;
            bf16_t* vt = Vt + (8 * dc) * kVStride + key;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                vt[(2 * t) * kVStride] = (bf16_t)(vv[t] & 0xffffu);
                vt[(2 * t + 1) * kVStride] = (bf16_t)(vv[t] >> 16);
            }
        }
        __syncthreads();

        // S^T tile: 4 key blocks of 16; lane holds keys kb*16 + 4g + e for query c16
        f32x4 sacc[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            const bf16_t* krow = Ks + (kb * 16 + c16) * kKStride + 8 * g;
#pragma unroll
            for (int s = 0; s < 4; ++s) acc = mfma16(*(const u32x4*)(krow + 32 * s), bq[s], acc);
            sacc[kb] = acc;
        }
        // online softmax over the tile for query c16
        float tmax = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = t0 + kb * 16 + 4 * g + e;
                const float sv = (j < j_end) ? sacc[kb][e] * scale : -INFINITY;
                sacc[kb][e] = sv;
                tmax = fmaxf(tmax, sv);
            }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
        const float m_new = fmaxf(m_run, tmax);
        const float corr = (m_new == -INFINITY) ? 1.f : expf(m_run - m_new);
        float tsum = 0.f;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float p = (m_new == -INFINITY) ? 0.f : expf(sacc[kb][e] - m_new);
                sacc[kb][e] = p;
                tsum += p;
            }
        tsum += __shfl_xor(tsum, 16, 64);
        tsum += __shfl_xor(tsum, 32, 64);
        l_run = l_run * corr + tsum;
        m_run = m_new;
#pragma unroll
        for (int db = 0; db < 8; ++db) oacc[db] *= corr;

        // O^T += V^T P^T: two key steps of 32; key order within a step: 4g+t (t<4) then 16+4g+(t-4)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            u32x4 bp;
            bp[0] = pack_bf16(sacc[2 * ks][0], sacc[2 * ks][1]);
            bp[1] = pack_bf16(sacc[2 * ks][2], sacc[2 * ks][3]);
            bp[2] = pack_bf16(sacc[2 * ks + 1][0], sacc[2 * ks + 1][1]);
            bp[3] = pack_bf16(sacc[2 * ks + 1][2], sacc[2 * ks + 1][3]);
#pragma unroll
            for (int db = 0; db < 8; ++db) {
                const bf16_t* vrow = Vt + (db * 16 + c16) * kVStride + 32 * ks + 4 * g;
                const u32x2 lo = *(const u32x2*)vrow;
                const u32x2 hi = *(const u32x2*)(vrow + 16);
                const u32x4 av = {lo[0], lo[1], hi[0], hi[1]};
                oacc[db] = mfma16(av, bp, oacc[db]);
            }
        }
    }

    // partial results for queries q0 + c16: O^T rows dims db*16 + 4g + e
    const long base = (((long)b * H + h) * nsplit + split) * Tpad + q0 + c16;
    float* po = part_o + base * kDh;
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
        for (int e = 0; e < 4; ++e) po[db * 16 + 4 * g + e] = oacc[db][e];
    if (g == 0) {
        part_ml[base * 2 + 0] = m_run;
        part_ml[base * 2 + 1] = l_run;
    }
}

// Merge the prefix partials with the node's tree keys. grid (T, H, B), block 64.
__global__ __launch_bounds__(64) void attn_combine(const bf16_t* __restrict__ q_rot, const bf16_t* __restrict__ k_rot,
                                                   const bf16_t* __restrict__ v, const float* __restrict__ part_o,
                                                   const float* __restrict__ part_ml,
                                                   const uint64_t* __restrict__ anc, int T, int Tpad, int H, int W,
                                                   int nsplit, bf16_t* __restrict__ out) {
    const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x;
    const float scale = 1.f / sqrtf((float)kDh);
    const bf16_t* qi = q_rot + (((long)b * H + h) * Tpad + i) * kDh;
    const float qa = bf16_to_f32(qi[lane]), qb = bf16_to_f32(qi[lane + 64]);
    // tree scores
    float ts[MDT_MAX_HEADS + 1];
    int tj[MDT_MAX_HEADS + 1];
    int nt = 0;
    float M = -INFINITY;
    for (int w = 0; w < W; ++w) {
        uint64_t bits = anc[(long)i * W + w];
        while (bits && nt <= MDT_MAX_HEADS) {
            const int j = w * 64 + __builtin_ctzll(bits);
            bits &= bits - 1;
            if (j >= T) break;
            const bf16_t* kj = k_rot + (((long)b * T + j) * H + h) * kDh;
            const float s = wave_sum(qa * bf16_to_f32(kj[lane]) + qb * bf16_to_f32(kj[lane + 64])) * scale;
            ts[nt] = s;
            tj[nt] = j;
            ++nt;
            M = fmaxf(M, s);
        }
    }
    const long pbase = ((long)b * H + h) * nsplit * Tpad + i;
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, part_ml[(pbase + (long)s * Tpad) * 2]);
    float den = 0.f, na = 0.f, nb = 0.f;
    for (int s = 0; s < nsplit; ++s) {
        const long p = pbase + (long)s * Tpad;
        const float ms = part_ml[p * 2];
        if (ms == -INFINITY) continue;
        const float wgt = expf(ms - M);
        den += part_ml[p * 2 + 1] * wgt;
        na += part_o[p * kDh + lane] * wgt;
        nb += part_o[p * kDh + lane + 64] * wgt;
    }
    for (int t = 0; t < nt; ++t) {
        const float wgt = expf(ts[t] - M);
        const bf16_t* vj = v + (((long)b * T + tj[t]) * H + h) * kDh;
        den += wgt;
        na += wgt * bf16_to_f32(vj[lane]);
        nb += wgt * bf16_to_f32(vj[lane + 64]);
    }
    bf16_t* o = out + (((long)b * T + i) * H + h) * kDh;
    o[lane] = f32_to_bf16(na / den);
    o[lane + 64] = f32_to_bf16(nb / den);
}

struct Plan {
    int Tpad, nsplit, tiles_per_split;
    size_t q_bytes, po_bytes, pml_bytes;
};

Plan plan(int B, int T, int H, int capacity) {
    Plan p;
    p.Tpad = (T + 15) / 16 * 16;
    const int tiles = capacity > 0 ? (capacity + kTile - 1) / kTile : 1;
    long want = (512 + (long)B * H - 1) / ((long)B * H);
    if (want < 1) want = 1;
    int tps = (int)((tiles + want - 1) / want);
    if (tps < kMinTilesPerSplit) tps = kMinTilesPerSplit;
    p.tiles_per_split = tps;
    p.nsplit = (tiles + tps - 1) / tps;
    p.q_bytes = ((size_t)B * H * p.Tpad * kDh * sizeof(bf16_t) + 255) & ~(size_t)255;
    p.po_bytes = ((size_t)B * H * p.nsplit * p.Tpad * kDh * sizeof(float) + 255) & ~(size_t)255;
    p.pml_bytes = (size_t)B * H * p.nsplit * p.Tpad * 2 * sizeof(float);
    return p;
}

}  // namespace

extern "C" size_t mdt_tree_attention_workspace(mdt_dtype dt, int B, int T, int H, int Dh, int capacity) {
    if (dt != MDT_BF16 || B < 1 || T < 1 || H < 1) return 0;
    (void)Dh;
    const Plan p = plan(B, T, H, capacity);
    return p.q_bytes + p.po_bytes + p.pml_bytes;
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
        hipLaunchKernelGGL(attn_valu<float>, dim3(T, H, B), dim3(64), 0, s, kv, (const float*)q, (const float*)k,
                           (const float*)v, prefix_len, tree->depth, tree->anc, T, H, Dh, tree->anc_words, theta,
                           (float*)out, (float*)k_rot);
        return mdt_check_launch("tree_attention");
    }
    const Plan p = plan(B, T, H, cache->capacity);
    MDT_REQUIRE(ws, MDT_ERR_WORKSPACE, "workspace is NULL");
    MDT_REQUIRE(mdt_aligned16(ws), MDT_ERR_ALIGN, "workspace must be 16-byte aligned");
    MDT_REQUIRE(ws_bytes >= p.q_bytes + p.po_bytes + p.pml_bytes, MDT_ERR_WORKSPACE, "workspace too small");
    bf16_t* q_rot = (bf16_t*)ws;
    float* part_o = (float*)((char*)ws + p.q_bytes);
    float* part_ml = (float*)((char*)ws + p.q_bytes + p.po_bytes);
    hipLaunchKernelGGL(attn_rope, dim3(p.Tpad, B), dim3(256), 0, s, (const bf16_t*)q, (const bf16_t*)k, prefix_len,
                       tree->depth, cache->capacity, T, p.Tpad, H, theta, q_rot, (bf16_t*)k_rot);
    st = mdt_check_launch("tree_attention rope");
    if (st != MDT_OK) return st;
    hipLaunchKernelGGL(attn_prefix_mfma, dim3(p.nsplit, H, B), dim3(64 * (p.Tpad / 16)), 0, s, kv, q_rot,
                       prefix_len, H, p.Tpad, p.tiles_per_split, p.nsplit, part_o, part_ml);
    st = mdt_check_launch("tree_attention prefix");
    if (st != MDT_OK) return st;
    hipLaunchKernelGGL(attn_combine, dim3(T, H, B), dim3(64), 0, s, q_rot, (const bf16_t*)k_rot, (const bf16_t*)v,
                       part_o, part_ml, tree->anc, T, p.Tpad, H, tree->anc_words, p.nsplit, (bf16_t*)out);
    return mdt_check_launch("tree_attention combine");
}
