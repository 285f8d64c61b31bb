// The decoder layers of the verify forward: the backbone pass that the packed tree goes
// through before the LM head (summary page, section 3.2 step 4 and "Tree Attention"
// steps 3-5: all candidates are processed by the full model in one forward pass with
// the tree mask; "Notes on Medusa", section 3).  The pages name the backbone
// (Vicuna, a Llama model) but not its layer; the layer here is the Llama one:
// pre-norm RMSNorm, q/k/v projections, tree attention with rotary positions, output
// projection with residual, RMSNorm, SwiGLU feed-forward with residual.
//
//   mdt_embed        x0[m] = E[token[m]]
//   mdt_rmsnorm      h = x / sqrt(mean(x^2) + eps) * g
//   mdt_add_rmsnorm  x += sum of fp32 partial products; h = rmsnorm(x) * g
//   mdt_linear       y = x W^T (+ residual), q|k|v segments, or the SwiGLU of an
//                    interleaved gate/up product
//   mdt_linear_split the products of nsplit slices of the inner dimension, in fp32
//
// The linear calls stream W once: with M <= 64 rows (a 64-node tree) every weight byte
// is read once and used for 64 rows, so a product is bound by HBM, not by the matrix
// cores.  Each workgroup multiplies 64 x rows by 48 to 128 weight rows (dma_tile.h; the
// narrowest width whose grid still has one workgroup per CU).  A weight with few
// 64-row blocks (the d x d output projection: 64 blocks for 256 CUs) has its inner
// dimension cut into slices on more workgroups; their fp32 partial tiles are added
// by the next call, which reads whole rows anyway (mdt_add_rmsnorm: the residual add
// and the following RMSNorm), so no workgroup waits for another.
#include <math.h>

#include "dma_tile.h"

namespace {

constexpr int kMBL = 64;  // x rows per workgroup

enum Epi { kStore = 0, kResidual = 1, kSwiglu = 2, kPartial = 3 };

struct LinArgs {
    const bf16_t* x;
    const bf16_t* W;
    const bf16_t* res;
    bf16_t* y;
    float* part;  // kPartial: [nsplit][M][N]
    int M, N, K, kslice, nseg;
};

__device__ __forceinline__ uint32_t pack2(float a, float b) {
    return (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
}

__device__ __forceinline__ float lo16(uint32_t u) { return bf16_to_f32(u & 0xffffu); }
__device__ __forceinline__ float hi16(uint32_t u) { return bf16_to_f32(u >> 16); }

// x SiLU(x)-gated: silu(g) * u, silu(g) = g / (1 + e^-g).
__device__ __forceinline__ float swiglu(float g, float u) { return g / (1.f + __expf(-g)) * u; }

// The stores of a product's 64 x NB result tile zt (row stride NB + 1, in LDS) by NTH
// threads: fp32 slices (kPartial), the SwiGLU of gate/up column pairs, or bf16 columns in
// nseg segments (optionally plus the residual).
template <int EPI, int NB, int NTH>
__device__ __forceinline__ void linear_epilogue(const LinArgs& a, const float* zt, int m0, int n0, int s) {
    constexpr int kZs = NB + 1;
    if constexpr (EPI == kPartial) {
        // four consecutive columns per item, 16-byte stores
        constexpr int kItems = NB / 4;
        float* ps = a.part + (size_t)s * a.M * a.N;
        for (int it = threadIdx.x; it < kMBL * kItems; it += NTH) {
            const int row = it / kItems, c0 = 4 * (it % kItems);
            const int m = m0 + row, n = n0 + c0;
            if (m >= a.M || n >= a.N) continue;
            const float* zr = zt + row * kZs + c0;
            *(float4*)(ps + (size_t)m * a.N + n) = make_float4(zr[0], zr[1], zr[2], zr[3]);
        }
        return;
    }

    if constexpr (EPI == kSwiglu) {
        // Weight rows 32j..32j+15 are gate rows 16j.., rows 32j+16..32j+31 the matching up
        // rows: output column 16j + i = silu(gate_i) * up_i.  One item, eight outputs.
        constexpr int kItems = NB / 16;
        const int F = a.N >> 1;
        for (int it = threadIdx.x; it < kMBL * kItems; it += NTH) {
            const int row = it / kItems, og = it % kItems;
            const int jj = og >> 1, i0 = 8 * (og & 1);
            const int m = m0 + row;
            if (m >= a.M || n0 + 32 * jj >= a.N) continue;
            const float* zr = zt + row * kZs + 32 * jj + i0;
            uint4 o;
            o.x = pack2(swiglu(zr[0], zr[16]), swiglu(zr[1], zr[17]));
            o.y = pack2(swiglu(zr[2], zr[18]), swiglu(zr[3], zr[19]));
            o.z = pack2(swiglu(zr[4], zr[20]), swiglu(zr[5], zr[21]));
            o.w = pack2(swiglu(zr[6], zr[22]), swiglu(zr[7], zr[23]));
            *(uint4*)(a.y + (size_t)m * F + (n0 >> 1) + 16 * jj + i0) = o;
        }
    } else {
        // Eight consecutive columns per item; the columns are cut into nseg equal
        // segments, segment q going to y + q*M*(N/nseg) as its own [M][N/nseg] matrix.
        constexpr int kItems = NB / 8;
        const int nsegc = a.N / a.nseg;
        for (int it = threadIdx.x; it < kMBL * kItems; it += NTH) {
            const int row = it / kItems, c0 = 8 * (it % kItems);
            const int m = m0 + row, n = n0 + c0;
            if (m >= a.M || n >= a.N) continue;
            const float* zr = zt + row * kZs + c0;
            float v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = zr[j];
            if constexpr (EPI == kResidual) {
                const uint4 r = *(const uint4*)(a.res + (size_t)m * a.N + n);
                v[0] += lo16(r.x), v[1] += hi16(r.x), v[2] += lo16(r.y), v[3] += hi16(r.y);
                v[4] += lo16(r.z), v[5] += hi16(r.z), v[6] += lo16(r.w), v[7] += hi16(r.w);
            }
            const int q = n / nsegc;
            uint4 o;
            o.x = pack2(v[0], v[1]);
            o.y = pack2(v[2], v[3]);
            o.z = pack2(v[4], v[5]);
            o.w = pack2(v[6], v[7]);
            *(uint4*)(a.y + (size_t)q * a.M * nsegc + (size_t)m * nsegc + (n - q * nsegc)) = o;
        }
    }
}

// One 64 x NB tile of a product on dma_tile: both operands staged by direct global-to-LDS
// loads through an S-stage ring of 128-dim chunks, CG column groups x KS k-groups of waves
// (chosen per tile width so that the loads divide evenly among the waves).  Column block b
// walks its chunks from chunk b on, so that neighbouring workgroups read different parts of
// their weight rows at any one time.
// grid (ceil(N/NB), ceil(M/64), nsplit); blockIdx.z > 0 only for kPartial.
template <int EPI, int NB, int CG, int KS, int S>
__global__ __launch_bounds__(64 * CG * KS) void linear_dma(LinArgs a) {
    using P = DmaTile<128, NB, CG, KS, S>;
    constexpr int NTH = P::NT;
    constexpr int kZs = NB + 1;
    constexpr int kZOff = P::kRedBytes;  // the result tile after the k-groups' partials
    constexpr int kEpi = kZOff + kMBL * kZs * 4;
    constexpr int kLds = P::kRingBytes > kEpi ? P::kRingBytes : kEpi;
    static_assert(EPI != kSwiglu || NB % 32 == 0, "SwiGLU tiles hold whole gate/up pairs");
    __shared__ __attribute__((aligned(1024))) char smem[kLds];
    const int n0 = blockIdx.x * NB, m0 = blockIdx.y * kMBL, s = blockIdx.z;
    const int k0 = s * a.kslice;
    const int klen = min(a.kslice, a.K - k0);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, c16 = lane & 15, cg = wave % CG;
    float* zt = (float*)(smem + kZOff);
    dma_tile<128, NB, CG, KS, S, 2>(a.x + (size_t)m0 * a.K + k0, a.W + k0, a.M - m0, klen, a.K, a.N, n0, smem,
                                    [&](const f32x4 (&acc)[NB / CG / 16][4]) {
#pragma unroll
                                        for (int nt = 0; nt < NB / CG / 16; ++nt)
#pragma unroll
                                            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                                                for (int e = 0; e < 4; ++e)
                                                    zt[(mt * 16 + 4 * g + e) * kZs + cg * (NB / CG) + 16 * nt +
                                                       c16] = acc[nt][mt][e];
                                    },
                                    blockIdx.x);
    __syncthreads();
    linear_epilogue<EPI, NB, NTH>(a, zt, m0, n0, s);
}

// One workgroup of kNormThreads per row.  With nparts > 0 the row first becomes
// x + part[0] + ... + part[nparts-1] (fp32, in that order), rounded once to bf16 and
// written back; the norm is taken of the stored row.
//
// A row of at most NP * kNormThreads 16-byte pieces (d = 4096: 512 pieces, one per thread)
// is held in registers: every load of the row (x, the first kPartsHeld partial slices and
// g) is issued before the first is used, so the call costs about one memory latency, and
// the stored row is not read back.  NP = 0 walks longer rows piece by piece.
constexpr int kNormThreads = 512;
constexpr int kPartsHeld = 8;

template <int NP>
__global__ __launch_bounds__(kNormThreads) void rmsnorm_kernel(uint4* __restrict__ x, const float4* __restrict__ part,
                                                               int nparts, long part_stride,
                                                               const uint4* __restrict__ g, int nvec, float inv_d,
                                                               float eps, uint4* __restrict__ y) {
    __shared__ float red[kNormThreads / 64];
    uint4* xr = x + (size_t)blockIdx.x * nvec;
    uint4* yr = y + (size_t)blockIdx.x * nvec;
    const float4* prow = part + (size_t)blockIdx.x * nvec * 2;
    // x (+ the partial slices) of one piece, rounded to bf16
    auto add_parts = [&](uint4 q, float4 sa, float4 sb) {
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
        float v[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[2 * j] = lo16(w[j]), v[2 * j + 1] = hi16(w[j]);
        q.x = pack2(v[0] + sa.x, v[1] + sa.y);
        q.y = pack2(v[2] + sa.z, v[3] + sa.w);
        q.z = pack2(v[4] + sb.x, v[5] + sb.y);
        q.w = pack2(v[6] + sb.z, v[7] + sb.w);
        return q;
    };
    auto add4 = [](float4& s, const float4& t) { s.x += t.x, s.y += t.y, s.z += t.z, s.w += t.w; };
    auto sumsq = [](const uint4& q) {
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float a = lo16(w[j]), b = hi16(w[j]);
            ss += a * a + b * b;
        }
        return ss;
    };
    auto normed = [](const uint4& q, const uint4& gg, float r) {
        const uint32_t w[4] = {q.x, q.y, q.z, q.w}, gw[4] = {gg.x, gg.y, gg.z, gg.w};
        uint32_t o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = pack2(lo16(w[j]) * r * lo16(gw[j]), hi16(w[j]) * r * hi16(gw[j]));
        return make_uint4(o[0], o[1], o[2], o[3]);
    };
    auto finish = [&](float ss) {
        ss = wave_sum(ss);
        if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
        __syncthreads();
        float tot = 0.f;
#pragma unroll
        for (int w = 0; w < kNormThreads / 64; ++w) tot += red[w];
        return rsqrtf(tot * inv_d + eps);
    };

    if constexpr (NP > 0) {
        uint4 q[NP], gg[NP];
        float4 pa[kPartsHeld][NP], pb[kPartsHeld][NP];
#pragma unroll
        for (int j = 0; j < NP; ++j) {
            const int i = min((int)threadIdx.x + j * kNormThreads, nvec - 1);
            q[j] = xr[i];
            gg[j] = g[i];
        }
#pragma unroll
        for (int p = 0; p < kPartsHeld; ++p)
            if (p < nparts)
#pragma unroll
                for (int j = 0; j < NP; ++j) {
                    const float4* pr = prow + (size_t)min((int)threadIdx.x + j * kNormThreads, nvec - 1) * 2;
                    pa[p][j] = pr[p * part_stride];
                    pb[p][j] = pr[p * part_stride + 1];
                }
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < NP; ++j) {
            const int i = threadIdx.x + j * kNormThreads;
            if (i >= nvec) continue;
            if (nparts > 0) {
                float4 sa = pa[0][j], sb = pb[0][j];
#pragma unroll
                for (int p = 1; p < kPartsHeld; ++p)
                    if (p < nparts) add4(sa, pa[p][j]), add4(sb, pb[p][j]);
                for (int p = kPartsHeld; p < nparts; ++p)
                    add4(sa, prow[(size_t)i * 2 + p * part_stride]), add4(sb, prow[(size_t)i * 2 + p * part_stride + 1]);
                q[j] = add_parts(q[j], sa, sb);
                xr[i] = q[j];
            }
            ss += sumsq(q[j]);
        }
        const float r = finish(ss);
#pragma unroll
        for (int j = 0; j < NP; ++j) {
            const int i = threadIdx.x + j * kNormThreads;
            if (i < nvec) yr[i] = normed(q[j], gg[j], r);
        }
    } else {
        float ss = 0.f;
        for (int i = threadIdx.x; i < nvec; i += kNormThreads) {
            uint4 q = xr[i];
            if (nparts > 0) {
                const float4* pr = prow + (size_t)i * 2;
                float4 sa = pr[0], sb = pr[1];
                for (int p = 1; p < nparts; ++p) add4(sa, pr[p * part_stride]), add4(sb, pr[p * part_stride + 1]);
                q = add_parts(q, sa, sb);
                xr[i] = q;
            }
            ss += sumsq(q);
        }
        const float r = finish(ss);
        for (int i = threadIdx.x; i < nvec; i += kNormThreads) yr[i] = normed(xr[i], g[i], r);
    }
}

// One workgroup per row; a token outside [0, V) gives a zero row.
__global__ __launch_bounds__(256) void embed_kernel(const int32_t* __restrict__ tokens, const uint4* __restrict__ E,
                                                    int V, int nvec, uint4* __restrict__ y) {
    const int t = tokens[blockIdx.x];
    const bool ok = t >= 0 && t < V;
    const uint4* src = E + (size_t)(ok ? t : 0) * nvec;
    uint4* dst = y + (size_t)blockIdx.x * nvec;
    for (int i = threadIdx.x; i < nvec; i += 256) dst[i] = ok ? src[i] : make_uint4(0, 0, 0, 0);
}

// Launches the product with the narrowest tile (3, 4, 6 or 8 groups of 16 weight rows, on
// twice as many waves) whose grid fits one workgroup per CU, so that one round covers the
// CUs; a wider grid takes the 4-wave 64 x 64 tile.
template <int EPI>
mdt_status launch_linear(const LinArgs& a, int nsplit, hipStream_t hs) {
    const long rows = (long)((a.M + kMBL - 1) / kMBL) * nsplit;
    const long cus = mdt_num_cus();
    auto fits = [&](int nb) { return (a.N + nb - 1) / nb * rows <= cus; };
    auto go = [&](auto kern, int nb, int threads) {
        MDT_LAUNCH("linear_mfma", kern, dim3((a.N + nb - 1) / nb, (a.M + kMBL - 1) / kMBL, nsplit), dim3(threads), 0,
                   hs, a);
        return mdt_launched("linear_mfma");
    };
    // check_linear and kslice_for keep K and every slice a multiple of 32
    if constexpr (EPI != kSwiglu)  // a SwiGLU tile holds whole 32-row gate/up pairs
        if (fits(48)) return go(linear_dma<EPI, 48, 1, 4, 4>, 48, 256);
    if (fits(64)) return go(linear_dma<EPI, 64, 4, 2, 4>, 64, 512);
    if (fits(96)) return go(linear_dma<EPI, 96, 2, 4, 3>, 96, 512);
    return go(linear_dma<EPI, 128, 4, 2, 3>, 128, 512);
}

int kslice_for(int K, int nsplit) {
    int ks = (K + nsplit - 1) / nsplit;
    return (ks + 31) / 32 * 32;
}

mdt_status check_linear(int M, int N, int K, const void* x, const void* W, const void* y) {
    MDT_REQUIRE(M >= 1 && N >= 1 && K >= 1, MDT_ERR_SHAPE, "bad shape M=%d N=%d K=%d", M, N, K);
    MDT_REQUIRE((M + kMBL - 1) / kMBL <= 65535, MDT_ERR_SHAPE, "M=%d too large", M);
    MDT_REQUIRE(K % 32 == 0 && N % 8 == 0, MDT_ERR_SHAPE, "K=%d must be a multiple of 32 and N=%d of 8", K, N);
    MDT_REQUIRE(x && W && y, MDT_ERR_NULL, "a tensor pointer is NULL");
    MDT_REQUIRE(mdt_aligned16(x) && mdt_aligned16(W) && mdt_aligned16(y), MDT_ERR_ALIGN,
                "tensor pointers must be 16-byte aligned");
    return MDT_OK;
}

mdt_status launch_rmsnorm(void* stream, int M, int d, void* x, const float* part, int nparts, const void* g,
                          float eps, void* y) {
    MDT_REQUIRE(M >= 1 && d >= 8 && d % 8 == 0, MDT_ERR_SHAPE, "bad shape M=%d d=%d (d a multiple of 8)", M, d);
    MDT_REQUIRE(eps >= 0.f, MDT_ERR_VALUE, "eps must be >= 0");
    MDT_REQUIRE(nparts >= 0 && nparts <= 64, MDT_ERR_VALUE, "nparts=%d out of range 0..64", nparts);
    MDT_REQUIRE(x && g && y && (nparts == 0 || part), MDT_ERR_NULL, "a tensor pointer is NULL");
    MDT_REQUIRE(mdt_aligned16(x) && mdt_aligned16(g) && mdt_aligned16(y) && mdt_aligned16(part), MDT_ERR_ALIGN,
                "tensor pointers must be 16-byte aligned");
    const int nvec = d / 8, np = (nvec + kNormThreads - 1) / kNormThreads;
    auto go = [&](auto kern) {
        MDT_LAUNCH("rmsnorm_kernel", kern, dim3(M), dim3(kNormThreads), 0, (hipStream_t)stream, (uint4*)x,
                   (const float4*)part, nparts, (long)M * d / 4, (const uint4*)g, nvec, 1.f / (float)d, eps, (uint4*)y);
        return mdt_launched("rmsnorm_kernel");
    };
    if (np == 1) return go(rmsnorm_kernel<1>);
    if (np == 2) return go(rmsnorm_kernel<2>);
    if (np <= 4) return go(rmsnorm_kernel<4>);
    return go(rmsnorm_kernel<0>);
}

}  // namespace

extern "C" mdt_status mdt_linear(void* stream, int M, int N, int K, const void* x, const void* W,
                                 const void* residual, int nseg, int act, void* y) {
    mdt_status st = check_linear(M, N, K, x, W, y);
    if (st != MDT_OK) return st;
    MDT_REQUIRE(act == MDT_ACT_NONE || act == MDT_ACT_SWIGLU, MDT_ERR_VALUE, "unknown activation %d", act);
    MDT_REQUIRE(mdt_aligned16(residual), MDT_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
    if (act == MDT_ACT_SWIGLU) {
        MDT_REQUIRE(N % 32 == 0, MDT_ERR_SHAPE, "SwiGLU needs N=%d to be a multiple of 32", N);
        MDT_REQUIRE(!residual && nseg == 1, MDT_ERR_VALUE, "SwiGLU takes no residual and one segment");
    } else {
        MDT_REQUIRE(nseg >= 1 && N % nseg == 0 && (N / nseg) % 8 == 0, MDT_ERR_SHAPE,
                    "nseg=%d must split N=%d into multiples of 8", nseg, N);
        MDT_REQUIRE(!residual || nseg == 1, MDT_ERR_VALUE, "a residual needs nseg == 1");
    }
    LinArgs a{(const bf16_t*)x, (const bf16_t*)W, (const bf16_t*)residual, (bf16_t*)y, nullptr, M, N, K, K, nseg};
    const hipStream_t hs = (hipStream_t)stream;
    if (act == MDT_ACT_SWIGLU) return launch_linear<kSwiglu>(a, 1, hs);
    if (residual) return launch_linear<kResidual>(a, 1, hs);
    return launch_linear<kStore>(a, 1, hs);
}

extern "C" mdt_status mdt_linear_split(void* stream, int M, int N, int K, const void* x, const void* W, int nsplit,
                                       float* part) {
    mdt_status st = check_linear(M, N, K, x, W, part);
    if (st != MDT_OK) return st;
    MDT_REQUIRE(nsplit >= 1 && nsplit <= 64 && nsplit * 32 <= K, MDT_ERR_VALUE,
                "nsplit=%d out of range 1..min(64, K/32)", nsplit);
    const int ks = kslice_for(K, nsplit);
    MDT_REQUIRE((K + ks - 1) / ks == nsplit, MDT_ERR_VALUE, "K=%d cannot be cut into %d slices of 32-multiples", K,
                nsplit);
    LinArgs a{(const bf16_t*)x, (const bf16_t*)W, nullptr, nullptr, part, M, N, K, ks, 1};
    return launch_linear<kPartial>(a, nsplit, (hipStream_t)stream);
}

extern "C" mdt_status mdt_rmsnorm(void* stream, int M, int d, const void* x, const void* g, float eps, void* y) {
    return launch_rmsnorm(stream, M, d, (void*)x, nullptr, 0, g, eps, y);
}

extern "C" mdt_status mdt_add_rmsnorm(void* stream, int M, int d, int nparts, const float* part, void* x,
                                      const void* g, float eps, void* y) {
    MDT_REQUIRE(nparts >= 1, MDT_ERR_VALUE, "nparts=%d must be >= 1", nparts);
    MDT_REQUIRE(!part || (part + (size_t)nparts * M * d <= (const float*)x || (const float*)x + (size_t)M * d / 2 <= part),
                MDT_ERR_VALUE, "part must not overlap x");
    return launch_rmsnorm(stream, M, d, x, part, nparts, g, eps, y);
}

extern "C" mdt_status mdt_embed(void* stream, int M, int d, int V, const int32_t* tokens, const void* E, void* y) {
    MDT_REQUIRE(M >= 1 && V >= 1 && d >= 8 && d % 8 == 0, MDT_ERR_SHAPE,
                "bad shape M=%d d=%d V=%d (d a multiple of 8)", M, d, V);
    MDT_REQUIRE(tokens && E && y, MDT_ERR_NULL, "a tensor pointer is NULL");
    MDT_REQUIRE(mdt_aligned16(E) && mdt_aligned16(y), MDT_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
    MDT_LAUNCH("embed_kernel", embed_kernel, dim3(M), dim3(256), 0, (hipStream_t)stream, tokens, (const uint4*)E, V,
               d / 8, (uint4*)y);
    return mdt_launched("embed_kernel");
}
