// The heads of a batch of sequences on the matrix cores (bf16, B >= 4).
//
// Same arithmetic as the GEMV path of mdt_medusa_heads (summary page, "MEDUSA Heads":
// logits_k = W2_k (SiLU(W1_k h) + h), the LM head logits_0 = W_lm h), but every weight
// byte now serves B sequences: a GEMV that keeps up to 8 activation vectors in LDS
// re-streams the weights once per 8 sequences and spends B multiply-adds per weight
// element on the vector ALUs, while an MFMA tile reads each weight row once for all B
// rows of h.  Hidden sizes that are a multiple of 128 take the DMA-staged tile
// (dma_tile.h: 96 or 128 weight rows per workgroup, both operands loaded straight into
// LDS); other multiples of 64 the register-staged 64 x 64 tile (mfma_tile.h).
//
// Launch 1 streams the rows of W1_0..W1_{K-1} (stacked, K*d rows) and of W_lm: the W1
// epilogue forms a = SiLU(u) + h in fp32 and stores it as two bf16 rows, a_hi = bf16(a)
// and a_lo = bf16(a - a_hi), so that launch 2 can multiply a with bf16 operands and
// still keep about 16 significant bits of a (a_hi + a_lo); the W_lm epilogue writes
// logits_0.  Launch 2 streams W2_k against the 2B rows [a_hi; a_lo] of head k and adds
// the two halves of each product in its epilogue.
#include <math.h>

#include "dma_tile.h"
#include "heads_mfma.h"

namespace {

constexpr int kKC = 256;
constexpr int kNB = 64;
constexpr int kThreads = 4 * kNB;

struct HeadsArgs {
    const bf16_t* h;    // [B][d]
    const bf16_t* W1;   // [K][d][d]
    const bf16_t* W2;   // [K][V][d]
    const bf16_t* Wlm;  // [V][d]
    float* logits;      // [B][K+1][V]
    bf16_t* ahl;        // [K][2B][d]: rows 0..B-1 a_hi, rows B..2B-1 a_lo
    int B, d, V, K, w1_tiles;
};

// grid (K*d/64 + ceil(V/64)): W1 tiles first, then W_lm tiles.
template <int MT>
__global__ __launch_bounds__(kThreads) void heads_mfma_w1_lm(HeadsArgs a) {
    __shared__ __attribute__((aligned(16))) char smem[MfmaTile<kKC, kNB, MT>::kBytes];
    static_assert(MfmaTile<kKC, kNB, MT>::kBytes >= 16 * MT * (kNB + 1) * 4, "the result tile must fit");
    const bool w1 = (int)blockIdx.x < a.w1_tiles;
    const int n0 = (w1 ? blockIdx.x : blockIdx.x - a.w1_tiles) * kNB;
    const int nrows = w1 ? a.K * a.d : a.V;
    const bf16_t* W = w1 ? a.W1 : a.Wlm;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, c16 = lane & 15;
    float* zt = (float*)smem;  // [16*MT][kNB + 1]
    mfma_tile<kKC, kNB, MT>(a.h, W, a.B, a.d, a.d, nrows, 0, n0, smem, [&](const f32x4 (&acc)[MT]) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int e = 0; e < 4; ++e) zt[(mt * 16 + 4 * g + e) * (kNB + 1) + wave * 16 + c16] = acc[mt][e];
    });
    __syncthreads();
    for (int it = threadIdx.x; it < a.B * kNB; it += kThreads) {
        const int b = it / kNB, c = it % kNB;
        const float u = zt[b * (kNB + 1) + c];
        if (w1) {
            const int k = n0 / a.d, j = n0 % a.d + c;  // a 64-row tile lies in one head (d % 64 == 0)
            const float v = u / (1.f + __expf(-u)) + bf16_to_f32(a.h[(size_t)b * a.d + j]);
            const bf16_t hi = f32_to_bf16(v);
            const bf16_t lo = f32_to_bf16(v - bf16_to_f32(hi));
            bf16_t* row = a.ahl + ((size_t)k * 2 * a.B + b) * a.d + j;
            row[0] = hi;
            row[(size_t)a.B * a.d] = lo;
        } else if (n0 + c < a.V) {
            a.logits[(size_t)b * (a.K + 1) * a.V + n0 + c] = u;
        }
    }
}

// grid (ceil(V/64), K).
template <int MT>
__global__ __launch_bounds__(kThreads) void heads_mfma_w2(HeadsArgs a) {
    __shared__ __attribute__((aligned(16))) char smem[MfmaTile<kKC, kNB, MT>::kBytes];
    static_assert(MfmaTile<kKC, kNB, MT>::kBytes >= 16 * MT * (kNB + 1) * 4, "the result tile must fit");
    const int n0 = blockIdx.x * kNB, k = blockIdx.y;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, c16 = lane & 15;
    float* zt = (float*)smem;
    const bf16_t* x = a.ahl + (size_t)k * 2 * a.B * a.d;
    const bf16_t* W = a.W2 + (size_t)k * a.V * a.d;
    mfma_tile<kKC, kNB, MT>(x, W, 2 * a.B, a.d, a.d, a.V, 0, n0, smem, [&](const f32x4 (&acc)[MT]) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int e = 0; e < 4; ++e) zt[(mt * 16 + 4 * g + e) * (kNB + 1) + wave * 16 + c16] = acc[mt][e];
    });
    __syncthreads();
    for (int it = threadIdx.x; it < a.B * kNB; it += kThreads) {
        const int b = it / kNB, c = it % kNB;
        if (n0 + c < a.V)
            a.logits[((size_t)b * (a.K + 1) + k + 1) * a.V + n0 + c] =
                zt[b * (kNB + 1) + c] + zt[(a.B + b) * (kNB + 1) + c];
    }
}

// The same two launches on the DMA-staged tile (dma_tile.h): NB weight rows against the
// 16 MT x rows per workgroup, both fed by direct global-to-LDS loads through a 4-stage ring
// (3 stages where 4 do not fit the LDS) of 128-dim chunks on four waves, weights streamed
// non-temporally.  Block b walks the chunks from chunk b on, so that neighbouring
// workgroups read different parts of their weight rows at any one time.  Launch 2 (W2) uses
// 128-row tiles; launch 1 (W1 + W_lm) 96- or 128-row tiles, whichever grid fills the last
// round of workgroups (one per CU) better, since the CUs left idle in a short last round
// stream nothing (a W1 tile may then span two heads; the epilogue places each column).
// Whole heads calls against the register-staged tiles (both launches, weights from HBM):
// 397 -> 384 us at B = 4, d = 6656 (2.48 GB, 6.5 TB/s); 258 -> 251 us at B = 16, d = 4096.
// 64-row tiles (two workgroups per CU) were slower: 326 against 319 us for W2 at 33B.
template <int NB, int MT, int CG, int KS>
constexpr int kHS = (NB + 16 * MT) * 256 * 4 + (KS - 1) * NB * MT * 64 <= 160 * 1024 ? 4 : 3;
template <int NB, int MT, int CG, int KS>
using HDma = DmaTile<128, NB, CG, KS, kHS<NB, MT, CG, KS>, MT>;
template <int NB, int MT, int CG, int KS>
constexpr int kHLds = HDma<NB, MT, CG, KS>::kRingBytes > 16 * MT * (NB + 1) * 4 + HDma<NB, MT, CG, KS>::kRedBytes
                          ? HDma<NB, MT, CG, KS>::kRingBytes
                          : 16 * MT * (NB + 1) * 4 + HDma<NB, MT, CG, KS>::kRedBytes;

// The product tile of x (at most 16 MT valid rows: M) against weight rows n0.. of W (V rows),
// left as [16 MT][NB + 1] fp32 at the returned address in smem.
template <int NB, int MT, int CG, int KS>
__device__ __forceinline__ const float* head_tile(const bf16_t* x, int M, const bf16_t* W, int V, int d, int n0,
                                                  int rot, char* smem) {
    using P = HDma<NB, MT, CG, KS>;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, c16 = lane & 15, cg = wave % CG;
    float* zt = (float*)(smem + P::kRedBytes);  // after the k-groups' partials
    dma_tile<128, NB, CG, KS, kHS<NB, MT, CG, KS>, 2, MT>(
        x, W, M, d, d, V, n0, smem,
        [&](const f32x4 (&acc)[NB / CG / 16][MT]) {
#pragma unroll
            for (int nt = 0; nt < NB / CG / 16; ++nt)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        zt[(mt * 16 + 4 * g + e) * (NB + 1) + cg * (NB / CG) + 16 * nt + c16] = acc[nt][mt][e];
        },
        rot);
    __syncthreads();
    return zt;
}

// grid (ceil(K*d/NB) + ceil(V/NB)): W1 tiles first, then W_lm tiles.
template <int NB, int MT, int CG, int KS>
__global__ __launch_bounds__(256) void heads_dma_w1_lm(HeadsArgs a) {
    __shared__ __attribute__((aligned(1024))) char smem[kHLds<NB, MT, CG, KS>];
    const bool w1 = (int)blockIdx.x < a.w1_tiles;
    const int n0 = (w1 ? blockIdx.x : blockIdx.x - a.w1_tiles) * NB;
    const int nrows = w1 ? a.K * a.d : a.V;
    const float* zt = head_tile<NB, MT, CG, KS>(a.h, a.B, w1 ? a.W1 : a.Wlm, nrows, a.d, n0, blockIdx.x, smem);
    for (int it = threadIdx.x; it < a.B * NB; it += 256) {
        const int b = it / NB, c = it % NB, n = n0 + c;
        if (n >= nrows) continue;
        const float u = zt[b * (NB + 1) + c];
        if (w1) {
            const int k = n / a.d, j = n - k * a.d;
            const float v = u / (1.f + __expf(-u)) + bf16_to_f32(a.h[(size_t)b * a.d + j]);
            const bf16_t hi = f32_to_bf16(v);
            const bf16_t lo = f32_to_bf16(v - bf16_to_f32(hi));
            bf16_t* row = a.ahl + ((size_t)k * 2 * a.B + b) * a.d + j;
            row[0] = hi;
            row[(size_t)a.B * a.d] = lo;
        } else {
            a.logits[(size_t)b * (a.K + 1) * a.V + n] = u;
        }
    }
}

// grid (ceil(V/128), K).
template <int MT>
__global__ __launch_bounds__(256) void heads_dma_w2(HeadsArgs a) {
    __shared__ __attribute__((aligned(1024))) char smem[kHLds<128, MT, 4, 1>];
    const int n0 = blockIdx.x * 128, k = blockIdx.y;
    const float* zt = head_tile<128, MT, 4, 1>(a.ahl + (size_t)k * 2 * a.B * a.d, 2 * a.B,
                                               a.W2 + (size_t)k * a.V * a.d, a.V, a.d, n0,
                                               blockIdx.x + 5 * blockIdx.y, smem);
    for (int it = threadIdx.x; it < a.B * 128; it += 256) {
        const int b = it / 128, c = it % 128;
        if (n0 + c < a.V)
            a.logits[((size_t)b * (a.K + 1) + k + 1) * a.V + n0 + c] = zt[b * 129 + c] + zt[(a.B + b) * 129 + c];
    }
}

// Fraction of the CUs busy over the rounds of `tiles` workgroups, one per CU.
double round_fill(long tiles, long cus) { return (double)tiles / (double)(((tiles + cus - 1) / cus) * cus); }

template <int MT1, int MT2>
mdt_status launch_dma(HeadsArgs a, hipStream_t s) {
    const long cus = mdt_num_cus();
    auto tiles = [&](int nb) { return (a.K * a.d + nb - 1) / nb + (a.Wlm ? (a.V + nb - 1) / nb : 0); };
    auto go1 = [&](auto kern, int nb) {
        a.w1_tiles = (a.K * a.d + nb - 1) / nb;
        MDT_LAUNCH("heads_mfma_w1_lm", kern, dim3(tiles(nb)), dim3(256), 0, s, a);
        return mdt_launched("heads_mfma_w1_lm");
    };
    // 128-row tiles unless 96-row ones fill the last round clearly better (7B, K = 4: 505
    // workgroups against 378 on 256 CUs)
    const mdt_status st = round_fill(tiles(128), cus) >= round_fill(tiles(96), cus) - 0.02
                              ? go1(heads_dma_w1_lm<128, MT1, 4, 1>, 128)
                              : go1(heads_dma_w1_lm<96, MT1, 2, 2>, 96);
    if (st != MDT_OK) return st;
    MDT_LAUNCH("heads_mfma_w2", heads_dma_w2<MT2>, dim3((a.V + 127) / 128, a.K), dim3(256), 0, s, a);
    return mdt_launched("heads_mfma_w2");
}

template <int MT1, int MT2>
mdt_status launch_pair(const HeadsArgs& a, hipStream_t s) {
    const int lm_tiles = (a.V + kNB - 1) / kNB;
    // no W_lm: launch 1 streams W1 only and the LM-head slot is left as it is
    MDT_LAUNCH("heads_mfma_w1_lm", heads_mfma_w1_lm<MT1>, dim3(a.w1_tiles + (a.Wlm ? lm_tiles : 0)), dim3(kThreads),
               0, s, a);
    mdt_status st = mdt_launched("heads_mfma_w1_lm");
    if (st != MDT_OK) return st;
    MDT_LAUNCH("heads_mfma_w2", heads_mfma_w2<MT2>, dim3(lm_tiles, a.K), dim3(kThreads), 0, s, a);
    return mdt_launched("heads_mfma_w2");
}

}  // namespace

bool mdt_heads_mfma_applies(int B, int d) { return B >= kHeadsMfmaMinB && B <= 32 && d % 64 == 0; }

mdt_status mdt_heads_mfma(hipStream_t s, int B, int d, int V, int K, const void* h, const void* W1, const void* W2,
                          const void* Wlm, float* logits, void* ws) {
    HeadsArgs a{(const bf16_t*)h, (const bf16_t*)W1, (const bf16_t*)W2, (const bf16_t*)Wlm, logits, (bf16_t*)ws,
                B, d, V, K, K * d / kNB};
    if (d % 128 == 0) {
        if (B <= 8) return launch_dma<1, 1>(a, s);
        if (B <= 16) return launch_dma<1, 2>(a, s);
        return launch_dma<2, 4>(a, s);
    }
    // 16-row m-tiles: B rows of h in launch 1, 2B rows of [a_hi; a_lo] in launch 2
    if (B <= 8) return launch_pair<1, 1>(a, s);
    if (B <= 16) return launch_pair<1, 2>(a, s);
    return launch_pair<2, 4>(a, s);
}
