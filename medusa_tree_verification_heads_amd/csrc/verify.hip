// mdt_verify_logits: LM head on every tree node, with per-row statistics and edge logits.
//
// Summary page "Medusa: Simple LLM Inference Acceleration Framework with Multiple
// Decoding Heads", section "Tree Attention", steps 5-6 (one pass gives logits
// for every candidate, conditioned on its branch) and section "Typical
// Acceptance Scheme" (the verifier's probability of the candidate and the
// entropy in nats of its distribution); "Notes on Medusa", section 3 (the node
// outputs go through the LM head).
//
// The rows of x (B*T nodes) share every weight row, so this is a real dense
// contraction: bf16 MFMA 16x16x32 with fp32 accumulation.  A workgroup owns 64
// vocabulary columns and 64 node rows.  Weight rows are read from HBM in long
// row-contiguous runs and transposed into MFMA fragments through LDS, together
// with the 64 x rows (shared by the four waves, each owning 16 columns).  The epilogue
// keeps the logits tile in LDS and reduces it to per-row partial statistics over
// the 64 columns -- max, argmax, s = sum exp((z-m)/tau), u = sum exp((z-m)/tau) (z-m)/tau --
// and picks the edge logits whose token falls in the tile.  A second kernel
// merges the partials of a row in column-block order:
//   logZ = M/tau + ln S,  H = ln S - U/S.
#include <climits>
#include <math.h>

#include "dma_tile.h"
#include "mfma_tile.h"
#include "verify_core.h"

namespace {

constexpr int kNB = 64;          // vocabulary columns per workgroup
constexpr int kMB = 64;          // node rows per workgroup (bf16 path)
constexpr int kBigRows = 256;    // from this many node rows on: the compute-bound tiles
constexpr int kZStride = kNB + 1;
#ifndef MDT_VERIFY_KC
#define MDT_VERIFY_KC 256        // dims per staged chunk (LDS holds one 64-row tile of x and of W)
#endif
#ifndef MDT_VERIFY_NB
#define MDT_VERIFY_NB 64         // vocabulary columns per MFMA workgroup (4 waves of 16 per 64)
#endif

// Reduce a logits tile zt[MT][NB + 1] (rows m0.., cols n0..) to per-row partials,
// write optional full logits and the edge logits that fall inside the tile.
// Edge inputs of this thread's first node of the tile's sequences, requested before the
// weight stream so that the epilogue does not wait for them.
struct EdgePre {
    int par, tok;
};

template <int MT>
__device__ EdgePre edge_preload(int m0, int M, const int32_t* __restrict__ parent, const int32_t* __restrict__ tokens,
                                int T) {
    const int idx = min(m0 / T * T + (int)threadIdx.x, M - 1);
    return EdgePre{parent[idx % T], tokens[idx]};
}

template <int MT, int NB, int NT>
__device__ void tile_epilogue(const float* zt, int m0, int n0, int M, int V, float tau, int nblk_n,
                              Part* __restrict__ part, float* __restrict__ logits_opt,
                              const int32_t* __restrict__ parent, const int32_t* __restrict__ tokens, int T,
                              float* __restrict__ edge, EdgePre pre) {
    constexpr int kZS = NB + 1;         // row stride of zt
    // threads per row: the largest power of two with TPR * MT <= NT (with 224 rows on 512
    // threads the last 64 threads only take part in the edge pass)
    constexpr int TPR = NT / MT >= 16 ? 16 : NT / MT >= 8 ? 8 : NT / MT >= 4 ? 4 : NT / MT >= 2 ? 2 : 1;
    constexpr int CPT = NB / TPR;       // columns per thread
    static_assert(NB % TPR == 0, "columns divide among a row's threads");
    const int t = threadIdx.x;
    const int r = t / TPR, q = t % TPR;
    const bool has_row = r < MT;
    const int row = m0 + r;
    const int ncol = has_row ? min(NB, V - n0) : 0;
    Part p{-INFINITY, INT_MAX, 0.f, 0.f};
    const float* z = zt + min(r, MT - 1) * kZS;
    for (int c = q * CPT; c < q * CPT + CPT; ++c) {
        if (c >= ncol) break;
        if (better(z[c], n0 + c, p.m, p.a)) {
            p.m = z[c];
            p.a = n0 + c;
        }
    }
    if (tau > 0.f && p.m != -INFINITY) {
        for (int c = q * CPT; c < q * CPT + CPT; ++c) {
            if (c >= ncol) break;
            const float dz = (z[c] - p.m) / tau;
            const float e = __expf(dz);
            p.s += e;
            p.u += e * dz;
        }
    }
#pragma unroll
    for (int off = 1; off < TPR; off <<= 1) p = part_merge(p, shfl_xor_part(p, off), tau > 0.f ? 1.f / tau : 0.f);
    if (has_row && q == 0 && row < M) part[(long)row * nblk_n + n0 / NB] = p;
    if (logits_opt && has_row && row < M)
        for (int c = q * CPT; c < q * CPT + CPT && c < ncol; ++c) logits_opt[(long)row * V + n0 + c] = z[c];
    // edges: node c of sequence b reads row b*T + parent(c) at column token(b, c)
    const int first_b = m0 / T, last_b = min(M - 1, m0 + MT - 1) / T;
    for (int idx = first_b * T + t; idx <= last_b * T + T - 1; idx += NT) {
        const int b = idx / T, c = idx % T;
        if (c == 0 || idx >= M) continue;
        const bool first = idx == first_b * T + t;  // preloaded
        const int pr = first ? pre.par : parent[c];
        if (pr < 0 || pr >= T) continue;
        const int rr = b * T + pr;
        const int tok = first ? pre.tok : tokens[idx];
        if (rr >= m0 && rr < m0 + MT && rr < M && tok >= n0 && tok < n0 + ncol) edge[idx] = zt[(rr - m0) * kZS + tok - n0];
    }
}

// grid (ceil(V/NB), ceil(M/(16*MT))), block 4*NB: the tile of mfma_tile (16*MT node rows),
// then the statistics epilogue.  MT = 4 (64 rows) is used for every M: with 256 rows per
// workgroup (MT = 16, 128-dim chunks) the batched shapes ran slower (one wave per SIMD
// at 284 registers), the repeated weight streams being served largely from the
// last-level cache.
template <int KC, int NB, int MT = 4, bool MMAJOR = false>
__global__ __launch_bounds__(4 * NB) void verify_mfma(const bf16_t* __restrict__ x, const bf16_t* __restrict__ W,
                                                      int M, int d, int V, float tau, int nblk_n,
                                                      Part* __restrict__ part, float* __restrict__ logits_opt,
                                                      const int32_t* __restrict__ parent,
                                                      const int32_t* __restrict__ tokens, int T,
                                                      float* __restrict__ edge) {
    constexpr int NT = 4 * NB;
    constexpr int MB = 16 * MT;
    static_assert(MfmaTile<KC, NB, MT>::kBytes >= MB * (NB + 1) * 4, "the logits tile must fit");
    __shared__ __attribute__((aligned(16))) char smem[MfmaTile<KC, NB, MT>::kBytes];
    // MMAJOR: the workgroups that read one block of weight rows run on one XCD, one after
    // another, and share it through its L2
    int mb = blockIdx.y, nb = blockIdx.x;
    if (MMAJOR) xcd_tile(blockIdx.x + blockIdx.y * gridDim.x, gridDim.x, gridDim.y, mb, nb);
    const int n0 = nb * NB, m0 = mb * MB;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, c16 = lane & 15;
    const EdgePre pre = edge_preload<MB>(m0, M, parent, tokens, T);
    float* zt = (float*)smem;  // [MB][NB + 1], reuses the tiles
    mfma_tile<KC, NB, MT>(x, W, M, d, d, V, m0, n0, smem, [&](const f32x4 (&acc)[MT]) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int e = 0; e < 4; ++e) zt[(mt * 16 + 4 * g + e) * (NB + 1) + wave * 16 + c16] = acc[mt][e];
    });
    __syncthreads();
    tile_epilogue<MB, NB, NT>(zt, m0, n0, M, V, tau, nblk_n, part, logits_opt, parent, tokens, T, edge, pre);
}

// At most 64 node rows (one tree of a single sequence, the batch-1 shapes): dma_tile, the
// 64 x NB tile fed by direct global-to-LDS loads through an S-stage ring, then the
// statistics epilogue over NB columns on all threads.  Column block b walks the chunks from
// chunk b on (spreading the weight reads over the memory channels).  grid ceil(V / NB),
// block 64 CG KS.
#ifndef MDT_VDMA_KC
#define MDT_VDMA_KC 128
#endif
#ifndef MDT_VDMA_CG
#define MDT_VDMA_CG 4
#endif
#ifndef MDT_VDMA_KS
#define MDT_VDMA_KS 2
#endif
#ifndef MDT_VDMA_S
#define MDT_VDMA_S 3
#endif
#ifndef MDT_VDMA_AUX
#define MDT_VDMA_AUX 2  // cache policy of the weight loads: streamed (read once)
#endif
constexpr int kDmaNB = 128;
using VDma = DmaTile<MDT_VDMA_KC, kDmaNB, MDT_VDMA_CG, MDT_VDMA_KS, MDT_VDMA_S>;

__global__ __launch_bounds__(VDma::NT) void verify_dma(const bf16_t* __restrict__ x, const bf16_t* __restrict__ W,
                                                       int M, int d, int V, float tau, int nblk_n,
                                                       Part* __restrict__ part, float* __restrict__ logits_opt,
                                                       const int32_t* __restrict__ parent,
                                                       const int32_t* __restrict__ tokens, int T,
                                                       float* __restrict__ edge) {
    constexpr int NB = kDmaNB, CG = MDT_VDMA_CG;
    constexpr int kZOff = VDma::kRedBytes;  // the logits tile after the k-groups' partials
    constexpr int kEpi = kZOff + kMB * (NB + 1) * 4;
    constexpr int kLds = VDma::kRingBytes > kEpi ? VDma::kRingBytes : kEpi;
    __shared__ __attribute__((aligned(1024))) char smem[kLds];
    const int n0 = blockIdx.x * NB;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, c16 = lane & 15, cg = wave % CG;
    const EdgePre pre = edge_preload<kMB>(0, M, parent, tokens, T);
    float* zt = (float*)(smem + kZOff);  // [64][NB + 1]
    dma_tile<MDT_VDMA_KC, NB, CG, MDT_VDMA_KS, MDT_VDMA_S, MDT_VDMA_AUX>(
        x, W, M, d, d, V, n0, smem, [&](const f32x4 (&acc)[NB / CG / 16][4]) {
#pragma unroll
            for (int nt = 0; nt < NB / CG / 16; ++nt)
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        zt[(mt * 16 + 4 * g + e) * (NB + 1) + cg * (NB / CG) + 16 * nt + c16] = acc[nt][mt][e];
        }, blockIdx.x);
    __syncthreads();
    tile_epilogue<kMB, NB, VDma::NT>(zt, 0, n0, M, V, tau, nblk_n, part, logits_opt, parent, tokens, T, edge, pre);
}

// Many node rows (batches, 256-node trees) with the DMA-staged tile: 256 x 128 tiles on 8
// waves (4 x 2, each 64 x 64: two waves per SIMD hide each other's LDS and barrier waits;
// four waves of 128 x 64 were 12 % slower, 128-row tiles slower still), 64-dim chunks in a
// 3-stage ring, the row blocks of one weight block together on one XCD, partials per 128
// columns.  grid (ceil(M/256), ceil(V/128)).
#ifndef MDT_VBIG_MB
#define MDT_VBIG_MB 256
#endif
#ifndef MDT_VBIG_S
#define MDT_VBIG_S 3
#endif
#ifndef MDT_VBIG_AUX
#define MDT_VBIG_AUX 0
#endif
#ifndef MDT_VBIG_WM
#define MDT_VBIG_WM 4
#endif
#ifndef MDT_VBIG_WN
#define MDT_VBIG_WN 2
#endif
#ifndef MDT_VBIG_KC
#define MDT_VBIG_KC 64
#endif
constexpr int kBigMB = MDT_VBIG_MB;
using VBig = DmaGemm<kBigMB, 128, MDT_VBIG_WM, MDT_VBIG_WN, MDT_VBIG_KC, MDT_VBIG_S>;

__global__ __launch_bounds__(VBig::NT) void verify_dma_big(const bf16_t* __restrict__ x, const bf16_t* __restrict__ W,
                                                           int M, int d, int V, float tau, int nblk_n,
                                                           Part* __restrict__ part, float* __restrict__ logits_opt,
                                                           const int32_t* __restrict__ parent,
                                                           const int32_t* __restrict__ tokens, int T,
                                                           float* __restrict__ edge) {
    constexpr int MB = kBigMB, NB = 128, kZ = NB + 1;
    constexpr int kEpi = MB * kZ * 4;
    constexpr int kLds = VBig::kRingBytes > kEpi ? VBig::kRingBytes : kEpi;
    __shared__ __attribute__((aligned(1024))) char smem[kLds];
    int mb, nb;  // the row blocks of one weight block together, on one XCD
    xcd_tile(blockIdx.x + blockIdx.y * gridDim.x, gridDim.x, gridDim.y, mb, nb);
    const int m0 = mb * MB, n0 = nb * NB;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, c16 = lane & 15;
    constexpr int WM = MDT_VBIG_WM, WN = MDT_VBIG_WN;
    const int wm = wave / WN, wn = wave % WN;
    const EdgePre pre = edge_preload<MB>(m0, M, parent, tokens, T);
    float* zt = (float*)smem;  // [MB][NB + 1], reuses the ring
    dma_gemm_tile<MB, NB, WM, WN, MDT_VBIG_KC, MDT_VBIG_S, MDT_VBIG_AUX>(
        x, W, M, d, V, m0, n0, smem, [&](const f32x4 (&acc)[VBig::NTW][VBig::MTW]) {
#pragma unroll
            for (int nt = 0; nt < VBig::NTW; ++nt)
#pragma unroll
                for (int mt = 0; mt < VBig::MTW; ++mt)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        zt[((MB / WM) * wm + 16 * mt + 4 * g + e) * kZ + (NB / WN) * wn + 16 * nt + c16] =
                            acc[nt][mt][e];
        });
    __syncthreads();
    tile_epilogue<MB, NB, VBig::NT>(zt, m0, n0, M, V, tau, nblk_n, part, logits_opt, parent, tokens, T, edge, pre);
}

// The most node rows: tiles of dma_gemm_wide on 8 waves, 64-dim chunks in a 2-stage ring:
// 256 x 256 (4 x 2 waves of 64 x 128) from kWideRows node rows on; from kWide192Rows on,
// NB = 192 weight rows (501 workgroups for three row blocks, two rounds of the CUs, where
// 256-column tiles would make 1.5) with 256 x rows (4 x 2 waves of 64 x 96) or, when that
// takes as many row blocks and pads fewer rows, 224 (2 x 4 waves of 112 x 48; 672 rows are
// three blocks exactly).  The epilogue runs once per PW columns (the result tile of all NB
// columns does not fit the LDS), partials per PW columns.  grid (ceil(M/MB), ceil(V/NB)).
#ifndef MDT_VWIDE_MIN_ROWS
#define MDT_VWIDE_MIN_ROWS 1024
#endif
#ifndef MDT_VWIDE192_MIN_ROWS
#define MDT_VWIDE192_MIN_ROWS 512
#endif
constexpr int kWideRows = MDT_VWIDE_MIN_ROWS;
constexpr int kWide192Rows = MDT_VWIDE192_MIN_ROWS;

template <int MB, int NB, int WM, int WN, int PW>
__global__ __launch_bounds__(512) void verify_dma_wide(const bf16_t* __restrict__ x, const bf16_t* __restrict__ W,
                                                       int M, int d, int V, float tau, int nblk_n,
                                                       Part* __restrict__ part, float* __restrict__ logits_opt,
                                                       const int32_t* __restrict__ parent,
                                                       const int32_t* __restrict__ tokens, int T,
                                                       float* __restrict__ edge) {
    using G = DmaGemmWide<MB, NB, WM, WN, 64, 2>;
    static_assert(G::NT == 512 && NB % PW == 0 && PW % 16 == 0, "tile shape");
    constexpr int kZ = PW + 1, RW = MB / WM, CW = NB / WN;  // rows / columns per wave
    constexpr int kEpi = MB * kZ * 4;
    constexpr int kLds = G::kRingBytes > kEpi ? G::kRingBytes : kEpi;
    __shared__ __attribute__((aligned(1024))) char smem[kLds];
    int mb, nb;  // the row blocks of one weight block together, on one XCD
    xcd_tile(blockIdx.x + blockIdx.y * gridDim.x, gridDim.x, gridDim.y, mb, nb);
    const int m0 = mb * MB, n0 = nb * NB;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, c16 = lane & 15;
    const int wm = wave / WN, wn = wave % WN;
    const EdgePre pre = edge_preload<MB>(m0, M, parent, tokens, T);
    float* zt = (float*)smem;  // [MB][PW + 1], reuses the ring
    dma_gemm_wide<MB, NB, WM, WN, 64, 2, MDT_VBIG_AUX>(
        x, W, M, d, V, m0, n0, smem, [&](const f32x4 (&acc)[G::NTW][G::MTW]) {
            for (int pass = 0; pass < NB / PW; ++pass) {
                if (n0 + PW * pass >= V) break;  // uniform: columns past the vocabulary have no partial
#pragma unroll
                for (int nt = 0; nt < G::NTW; ++nt) {
                    const int col = CW * wn + 16 * nt - PW * pass;  // this fragment's first column in the pass
                    if (col >= 0 && col < PW)
#pragma unroll
                        for (int mt = 0; mt < G::MTW; ++mt)
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                zt[(RW * wm + 16 * mt + 4 * g + e) * kZ + col + c16] = acc[nt][mt][e];
                }
                __syncthreads();
                tile_epilogue<MB, PW, G::NT>(zt, m0, n0 + PW * pass, M, V, tau, nblk_n, part, logits_opt, parent,
                                             tokens, T, edge, pre);
                __syncthreads();
            }
        });
}

// Many node rows (batches, 256-node trees): 128 x 128 tiles (mfma_tile128), grid
// (ceil(M/128), ceil(V/128)) row-block-major, partials per 128 vocabulary columns.
template <int KC>
__global__ __launch_bounds__(256) void verify_mfma128(const bf16_t* __restrict__ x, const bf16_t* __restrict__ W,
                                                      int M, int d, int V, float tau, int nblk_n,
                                                      Part* __restrict__ part, float* __restrict__ logits_opt,
                                                      const int32_t* __restrict__ parent,
                                                      const int32_t* __restrict__ tokens, int T,
                                                      float* __restrict__ edge) {
    constexpr int kZ = 128 + 1;
    constexpr int kLds = MfmaTile128<KC>::kBytes > 128 * kZ * 4 ? MfmaTile128<KC>::kBytes : 128 * kZ * 4;
    __shared__ __attribute__((aligned(16))) char smem[kLds];
    int mb, nb;  // the row blocks of one weight block together, on one XCD
    xcd_tile(blockIdx.x + blockIdx.y * gridDim.x, gridDim.x, gridDim.y, mb, nb);
    const int m0 = mb * 128, n0 = nb * 128;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, c16 = lane & 15;
    const int wm = wave >> 1, wn = wave & 1;
    const EdgePre pre = edge_preload<128>(m0, M, parent, tokens, T);
    float* zt = (float*)smem;  // [128][129], reuses the tiles
    mfma_tile128<KC>(x, W, M, d, d, V, m0, n0, smem, [&](const f32x4 (&acc)[4][4]) {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    zt[(64 * wm + 16 * mt + 4 * g + e) * kZ + 64 * wn + 16 * nt + c16] = acc[nt][mt][e];
    });
    __syncthreads();
    tile_epilogue<128, 128, 256>(zt, m0, n0, M, V, tau, nblk_n, part, logits_opt, parent, tokens, T, edge, pre);
}

// fp32 path: grid (ceil(V/64), ceil(M/16)), block 256; x rows staged in LDS as fp32.
__global__ __launch_bounds__(256) void verify_f32(const float* __restrict__ x, const float* __restrict__ W, int M,
                                                  int d, int V, float tau, int nblk_n, Part* __restrict__ part,
                                                  float* __restrict__ logits_opt, const int32_t* __restrict__ parent,
                                                  const int32_t* __restrict__ tokens, int T,
                                                  float* __restrict__ edge) {
    extern __shared__ float xsf[];  // [16][d], then reused as zt[16][kZStride]
    const int n0 = blockIdx.x * kNB, m0 = blockIdx.y * 16;
    for (int e = threadIdx.x; e < 16 * d; e += 256) {
        const int r = e / d, k = e % d;
        xsf[e] = (m0 + r < M) ? x[(size_t)(m0 + r) * d + k] : 0.f;
    }
    __syncthreads();
    const int cl = threadIdx.x % kNB, rg = threadIdx.x / kNB;  // 4 row groups of 4 rows
    const int col = n0 + cl;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    if (col < V) {
        const float* w = W + (size_t)col * d;
        for (int k = 0; k < d; ++k) {
            const float wv = w[k];
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[j] = fmaf(xsf[(rg * 4 + j) * d + k], wv, acc[j]);
        }
    }
    __syncthreads();
    float* zt = xsf;
#pragma unroll
    for (int j = 0; j < 4; ++j) zt[(rg * 4 + j) * kZStride + cl] = acc[j];
    __syncthreads();
    tile_epilogue<16, kNB, 256>(zt, m0, n0, M, V, tau, nblk_n, part, logits_opt, parent, tokens, T, edge,
                      edge_preload<16>(m0, M, parent, tokens, T));
}

// Merge row partials; grid ceil(M / 4), block 64: each 16-lane group of the wave merges one
// row (merge_row).  Also writes the edge entries that no tile owns (root, out-of-range
// tokens).
__global__ __launch_bounds__(64) void verify_merge(const Part* __restrict__ part, int M, int nblk_n, int V,
                                                   float tau, mdt_row_stats* __restrict__ stats,
                                                   const int32_t* __restrict__ tokens,
                                                   const int32_t* __restrict__ parent, int T,
                                                   float* __restrict__ edge) {
    const int row = blockIdx.x * (64 / kMergeLanes) + (int)threadIdx.x / kMergeLanes;
    const int sub = threadIdx.x % kMergeLanes;
    const Part p = merge_row(part + (long)min(row, M - 1) * nblk_n, nblk_n, tau > 0.f ? 1.f / tau : 0.f, sub);
    if (sub == 0 && row < M) {
        stats[row] = row_stats_of(p, tau);
        edge_defaults(row, T, V, tokens, parent, edge);
    }
}

}  // namespace

extern "C" size_t mdt_verify_logits_workspace(mdt_dtype dt, int B, int T, int d, int V) {
    (void)dt;
    (void)d;
    if (B < 1 || T < 1 || V < 1) return 0;
    return (size_t)B * T * ((V + kNB - 1) / kNB) * sizeof(Part);
}

mdt_status mdt_verify_tiles(hipStream_t s, mdt_dtype dt, int B, int T, int d, int V, const void* x, const void* Wlm,
                            const mdt_tree_dev* tree, const int32_t* tree_tokens, float temperature,
                            mdt_row_stats* stats, float* edge_logit, float* logits_opt, void* ws, size_t ws_bytes,
                            int* nblk_n_out) {
    MDT_REQUIRE(dt == MDT_F32 || dt == MDT_BF16, MDT_ERR_DTYPE, "dtype %d not supported", (int)dt);
    mdt_status st = mdt_check_tree(tree);
    if (st != MDT_OK) return st;
    MDT_REQUIRE(T == tree->T, MDT_ERR_SHAPE, "T=%d differs from the tree's %d nodes", T, tree->T);
    MDT_REQUIRE(B >= 1 && (long)B * T <= 65535L * kMB, MDT_ERR_SHAPE, "B=%d out of range", B);
    MDT_REQUIRE(V >= 1 && V <= 64 * 65535, MDT_ERR_SHAPE, "V=%d out of range", V);
    if (dt == MDT_BF16)
        MDT_REQUIRE(d >= 32 && d % 32 == 0, MDT_ERR_SHAPE, "bf16 verify needs d a multiple of 32 (got %d)", d);
    else
        MDT_REQUIRE(d >= 1 && d <= 1024, MDT_ERR_UNSUPPORTED, "fp32 verify supports d <= 1024 (got %d)", d);
    MDT_REQUIRE(temperature >= 0.f && temperature == temperature, MDT_ERR_VALUE, "temperature must be >= 0");
    MDT_REQUIRE(x && Wlm && tree_tokens && stats && edge_logit, MDT_ERR_NULL, "a tensor pointer is NULL");
    MDT_REQUIRE(mdt_aligned16(x) && mdt_aligned16(Wlm) && (!logits_opt || mdt_aligned16(logits_opt)), MDT_ERR_ALIGN,
                "tensor pointers must be 16-byte aligned");
    MDT_REQUIRE(ws, MDT_ERR_WORKSPACE, "workspace is NULL");
    MDT_REQUIRE(ws_bytes >= mdt_verify_logits_workspace(dt, B, T, d, V), MDT_ERR_WORKSPACE, "workspace too small");
    MDT_REQUIRE(mdt_aligned16(ws), MDT_ERR_ALIGN, "workspace must be 16-byte aligned");
    const int M = B * T;
    const bool big = dt == MDT_BF16 && M >= kBigRows;
#ifndef MDT_VERIFY_NO_DMA
    const bool dma = dt == MDT_BF16 && M <= kMB;
#else
    const bool dma = false;
#endif
    const bool wide = big && d % 64 == 0 && M >= kWideRows;
    const bool wide192 = big && d % 64 == 0 && !wide && M >= kWide192Rows;
    // columns per partial
    const int nb_cols = wide192 ? 64 : big || dma ? 128 : dt == MDT_BF16 ? MDT_VERIFY_NB : kNB;
    const int nblk_n = (V + nb_cols - 1) / nb_cols;
    Part* part = (Part*)ws;
    if (wide) {
        auto kern = verify_dma_wide<256, 256, 4, 2, 128>;
        MDT_LAUNCH("verify_mfma", kern, dim3((M + 255) / 256, (V + 255) / 256), dim3(512), 0, s, (const bf16_t*)x,
                   (const bf16_t*)Wlm, M, d, V, temperature, nblk_n, part, logits_opt, tree->parent, tree_tokens, T,
                   edge_logit);
    } else if (wide192 && (M + 223) / 224 == (M + 255) / 256) {
        auto kern = verify_dma_wide<224, 192, 2, 4, 64>;
        MDT_LAUNCH("verify_mfma", kern, dim3((M + 223) / 224, (V + 191) / 192), dim3(512), 0, s, (const bf16_t*)x,
                   (const bf16_t*)Wlm, M, d, V, temperature, nblk_n, part, logits_opt, tree->parent, tree_tokens, T,
                   edge_logit);
    } else if (wide192) {
        auto kern = verify_dma_wide<256, 192, 4, 2, 64>;
        MDT_LAUNCH("verify_mfma", kern, dim3((M + 255) / 256, (V + 191) / 192), dim3(512), 0, s, (const bf16_t*)x,
                   (const bf16_t*)Wlm, M, d, V, temperature, nblk_n, part, logits_opt, tree->parent, tree_tokens, T,
                   edge_logit);
    } else if (big && d % MDT_VBIG_KC == 0) {
        MDT_LAUNCH("verify_mfma", verify_dma_big, dim3((M + kBigMB - 1) / kBigMB, nblk_n), dim3(VBig::NT), 0, s,
                   (const bf16_t*)x, (const bf16_t*)Wlm, M, d, V, temperature, nblk_n, part, logits_opt, tree->parent,
                   tree_tokens, T, edge_logit);
    } else if (big) {  // inner dimension not a multiple of the chunk
        auto kern = verify_mfma128<64>;
        MDT_LAUNCH("verify_mfma", kern, dim3((M + 127) / 128, nblk_n), dim3(256), 0, s, (const bf16_t*)x,
                   (const bf16_t*)Wlm, M, d, V, temperature, nblk_n, part, logits_opt, tree->parent, tree_tokens, T,
                   edge_logit);
    } else if (dma) {
        MDT_LAUNCH("verify_mfma", verify_dma, dim3(nblk_n), dim3(VDma::NT), 0, s, (const bf16_t*)x, (const bf16_t*)Wlm,
                   M, d, V, temperature, nblk_n, part, logits_opt, tree->parent, tree_tokens, T, edge_logit);
    } else if (dt == MDT_BF16 && M > kMB) {
        // several node-row blocks: row-block-major grid (each weight block streamed once)
        auto kern = verify_mfma<MDT_VERIFY_KC, MDT_VERIFY_NB, 4, true>;
        MDT_LAUNCH("verify_mfma", kern, dim3((M + kMB - 1) / kMB, nblk_n), dim3(4 * MDT_VERIFY_NB), 0, s,
                   (const bf16_t*)x, (const bf16_t*)Wlm, M, d, V, temperature, nblk_n, part, logits_opt,
                   tree->parent, tree_tokens, T, edge_logit);
    } else if (dt == MDT_BF16) {
        auto kern = verify_mfma<MDT_VERIFY_KC, MDT_VERIFY_NB>;
        MDT_LAUNCH("verify_mfma", kern, dim3(nblk_n, (M + kMB - 1) / kMB), dim3(4 * MDT_VERIFY_NB), 0, s,
                   (const bf16_t*)x,
                           (const bf16_t*)Wlm, M, d, V, temperature, nblk_n, part, logits_opt, tree->parent,
                           tree_tokens, T, edge_logit);
    } else {
        const size_t lds = (size_t)16 * (d > kZStride ? d : kZStride) * sizeof(float);
        MDT_LAUNCH("verify_f32", verify_f32, dim3(nblk_n, (M + 15) / 16), dim3(256), lds, s, (const float*)x,
                           (const float*)Wlm, M, d, V, temperature, nblk_n, part, logits_opt, tree->parent,
                           tree_tokens, T, edge_logit);
    }
    *nblk_n_out = nblk_n;
    return mdt_launched(dt == MDT_BF16 ? "verify_mfma" : "verify_f32");
}

extern "C" mdt_status mdt_verify_logits(void* stream, mdt_dtype dt, int B, int T, int d, int V, const void* x,
                                        const void* Wlm, const mdt_tree_dev* tree, const int32_t* tree_tokens,
                                        float temperature, mdt_row_stats* stats, float* edge_logit,
                                        float* logits_opt, void* ws, size_t ws_bytes) {
    hipStream_t s = (hipStream_t)stream;
    int nblk_n = 0;
    const mdt_status st = mdt_verify_tiles(s, dt, B, T, d, V, x, Wlm, tree, tree_tokens, temperature, stats,
                                           edge_logit, logits_opt, ws, ws_bytes, &nblk_n);
    if (st != MDT_OK) return st;
    constexpr int kRowsPerWave = 64 / kMergeLanes;
    MDT_LAUNCH("verify_merge", verify_merge, dim3((B * T + kRowsPerWave - 1) / kRowsPerWave), dim3(64), 0, s, (const Part*)ws, B * T, nblk_n, V,
               temperature, stats, tree_tokens, tree->parent, T, edge_logit);
    return mdt_launched("verify_merge");
}
