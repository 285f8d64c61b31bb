// A 64 x NB tile of x W^T (bf16 inputs, fp32 MFMA accumulation) over the full inner
// dimension: the verifier for 65 to 255 node rows and the heads of a batch.
//
// grid.x walks NB-row blocks of W, grid.y 64-row blocks of x; NB/16 waves.  Per chunk of
// KC dims, the workgroup moves its NB weight rows and 64 x rows into LDS with
// row-contiguous 16-byte loads (each wave instruction covers whole row runs, the pattern
// HBM streams best), then every wave reads MFMA fragments out of LDS: B = its 16 weight
// rows, A = the 64 x rows.  Two register buffers alternate statically (the loop handles
// chunks c and c+1), so while chunk c is multiplied the weights of chunks c+1 and c+2
// and the x rows of chunk c+1 are in flight.
#pragma once

#include "common.h"

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
}

__device__ __forceinline__ u32x4 ld_stream(const void* p) { return __builtin_nontemporal_load((const u32x4*)p); }

template <int KC, int NB, int MT = 4>
struct MfmaTile {
    static constexpr int NT = 4 * NB;                  // one wave per 16 weight rows
    static constexpr int kStride = KC + 8;             // LDS row stride (elements)
    static constexpr int kXBytes = 16 * MT * kStride * 2;  // the 16*MT-row x tile
    static constexpr int kWBytes = NB * kStride * 2;   // the NB-row weight tile
    static constexpr int kBytes = kXBytes + kWBytes;
};

// Multiplies the tile (x rows m0.., weight rows n0..; x is [M][ld], W is [V][ld], the
// product runs over the first d columns of both) and hands
// the fp32 accumulators to epi(acc): wave w owns weight rows 16w..16w+15 against all
// 16*MT x rows, acc[mt] holding x rows 16mt..16mt+15 in the 16x16 MFMA output layout
// (lane l: column 16w + l%16, rows 16mt + 4(l/16) + e).  `smem` holds
// MfmaTile<KC, NB, MT>::kBytes bytes; rows of x past M and of W past V read as zero.
// d must be a multiple of 32 and ld of 8.
template <int KC, int NB, int MT = 4, typename Epi>
__device__ __forceinline__ void mfma_tile(const bf16_t* __restrict__ x, const bf16_t* __restrict__ W, int M, int d,
                                          int ld, int V, int m0, int n0, char* smem, Epi&& epi) {
    constexpr int NT = MfmaTile<KC, NB, MT>::NT;
    constexpr int kStride = MfmaTile<KC, NB, MT>::kStride;
    constexpr int kPR = KC / 8;                   // 16-byte pieces per row per chunk
    constexpr int kPPT = NB * kPR / NT;           // weight pieces per thread per chunk
    constexpr int kXPT = 16 * MT * kPR / NT;      // x pieces per thread per chunk
    static_assert(KC % 32 == 0, "k-steps of 32");
    static_assert(16 * MT * kPR % NT == 0, "x pieces must divide among the threads");
    bf16_t* xs = (bf16_t*)smem;
    bf16_t* ws = (bf16_t*)(smem + MfmaTile<KC, NB, MT>::kXBytes);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, c16 = lane & 15;
    const int nchunks = (d + KC - 1) / KC;

    // No load is under a branch and no loaded register is touched before its LDS store
    // (either would make the compiler wait for the loads still in flight): a piece
    // outside the matrix, or of a chunk past the end, reads element 0 and is replaced
    // by zero when it is stored.
    u32x4 wA[kPPT], wB[kPPT], xr[kXPT];
    auto piece_in = [&](int c, int j, int rows0, int nrows) {
        const int p = threadIdx.x + NT * j;
        const int r = p / kPR, off = 8 * (p % kPR);
        return c < nchunks && off < d - c * KC && rows0 + r < nrows;
    };
    auto piece_at = [&](int c, int j, int rows0) {
        const int p = threadIdx.x + NT * j;
        return (size_t)(rows0 + p / kPR) * ld + c * KC + 8 * (p % kPR);
    };
    auto load_w = [&](int c, u32x4 (&wr)[kPPT]) {
#pragma unroll
        for (int j = 0; j < kPPT; ++j) wr[j] = ld_stream(W + (piece_in(c, j, n0, V) ? piece_at(c, j, n0) : 0));
    };
    auto load_x = [&](int c, u32x4 (&xb)[kXPT]) {
#pragma unroll
        for (int j = 0; j < kXPT; ++j) xb[j] = *(const u32x4*)(x + (piece_in(c, j, m0, M) ? piece_at(c, j, m0) : 0));
    };
    auto store = [&](int c, const u32x4 (&wr)[kPPT], const u32x4 (&xb)[kXPT]) {
        const u32x4 z{0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < kPPT; ++j) {
            const int p = threadIdx.x + NT * j;
            *(u32x4*)(ws + (p / kPR) * kStride + 8 * (p % kPR)) = piece_in(c, j, n0, V) ? wr[j] : z;
        }
#pragma unroll
        for (int j = 0; j < kXPT; ++j) {
            const int p = threadIdx.x + NT * j;
            *(u32x4*)(xs + (p / kPR) * kStride + 8 * (p % kPR)) = piece_in(c, j, m0, M) ? xb[j] : z;
        }
    };

    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto compute = [&](int c) {
        const int nsteps = min(KC, d - c * KC) / 32;  // <= 0 past the end
        const bf16_t* wrow = ws + (wave * 16 + c16) * kStride + 8 * g;
#pragma unroll 4
        for (int s = 0; s < KC / 32; ++s) {
            if (s < nsteps) {
                const u32x4 b = *(const u32x4*)(wrow + 32 * s);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const u32x4 a = *(const u32x4*)(xs + (mt * 16 + c16) * kStride + 32 * s + 8 * g);
                    acc[mt] = mfma16(a, b, acc[mt]);
                }
            }
        }
    };
    load_w(0, wA);
    load_x(0, xr);
    load_w(1, wB);
    store(0, wA, xr);
    __syncthreads();
    for (int c = 0; c < nchunks; c += 2) {
        // LDS: chunk c; wB: chunk c+1
        load_x(c + 1, xr);
        load_w(c + 2, wA);
        compute(c);
        __syncthreads();
        store(c + 1, wB, xr);
        __syncthreads();
        // LDS: chunk c+1; wA: chunk c+2
        load_x(c + 2, xr);
        load_w(c + 3, wB);
        compute(c + 1);
        __syncthreads();
        store(c + 2, wA, xr);
        __syncthreads();
    }
    epi(acc);
}



// A 128 x 128 tile for products with many x rows (compute-bound when both sides are
// large): 4 waves in a 2 x 2 grid, wave (wm, wn) = (w / 2, w % 2) multiplying x rows
// 64 wm .. +64 against weight rows 64 wn .. +64, i.e. 4 x 4 MFMA 16x16 fragments, so
// every fragment read from LDS feeds four products (the 64 x 64 tile's waves read all
// 64 x rows for 16 weight rows: 1.25 reads per product).  Same staging as mfma_tile:
// row-contiguous 16-byte loads, two register buffers, pieces outside the matrices
// zeroed in LDS.  acc[nt][mt]: weight rows 64 wn + 16 nt + l%16, x rows
// 64 wm + 16 mt + 4(l/16) + e.  LDS: MfmaTile128<KC>::kBytes.
template <int KC>
struct MfmaTile128 {
    static constexpr int kStride = KC + 8;
    static constexpr int kXBytes = 128 * kStride * 2;
    static constexpr int kBytes = 2 * kXBytes;
};

template <int KC, typename Epi>
__device__ __forceinline__ void mfma_tile128(const bf16_t* __restrict__ x, const bf16_t* __restrict__ W, int M,
                                             int d, int ld, int V, int m0, int n0, char* smem, Epi&& epi) {
    constexpr int NT = 256;
    constexpr int kStride = MfmaTile128<KC>::kStride;
    constexpr int kPR = KC / 8;
    constexpr int kPT = 128 * kPR / NT;  // pieces per thread per chunk, each operand
    static_assert(KC % 32 == 0 && 128 * kPR % NT == 0, "chunk shape");
    bf16_t* xs = (bf16_t*)smem;
    bf16_t* ws = (bf16_t*)(smem + MfmaTile128<KC>::kXBytes);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, c16 = lane & 15;
    const int wm = wave >> 1, wn = wave & 1;
    const int nchunks = (d + KC - 1) / KC;

    u32x4 wA[kPT], wB[kPT], xr[kPT];
    auto piece_in = [&](int c, int j, int rows0, int nrows) {
        const int p = threadIdx.x + NT * j;
        return c < nchunks && 8 * (p % kPR) < d - c * KC && rows0 + p / kPR < nrows;
    };
    auto piece_at = [&](int c, int j, int rows0) {
        const int p = threadIdx.x + NT * j;
        return (size_t)(rows0 + p / kPR) * ld + c * KC + 8 * (p % kPR);
    };
    auto load_w = [&](int c, u32x4 (&wr)[kPT]) {
#pragma unroll
        for (int j = 0; j < kPT; ++j) wr[j] = ld_stream(W + (piece_in(c, j, n0, V) ? piece_at(c, j, n0) : 0));
    };
    auto load_x = [&](int c) {
#pragma unroll
        for (int j = 0; j < kPT; ++j) xr[j] = *(const u32x4*)(x + (piece_in(c, j, m0, M) ? piece_at(c, j, m0) : 0));
    };
    auto store = [&](int c, const u32x4 (&wr)[kPT]) {
        const u32x4 z{0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < kPT; ++j) {
            const int p = threadIdx.x + NT * j;
            *(u32x4*)(ws + (p / kPR) * kStride + 8 * (p % kPR)) = piece_in(c, j, n0, V) ? wr[j] : z;
            *(u32x4*)(xs + (p / kPR) * kStride + 8 * (p % kPR)) = piece_in(c, j, m0, M) ? xr[j] : z;
        }
    };
    f32x4 acc[4][4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc[nt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto compute = [&](int c) {
        const int nsteps = min(KC, d - c * KC) / 32;  // <= 0 past the end
#pragma unroll
        for (int s = 0; s < KC / 32; ++s) {
            if (s < nsteps) {
                u32x4 a[4], b[4];
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
                    a[mt] = *(const u32x4*)(xs + (64 * wm + 16 * mt + c16) * kStride + 32 * s + 8 * g);
#pragma unroll
                for (int nt = 0; nt < 4; ++nt)
                    b[nt] = *(const u32x4*)(ws + (64 * wn + 16 * nt + c16) * kStride + 32 * s + 8 * g);
#pragma unroll
                for (int nt = 0; nt < 4; ++nt)
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt) acc[nt][mt] = mfma16(a[mt], b[nt], acc[nt][mt]);
            }
        }
    };
    load_w(0, wA);
    load_x(0);
    load_w(1, wB);
    store(0, wA);
    __syncthreads();
    for (int c = 0; c < nchunks; c += 2) {
        load_x(c + 1);
        load_w(c + 2, wA);
        compute(c);
        __syncthreads();
        store(c + 1, wB);
        __syncthreads();
        load_x(c + 2);
        load_w(c + 3, wB);
        compute(c + 1);
        __syncthreads();
        store(c + 2, wA);
        __syncthreads();
    }
    epi(acc);
}
