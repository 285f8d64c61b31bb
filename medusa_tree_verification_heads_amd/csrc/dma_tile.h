// A 16 MT x NB tile of x W^T for at most 16 MT x rows (MT = 4 unless stated: 64 rows),
// with both operands staged in LDS by direct global-to-LDS loads (global_load_lds_dwordx4:
// each lane's 16 bytes land in LDS without passing through registers).
//
// The inner dimension is walked in chunks of KC dims held in an S-stage ring: while the
// waves multiply chunk c out of LDS, the loads of chunks c+1 .. c+S-1 are in flight, and
// one barrier per chunk both publishes chunk c and frees the buffer that chunk c+S-1 is
// then loaded into.  A load instruction fills 1 KiB of LDS contiguously (lane l at
// +16 l), so the layout is chosen through the global addresses: row r of a chunk takes
// KC/8 consecutive 16-byte slots, and slot j of the row holds the row's piece
// j ^ (r mod 16).  Every instruction still reads whole rows of the chunk (runs of 2 KC
// bytes), and the 16 rows of an MFMA fragment read fall into 16 distinct bank groups.
//
// Waves: CG column groups x KS inner-dimension groups.  Wave (cg, kh) multiplies x rows
// 0..16 MT - 1 against weight rows cg NB/CG .. +NB/CG over the k-steps kh, kh + KS, ... of each
// chunk; the KS partial products are then summed through LDS in kh order, and epi(acc)
// runs on the kh = 0 waves with acc[nt][mt] holding weight rows cg NB/CG + 16 nt + l%16 and
// x rows 16 mt + 4 (l/16) + e (the 16x16 MFMA output layout).
//
// Rows of x past M and of W past V read the last valid row (their products are never
// stored by a caller that honours M and V); pieces past d read the row's first piece and
// the k-steps past d are skipped.  The product runs over the first d columns of rows that
// are ld elements apart (a slice of a longer inner dimension); d must be a multiple of 32.
//
// The chunks are walked starting from chunk rot (mod the chunk count) and wrapping round.
// When every workgroup of a grid starts at chunk 0, the whole GPU requests the same 2 KC
// bytes of every weight row at once, which spreads unevenly over the memory channels; a
// start that differs between neighbouring workgroups spreads it (a plain load stream of a
// 96-row x 256-byte chunk shape: 4.9 -> 6.3 TB/s in one pass over 180 MB).
#pragma once

#include "mfma_tile.h"

typedef __attribute__((address_space(3))) void lds_void_t;

// Wait until at most N vector-memory operations of this wave are outstanding and every LDS
// operation is done (s_waitcnt vmcnt(N) lgkmcnt(0)), then meet the workgroup at a barrier.
// __syncthreads() would also wait for every load still in flight (its fence covers the
// direct-to-LDS loads), which is exactly the overlap the ring exists for.  The empty asm
// statements keep the compiler from moving memory accesses across the barrier; the
// lgkmcnt(0) makes every LDS read of the previous chunk complete before any wave can
// refill that buffer.
template <int N>
__device__ __forceinline__ void ring_barrier() {
    static_assert(N >= 0 && N < 64, "vmcnt is six bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// s_waitcnt lgkmcnt(0) alone.  At the end of a pipelined iteration the next iteration's
// first fragments are complete by then (the MFMAs issued in between take longer); with
// nothing pending across the loop's back edge, the compiler's own wait before the next
// MFMAs covers only the reads issued in the same iteration.
__device__ __forceinline__ void lds_done() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8)); }

// Wait until at most `later` chunks of I load instructions each, issued after the awaited
// one, are outstanding (0 <= later <= L), then meet the workgroup at the barrier.
template <int I, int L>
__device__ __forceinline__ void chunk_landed(int later) {
    if constexpr (L == 0) {
        ring_barrier<0>();
    } else {
        if (later >= L)
            ring_barrier<L * I>();
        else
            chunk_landed<I, L - 1>(later);
    }
}

template <int KC, int NB, int CG, int KS, int S, int MT = 4>
struct DmaTile {
    static constexpr int NW = CG * KS;
    static constexpr int NT = 64 * NW;
    static constexpr int MX = 16 * MT;                 // x rows
    static constexpr int kPR = KC / 8;                 // 16-byte pieces per row per chunk
    static constexpr int kWBytes = NB * KC * 2;
    static constexpr int kXBytes = MX * KC * 2;
    static constexpr int kStage = kWBytes + kXBytes;
    static constexpr int kIW = NB * kPR / 64 / NW;     // weight load instructions per wave per chunk
    static constexpr int kIX = MX * kPR / 64 / NW;     // x load instructions per wave per chunk
    static constexpr int kLoads = kIW + kIX;
    static constexpr int kRedBytes = (KS - 1) * (NB / 16) * MT * 64 * 16;  // k-group partials
    static constexpr int kRingBytes = S * kStage;
    static_assert(KC % 128 == 0, "a chunk row spans at least 16 pieces (the swizzle's period)");
    static_assert((KC / 32) % KS == 0, "k-steps divide among the k-groups");
    static_assert(NB % (16 * CG) == 0, "columns divide among the column groups");
    static_assert(NB * kPR % (64 * NW) == 0 && MX * kPR % (64 * NW) == 0, "loads divide among the waves");
    static_assert(S >= 2 && S <= 4, "2 to 4 stages");
    static_assert(kLoads * (S - 2) < 64, "vmcnt range");
};

template <int KC, int NB, int CG, int KS, int S, int AUX = 0, int MT = 4, typename Epi>
__device__ __forceinline__ void dma_tile(const bf16_t* __restrict__ x, const bf16_t* __restrict__ W, int M, int d,
                                         int ld, int V, int n0, char* smem, Epi&& epi, int rot = 0) {
    using P = DmaTile<KC, NB, CG, KS, S, MT>;
    constexpr int kPR = P::kPR;
    constexpr int NTW = NB / CG / 16;   // weight fragments per wave
    constexpr int KSS = KC / 32 / KS;   // k-steps per wave per chunk
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, c16 = lane & 15;
    const int cg = wave % CG, kh = wave / CG;
    const int nch = (d + KC - 1) / KC;
    rot %= nch;
    auto chunk_of = [&](int c) { return c + rot < nch ? c + rot : c + rot - nch; };

    // the c-th chunk walked into ring slot c % S: instruction i of the chunk covers linear
    // slots 64 i .. 64 i + 63, slot q holding piece (q % kPR) ^ (row % 16) of row q / kPR
    auto issue = [&](int c) {
        char* st = smem + (c % S) * P::kStage;
        const int kc = chunk_of(c) * KC;
#pragma unroll
        for (int j = 0; j < P::kIW; ++j) {
            const int i = wave * P::kIW + j;
            const int q = 64 * i + lane;
            const int r = q / kPR, p = (q % kPR) ^ (r & 15);
            const int k = kc + 8 * p;
            const bf16_t* src = W + (size_t)min(n0 + r, V - 1) * ld + (k < d ? k : 0);
            __builtin_amdgcn_global_load_lds((const void*)src, (lds_void_t*)(st + 1024 * i), 16, 0, AUX);
        }
#pragma unroll
        for (int j = 0; j < P::kIX; ++j) {
            const int i = wave * P::kIX + j;
            const int q = 64 * i + lane;
            const int r = q / kPR, p = (q % kPR) ^ (r & 15);
            const int k = kc + 8 * p;
            const bf16_t* src = x + (size_t)min(r, M - 1) * ld + (k < d ? k : 0);
            __builtin_amdgcn_global_load_lds((const void*)src, (lds_void_t*)(st + P::kWBytes + 1024 * i), 16, 0, 0);
        }
    };

    f32x4 acc[NTW][MT];
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[nt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto compute = [&](int c) {
        const char* st = smem + (c % S) * P::kStage;
        const bf16_t* ws = (const bf16_t*)st;
        const bf16_t* xs = (const bf16_t*)(st + P::kWBytes);
        const int nsteps = min(KC, d - chunk_of(c) * KC) / 32;
        if (KSS >= 4 && nsteps == KC / 32) {
            // a whole chunk with four or more k-steps per wave: every fragment read first,
            // then the MFMAs (the guarded loop below waits for each step's reads in turn;
            // with fewer steps per wave it measured as fast or faster)
            u32x4 a[KSS][MT], b[KSS][NTW];
#pragma unroll
            for (int s2 = 0; s2 < KSS; ++s2) {
                const int pp = (4 * (kh + KS * s2) + g) ^ c16;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) a[s2][mt] = *(const u32x4*)(xs + ((16 * mt + c16) * kPR + pp) * 8);
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt)
                    b[s2][nt] = *(const u32x4*)(ws + ((cg * (NB / CG) + 16 * nt + c16) * kPR + pp) * 8);
            }
#pragma unroll
            for (int s2 = 0; s2 < KSS; ++s2)
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) acc[nt][mt] = mfma16(a[s2][mt], b[s2][nt], acc[nt][mt]);
            return;
        }
#pragma unroll
        for (int s2 = 0; s2 < KSS; ++s2) {
            const int s = kh + KS * s2;
            if (s < nsteps) {
                const int pp = (4 * s + g) ^ c16;  // rows of a fragment start at multiples of 16
                u32x4 a[MT], b[NTW];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) a[mt] = *(const u32x4*)(xs + ((16 * mt + c16) * kPR + pp) * 8);
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt)
                    b[nt] = *(const u32x4*)(ws + ((cg * (NB / CG) + 16 * nt + c16) * kPR + pp) * 8);
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) acc[nt][mt] = mfma16(a[mt], b[nt], acc[nt][mt]);
            }
        }
    };

#pragma unroll
    for (int c = 0; c < S - 1; ++c)
        if (c < nch) issue(c);
    for (int c = 0; c < nch; ++c) {
        // chunk c has landed once at most min(S - 2, nch - 1 - c) later chunks are outstanding
        const int later = min(S - 2, nch - 1 - c);
        if (later >= 2)
            ring_barrier<2 * P::kLoads>();
        else if (later == 1)
            ring_barrier<P::kLoads>();
        else
            ring_barrier<0>();
        if (c + S - 1 < nch) issue(c + S - 1);
        compute(c);
    }
    __syncthreads();  // every wave is done with the ring: it becomes the reduction buffer
    if (KS > 1) {
        float* red = (float*)smem;  // [KS-1][CG][NTW][MT][4 e][64 lanes]
        if (kh > 0) {
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        red[(((((kh - 1) * CG + cg) * NTW + nt) * MT + mt) * 4 + e) * 64 + lane] = acc[nt][mt][e];
        }
        __syncthreads();
        if (kh == 0) {
#pragma unroll
            for (int k2 = 1; k2 < KS; ++k2)
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            acc[nt][mt][e] += red[(((((k2 - 1) * CG + cg) * NTW + nt) * MT + mt) * 4 + e) * 64 + lane];
        }
    }
    if (kh == 0) epi(acc);
}

// The 16-byte piece of a chunk row that sits in slot j of the row's LDS slots: rows of
// 16 or more pieces XOR with the row's low four bits; rows of 8 pieces (128 bytes, half a
// bank window) with bits 1..3, the row's parity already splitting the window.  Either way
// the 16 rows of an MFMA fragment read land in 16 distinct bank groups.
template <int kPR>
__device__ __forceinline__ int dma_swz(int j, int r) {
    static_assert(kPR == 8 || kPR % 16 == 0, "8 or a multiple of 16 pieces per row");
    return kPR >= 16 ? (j ^ (r & 15)) : (j ^ ((r >> 1) & 7));
}

// An MB x NB tile of x W^T (x rows m0.., weight rows n0..) for products with many x rows,
// staged like dma_tile (direct global-to-LDS loads into an S-stage ring of KC-dim chunks)
// without splitting the inner dimension: WM x WN waves, wave (wm, wn) = (w / WN, w % WN)
// owns x rows wm MB/WM .. and weight rows wn NB/WN .., i.e. MTW x NTW MFMA fragments.
//
// Software pipeline: the fragments of k-step s+1 are read from LDS while the MFMAs of step
// s run (two register sets), and the one barrier per chunk sits before the chunk's last
// k-step -- its fragments are already in registers, so the barrier both publishes chunk
// c+1 and frees chunk c's buffer, which is refilled with chunk c+S right away, and the
// first fragments of chunk c+1 are read while the last MFMAs of chunk c run.
// epi(acc) runs on every wave: acc[nt][mt] holds weight rows wn NB/WN + 16 nt + l%16 and x
// rows wm MB/WM + 16 mt + 4 (l/16) + e.  Rows past M / V read the last valid row; d must be
// a multiple of KC.
template <int MB, int NB, int WM, int WN, int KC, int S>
struct DmaGemm {
    static constexpr int NW = WM * WN;
    static constexpr int NT = 64 * NW;
    static constexpr int kPR = KC / 8;
    static constexpr int kXBytes = MB * KC * 2;
    static constexpr int kWBytes = NB * KC * 2;
    static constexpr int kStage = kXBytes + kWBytes;
    static constexpr int kIX = MB * kPR / 64 / NW;
    static constexpr int kIW = NB * kPR / 64 / NW;
    static constexpr int kLoads = kIX + kIW;
    static constexpr int kRingBytes = S * kStage;
    static constexpr int MTW = MB / WM / 16;
    static constexpr int NTW = NB / WN / 16;
    static constexpr int KSTEPS = KC / 32;
    static_assert(KC % 64 == 0 && (kPR == 8 || kPR % 16 == 0), "chunk shape");
    static_assert(MB * kPR % (64 * NW) == 0 && NB * kPR % (64 * NW) == 0, "loads divide among the waves");
    static_assert(MB % (16 * WM) == 0 && NB % (16 * WN) == 0, "fragments divide among the waves");
    static_assert(S >= 2 && S <= 4 && kLoads * (S - 1) < 64, "stages / vmcnt range");
};

template <int MB, int NB, int WM, int WN, int KC, int S, int AUX = 0, typename Epi>
__device__ __forceinline__ void dma_gemm_tile(const bf16_t* __restrict__ x, const bf16_t* __restrict__ W, int M,
                                              int d, int V, int m0, int n0, char* smem, Epi&& epi) {
    using P = DmaGemm<MB, NB, WM, WN, KC, S>;
    constexpr int kPR = P::kPR, MTW = P::MTW, NTW = P::NTW, KSTEPS = P::KSTEPS;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, c16 = lane & 15;
    const int wm = wave / WN, wn = wave % WN;
    const int nch = d / KC;

    auto issue = [&](int c) {
        char* st = smem + (c % S) * P::kStage;
#pragma unroll
        for (int j = 0; j < P::kIX; ++j) {
            const int i = wave * P::kIX + j;
            const int q = 64 * i + lane;
            const int r = q / kPR, p = dma_swz<kPR>(q % kPR, r);
            const bf16_t* src = x + (size_t)min(m0 + r, M - 1) * d + c * KC + 8 * p;
            __builtin_amdgcn_global_load_lds((const void*)src, (lds_void_t*)(st + 1024 * i), 16, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < P::kIW; ++j) {
            const int i = wave * P::kIW + j;
            const int q = 64 * i + lane;
            const int r = q / kPR, p = dma_swz<kPR>(q % kPR, r);
            const bf16_t* src = W + (size_t)min(n0 + r, V - 1) * d + c * KC + 8 * p;
            __builtin_amdgcn_global_load_lds((const void*)src, (lds_void_t*)(st + P::kXBytes + 1024 * i), 16, 0,
                                             AUX);
        }
    };
    // wait until chunk c has landed (at most `later` chunks issued after it outstanding),
    // then meet at the barrier
    auto landed = [&](int later) {
        if (later >= 3)
            ring_barrier<3 * P::kLoads>();
        else if (later == 2)
            ring_barrier<2 * P::kLoads>();
        else if (later == 1)
            ring_barrier<P::kLoads>();
        else
            ring_barrier<0>();
    };

    f32x4 acc[NTW][MTW];
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
        for (int mt = 0; mt < MTW; ++mt) acc[nt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    u32x4 fa[2][MTW], fb[2][NTW];
    // fragments of k-step s of the chunk in ring slot `slot` into register set `set`
    auto read = [&](int slot, int s, int set) {
        const bf16_t* xs = (const bf16_t*)(smem + slot * P::kStage);
        const bf16_t* ws = (const bf16_t*)(smem + slot * P::kStage + P::kXBytes);
#pragma unroll
        for (int mt = 0; mt < MTW; ++mt) {
            const int row = wm * (MB / WM) + 16 * mt + c16;
            fa[set][mt] = *(const u32x4*)(xs + (row * kPR + dma_swz<kPR>(4 * s + g, row)) * 8);
        }
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
            const int row = wn * (NB / WN) + 16 * nt + c16;
            fb[set][nt] = *(const u32x4*)(ws + (row * kPR + dma_swz<kPR>(4 * s + g, row)) * 8);
        }
    };
    auto mma = [&](int set) {
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
            for (int mt = 0; mt < MTW; ++mt) acc[nt][mt] = mfma16(fa[set][mt], fb[set][nt], acc[nt][mt]);
    };

#pragma unroll
    for (int c = 0; c < S; ++c)
        if (c < nch) issue(c);
    landed(min(S - 1, nch - 1));
    read(0, 0, 0);
    lds_done();
    for (int c = 0; c < nch; ++c) {
        const int slot = c % S;
#pragma unroll
        for (int s = 0; s + 1 < KSTEPS; ++s) {
            read(slot, s + 1, (s + 1) & 1);
            mma(s & 1);
        }
        // chunk c's last fragments are in registers: publish chunk c+1, free chunk c's buffer
        if (c + 1 < nch) {
            landed(min(S - 2, nch - 2 - c));
            if (c + S < nch) issue(c + S);
        }
        // The first fragments of chunk c+1 go out before the last MFMAs of chunk c.  The read
        // is unconditional (after the last chunk it reads a ring slot whose values are never
        // used) so that every path into the MFMAs below has the same LDS reads in flight:
        // otherwise the compiler's wait before them also covers these reads.
        read((c + 1) % S, 0, KSTEPS & 1);
        mma((KSTEPS - 1) & 1);
        lds_done();
    }
    __syncthreads();  // the ring is free for the caller's epilogue
    epi(acc);
}

// dma_gemm_tile's staging with a wider tile: each chunk brings MB + NB rows, so a 256 x 256
// tile moves a third fewer bytes through the L2 -> LDS path per MFMA than 256 x 128 (the x rows,
// re-read by every weight block, are the larger share).  Per k-step a wave reads its MTW x
// fragments into one of two register sets and refills each weight fragment register with
// the next step's fragment right after that fragment's MFMAs ("rolling"), which keeps the
// accumulators and the operands of two steps within two waves per SIMD.  The barrier sits
// before a chunk's last k-step, whose fragments are already in registers; the next chunk's
// first fragments are read during that step.  KC / 32 must be even (register sets alternate
// with the k-step's parity).  The x rows' load instructions need not divide among the waves
// (224-row tiles: 28 instructions on 8 waves): instruction i goes to wave i mod NW.
// epi(acc) as for dma_gemm_tile.
template <int MB, int NB, int WM, int WN, int KC, int S>
struct DmaGemmWide {
    static constexpr int NW = WM * WN;
    static constexpr int NT = 64 * NW;
    static constexpr int kPR = KC / 8;
    static constexpr int kXBytes = MB * KC * 2;
    static constexpr int kWBytes = NB * KC * 2;
    static constexpr int kStage = kXBytes + kWBytes;
    static constexpr int kRingBytes = S * kStage;
    static constexpr int kNIX = MB * kPR / 64;               // x load instructions per chunk
    static constexpr int kIXmax = (kNIX + NW - 1) / NW;      // per wave, at most
    static constexpr int kIXlow = kNIX % NW;                 // waves below this index issue kIXmax
    static constexpr int kIW = NB * kPR / 64 / NW;           // weight load instructions per wave
    static constexpr int MTW = MB / WM / 16;
    static constexpr int NTW = NB / WN / 16;
    static constexpr int KSTEPS = KC / 32;
    static_assert(KC % 64 == 0 && (kPR == 8 || kPR % 16 == 0), "chunk shape");
    static_assert(MB * kPR % 64 == 0 && NB * kPR % (64 * NW) == 0, "whole load instructions");
    static_assert(MB % (16 * WM) == 0 && NB % (16 * WN) == 0, "fragments divide among the waves");
    static_assert(S >= 2 && (kIXmax + kIW) * (S - 1) < 64, "stages / vmcnt range");
};

template <int MB, int NB, int WM, int WN, int KC, int S, int AUX = 0, typename Epi>
__device__ __forceinline__ void dma_gemm_wide(const bf16_t* __restrict__ x, const bf16_t* __restrict__ W, int M,
                                              int d, int V, int m0, int n0, char* smem, Epi&& epi) {
    using P = DmaGemmWide<MB, NB, WM, WN, KC, S>;
    constexpr int kPR = P::kPR, MTW = P::MTW, NTW = P::NTW, KSTEPS = P::KSTEPS;
    static_assert(KSTEPS % 2 == 0, "k-steps per chunk must be even");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, c16 = lane & 15;
    const int wm = wave / WN, wn = wave % WN;
    const int nch = d / KC;
    // this wave's load instructions per chunk (the first kIXlow waves issue one x load more)
    const bool xmore = P::kIXlow == 0 || wave < P::kIXlow;

    auto issue = [&](int c) {
        char* st = smem + (c % S) * P::kStage;
#pragma unroll
        for (int j = 0; j < P::kIXmax; ++j) {
            const int i = j * P::NW + wave;
            if (i < P::kNIX) {
                const int q = 64 * i + lane;
                const int r = q / kPR, p = dma_swz<kPR>(q % kPR, r);
                const bf16_t* src = x + (size_t)min(m0 + r, M - 1) * d + c * KC + 8 * p;
                __builtin_amdgcn_global_load_lds((const void*)src, (lds_void_t*)(st + 1024 * i), 16, 0, 0);
            }
        }
#pragma unroll
        for (int j = 0; j < P::kIW; ++j) {
            const int i = wave * P::kIW + j;
            const int q = 64 * i + lane;
            const int r = q / kPR, p = dma_swz<kPR>(q % kPR, r);
            const bf16_t* src = W + (size_t)min(n0 + r, V - 1) * d + c * KC + 8 * p;
            __builtin_amdgcn_global_load_lds((const void*)src, (lds_void_t*)(st + P::kXBytes + 1024 * i), 16, 0,
                                             AUX);
        }
    };
    // wait until at most `later` chunks issued after the awaited one are outstanding
    auto landed = [&](int later) {
        constexpr int kHi = P::kIXmax + P::kIW, kLo = (P::kIXlow ? P::kIXmax - 1 : P::kIXmax) + P::kIW;
        if (xmore)
            chunk_landed<kHi, S - 1>(min(later, S - 1));
        else
            chunk_landed<kLo, S - 1>(min(later, S - 1));
    };

    f32x4 acc[NTW][MTW];
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
        for (int mt = 0; mt < MTW; ++mt) acc[nt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    u32x4 fa[2][MTW], fb[NTW];
    auto read_a = [&](int slot, int s, int set) {
        const bf16_t* xs = (const bf16_t*)(smem + slot * P::kStage);
#pragma unroll
        for (int mt = 0; mt < MTW; ++mt) {
            const int row = wm * (MB / WM) + 16 * mt + c16;
            fa[set][mt] = *(const u32x4*)(xs + (row * kPR + dma_swz<kPR>(4 * s + g, row)) * 8);
        }
    };
    auto read_b = [&](int slot, int s, int nt) {
        const bf16_t* ws = (const bf16_t*)(smem + slot * P::kStage + P::kXBytes);
        const int row = wn * (NB / WN) + 16 * nt + c16;
        return *(const u32x4*)(ws + (row * kPR + dma_swz<kPR>(4 * s + g, row)) * 8);
    };
    // the MFMAs of one k-step (register set `set`, weight fragments fb), each weight
    // fragment refilled from (nslot, ns) once its MFMAs are issued
    auto step = [&](int set, int nslot, int ns) {
        read_a(nslot, ns, set ^ 1);
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
#pragma unroll
            for (int mt = 0; mt < MTW; ++mt) acc[nt][mt] = mfma16(fa[set][mt], fb[nt], acc[nt][mt]);
            fb[nt] = read_b(nslot, ns, nt);
        }
    };

#pragma unroll
    for (int c = 0; c < S; ++c)
        if (c < nch) issue(c);
    landed(nch - 1);
    read_a(0, 0, 0);
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) fb[nt] = read_b(0, 0, nt);
    lds_done();
    for (int c = 0; c < nch; ++c) {
        const int slot = c % S;
#pragma unroll
        for (int s = 0; s + 1 < KSTEPS; ++s) step(s & 1, slot, s + 1);
        // chunk c's last fragments are in registers: publish chunk c+1, free chunk c's buffer;
        // the last step reads chunk c+1's first fragments (after the last chunk: a ring slot
        // whose values are never used, so that every path has the same reads in flight)
        if (c + 1 < nch) {
            landed(min(S - 2, nch - 2 - c));
            if (c + S < nch) issue(c + S);
        }
        step((KSTEPS - 1) & 1, (c + 1) % S, 0);
        lds_done();
    }
    __syncthreads();  // the ring is free for the caller's epilogue
    epi(acc);
}
