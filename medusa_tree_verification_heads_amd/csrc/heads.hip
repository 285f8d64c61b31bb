// mdt_medusa_heads: the K Medusa heads and the LM head on the last hidden state.
//
// Summary page "Medusa: Simple LLM Inference Acceleration Framework with Multiple
// Decoding Heads", section "MEDUSA Heads": logits_k = W2_k (SiLU(W1_k h) + h); the
// LM head gives logits_0 = W_lm h (section 3.2).
//
// At batch 1 every weight byte is used for one multiply-add: the call is a pure
// HBM stream of K*d*d + (K+1)*d*V weights.  Each output row is a dot product of a
// contiguous weight row with an activation vector held in LDS as fp32.  A wave
// owns two rows at a time; each lane loads 16-byte chunks lane, lane+64, ... of
// both rows, so a wave instruction reads 1 KiB of contiguous weights per row, and
// the loads of the wave's next segment are in flight while it multiplies.
//
// Launch 1 streams W1 (-> a_k = SiLU(u) + h, fp32 in the workspace) together with
// W_lm (-> logits_0), which only needs h; launch 2 streams W2 (-> logits_1..K).
// Batches of 4 or more bf16 sequences take the matrix-core path instead
// (heads_mfma.hip), where each weight byte serves every sequence.
// Rows of all heads of a launch form one grid; a workgroup owns a contiguous row
// block of one head.
#include <atomic>
#include <mutex>
#include <type_traits>

#include "common.h"
#include "heads_mfma.h"

namespace {

constexpr int kThreads = 256;
constexpr int kMaxSeg = 2 * MDT_MAX_HEADS + 1;
constexpr int kRowsPerWg = 16;  // rows per workgroup per activation vector (launch planning)
constexpr int kLdsBytes = 64 * 1024;

struct GemvSeg {
    const void* W;        // [nrows][d], storage type
    const void* x;        // activations x + b * x_bstride: storage type in launch 1, fp32 in launch 2
    const void* resid;    // SiLU epilogue residual: must be x itself (read from LDS)
    float* out;           // out + b * out_bstride + row
    long x_bstride;
    long resid_bstride;
    long out_bstride;
    int nrows;
    int rows_per_wg;
    int wg_begin;
    int silu;             // epilogue: SiLU(u) + resid
    int pad;
};

struct GemvLaunch {
    GemvSeg seg[kMaxSeg];
    int nseg;
    int d;
    int B;
    int pad;
};

// Multiply-add one 16-byte weight chunk with the matching activations.
template <typename WT> struct Chunk;
template <> struct Chunk<bf16_t> {
    static constexpr int kElems = 8;
    static __device__ __forceinline__ float dot(const uint4& w, const float* x) {
        const float4 a = *(const float4*)x;
        const float4 b = *(const float4*)(x + 4);
        float s = __uint_as_float(w.x << 16) * a.x;
        s = fmaf(__uint_as_float(w.x & 0xffff0000u), a.y, s);
        s = fmaf(__uint_as_float(w.y << 16), a.z, s);
        s = fmaf(__uint_as_float(w.y & 0xffff0000u), a.w, s);
        s = fmaf(__uint_as_float(w.z << 16), b.x, s);
        s = fmaf(__uint_as_float(w.z & 0xffff0000u), b.y, s);
        s = fmaf(__uint_as_float(w.w << 16), b.z, s);
        s = fmaf(__uint_as_float(w.w & 0xffff0000u), b.w, s);
        return s;
    }
};
template <> struct Chunk<float> {
    static constexpr int kElems = 4;
    static __device__ __forceinline__ float dot(const uint4& w, const float* x) {
        const float4 a = *(const float4*)x;
        float s = __uint_as_float(w.x) * a.x;
        s = fmaf(__uint_as_float(w.y), a.y, s);
        s = fmaf(__uint_as_float(w.z), a.z, s);
        s = fmaf(__uint_as_float(w.w), a.w, s);
        return s;
    }
};

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Weights are read exactly once per call: load them non-temporally.
__device__ __forceinline__ uint4 ld_stream(const uint4* p) {
    const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// STAGE only names the launch (1: W1 + LM head, 2: W2) so that profiles separate the two.
// The wave walks (row pair, segment) items in order, a segment being SEG chunks of
// 16 bytes per lane of both rows (64*SEG chunks per row); the next item's loads are
// issued before the current item's multiply-adds, so every wave keeps 4*SEG loads in
// flight without gaps between rows.
template <typename WT, int NV, int STAGE, int SEG>
__global__ __launch_bounds__(kThreads) void heads_gemv(GemvLaunch P) {
    extern __shared__ float xs[];  // [NV][d]
    const int wg = blockIdx.x;
    int s = 0;
    while (s + 1 < P.nseg && wg >= P.seg[s + 1].wg_begin) ++s;
    const GemvSeg S = P.seg[s];
    const int d = P.d;
    const int b0 = blockIdx.y * NV;
    const int nv = min(NV, P.B - b0);

    constexpr int VEC = Chunk<WT>::kElems;
    const int nchunk = d / VEC;
    const int nseg = (nchunk + 64 * SEG - 1) / (64 * SEG);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r0 = (wg - S.wg_begin) * S.rows_per_wg;
    const int r1 = min(S.nrows, r0 + S.rows_per_wg);
    const int first = r0 + 2 * wave;  // pairs first, first + 8, ...
    const int npairs = first < r1 ? (r1 - first + 7) / 8 : 0;
    const int items = npairs * nseg;
    const WT* W = (const WT*)S.W;

    uint4 a0[SEG], a1[SEG], b0r[SEG], b1r[SEG];  // two static buffers: items it (A) and it+1 (B)
    // Loads are never under a branch and buffers are never copied (either would make the
    // compiler wait for every load in flight): addresses are clamped, a tail chunk
    // multiplies as zero, and a dummy item (real == false) makes all lanes read one piece.
    auto load = [&](int it, bool real, uint4 (&p)[SEG], uint4 (&q)[SEG]) {
        const int itc = real ? it : 0;
        const int pair = itc / nseg, sg = itc - pair * nseg;
        const int r = first + 8 * pair;
        const bool two = r + 1 < r1;
        const uint4* w0 = (const uint4*)(W + (size_t)(real ? r : r0) * d);
        const uint4* w1 = (const uint4*)(W + (size_t)(real && two ? r + 1 : (real ? r : r0)) * d);
#pragma unroll
        for (int u = 0; u < SEG; ++u) {
            const int c = real ? min(sg * 64 * SEG + lane + 64 * u, nchunk - 1) : 0;
            p[u] = ld_stream(w0 + c);
            q[u] = ld_stream(w1 + c);
        }
    };
    float acc0[NV], acc1[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) acc0[v] = acc1[v] = 0.f;
    auto process = [&](int it, const uint4 (&p)[SEG], const uint4 (&q)[SEG]) {
        const int pair = it / nseg, sg = it - pair * nseg;
#pragma unroll
        for (int u = 0; u < SEG; ++u) {
            const int c = sg * 64 * SEG + lane + 64 * u;
            const bool in = c < nchunk;
            const int cc = in ? c : nchunk - 1;
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const float* xp = xs + v * d + cc * VEC;
                const float d0 = Chunk<WT>::dot(p[u], xp), d1 = Chunk<WT>::dot(q[u], xp);
                acc0[v] += in ? d0 : 0.f;
                acc1[v] += in ? d1 : 0.f;
            }
        }
        if (sg == nseg - 1) {
            const int r = first + 8 * pair;
            const bool two = r + 1 < r1;
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                acc0[v] = wave_sum(acc0[v]);
                acc1[v] = wave_sum(acc1[v]);
            }
            if (lane == 0) {
                for (int v = 0; v < nv; ++v) {
                    const long b = b0 + v;
                    for (int q2 = 0; q2 < (two ? 2 : 1); ++q2) {
                        const int row = r + q2;
                        float u = q2 ? acc1[v] : acc0[v];
                        // the residual is the activation itself (h, staged in LDS), so the
                        // epilogue issues no global load that would wait for the prefetch
                        if (S.silu) u = u / (1.f + expf(-u)) + xs[v * d + row];
                        S.out[b * S.out_bstride + row] = u;
                    }
                }
            }
#pragma unroll
            for (int v = 0; v < NV; ++v) acc0[v] = acc1[v] = 0.f;
        }
    };

    // Activations (stage 1: the hidden state in the storage type; stage 2: fp32) go to LDS
    // as fp32.  The first kXB 16-byte pieces per thread are requested before the first
    // weight segment, so waiting for them waits for nothing newer and both latencies overlap.
    using XT = typename std::conditional<STAGE == 1, WT, float>::type;
    constexpr int XV = 16 / (int)sizeof(XT);  // elements per piece
    constexpr int kXB = 4;
    const int npieces = nv * d / XV;
    auto x_piece = [&](int p) -> const uint4* {
        const int e0 = p * XV, v = e0 / d, e = e0 - v * d;
        return (const uint4*)((const XT*)S.x + (long)(b0 + v) * S.x_bstride + e);
    };
    auto x_store = [&](int p, const uint4& w) {
        float* dst = xs + p * XV;
        if constexpr (sizeof(XT) == 4) {
            *(float4*)dst = make_float4(__uint_as_float(w.x), __uint_as_float(w.y), __uint_as_float(w.z),
                                        __uint_as_float(w.w));
        } else {
            *(float4*)dst = make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                                        __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u));
            *(float4*)(dst + 4) = make_float4(__uint_as_float(w.z << 16), __uint_as_float(w.z & 0xffff0000u),
                                              __uint_as_float(w.w << 16), __uint_as_float(w.w & 0xffff0000u));
        }
    };
    uint4 xb[kXB];
#pragma unroll
    for (int j = 0; j < kXB; ++j) xb[j] = *x_piece(min((int)threadIdx.x + kThreads * j, npieces - 1));
    load(0, items > 0, a0, a1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < kXB; ++j)
        if ((int)threadIdx.x + kThreads * j < npieces) x_store(threadIdx.x + kThreads * j, xb[j]);
    for (int p = threadIdx.x + kThreads * kXB; p < npieces; p += kThreads) x_store(p, *x_piece(p));
    __syncthreads();

    for (int it = 0; it < items; it += 2) {
        // A holds item it; B gets it+1 while A is used, then A gets it+2 while B is used.
        // The scheduling barriers keep the loads ahead of the math that precedes them in
        // the wait order.
        load(it + 1, it + 1 < items, b0r, b1r);
        __builtin_amdgcn_sched_barrier(0);
        process(it, a0, a1);
        load(it + 2, it + 2 < items, a0, a1);
        __builtin_amdgcn_sched_barrier(0);
        if (it + 1 < items) process(it + 1, b0r, b1r);
    }
}

// Split a launch's rows into workgroups: about `target` workgroups in total,
// proportional to each segment's rows, each block a multiple of 8 rows.
int plan_segments(GemvLaunch& P, int target) {
    long total = 0;
    for (int s = 0; s < P.nseg; ++s) total += P.seg[s].nrows;
    int wg = 0;
    for (int s = 0; s < P.nseg; ++s) {
        GemvSeg& S = P.seg[s];
        long g = (long)((double)target * S.nrows / (double)total + 0.5);
        if (g < 1) g = 1;
        long rpw = (S.nrows + g - 1) / g;
        rpw = (rpw + 7) / 8 * 8;
        S.rows_per_wg = (int)rpw;
        S.wg_begin = wg;
        wg += (int)((S.nrows + rpw - 1) / rpw);
    }
    return wg;
}

template <typename WT, int STAGE>
mdt_status launch(GemvLaunch& P, hipStream_t stream) {
    const int d = P.d;
    int nv = 1;
    while (nv * 2 <= 8 && nv * 2 <= P.B && (size_t)(nv * 2) * d * sizeof(float) <= (size_t)kLdsBytes) nv *= 2;
    // Short workgroups of about kRowsPerWg rows (two row pairs per wave): far more
    // workgroups than resident slots, so the dispatcher refills a CU as soon as one of its
    // workgroups retires.  With one long block per slot, the SIMD arbiter's preference for
    // older waves made the first workgroup on every CU finish long before the last, which
    // then streamed the tail with few loads in flight.
    long rows_total = 0;
    for (int q = 0; q < P.nseg; ++q) rows_total += P.seg[q].nrows;
    // a workgroup stages nv activation vectors, so its row block grows with nv
    const long rows_per_wg = (long)kRowsPerWg * nv;
    const int nwg = plan_segments(P, (int)((rows_total + rows_per_wg - 1) / rows_per_wg));
    dim3 grid(nwg, (P.B + nv - 1) / nv);
    const size_t lds = (size_t)nv * d * sizeof(float);
    const char* name = STAGE == 1 ? "heads_gemv_w1_lm" : "heads_gemv_w2";
    switch (nv) {
        case 1: MDT_LAUNCH(name, (heads_gemv<WT, 1, STAGE, 8>), grid, dim3(kThreads), lds, stream, P); break;
        case 2: MDT_LAUNCH(name, (heads_gemv<WT, 2, STAGE, 8>), grid, dim3(kThreads), lds, stream, P); break;
        case 4: MDT_LAUNCH(name, (heads_gemv<WT, 4, STAGE, 4>), grid, dim3(kThreads), lds, stream, P); break;
        default: MDT_LAUNCH(name, (heads_gemv<WT, 8, STAGE, 4>), grid, dim3(kThreads), lds, stream, P); break;
    }
    return mdt_launched(name);
}

template <typename WT>
mdt_status run(hipStream_t stream, int B, int d, int V, int K, const void* h, const void* W1, const void* W2,
               const void* Wlm, float* logits, float* a) {
    GemvLaunch P1{};
    P1.d = d;
    P1.B = B;
    for (int k = 0; k < K; ++k) {
        GemvSeg& S = P1.seg[P1.nseg++];
        S.W = (const WT*)W1 + (size_t)k * d * d;
        S.x = h;
        S.x_bstride = d;
        S.resid = h;
        S.resid_bstride = d;
        S.out = a + (size_t)k * d;
        S.out_bstride = (long)K * d;
        S.nrows = d;
        S.silu = 1;
    }
    if (Wlm) {  // NULL: the LM-head slot is left as it is
        GemvSeg& S = P1.seg[P1.nseg++];
        S.W = Wlm;
        S.x = h;
        S.x_bstride = d;
        S.out = logits;
        S.out_bstride = (long)(K + 1) * V;
        S.nrows = V;
    }
    mdt_status st = launch<WT, 1>(P1, stream);
    if (st != MDT_OK) return st;

    GemvLaunch P2{};
    P2.d = d;
    P2.B = B;
    for (int k = 0; k < K; ++k) {
        GemvSeg& S = P2.seg[P2.nseg++];
        S.W = (const WT*)W2 + (size_t)k * V * d;
        S.x = a + (size_t)k * d;
        S.x_bstride = (long)K * d;
        S.out = logits + (size_t)(k + 1) * V;
        S.out_bstride = (long)(K + 1) * V;
        S.nrows = V;
    }
    return launch<WT, 2>(P2, stream);
}

}  // namespace

extern "C" size_t mdt_medusa_heads_workspace(int B, int d, int K) {
    if (B < 1 || d < 1 || K < 1) return 0;
    return (size_t)B * K * d * sizeof(float);
}

extern "C" mdt_status mdt_medusa_heads(void* stream, mdt_dtype dt, int B, int d, int V, int K, const void* h,
                                       const void* W1, const void* W2, const void* Wlm, float* logits, void* ws,
                                       size_t ws_bytes) {
    MDT_REQUIRE(dt == MDT_F32 || dt == MDT_BF16, MDT_ERR_DTYPE, "dtype %d not supported", (int)dt);
    MDT_REQUIRE(B >= 1 && B <= 1024, MDT_ERR_SHAPE, "B=%d out of range 1..1024", B);
    MDT_REQUIRE(d >= 8 && d % 8 == 0 && d <= 16384, MDT_ERR_SHAPE, "d=%d must be a multiple of 8 in 8..16384", d);
    MDT_REQUIRE(V >= 1, MDT_ERR_SHAPE, "V=%d must be >= 1", V);
    MDT_REQUIRE(K >= 1 && K <= MDT_MAX_HEADS, MDT_ERR_SHAPE, "K=%d out of range 1..%d", K, MDT_MAX_HEADS);
    MDT_REQUIRE(h && W1 && W2 && logits, MDT_ERR_NULL, "a tensor pointer is NULL");
    MDT_REQUIRE(mdt_aligned16(h) && mdt_aligned16(W1) && mdt_aligned16(W2) && mdt_aligned16(Wlm) &&
                    mdt_aligned16(logits),
                MDT_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
    MDT_REQUIRE(ws, MDT_ERR_WORKSPACE, "workspace is NULL");
    MDT_REQUIRE(ws_bytes >= mdt_medusa_heads_workspace(B, d, K), MDT_ERR_WORKSPACE, "workspace %zu < %zu bytes",
                ws_bytes, mdt_medusa_heads_workspace(B, d, K));
    MDT_REQUIRE(mdt_aligned16(ws), MDT_ERR_ALIGN, "workspace must be 16-byte aligned");
    hipStream_t s = (hipStream_t)stream;
    if (dt == MDT_BF16 && mdt_heads_mfma_applies(B, d)) return mdt_heads_mfma(s, B, d, V, K, h, W1, W2, Wlm, logits, ws);
    if (dt == MDT_BF16) return run<bf16_t>(s, B, d, V, K, h, W1, W2, Wlm, logits, (float*)ws);
    return run<float>(s, B, d, V, K, h, W1, W2, Wlm, logits, (float*)ws);
}

// ---------------------------------------------------------------------------
// mdt_medusa_heads_noalloc: the same two kernels with their activations in a fixed
// device array of this library instead of a caller workspace.
// ---------------------------------------------------------------------------

// One copy per device, alive until the process ends.  Host code never passes this name
// to a kernel (on the host it is only a stand-in for the device symbol): the device
// address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[MDT_HEADS_NOALLOC_MAX_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the current device (looked up on the first call there).
mdt_status scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    MDT_REQUIRE(e == hipSuccess, MDT_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    MDT_REQUIRE(dev >= 0 && dev < kMaxDevices, MDT_ERR_UNSUPPORTED, "device %d beyond %d devices", dev, kMaxDevices);
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            MDT_REQUIRE(e == hipSuccess && p, MDT_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return MDT_OK;
}
}  // namespace

extern "C" mdt_status mdt_medusa_heads_noalloc(void* stream, mdt_dtype dt, int B, int d, int V, int K, const void* h,
                                               const void* W1, const void* W2, const void* Wlm, float* logits) {
    MDT_REQUIRE(B >= 1 && d >= 1 && K >= 1, MDT_ERR_SHAPE, "B=%d d=%d K=%d must be >= 1", B, d, K);
    const size_t need = mdt_medusa_heads_workspace(B, d, K);
    MDT_REQUIRE(need <= (size_t)MDT_HEADS_NOALLOC_MAX_BYTES, MDT_ERR_WORKSPACE,
                "B*K*d*4 = %zu bytes exceeds the fixed scratch of %u bytes (use mdt_medusa_heads with a workspace)",
                need, (unsigned)MDT_HEADS_NOALLOC_MAX_BYTES);
    void* ws = nullptr;
    const mdt_status st = scratch_address(&ws);
    if (st != MDT_OK) return st;
    return mdt_medusa_heads(stream, dt, B, d, V, K, h, W1, W2, Wlm, logits, ws, MDT_HEADS_NOALLOC_MAX_BYTES);
}
