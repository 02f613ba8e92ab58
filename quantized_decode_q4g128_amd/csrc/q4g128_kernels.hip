// HIP kernels for the int4-g128 weight-streaming product on gfx950.
//
//   y[m][n] = sum_k x[m][k] * (q[n][k] * s[n][k/128] + mn[n][k/128])
//
// Decode streams every weight byte once per step (Token Rush README,
// bandwidth paragraph); an M-row verify step does the same with M activation
// rows (steps table rows 13-14, 28).  One kernel serves every M in 1..8.
//
// Per 128-group the sum is factored as
//   sum_k x*(q*s + mn) = s * sum_k x*(128 + q) + (mn - 128*s) * sum_k x
// The codes enter a bf16 MFMA as the exact bf16 values 128 + q (a mask and an
// OR per pair, no conversion); the x rows are the A operand, padded with zero
// rows to 16; the row sums sum_k x come from a second MFMA against an all-ones
// B operand.  Every output element is its own dot product inside the MFMA,
// and the schedule of instructions depends on (K, N) only, so row m of an
// M-row call is bit-identical to the one-row call (bw24 article, exactness
// paragraph).
//
// Work layout: a workgroup of 4 waves owns 64*TPW output columns and one
// contiguous range of 128-groups (the K split).  Each wave owns TPW tiles of
// 16 columns; lane (i = l%16, h = l/16) streams column i's 16-byte code piece
// h of every group (words 16g+4h .. 16g+4h+3), so the four lanes of a column
// read its 64 contiguous bytes per group.  x for kChunk groups at a time sits
// in LDS (double buffered), reordered into the pair order of the codes.
#include "q4g128_device.h"
#include "q4g128_launch.h"

namespace q4g128 {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kChunk = 8;                      // groups per LDS x chunk; also prefetch depth
constexpr int kRowStride = kChunk * 128 + 8;   // bf16 per LDS row: 16-byte pad vs bank conflicts
constexpr int kPiecesPerRow = kChunk * 16;     // 16-byte x pieces per row per chunk
constexpr int kStagePerThread = (kMaxM * kPiecesPerRow + kThreads - 1) / kThreads;

static_assert(kPiecesPerRow == 128, "piece index math below assumes 128 pieces per row");

// All outstanding LDS operations of this wave complete, then a workgroup
// barrier.  Outstanding global loads (the code prefetch) are left in flight.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int TPW>
__global__ __launch_bounds__(kThreads) void gemv_q4g128(
    const uint16_t *__restrict__ x, int M, int K, const uint32_t *__restrict__ W,
    const uint16_t *__restrict__ scale, const uint16_t *__restrict__ mn, int N,
    float *__restrict__ out, int S)
{
    __shared__ __attribute__((aligned(16))) uint16_t xs[2][kMaxM * kRowStride];
    __shared__ __attribute__((aligned(16))) uint16_t xzero[kChunk * 128];   // A rows >= M read here

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int i = lane & 15;    // column within a tile; A row
    const int h = lane >> 4;    // 16-byte code piece within a group; D row block
    const int G = K >> 7;
    const size_t K8 = (size_t)(K >> 3);
    const int split = blockIdx.y;
    const int gs = (int)(((long)split * G) / S);
    const int ge = (int)(((long)(split + 1) * G) / S);
    const int ng = ge - gs;
    const int nchunks = (ng + kChunk - 1) / kChunk;

    const int col0 = (blockIdx.x * kWaves + wave) * TPW * 16;
    const bool wave_live = col0 < N;   // wave-uniform

    // Wave-local buffer descriptors: codes, scales and minimums of this wave's
    // 16*TPW columns; the group offset of every load is a scalar (soffset),
    // the column offset a per-lane constant (voffset).
    const int ncols = __builtin_amdgcn_readfirstlane(max(0, min(16 * TPW, N - col0)));
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(W + (size_t)col0 * K8, (uint32_t)((size_t)ncols * K8 * 4));
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(scale + (size_t)col0 * G, (uint32_t)(ncols * G * 2));
    const __amdgpu_buffer_rsrc_t rm = make_rsrc(mn + (size_t)col0 * G, (uint32_t)(ncols * G * 2));
    uint32_t vw[TPW], vs[TPW];
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        const int c = min(16 * u + i, ncols - 1);   // ragged tail: read a real column, store nothing
        vw[u] = (uint32_t)((size_t)c * K8 * 4 + 16 * h);
        vs[u] = (uint32_t)(c * G * 2);
    }

    // Code / scale / minimum prefetch ring: slot q holds group gs + c*kChunk + q.
    // Loads past the end of the range re-read its last group (clamped), so the
    // ring is refilled unconditionally.
    u32x4 cb[kChunk][TPW];
    uint32_t sb[kChunk][TPW], mb[kChunk][TPW];
    auto fetch = [&](int q, int g) {
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
            cb[q][u] = __builtin_amdgcn_raw_buffer_load_b128(rw, vw[u], 64 * g, 0);
            sb[q][u] = __builtin_amdgcn_raw_buffer_load_b16(rs, vs[u], 2 * g, 0);
            mb[q][u] = __builtin_amdgcn_raw_buffer_load_b16(rm, vs[u], 2 * g, 0);
        }
    };
    if (wave_live) {
#pragma unroll
        for (int q = 0; q < kChunk; ++q) fetch(q, min(gs + q, ge - 1));
    }

    // x staging: piece p = (row p/128, 16-byte block p%128 of the chunk).
    const int pieces = M * kPiecesPerRow;
    u32x4 st[kStagePerThread];
    auto load_chunk = [&](int c) {
#pragma unroll
        for (int j = 0; j < kStagePerThread; ++j) {
            const int p = tid + kThreads * j;
            const int g = gs + c * kChunk + ((p & 127) >> 4);
            if (p < pieces && g < ge)
                st[j] = *reinterpret_cast<const u32x4 *>(x + (size_t)(p >> 7) * K + (size_t)g * 128 +
                                                         (p & 15) * 8);
        }
    };
    auto store_chunk = [&](int c, int buf) {
#pragma unroll
        for (int j = 0; j < kStagePerThread; ++j) {
            const int p = tid + kThreads * j;
            const int g = gs + c * kChunk + ((p & 127) >> 4);
            if (p < pieces && g < ge)
                *reinterpret_cast<u32x4 *>(&xs[buf][(p >> 7) * kRowStride + (p & 127) * 8]) =
                    pair_order(st[j]);
        }
    };

    static_assert(kChunk * 128 * 2 == kThreads * 8, "one 8-byte zero store per thread");
    reinterpret_cast<uint2 *>(xzero)[tid] = make_uint2(0u, 0u);
    load_chunk(0);
    store_chunk(0, 0);
    lds_barrier();

    float acc[TPW][4];
#pragma unroll
    for (int u = 0; u < TPW; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[u][r] = 0.0f;

    const u32x4 ones = {kOnePair, kOnePair, kOnePair, kOnePair};
    const UnpackConsts uc = unpack_consts();

    // One 128-group: A fragments from LDS, row sums, then per tile the code
    // MFMAs and the scale/minimum epilogue.  `q` is the ring slot.
    auto do_group = [&](const uint16_t *abase, int q, int g) {
        u32x4 a[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) a[t] = *reinterpret_cast<const u32x4 *>(abase + q * 128 + 8 * t);
        f32x4 xsum = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int t = 0; t < 4; ++t) xsum = mfma_16x16x32(a[t], ones, xsum);
        u32x4 cw[TPW];
        uint32_t sv[TPW], mv[TPW];
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
            cw[u] = cb[q][u];
            sv[u] = sb[q][u];
            mv[u] = mb[q][u];
        }
        fetch(q, min(g + kChunk, ge - 1));
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
            f32x4 d = {0.0f, 0.0f, 0.0f, 0.0f};
            d = mfma_16x16x32(a[0], unpack_biased(cw[u].x, uc), d);
            d = mfma_16x16x32(a[1], unpack_biased(cw[u].y, uc), d);
            d = mfma_16x16x32(a[2], unpack_biased(cw[u].z, uc), d);
            d = mfma_16x16x32(a[3], unpack_biased(cw[u].w, uc), d);
            const float s = bf16_lo(sv[u]);
            const float m = bf16_lo(mv[u]);
            const float m_adj = fmaf(-kBias, s, m);   // mn - 128*s, one rounding
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                acc[u][r] = fmaf(s, d[r], acc[u][r]);
                acc[u][r] = fmaf(m_adj, xsum[r], acc[u][r]);
            }
        }
    };

    const bool row_live = i < M;
    for (int c = 0; c < nchunks; ++c) {
        const bool more = c + 1 < nchunks;
        if (more) load_chunk(c + 1);
        if (wave_live) {
            const uint16_t *abase =
                row_live ? &xs[c & 1][i * kRowStride + 32 * h] : &xzero[32 * h];
            const int g0 = gs + c * kChunk;
            if (g0 + kChunk <= ge) {
#pragma unroll
                for (int q = 0; q < kChunk; ++q) do_group(abase, q, g0 + q);
            } else {
#pragma unroll
                for (int q = 0; q < kChunk; ++q)
                    if (g0 + q < ge) do_group(abase, q, g0 + q);
            }
        }
        if (more) store_chunk(c + 1, (c + 1) & 1);
        lds_barrier();
    }

    if (!wave_live) return;
    float *o = out + (size_t)split * (size_t)M * (size_t)N;
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        const int n = col0 + 16 * u + i;
        if (n < N) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 4 * h + r;
                if (row < M) o[(size_t)row * N + n] = acc[u][r];
            }
        }
    }
}

// y[e] = P[0][e] + P[1][e] + ... + P[S-1][e], in ascending s.
__global__ __launch_bounds__(256) void splitk_sum(const float *__restrict__ P, int S, size_t MN,
                                                  float *__restrict__ y)
{
    const size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= MN) return;
    float v = P[e];
    for (int s = 1; s < S; ++s) v += P[(size_t)s * MN + e];
    y[e] = v;
}

// One thread per packed word: eight weights fp32(q*s + mn), one rounding each.
__global__ __launch_bounds__(256) void dequant_q4g128(const uint32_t *__restrict__ W,
                                                      const uint16_t *__restrict__ scale,
                                                      const uint16_t *__restrict__ mn, int K, int N,
                                                      float *__restrict__ w)
{
    const size_t K8 = (size_t)(K >> 3);
    const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (size_t)N * K8) return;
    const size_t n = idx / K8;
    const size_t j = idx - n * K8;
    const size_t gi = n * (size_t)(K >> 7) + (j >> 4);
    const float s = bf16_lo(scale[gi]);
    const float m = bf16_lo(mn[gi]);
    const u32x4 p = unpack_biased(W[idx], unpack_consts());
    // pair p: low half = code p, high half = code p+4 (each as 128 + q; exact - 128).
    float4 lo, hi;
    lo.x = fmaf(bf16_lo(p.x) - kBias, s, m);
    lo.y = fmaf(bf16_lo(p.y) - kBias, s, m);
    lo.z = fmaf(bf16_lo(p.z) - kBias, s, m);
    lo.w = fmaf(bf16_lo(p.w) - kBias, s, m);
    hi.x = fmaf(bf16_hi(p.x) - kBias, s, m);
    hi.y = fmaf(bf16_hi(p.y) - kBias, s, m);
    hi.z = fmaf(bf16_hi(p.z) - kBias, s, m);
    hi.w = fmaf(bf16_hi(p.w) - kBias, s, m);
    float4 *dst = reinterpret_cast<float4 *>(w + n * (size_t)K + 8 * j);
    dst[0] = lo;
    dst[1] = hi;
}

// ---- launchers ---------------------------------------------------------------

int columns_per_block(int tpw) { return kWaves * 16 * tpw; }

hipError_t launch_gemv(const GemvArgs &a, int tpw, hipStream_t stream)
{
    const int cpb = columns_per_block(tpw);
    dim3 grid((unsigned)((a.N + cpb - 1) / cpb), (unsigned)a.S, 1);
    dim3 block(kThreads, 1, 1);
    switch (tpw) {
    case 1:
        hipLaunchKernelGGL(gemv_q4g128<1>, grid, block, 0, stream, a.x, a.M, a.K, a.W, a.scale, a.mn,
                           a.N, a.out, a.S);
        break;
    case 2:
        hipLaunchKernelGGL(gemv_q4g128<2>, grid, block, 0, stream, a.x, a.M, a.K, a.W, a.scale, a.mn,
                           a.N, a.out, a.S);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_splitk_sum(const float *P, int S, size_t MN, float *y, hipStream_t stream)
{
    dim3 grid((unsigned)((MN + 255) / 256), 1, 1);
    hipLaunchKernelGGL(splitk_sum, grid, dim3(256, 1, 1), 0, stream, P, S, MN, y);
    return hipGetLastError();
}

hipError_t launch_dequant(const uint32_t *W, const uint16_t *scale, const uint16_t *mn, int K, int N,
                          float *w, hipStream_t stream)
{
    const size_t words = (size_t)N * (size_t)(K >> 3);
    dim3 grid((unsigned)((words + 255) / 256), 1, 1);
    hipLaunchKernelGGL(dequant_q4g128, grid, dim3(256, 1, 1), 0, stream, W, scale, mn, K, N, w);
    return hipGetLastError();
}

}  // namespace q4g128
