// Work-balanced ("stream-K") variant of the int4-g128 weight-streaming
// product for gfx950.  Same arithmetic per group as gemv_q4g128 (codes as the
// exact bf16 values 128 + q into a 16x16x32 bf16 MFMA, per-group epilogue
// s*D + (mn - 128*s)*X); what changes is how the work is spread.
//
// Decode is bound by streaming the weights (Token Rush README, bandwidth
// paragraph), and on MI355X a stream only reaches full rate when every
// compute unit moves the same number of bytes: with one 16-column tile per
// wave, N = 34816 gives 2176 tiles for 256 CUs and the busiest CUs carry
// 3/2.125 of the average.  Here the launch has exactly one 8-wave workgroup
// per CU (its LDS request is sized so two never share a CU), and the units
// (tile of 16 columns, block of 8 groups = 1024 k) are cut into equal
// contiguous ranges, one per wave.
//
// A tile whose blocks land in several waves is summed in parts: each wave
// writes its part (fp32, 16 columns x 8 rows) to the workspace, and the last
// wave to finish the tile (an agent-scope counter per tile) adds the parts in
// ascending part order and writes y.  Parts and counters move through
// device-coherent buffer accesses (not device-scope fences, which write back
// and invalidate whole L2 caches).  The part order is fixed by (K, N) and
// the CU count only, so results are deterministic and every row of an M-row
// call equals the one-row call bit for bit (bw24 article, exactness
// paragraph).  Counters are reset by the wave that consumes them, so a
// zero-filled workspace stays zero-filled between calls.
//
// K is cut into SK slices of whole blocks when 8 rows of x for all of K would
// not fit in LDS; each slice has its own workgroups and contributes parts of
// every tile.
#include "q4g128_device.h"
#include "q4g128_launch.h"
#include "q4g128_stage.h"

namespace q4g128 {

// Wave-uniform values computed with 64-bit arithmetic land in vector
// registers; these pin them to scalar registers (buffer descriptors and
// scalar offsets must be scalar).
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ long uni64(long v)
{
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((unsigned long)v >> 32));
    return (long)(((unsigned long)hi << 32) | lo);
}

__host__ __device__ inline int sk_b0(const SkShape &p, int s) { return (int)((long)s * p.nb / p.SK); }
__host__ __device__ inline int sk_nbs(const SkShape &p, int s) { return sk_b0(p, s + 1) - sk_b0(p, s); }
// Units of slice s and the waves that share them (never more waves than units).
__host__ __device__ inline long sk_units(const SkShape &p, int s) { return (long)p.T * sk_nbs(p, s); }
__host__ __device__ inline int sk_waves(const SkShape &p, long units)
{
    return (int)(units < (long)p.Wsl ? units : (long)p.Wsl);
}
// Wave v of Wv owns units [sk_start(v), sk_start(v + 1)); sk_owner inverts it.
__host__ __device__ inline long sk_start(long units, int Wv, int v) { return (long)v * units / Wv; }
__host__ __device__ inline int sk_owner(long units, int Wv, long u) { return (int)(((u + 1) * Wv - 1) / units); }

// Number of parts tile t is summed from, over all slices.
__device__ __forceinline__ int sk_nparts(const SkShape &p, int t)
{
    int n = 0;
    for (int s = 0; s < p.SK; ++s) {
        const int nbs = sk_nbs(p, s);
        const long U = sk_units(p, s);
        const int Wv = sk_waves(p, U);
        n += sk_owner(U, Wv, (long)(t + 1) * nbs - 1) - sk_owner(U, Wv, (long)t * nbs) + 1;
    }
    return n;
}

// A wave writes at most two parts: slot 0 for the tile its range starts in,
// slot 1 for the tile it ends in (when different).  Slot (wave v of slice s,
// which) holds 512 bytes at ((s * Wsl + v) * 2 + which) * 512 of the part
// area, laid out fp32 [column 0..15][row 0..7].

struct SkWave {
    // geometry
    int i, h, lane, M, N, G;
    uint32_t rowbytes;                 // K / 2
    __amdgpu_buffer_rsrc_t rw, rs, rm;
    int tw0;                           // first tile of this wave's range
    // ring: slot q holds the codes of group q of the next block
    u32x4 cb[8];
    u32x4 sm[2][2];                    // [set][scale, min]: 8 groups each
    float acc[4];

    // Lane offsets for tile t (columns past N read the last column).
    __device__ __forceinline__ uint32_t vcode(int t) const
    {
        return (uint32_t)min(i, N - 1 - 16 * t) * rowbytes + 16 * h;
    }
    __device__ __forceinline__ uint32_t vsm(int t) const { return (uint32_t)min(i, N - 1 - 16 * t) * (G * 2); }

    // Issue the loads of group q of block (t, g8) into ring slot q.
    __device__ __forceinline__ void fetch(int q, int t, int g8)
    {
        const uint32_t so = (uint32_t)(t - tw0) * 16 * rowbytes + (uint32_t)(g8 + q) * 64;
        cb[q] = __builtin_amdgcn_raw_buffer_load_b128(rw, vcode(t), so, 0);
    }
    __device__ __forceinline__ void fetch_sm(int set, int t, int g8)
    {
        const uint32_t so = (uint32_t)(t - tw0) * 16 * G * 2 + (uint32_t)g8 * 2;
        sm[set][0] = __builtin_amdgcn_raw_buffer_load_b128(rs, vsm(t), so, 0);
        sm[set][1] = __builtin_amdgcn_raw_buffer_load_b128(rm, vsm(t), so, 0);
    }
};

// One block of 8 groups: A fragments and row sums from LDS (group lg0 + q of
// the staged slice), codes from the ring (each slot refilled with the same
// group of block (tn, gn8) right after it is unpacked), scales and minimums
// from register set `set`.
__device__ __forceinline__ void sk_block(SkWave &w, const uint16_t *rbase, const int (&aoff)[4], const float *xrow,
                                         int lg0, int set, int tn, int gn8, UnpackConsts uc)
{
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int lg = lg0 + q;
        const uint16_t *gp = rbase + lg * 128;
        u32x4 a[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) a[t] = *reinterpret_cast<const u32x4 *>(gp + aoff[t]);
        const f32x4 xsum = *reinterpret_cast<const f32x4 *>(xrow + lg * kXsRows);
        u32x4 bq[4];
        bq[0] = unpack_biased(w.cb[q].x, uc);
        bq[1] = unpack_biased(w.cb[q].y, uc);
        bq[2] = unpack_biased(w.cb[q].z, uc);
        bq[3] = unpack_biased(w.cb[q].w, uc);
        const float s = bf16_at(w.sm[set][0], q);
        const float m = bf16_at(w.sm[set][1], q);
        w.fetch(q, tn, gn8);
        f32x4 d = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int t = 0; t < 4; ++t) d = mfma_16x16x32(a[t], bq[t], d);
        const float m_adj = fmaf(-kBias, s, m);          // mn - 128*s, one rounding
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            w.acc[r] = fmaf(s, d[r], w.acc[r]);
            w.acc[r] = fmaf(m_adj, xsum[r], w.acc[r]);
        }
    }
}

// Store the accumulators of tile t as y (rows < M, columns < N).
__device__ __forceinline__ void sk_store(const float (&v)[4], float *y, int M, int N, int t, int i, int h)
{
    const int n = 16 * t + i;
    if (h < 2 && n < N) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (4 * h + r < M) y[(size_t)(4 * h + r) * N + n] = v[r];
    }
}

// Cache-policy bit of a buffer access: device (agent) coherence.  Such
// stores and loads are coherent across the XCDs' separate L2 caches without
// the whole-L2 write-back and invalidate a device-scope fence costs.
constexpr int kAgentCoherent = 16;

// Store this wave's part of tile t, device-coherent (past this CU's caches).
__device__ __forceinline__ void sk_put_part(const SkShape &p, int s, int v, int which, const float (&acc)[4],
                                            __amdgpu_buffer_rsrc_t rparts, int i, int h)
{
    if (h < 2) {
        const f32x4 a = {acc[0], acc[1], acc[2], acc[3]};
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, a), rparts, (uint32_t)(i * 8 + 4 * h) * 4,
                                               (uint32_t)((s * p.Wsl + v) * 2 + which) * 512, kAgentCoherent);
    }
}

// Once the wave's part of tile t is complete in memory: count it; if it is the
// tile's last part to arrive, sum all parts in part order and write y, then
// reset the counter for the next call.
__device__ __forceinline__ void sk_settle(const SkShape &p, int t, __amdgpu_buffer_rsrc_t rparts, uint32_t *cnt,
                                          float *y, int M, int N, int i, int h, int lane)
{
    uint32_t old = 0;
    if (lane == 0) old = __hip_atomic_fetch_add(cnt + t, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    old = __builtin_amdgcn_readfirstlane(old);
    if ((int)old != uni(sk_nparts(p, t)) - 1) return;
    const uint32_t lane_off = (uint32_t)(i * 8 + 4 * (h & 1)) * 4;
    f32x4 sum = {0.0f, 0.0f, 0.0f, 0.0f};
    bool first = true;
    for (int s2 = 0; s2 < p.SK; ++s2) {
        const int nbs = sk_nbs(p, s2);
        const long U = sk_units(p, s2);
        const int Wv = sk_waves(p, U);
        const int vf = uni(sk_owner(U, Wv, (long)t * nbs)), vl = uni(sk_owner(U, Wv, (long)(t + 1) * nbs - 1));
        for (int v2 = vf; v2 <= vl; ++v2) {
            const int w2 = uni((t == (int)(sk_start(U, Wv, v2) / nbs)) ? 0 : 1);
            const f32x4 part = __builtin_bit_cast(
                f32x4, __builtin_amdgcn_raw_buffer_load_b128(rparts, lane_off, (uint32_t)((s2 * p.Wsl + v2) * 2 + w2) * 512,
                                                             kAgentCoherent));
            sum = first ? part : sum + part;
            first = false;
        }
    }
    const float out[4] = {sum[0], sum[1], sum[2], sum[3]};
    sk_store(out, y, M, N, t, i, h);
    if (lane == 0) __hip_atomic_store(cnt + t, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ __launch_bounds__(kSkThreads) void gemv_q4g128_streamk(
    const uint16_t *__restrict__ x, int M, int K, const uint32_t *__restrict__ W,
    const uint16_t *__restrict__ scale, const uint16_t *__restrict__ mn, int N, float *__restrict__ y,
    float *parts, uint32_t *cnt, SkShape P)
{
    extern __shared__ __attribute__((aligned(16))) uint16_t xs[];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wgs = P.Wsl / kSkWaves;                      // workgroups per slice
    const int s = uni(blockIdx.x / wgs);
    const int v = uni((blockIdx.x - s * wgs) * kSkWaves + wave);   // wave index within the slice
    const int b0 = uni(sk_b0(P, s)), nbs = uni(sk_nbs(P, s));
    const long U = uni64(sk_units(P, s));
    const int Wv = uni(sk_waves(P, U));
    if ((blockIdx.x - s * wgs) * kSkWaves >= Wv) return;   // whole workgroup idle
    const bool active = v < Wv;                            // wave-uniform

    SkWave w;
    w.lane = tid & 63;
    w.i = w.lane & 15;
    w.h = w.lane >> 4;
    w.M = M;
    w.N = N;
    w.G = K >> 7;
    w.rowbytes = (uint32_t)(K >> 1);
    const size_t K8 = (size_t)(K >> 3);
    int nu = 0, bb = 0;                                    // units in this wave's range; first block
    if (active) {
        const long ua = uni64(sk_start(U, Wv, v));
        nu = uni((int)(uni64(sk_start(U, Wv, v + 1)) - ua));
        w.tw0 = uni((int)(ua / nbs));
        bb = uni((int)(ua - (long)w.tw0 * nbs));
        const int twl = uni(w.tw0 + (bb + nu - 1) / nbs);
        const int c0 = 16 * w.tw0;
        const int ncols = uni(min(16 * (twl - w.tw0 + 1), N - c0));
        w.rw = make_rsrc(W + (size_t)c0 * K8, (uint32_t)((size_t)ncols * K8 * 4));
        w.rs = make_rsrc(scale + (size_t)c0 * w.G, (uint32_t)(ncols * w.G * 2));
        w.rm = make_rsrc(mn + (size_t)c0 * w.G, (uint32_t)(ncols * w.G * 2));
        // prime: the first block of the range
        const int g80 = (b0 + bb) * 8;
#pragma unroll
        for (int q = 0; q < 8; ++q) w.fetch(q, w.tw0, g80);
        w.fetch_sm(0, w.tw0, g80);
    }

    stage_x<kSkThreads, kSkStage>(xs, x, M, K, b0 * 8, (b0 + nbs) * 8);
    lds_barrier();
    if (!active) return;

    const UnpackConsts uc = unpack_consts();
    const int ng = nbs * 8;
    const int arow = min(w.i, M - 1);                      // rows >= M read a real row; never stored
    const uint16_t *rbase = xs + arow * ng * 128;
    const float *xrow = reinterpret_cast<const float *>(xs + M * ng * 128) + 4 * (w.h & 1);
    int aoff[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) aoff[t] = swz(4 * w.h + t, arow) * 8;
#pragma unroll
    for (int r = 0; r < 4; ++r) w.acc[r] = 0.0f;

    const __amdgpu_buffer_rsrc_t rparts = make_rsrc(parts, (uint32_t)(2 * kSkMaxWaves * 512));
    const bool whole = P.SK == 1;                          // a tile's blocks all in this slice
    int t = w.tw0;                                         // tile of the current block
    int left = nu;                                         // blocks of the range not yet done
    bool seg_whole = bb == 0;                              // open segment began at the tile's start
    for (;;) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            // next block of the range (the current one again if this is the last)
            int tn = t, bn = bb + 1;
            if (left == 1) bn = bb;
            else if (bn == nbs) { tn = t + 1; bn = 0; }
            const int gn8 = (b0 + bn) * 8;
            w.fetch_sm(half ^ 1, tn, gn8);
            sk_block(w, rbase, aoff, xrow, bb * 8, half, tn, gn8, uc);
            --left;
            ++bb;
            if (left == 0 || bb == nbs) {                  // segment of tile t ends
                if (whole && seg_whole && bb == nbs) {
                    sk_store(w.acc, y, M, N, t, w.i, w.h);
                } else {
                    sk_put_part(P, s, v, t == w.tw0 ? 0 : 1, w.acc, rparts, w.i, w.h);
                    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // part complete before it is counted
                    sk_settle(P, t, rparts, cnt, y, M, N, w.i, w.h, w.lane);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) w.acc[r] = 0.0f;
                if (left == 0) return;
                ++t;
                bb = 0;
                seg_whole = true;
            }
        }
    }
}

// ---- plan and launch ---------------------------------------------------------

bool streamk_plan(int K, int N, int ncu, SkShape *p)
{
    if (K % 1024 != 0 || N < 1 || ncu < kSkWaves) return false;
    int cus = 1;
    while (cus * 2 <= ncu && cus * 2 <= 256) cus *= 2;     // a power of two: slices share them evenly
    p->T = (N + 15) / 16;
    p->nb = K / 1024;
    p->SK = 1;
    while ((p->nb + p->SK - 1) / p->SK > kSkMaxBlocks) p->SK *= 2;
    if (p->SK > cus || p->SK > p->nb) return false;
    p->Wsl = cus / p->SK * kSkWaves;
    // Buffer offsets are 32-bit: the columns one wave touches must stay well
    // below 2 GiB of codes.
    const size_t per_wave = (size_t)N * (size_t)(K / 2) / (size_t)p->Wsl + (size_t)2 * 16 * (K / 2);
    return per_wave < ((size_t)1 << 31);
}

size_t streamk_lds_bytes(const SkShape &p, int M)
{
    const int nbmax = (p.nb + p.SK - 1) / p.SK;
    const size_t need = (size_t)M * nbmax * 1024 * 2 + (size_t)nbmax * 8 * kXsRows * 4;
    // More than half of the 160 KB LDS of a CU, so no two workgroups share one.
    const size_t own_cu = 80 * 1024 + 1024;
    return need > own_cu ? need : own_cu;
}

hipError_t launch_gemv_streamk(const GemvArgs &a, const SkShape &p, float *parts, uint32_t *cnt,
                               hipStream_t stream)
{
    static LdsRoom room;
    const hipError_t attr =
        lds_launch_ok(reinterpret_cast<const void *>(&gemv_q4g128_streamk), streamk_lds_bytes(p, a.M), room);
    if (attr != hipSuccess) return attr;
    dim3 grid((unsigned)(p.SK * (p.Wsl / kSkWaves)), 1, 1);
    hipLaunchKernelGGL(gemv_q4g128_streamk, grid, dim3(kSkThreads, 1, 1), streamk_lds_bytes(p, a.M), stream,
                       a.x, a.M, a.K, a.W, a.scale, a.mn, a.N, a.out, parts, cnt, p);
    return hipGetLastError();
}

}  // namespace q4g128
