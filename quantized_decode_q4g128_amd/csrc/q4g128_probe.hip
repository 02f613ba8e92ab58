// Read-bandwidth probes for the benchmark (not part of the product's C ABI;
// built into libq4g128_probe.so, which only bench.py loads).
//
// They read a code matrix W [N][K/8] uint32 and nothing else, so their
// rates are what HBM delivers for a given access pattern on this GPU:
//
//   probe_tile_read    the product's pattern and work split: one
//                      12-wave workgroup per compute unit owning an equal
//                      share of the rows (cut in units of 4, workgroups
//                      numbered XCD by XCD), tiles of 16 consecutive rows,
//                      one tile per wave at a time; per step each run of 8
//                      lanes reads 128 contiguous bytes (two 128-weight
//                      groups) of one row, 8 rows per wave instruction, two
//                      instructions per step, 2 steps (4 groups) in flight
//                      per wave;
//   probe_linear_read  the same bytes read contiguously: each wave owns an
//                      equal span of the buffer and reads 1 KB per step
//                      (16 bytes per lane); 8 steps in flight per wave.
//
// Both carry the non-temporal hint, as the product's code loads do: every
// line is read once.
//
// Every load is in bounds (indices are clamped, never left to the buffer
// descriptor); the loaded words are folded into one word per lane and
// written to a sink so that no load is dropped.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}

constexpr int kTileRing = 2;                    // steps of two groups
constexpr int kLinRing = 8;
constexpr int kNt = 2;                          // cache policy: non-temporal

constexpr int kTileWaves = 12;
constexpr int kOwnCuLds = 81 * 1024;

__global__ __launch_bounds__(64 * kTileWaves) void probe_tile_read(const uint32_t *__restrict__ W, int K, int N,
                                                                   uint32_t *__restrict__ sink)
{
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int gx = gridDim.x;
    const int c = (gx % 8 == 0) ? (int)(blockIdx.x % 8) * (gx / 8) + (int)(blockIdx.x / 8) : (int)blockIdx.x;
    const int N4 = (N + 3) >> 2;
    const int n0 = (int)((long)c * N4 / gx) * 4;
    const int n1 = min((int)((long)(c + 1) * N4 / gx) * 4, N);
    const int ntile = (n1 - n0 + 15) >> 4;
    const int G = K / 128;
    const uint32_t rowb = (uint32_t)(K / 2);         // bytes per row
    const __amdgpu_buffer_rsrc_t r = rsrc(W, (uint32_t)((size_t)N * rowb));
    uint32_t acc = 0;
    const int G2 = G >> 1;                         // steps of two groups (K % 256 == 0)
    for (int t = wave; t < ntile; t += kTileWaves) {
        const int rowa = min(n0 + 16 * t + (lane >> 3), n1 - 1);
        const int rowb8 = min(n0 + 16 * t + 8 + (lane >> 3), n1 - 1);
        const uint32_t ba = (uint32_t)rowa * rowb + 16 * (lane & 7);
        const uint32_t bb = (uint32_t)rowb8 * rowb + 16 * (lane & 7);
        u32x4 ra[kTileRing], rb[kTileRing];
#pragma unroll
        for (int u = 0; u < kTileRing; ++u) {
            ra[u] = __builtin_amdgcn_raw_buffer_load_b128(r, ba + 128 * (uint32_t)min(u, G2 - 1), 0, kNt);
            rb[u] = __builtin_amdgcn_raw_buffer_load_b128(r, bb + 128 * (uint32_t)min(u, G2 - 1), 0, kNt);
        }
        for (int g = 0; g < G2; g += kTileRing) {
#pragma unroll
            for (int u = 0; u < kTileRing; ++u) {
                acc ^= ra[u].x ^ ra[u].y ^ ra[u].z ^ ra[u].w ^ rb[u].x ^ rb[u].y ^ rb[u].z ^ rb[u].w;
                const int gn = min(g + u + kTileRing, G2 - 1);
                ra[u] = __builtin_amdgcn_raw_buffer_load_b128(r, ba + 128 * (uint32_t)gn, 0, kNt);
                rb[u] = __builtin_amdgcn_raw_buffer_load_b128(r, bb + 128 * (uint32_t)gn, 0, kNt);
            }
        }
#pragma unroll
        for (int u = 0; u < kTileRing; ++u)
            acc ^= ra[u].x ^ ra[u].y ^ ra[u].z ^ ra[u].w ^ rb[u].x ^ rb[u].y ^ rb[u].z ^ rb[u].w;
    }
    sink[((size_t)blockIdx.x * kTileWaves + wave) * 64 + lane] = acc;
}

int compute_units()
{
    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return -1;
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
    return ncu;
}

__global__ __launch_bounds__(256) void probe_linear_read(const uint32_t *__restrict__ W, size_t bytes, int waves,
                                                         uint32_t *__restrict__ sink)
{
    const int lane = threadIdx.x & 63;
    const int wave = (int)((blockIdx.x * blockDim.x + threadIdx.x) >> 6);
    if (wave >= waves) return;
    const size_t chunks = bytes / 1024;              // whole 1 KB steps
    const size_t c0 = chunks * wave / waves, c1 = chunks * (wave + 1) / waves;
    const int steps = (int)(c1 - c0);
    if (steps <= 0) return;
    const __amdgpu_buffer_rsrc_t r = rsrc(W, (uint32_t)bytes);
    const uint32_t base = (uint32_t)(c0 * 1024) + 16 * lane;
    uint32_t acc = 0;
    u32x4 ring[kLinRing];
#pragma unroll
    for (int u = 0; u < kLinRing; ++u)
        ring[u] = __builtin_amdgcn_raw_buffer_load_b128(r, base + 1024 * (uint32_t)min(u, steps - 1), 0, kNt);
    for (int k = 0; k < steps; k += kLinRing) {
#pragma unroll
        for (int u = 0; u < kLinRing; ++u) {
            acc ^= ring[u].x ^ ring[u].y ^ ring[u].z ^ ring[u].w;
            const int kn = min(k + u + kLinRing, steps - 1);
            ring[u] = __builtin_amdgcn_raw_buffer_load_b128(r, base + 1024 * (uint32_t)kn, 0, kNt);
        }
    }
#pragma unroll
    for (int u = 0; u < kLinRing; ++u) acc ^= ring[u].x ^ ring[u].y ^ ring[u].z ^ ring[u].w;
    sink[(size_t)wave * 64 + lane] = acc;
}

}  // namespace

extern "C" {

// Sink words the probes write: 64 per wave (the tile probe: 12 waves on
// each of at most 1024 compute units).
size_t q4g128_probe_sink_words(int K, int N, int linear_waves)
{
    (void)K;
    (void)N;
    const size_t w = (size_t)1024 * kTileWaves > (size_t)linear_waves ? (size_t)1024 * kTileWaves
                                                                        : (size_t)linear_waves;
    return w * 64;
}

// One launch of the tile-pattern probe over W [N][K/8] (K % 256 == 0,
// N * K / 2 < 2^32 bytes, W 16-byte aligned).  Returns a hipError_t.
int q4g128_probe_tile_read(const uint32_t *W, int K, int N, uint32_t *sink, void *stream)
{
    if (!W || !sink || K <= 0 || K % 256 || N <= 0 || (size_t)N * (size_t)(K / 2) >= (1ull << 32))
        return (int)hipErrorInvalidValue;
    const int ncu = compute_units();
    if (ncu < 1 || ncu > 1024) return (int)hipErrorInvalidDevice;
    const int N4 = (N + 3) / 4;
    const int gx = ncu < N4 ? ncu : N4;
    // The product's LDS request (over half the CU's 160 KB) keeps two
    // workgroups off one CU; the probe asks for the same.
    static bool done[64];                        // per device: the attribute is set once on each
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return (int)hipErrorInvalidDevice;
    if (!done[dev]) {
        const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(&probe_tile_read),
                                                    hipFuncAttributeMaxDynamicSharedMemorySize, kOwnCuLds);
        if (attr != hipSuccess) return (int)attr;
        done[dev] = true;
    }
    hipLaunchKernelGGL(probe_tile_read, dim3((unsigned)gx), dim3(64 * kTileWaves), kOwnCuLds,
                       static_cast<hipStream_t>(stream), W, K, N, sink);
    return (int)hipGetLastError();
}

// One launch of the contiguous probe over the same bytes with `waves` waves.
int q4g128_probe_linear_read(const uint32_t *W, int K, int N, int waves, uint32_t *sink, void *stream)
{
    const size_t bytes = (size_t)N * (size_t)(K / 2);
    if (!W || !sink || K <= 0 || K % 128 || N <= 0 || waves <= 0 || bytes >= (1ull << 32) || bytes < 1024)
        return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(probe_linear_read, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), W, bytes, waves, sink);
    return (int)hipGetLastError();
}

}  // extern "C"
