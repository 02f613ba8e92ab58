// Read-bandwidth probes for the benchmark (not part of the product's C ABI;
// built into libq4g128_probe.so, which only bench.py loads).
//
// They read a code matrix W [N][K/8] uint32 and nothing else, so their
// rates are what HBM delivers for a given access pattern on this GPU:
//
//   probe_tile_read    the product's pattern: one wave per tile of 16
//                      consecutive rows n; per step each lane quad reads 64
//                      contiguous bytes (one 128-weight group) of one row,
//                      16 rows per wave instruction; 4 groups in flight per
//                      wave; 4 waves per workgroup;
//   probe_linear_read  the same bytes read contiguously: each wave owns an
//                      equal span of the buffer and reads 1 KB per step
//                      (16 bytes per lane); 8 steps in flight per wave.
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

constexpr int kTileRing = 4;
constexpr int kLinRing = 8;

__global__ __launch_bounds__(256) void probe_tile_read(const uint32_t *__restrict__ W, int K, int N,
                                                       uint32_t *__restrict__ sink)
{
    const int lane = threadIdx.x & 63;
    const int wave = (int)((blockIdx.x * blockDim.x + threadIdx.x) >> 6);
    const int tiles = (N + 15) / 16;
    if (wave >= tiles) return;                       // wave-uniform
    const int G = K / 128;
    const uint32_t rowb = (uint32_t)(K / 2);         // bytes per row
    const int row = min(wave * 16 + (lane >> 2), N - 1);
    const __amdgpu_buffer_rsrc_t r = rsrc(W, (uint32_t)((size_t)N * rowb));
    const uint32_t base = (uint32_t)row * rowb + 16 * (lane & 3);
    uint32_t acc = 0;
    u32x4 ring[kTileRing];
#pragma unroll
    for (int u = 0; u < kTileRing; ++u)
        ring[u] = __builtin_amdgcn_raw_buffer_load_b128(r, base + 64 * (uint32_t)min(u, G - 1), 0, 0);
    for (int g = 0; g < G; g += kTileRing) {
#pragma unroll
        for (int u = 0; u < kTileRing; ++u) {
            acc ^= ring[u].x ^ ring[u].y ^ ring[u].z ^ ring[u].w;
            const int gn = min(g + u + kTileRing, G - 1);
            ring[u] = __builtin_amdgcn_raw_buffer_load_b128(r, base + 64 * (uint32_t)gn, 0, 0);
        }
    }
#pragma unroll
    for (int u = 0; u < kTileRing; ++u) acc ^= ring[u].x ^ ring[u].y ^ ring[u].z ^ ring[u].w;
    sink[(size_t)wave * 64 + lane] = acc;
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
        ring[u] = __builtin_amdgcn_raw_buffer_load_b128(r, base + 1024 * (uint32_t)min(u, steps - 1), 0, 0);
    for (int k = 0; k < steps; k += kLinRing) {
#pragma unroll
        for (int u = 0; u < kLinRing; ++u) {
            acc ^= ring[u].x ^ ring[u].y ^ ring[u].z ^ ring[u].w;
            const int kn = min(k + u + kLinRing, steps - 1);
            ring[u] = __builtin_amdgcn_raw_buffer_load_b128(r, base + 1024 * (uint32_t)kn, 0, 0);
        }
    }
#pragma unroll
    for (int u = 0; u < kLinRing; ++u) acc ^= ring[u].x ^ ring[u].y ^ ring[u].z ^ ring[u].w;
    sink[(size_t)wave * 64 + lane] = acc;
}

}  // namespace

extern "C" {

// Sink words the probes write: 64 per wave.
size_t q4g128_probe_sink_words(int K, int N, int linear_waves)
{
    const size_t tiles = ((size_t)N + 15) / 16;
    const size_t w = tiles > (size_t)linear_waves ? tiles : (size_t)linear_waves;
    return w * 64;
}

// One launch of the tile-pattern probe over W [N][K/8] (K % 128 == 0,
// N * K / 2 < 2^32 bytes, W 16-byte aligned).  Returns a hipError_t.
int q4g128_probe_tile_read(const uint32_t *W, int K, int N, uint32_t *sink, void *stream)
{
    if (!W || !sink || K <= 0 || K % 128 || N <= 0 || (size_t)N * (size_t)(K / 2) >= (1ull << 32))
        return (int)hipErrorInvalidValue;
    const int tiles = (N + 15) / 16;
    hipLaunchKernelGGL(probe_tile_read, dim3((unsigned)((tiles + 3) / 4)), dim3(256), 0,
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
