// Internal interface between the C ABI (q4g128_api.cpp) and the kernels
// (q4g128_kernels.hip).  Arguments reaching these launchers are validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

namespace q4g128 {

#ifndef Q4G128_WAVES_SMALL
#define Q4G128_WAVES_SMALL 2
#endif
#ifndef Q4G128_WAVES_LARGE
#define Q4G128_WAVES_LARGE 4
#endif
#ifndef Q4G128_SMALL_M
#define Q4G128_SMALL_M 2
#endif
#ifndef Q4G128_RING
#define Q4G128_RING 4
#endif
#ifndef Q4G128_STAGE
#define Q4G128_STAGE 16
#endif

// Dynamic LDS above 64 KiB has to be allowed per kernel and per device.
// Each call site keeps, per device, the room its kernel's own static LDS
// leaves of the CU's 160 KiB (0: not yet known), with the kernel's dynamic
// limit raised to that room the first time.  A launch asking for more than
// the room is refused here with hipErrorInvalidValue: the runtime does not
// check static plus dynamic LDS against the CU and would dispatch it, and
// the dispatch then fails as an invalid allocation that aborts the queue.
constexpr int kMaxDevices = 64;
constexpr int kCuLds = 160 * 1024;
typedef std::atomic<int> LdsRoom[kMaxDevices];

inline hipError_t lds_launch_ok(const void *kernel, size_t dyn, LdsRoom &room)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const bool cached = dev >= 0 && dev < kMaxDevices;
    int r = cached ? room[dev].load(std::memory_order_relaxed) : 0;
    if (r <= 0) {
        hipFuncAttributes fa;
        e = hipFuncGetAttributes(&fa, kernel);
        if (e != hipSuccess) return e;
        r = kCuLds - (int)fa.sharedSizeBytes;
        if (r <= 0) return hipErrorInvalidValue;
        e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, r);
        if (e != hipSuccess) return e;
        if (cached) room[dev].store(r, std::memory_order_relaxed);
    }
    return dyn <= (size_t)r ? hipSuccess : hipErrorInvalidValue;
}

constexpr int kMaxM = 16;                  // rows of one MFMA tile
constexpr int kSkMaxM = 8;                 // the stream-K kernel keeps 8 rows
// Waves per workgroup (they share one LDS copy of x): few for small M, where
// x is small and finer workgroups spread more evenly over the CUs; more for
// large M, whose x would not fit in LDS once per small workgroup.
constexpr int kWavesSmall = Q4G128_WAVES_SMALL;
constexpr int kWavesLarge = Q4G128_WAVES_LARGE;
constexpr int kSmallM = Q4G128_SMALL_M;
constexpr int kRing = 8;                   // K splits align to blocks of 8 groups (1024 k)
constexpr int kRingDepth = Q4G128_RING;    // groups of codes in flight per wave (4, 8 or 16)
constexpr int kStageMax = Q4G128_STAGE;    // 16-byte x pieces staged per thread per chunk
#ifndef Q4G128_TILE_PAIR
#define Q4G128_TILE_PAIR 1
#endif
constexpr bool kTilePair = Q4G128_TILE_PAIR; // per-tile kernel: codes two groups at a time where ranges are whole blocks

struct GemvArgs {
    const uint16_t *x;       // bf16 [M][K]
    int M, K;
    const uint32_t *W;       // [N][K/8]
    const uint16_t *scale;   // bf16 [N][K/128]
    const uint16_t *mn;      // bf16 [N][K/128]
    int N;
    float *out;              // S == 1: y [M][N]; S > 1: partials [S][M][N]
    int S;                   // K splits, 1..K/128: for S <= nb = ceil(K/1024) split s
                             // covers 8-group blocks [s*nb/S, (s+1)*nb/S), else
                             // groups [s*G/S, (s+1)*G/S), G = K/128
    uint16_t *act = nullptr; // balanced kernel only: if set, N = 2I is a fused gate/up
                             // product and bf16 silu(gate) * up [M][I] is written
                             // here instead of y (out unused)
};

// x chunk (in 128-groups, a multiple of kRing) staged in LDS for M rows.
int chunk_groups(int M);

// ---- balanced kernel: one workgroup per CU --------------------------------------
#ifndef Q4G128_BAL_WAVES
#define Q4G128_BAL_WAVES 12
#endif
#ifndef Q4G128_BAL_RING
#define Q4G128_BAL_RING 4
#endif
constexpr int kBalWaves = Q4G128_BAL_WAVES; // waves per workgroup; each takes one tile at a time
constexpr int kBalRing = Q4G128_BAL_RING;   // groups of codes in flight per wave
#ifndef Q4G128_BAL_SML
#define Q4G128_BAL_SML 1
#endif
constexpr bool kBalSml = Q4G128_BAL_SML;    // scales/minimums staged in LDS per tile (else loaded per block)
#ifndef Q4G128_BAL_PAIR
#define Q4G128_BAL_PAIR 1
#endif
constexpr bool kBalPair = Q4G128_BAL_PAIR;  // codes loaded two groups (128 B per column) at a time
// ... for workgroups of at least this many (tile, K part) units.  K = 5120,
// tiles per CU (us, paired / one group per load): 3: 11.31 / 10.35;
// 4: 11.70 / 11.80; 5: 13.73 / 14.30; 6: 14.45 / 16.28; 7: 15.56 / 18.35;
// 8.5 (gate/up) and the 131072-wide output projection: 1-13% faster paired.
#ifndef Q4G128_PAIR_UNITS
#define Q4G128_PAIR_UNITS 4
#endif
constexpr int kBalPairUnits = Q4G128_PAIR_UNITS;
#ifndef Q4G128_PAIR_CPOL
#define Q4G128_PAIR_CPOL 2
#endif
// Cache policy of the paired code loads: 2 = nt (non-temporal: the lines are
// read once per call; held in the caches, they only displace other data).
constexpr int kPairCpol = Q4G128_PAIR_CPOL;
#ifndef Q4G128_BAL_ONEROW
#define Q4G128_BAL_ONEROW 1
#endif
constexpr bool kBalOneRow = Q4G128_BAL_ONEROW;   // M <= 4: accumulate only the one D row per lane that is stored
#ifndef Q4G128_ROWPERM
#define Q4G128_ROWPERM 1
#endif
constexpr bool kRowPerm = Q4G128_ROWPERM;   // x row m in MFMA row rowpos(m) (product kernels)
constexpr int kBalThreads = 64 * kBalWaves;
constexpr int kBalStage = 8;                // x pieces per thread: M * ng * 16 <= 6144 (M = 8 at K = 6144, 9 at 5120)
constexpr int kBalSmRounds = 2;             // scale/min pieces per lane: 16 * nblk <= 128, nblk <= 8
constexpr size_t kBalOwnCu = 80 * 1024 + 1024;   // LDS request that keeps two workgroups off one CU
constexpr int kBalMinTiles = 8;             // fewer tiles per workgroup: cut each tile's K into parts
constexpr size_t kBalMaxLds = 160 * 1024;

// Launch geometry of the balanced kernel for M rows, S K splits, gx
// workgroups per split and P K parts per tile (P > 1 only with S == 1).
struct BalPlan {
    size_t lds;     // dynamic LDS bytes (at least kBalOwnCu: one workgroup per CU)
    int nblp;       // 8-group blocks per column row of a wave's scale/min area (odd)
    int nps;        // part-sum slots (P > 1)
    bool pair;      // codes loaded two groups at a time (workgroups of at least kBalPairUnits units)
};
BalPlan bal_plan(int M, int K, int N, int S, int gx, int P, bool act = false);
// y (S == 1) or partials [S][M][N] (S > 1) with gx workgroups per split.
// Requires K % 1024 == 0, 16-byte aligned scale/min, and the plan checks of
// plan_bal (x and LDS fit).
hipError_t launch_gemv_bal(const GemvArgs &a, int gx, int P, hipStream_t stream);

// ---- LDS-fed balanced kernel ------------------------------------------------------
// The balanced kernel's work split and arithmetic (same bits) with codes and
// scales/minimums brought into LDS by direct-to-LDS loads: a ring of rd (2 or
// 4) group pairs per wave; `burst` requests the first unit's weights before x.
// Needs S == 1, K % 1024 == 0, 16-byte aligned scale/min, and lds_plan().fits;
// built variants: rd 2 (plain or fused SwiGLU), burst with rd 2 or 4 (plain).
// nr (burst, rd 2, K not cut, at most 9 tiles, M = 5-16): ring slots and
// burst areas for the tile waves only, plus one spare the others share.
struct LdsPlan {
    size_t lds;     // dynamic LDS bytes
    size_t total;   // dynamic + the static LDS (rings; burst: scale/minimum areas)
    int nblm;       // most 8-group blocks of one unit
    int nps;        // part-sum slots (P > 1)
    bool fits;      // total <= 160 KiB, and (burst) units of at most 4 blocks
    int xcg = 0;    // chunked x (lds_plan_xch): groups per chunk
};
LdsPlan lds_plan(int M, int K, int N, int gx, int P, bool act, int rd, bool burst, bool nr = false);
hipError_t launch_gemv_lds(const GemvArgs &a, int gx, int P, int rd, bool burst, bool nr, hipStream_t stream);

// Chunked x on the LDS-fed kernel (ring 2, no burst, K not cut): for rows
// whose x does not fit the LDS whole, when every tile is one wave's and at
// least one wave has none (those load the chunks).  M <= 16.
LdsPlan lds_plan_xch(int M, int K, int N, int gx, bool act);
hipError_t launch_gemv_xch(const GemvArgs &a, int gx, hipStream_t stream);

// RMSNorm around the balanced kernels.
//
// Epilogue (K-part launch of the LDS-fed kernel, ring 2, burst): every
// workgroup stores its columns of h = r + y to a.out (h; may be r itself);
// epi 2: the workgroup that finishes last also computes x_out = bf16(h /
// sqrt(mean(h^2) + eps) * gamma) for whole rows.  cnt: a word of the
// caller's workspace that holds zero, counted up by every workgroup and left
// at zero again.  lds_epi_fits: the shape takes it (K parts, M <= 8, epi 2:
// one row of h and its group sums fitting the dynamic LDS).
//
// Prologue (xn): x = bf16(h / sqrt(mean(h^2) + eps) * gamma) made from fp32
// rows h (a.x points to h) while staging, then the product as usual: the LDS-
// fed kernel without burst (lds) or the register-ring kernel; M <= 8, S == 1.
// xn_fits: the plan (gx, P, kernel) takes it.
struct NormArgs {
    const float *r;
    const uint16_t *gamma;
    float eps;
    uint16_t *xo;
    uint32_t *cnt;
};
bool lds_epi_fits(int M, int K, int N, int gx, int P, int epi);
hipError_t launch_gemv_lds_epi(const GemvArgs &a, int gx, int P, int epi, const NormArgs &na, hipStream_t stream);
bool xn_fits(int M, int K, int N, int gx, int P, bool act, bool lds);
hipError_t launch_gemv_xn(const GemvArgs &a, int gx, int P, bool lds, const NormArgs &na, hipStream_t stream);

// ---- work-balanced (stream-K) kernel ----------------------------------------
constexpr int kSkWaves = 8;                 // waves per workgroup, one workgroup per CU
constexpr int kSkThreads = 64 * kSkWaves;
constexpr int kSkMaxBlocks = 9;             // blocks of 1024 k per K slice: 8 rows of x fit LDS
constexpr int kSkStage = 8 * kSkMaxBlocks * 8 * 16 / kSkThreads;   // x pieces per thread
constexpr int kSkMaxWaves = 256 * kSkWaves; // waves of the largest launch (256 CUs)

// Partition of the units (tile of 16 columns, block of 8 groups): K is cut
// into SK slices of whole blocks; each slice's units are split evenly over
// Wsl waves.
struct SkShape {
    int T;      // tiles, ceil(N / 16)
    int nb;     // blocks per column, K / 1024
    int SK;     // K slices
    int Wsl;    // waves per slice
};

// Plan for (K, N) on a device with `ncu` compute units; false if the shape
// is not supported (K not a multiple of 1024, too many slices, offsets).
bool streamk_plan(int K, int N, int ncu, SkShape *p);
size_t streamk_lds_bytes(const SkShape &p, int M);
// parts: 2 * kSkMaxWaves slots of 512 bytes; cnt: T zero-filled counters.
hipError_t launch_gemv_streamk(const GemvArgs &a, const SkShape &p, float *parts, uint32_t *cnt,
                               hipStream_t stream);

// Waves per workgroup and output columns per workgroup for M rows.
int waves_for(int M);
int columns_per_block(int tpw, int M);

hipError_t launch_gemv(const GemvArgs &a, int tpw, hipStream_t stream);

// Library-owned scratch for callers that cannot allocate: a file-scope
// device array of kScratchBytes on every GPU the library runs on (each GPU
// holds its own copy until the process ends).  scratch_pointer() returns
// this device's copy's address, looked up once per device; host code uses
// that address, never the array's name (a host-side stand-in).
constexpr size_t kScratchBytes = (size_t)8 << 20;
hipError_t scratch_pointer(float **p);
hipError_t launch_splitk_sum(const float *P, int S, size_t MN, float *y, hipStream_t stream);
hipError_t launch_dequant(const uint32_t *W, const uint16_t *scale, const uint16_t *mn, int K, int N,
                          float *w, hipStream_t stream);

// Epilogues over partial sums P [S][M][N] (summed in ascending s first):
// act [M][N/2] = bf16(silu(gate) * up) of the gate/up halves; and
// h = r + y, x_out = bf16(h / sqrt(mean(h^2) + eps) * gamma) per row (h may be
// r; xo == nullptr: h only).  launch_rmsnorm: x_out of given rows h alone.
hipError_t launch_sum_swiglu(const float *P, int S, int M, int N, uint16_t *act, hipStream_t stream);
hipError_t launch_sum_residual_rmsnorm(const float *P, int S, int M, int N, const float *r, const uint16_t *gamma,
                                       float eps, float *h, uint16_t *xo, hipStream_t stream);
hipError_t launch_rmsnorm(const float *h, int M, int N, const uint16_t *gamma, float eps, uint16_t *xo,
                          hipStream_t stream);

// Quantizer (q4g128_quant.hip): groups staged per workgroup for `ncand`, and
// the launch over `ngroups` consecutive 128-weight groups of w.
int quantize_groups_per_block(int ncand);
hipError_t launch_quantize(const uint16_t *w, long ngroups, int ncand, uint32_t *W, uint16_t *S, uint16_t *Mn,
                           double *err, hipStream_t stream);

}  // namespace q4g128
