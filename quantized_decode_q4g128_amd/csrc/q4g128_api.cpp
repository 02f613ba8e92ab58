// C ABI of libq4g128.so: argument checks, the (K, N) plan, kernel launches.
// Declarations and the contract of every entry point: include/q4g128.h.
#include "../../include/q4g128.h"

#include <hip/hip_runtime.h>
#include <stdio.h>
#include <string.h>

#include <atomic>

#include "q4g128_launch.h"

namespace {

thread_local char g_last_error[256] = "";

void set_error(const char *what, hipError_t e)
{
    snprintf(g_last_error, sizeof g_last_error, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Size limits keep every 32-bit offset inside the kernels (buffer offsets,
// grid dimensions) from overflowing.
constexpr int kMaxK = 1 << 24;
constexpr int kMaxN = 1 << 28;
constexpr int kMaxSplits = 65535;
// q4g128_gemm_rmsnorm's workspace starts with a control block (word 0: the
// one-launch form's arrival counter, zero between calls); its split-K
// partials follow.
constexpr size_t kNormCtlBytes = 256;

bool shape_ok(int M, int K, int N)
{
    return M >= 1 && M <= Q4G128_MAX_M && K > 0 && K <= kMaxK && K % Q4G128_GROUP == 0 && N > 0 &&
           N <= kMaxN;
}

bool operands_ok(const void *x, const uint32_t *W, const void *scale, const void *min, const float *y)
{
    return x && W && scale && min && y && aligned(x, 16) && aligned(W, 16) && aligned(scale, 2) &&
           aligned(min, 2) && aligned(y, 4);
}

// Up to one split per 128-group; splits of whole 8-group blocks (1024 k)
// while there are no more splits than blocks.
int max_splits(int K) { return K / Q4G128_GROUP; }

// Blocks of 8 groups (1024 k) along K: the default split count never
// exceeds it, so default splits are always whole blocks.
int k_blocks(int K) { return (K / Q4G128_GROUP + q4g128::kRing - 1) / q4g128::kRing; }

// Output tiles of 16 columns per wave.  One tile per wave for every shape.
int plan_tiles_per_wave(int /*K*/, int /*N*/) { return 1; }

// Waves the split-K planner aims for: 8 per compute unit on a 256-CU MI355X,
// enough loads in flight per CU to cover HBM latency.
constexpr long kTargetWaves = 2048;

// Compute units of the calling thread's current device, or -1.  Cached per
// device in atomics (every thread that fills an entry stores the same value,
// so relaxed ordering suffices).
int device_cus()
{
    static std::atomic<int> cache[q4g128::kMaxDevices];
    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return -1;
    const bool cached = dev >= 0 && dev < q4g128::kMaxDevices;
    if (cached) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
    if (cached && ncu > 0) cache[dev].store(ncu, std::memory_order_relaxed);
    return ncu;
}

// Clears an error an earlier, unrelated HIP call may have left pending on
// this thread, so that the launches of this call report their own.
void clear_pending_error() { (void)hipGetLastError(); }

// Balanced plan for gemv_q4g128_bal (one K split): workgroups (at most one
// per CU) and K parts per tile, or gx = 0 when the shape needs the per-tile
// kernel (K not a multiple of 1024, unaligned scale/min, x or LDS too large,
// huge y).
struct BalChoice {
    int gx;
    int P;
    int rb;         // P > 1: rows one launch can hold (1..kBalRowBlock); P == 1: M
};

// K-part shapes stage x for at most this many rows per launch: 9, a draft
// of 8 tokens plus the next one, fits at K <= 5120.
constexpr int kBalRowBlock = 9;

// Workgroups for N columns (ACT: N/2 pairs) shared out in units of 4.
int bal_gx(int N, bool act, int ncu)
{
    const int units = act ? (N / 2 + 3) / 4 : (N + 3) / 4;
    return ncu < units ? ncu : units;
}

// Tiles of at most 16 columns a workgroup gets when N is shared out in units of 4.
int bal_tiles(int N, int gx)
{
    const int N4 = (N + 3) / 4;
    return ((N4 + gx - 1) / gx * 4 + 15) / 16;
}

// K parts per tile, cut at the 8-group blocks: 1 when a workgroup has enough
// tiles for its waves (the many-tile shapes stream whole columns); else the
// count whose busiest wave has the fewest blocks to stream, units (tile,
// part) dealt to the waves in turn, and of those the one that keeps the
// fewest waves busy.  Measured against the alternatives at M = 1 (one box,
// interleaved): 5120 -> 12288 (3 tiles per CU) 3 parts 9.45 us against 10.28
// whole-K on the register-ring kernel, 10.21 in 2 parts, 10.41 in 4, 10.03 in
// 5; 5120 -> 8192 (2 tiles) 5 parts 0.80 of whole-K, 4 parts 0.89; 5120 ->
// 16384 (4 tiles) 3 parts 0.90, 2 parts 0.97; 5120 -> 20480 and 5120 -> 24576
// 2 parts 0.96 and 0.98; 17408 -> 5120 and 6144 -> 5120 (two whole tiles on
// 160 workgroups) 6 parts, 3-5 parts 8-14% slower.  The sums of a tile do not
// depend on M, so rows stay bit-identical across M; the price is in rows a
// launch cannot hold: q4g128_gemm then runs row blocks of up to 9 rows, each
// streaming the weights again (5120 -> 12288 at M = 10-16: 20.9-22.1 us
// against 13.0-15.8 us whole-K with x in chunks; M = 7 10.8 against 11.6, M = 9
// 11.7 against 12.2).
int bal_parts(int K, int N, int gx)
{
    using namespace q4g128;
    const int tiles = bal_tiles(N, gx);
    if (tiles >= kBalMinTiles) return 1;
    const int nb = K / 1024;
    int best = 1, bestc = 1 << 30, bestw = 1 << 30;
    for (int P = 1; P <= nb && P <= kBalWaves; ++P) {
        const int units = tiles * P;
        const int w = units < kBalWaves ? units : kBalWaves;
        int crit = 0;
        for (int v = 0; v < w; ++v) {
            int load = 0;
            for (int u = v; u < units; u += kBalWaves) {
                const int p = u % P;
                load += ((p + 1) * nb) / P - (p * nb) / P;
            }
            crit = load > crit ? load : crit;
        }
        if (crit < bestc || (crit == bestc && w < bestw)) {
            best = P;
            bestc = crit;
            bestw = w;
        }
    }
    return best;
}

struct BalGrid {
    int gx;
    int P;
};

BalGrid plain_grid(int K, int N, int ncu)
{
    using namespace q4g128;
    BalGrid g = {bal_gx(N, false, ncu), 1};
    if (bal_tiles(N, g.gx) >= kBalMinTiles) return g;
    if (N % 16 == 0 && N % (16 * g.gx) != 0) {
        const int n16 = N / 16;
        const int per = (n16 + ncu - 1) / ncu;                 // whole tiles per workgroup
        const int gw = (n16 + per - 1) / per;
        if (gw < g.gx) {
            g.gx = gw;
            g.P = bal_parts(K, N, gw);
            return g;
        }
    }
    g.P = bal_parts(K, N, g.gx);
    return g;
}

// Whether x for M rows over all of K fits the balanced kernel's staging and LDS.
bool bal_fits(int M, int K, int N, int gx, int P, bool act)
{
    using namespace q4g128;
    const int ng = K / 128;
    if ((long)M * ng * 16 > (long)kBalThreads * kBalStage) return false;       // x staging registers
    const int part = P > 1 ? (ng / 8 + P - 1) / P * 8 : ng;                     // longest part, groups
    if (16 * ((part + 7) / 8) > 64 * kBalSmRounds) return false;                 // scale/min pieces per lane
    return bal_plan(M, K, N, 1, gx, P, act).lds <= kBalMaxLds;
}

// With P > 1 the balanced kernel's sums are those of the per-tile kernel with
// P K splits and the split-order reduce (same block boundaries, same order),
// so a shape can take either path for any M: one balanced launch when it
// holds all M rows, else P splits.  With P == 1 both kernels compute every
// column the same way, so the choice may depend on M freely.
BalChoice plan_bal(int M, int K, int N, const void *scale, const void *min, bool act = false)
{
    BalChoice no = {0, 1, 0};
    if (K % 1024 != 0 || !aligned(scale, 16) || !aligned(min, 16)) return no;
    if ((long)M * N * 4 >= (1L << 31)) return no;
    // ACT tiles address gate and up columns N/2 apart through one descriptor.
    if (act && ((long)N / 2 + 8) * (K / 2) >= (1L << 31)) return no;
    const int ncu = device_cus();
    if (ncu < 1) return no;
    const BalGrid pg = plain_grid(K, N, ncu);
    const int gx = act ? bal_gx(N, true, ncu) : pg.gx;
    const int P = pg.P;                                        // the plain product's parts, also for ACT
    if (P == 1) {
        // Rows beyond what x staged whole allows: chunked x (M <= 16).
        if (!bal_fits(M, K, N, gx, 1, act) && !(M > 8 && q4g128::lds_plan_xch(M, K, N, gx, act).fits)) return no;
        BalChoice c = {gx, 1, M};
        return c;
    }
    int rb = 0;
    while (rb < kBalRowBlock && bal_fits(rb + 1, K, N, gx, P, act)) ++rb;
    if (rb == 0) return no;
    BalChoice c = {gx, P, rb};
    return c;
}

// Which balanced kernel runs a planned launch.  All give the same bits.
// Workgroups of many whole tiles (8 or more, K not cut: gate/up, the output
// projection, their SwiGLU and verify forms) take the LDS-fed kernel with a
// ring of 2 group pairs per wave, each wave's first tile requested before x
// is staged (burst): gate/up 18.33 -> 17.76 us against x first, M = 7 20.0
// -> 19.2 us, SwiGLU 18.34 -> 17.82 us (one box, interleaved); against the
// register-ring kernel 19.7-20.6 us.  K-part shapes take it in burst form
// too (17408 -> 5120 in 6 parts: 13.4 against 14.7 us; 6144 -> 5120: even),
// with SwiGLU x first.  Deeper rings (4 pairs) were slower on every shape.
// Few whole tiles per CU without parts (7 tiles per CU, or K = 1024, which
// has no block to cut at) stay on the register-ring kernel.  A shape whose
// LDS does not fit the burst form takes x first, then the register-ring
// kernel.
#ifndef Q4G128_LDS_MODE
#define Q4G128_LDS_MODE -1
#endif
int balanced_mode(int N, bool act, int gx, int P)
{
    const int tiles = act ? (((N / 2 + 3) / 4 + gx - 1) / gx * 4 + 7) / 8 : bal_tiles(N, gx);
    return P > 1 ? (act ? 1 : 2) : tiles >= q4g128::kBalMinTiles ? 2 : 0;
}

// The LDS-fed form a balanced launch of M rows takes: rd > 0 the ring depth
// (burst: the first tile requested before x; nr: ring slots and burst areas
// for the tile waves only, plus one spare the waves without a tile share),
// rd == 0 the register-ring kernel.
struct LdsForm {
    int rd;
    bool burst;
    bool nr;
};

LdsForm lds_form(int M, int K, int N, int gx, int P, bool act)
{
    using namespace q4g128;
    int mode = Q4G128_LDS_MODE;                 // 0: register ring; 1-4: LDS-fed (rd 2/2/4/4, burst on 2 and 4)
    if (mode < 0) mode = balanced_mode(N, act, gx, P);
    if (mode > 0) {
        const int rd = mode >= 3 ? 4 : 2;
        const bool burst = mode == 2 || mode == 4;
        if (lds_plan(M, K, N, gx, P, act, rd, burst).fits) return LdsForm{rd, burst, false};
        // Rows whose x leaves the burst form too little LDS with a slot and an
        // area for every wave (gate/up at M = 8, 9): the burst form with the
        // spare slot, 21.38 -> 20.46 us at M = 8 against x first, M = 9 21.77
        // -> 21.01 us against x in chunks (one box, interleaved).
        if (burst && P == 1 && M >= 5 && lds_plan(M, K, N, gx, P, act, 2, true, true).fits)
            return LdsForm{2, true, true};
        if (burst && lds_plan(M, K, N, gx, P, act, 2, false).fits) return LdsForm{2, false, false};
    }
    return LdsForm{0, false, false};
}

hipError_t launch_balanced(const q4g128::GemvArgs &a, int gx, int P, hipStream_t stream)
{
    using namespace q4g128;
    const LdsForm f = lds_form(a.M, a.K, a.N, gx, P, a.act != nullptr);
    if (f.rd > 0) return launch_gemv_lds(a, gx, P, f.rd, f.burst, f.nr, stream);
    const int mode = Q4G128_LDS_MODE < 0 ? balanced_mode(a.N, a.act != nullptr, gx, P) : Q4G128_LDS_MODE;
    // More rows than fit x whole (verify M = 9..16): chunked x, where the
    // LDS-fed kernel is the faster one or the register-ring kernel cannot
    // stage the rows.
    if (a.M > 8 && P == 1 && (mode > 0 || !bal_fits(a.M, a.K, a.N, gx, 1, a.act != nullptr)) &&
        lds_plan_xch(a.M, a.K, a.N, gx, a.act != nullptr).fits)
        return launch_gemv_xch(a, gx, stream);
    return launch_gemv_bal(a, gx, P, stream);
}

q4g128::GemvArgs gemv_args(const void *x, int M, int K, const uint32_t *W, const void *scale, const void *min, int N,
                           float *out, int S)
{
    q4g128::GemvArgs a;
    a.x = static_cast<const uint16_t *>(x);
    a.M = M;
    a.K = K;
    a.W = W;
    a.scale = static_cast<const uint16_t *>(scale);
    a.mn = static_cast<const uint16_t *>(min);
    a.N = N;
    a.out = out;
    a.S = S;
    return a;
}

// S == 1: y[M][N] in `out`, by the balanced kernel (K-part shapes in launches
// of at most rb rows) or the per-tile kernel.  S > 1: the per-tile kernel's
// S partial slices [S][M][N] in `out`.
q4g128_status run_gemv(const void *x, int M, int K, const uint32_t *W, const void *scale,
                       const void *min, int N, float *out, int S, hipStream_t stream)
{
    clear_pending_error();
    q4g128::GemvArgs a = gemv_args(x, M, K, W, scale, min, N, out, S);
    const BalChoice bc = S == 1 ? plan_bal(M, K, N, scale, min) : BalChoice{0, 1, 0};
    hipError_t e = hipSuccess;
    if (bc.gx > 0) {
        const int rows = bc.P > 1 ? bc.rb : M;
        for (int r0 = 0; r0 < M && e == hipSuccess; r0 += rows) {        // y rows are contiguous
            a.x = static_cast<const uint16_t *>(x) + (size_t)r0 * K;
            a.M = M - r0 < rows ? M - r0 : rows;
            a.out = out + (size_t)r0 * N;
            e = launch_balanced(a, bc.gx, bc.P, stream);
        }
    } else {
        e = q4g128::launch_gemv(a, plan_tiles_per_wave(K, N), stream);
    }
    if (e != hipSuccess) {
        set_error("gemv launch", e);
        return Q4G128_EHIP;
    }
    return Q4G128_OK;
}

// The product with K cut into S ranges of whole 8-group blocks.  When S is
// the shape's K-part count and one LDS-fed balanced launch holds all M rows,
// that launch writes the summed result to `dst` as a single slice; otherwise
// the per-tile kernel writes S partial slices to `ws`.  *slices tells which
// (1: in dst; S: in ws).  Both give the same bits after the split-order sum.
// Where the rows fit only the register-ring kernel (17408 -> 5120 at M = 2)
// the partial slices and their sum are the faster way: 13.71 against 14.39
// us; where the LDS-fed kernel holds them the one launch is (5120 -> 12288 at
// M = 2, 4, 8: 9.75 / 10.01 / 11.61 against 11.28 / 11.74 / 13.44 us; 8192
// -> 777 at M = 2: 7.01 against 8.13).
q4g128_status run_split(const void *x, int M, int K, const uint32_t *W, const void *scale, const void *min,
                        int N, int S, float *ws, float *dst, int *slices, hipStream_t stream)
{
    clear_pending_error();
    if (S == 1) {
        *slices = 1;
        return run_gemv(x, M, K, W, scale, min, N, dst, 1, stream);
    }
    const BalChoice bc = plan_bal(M, K, N, scale, min);
    if (bc.gx > 0 && bc.P == S && M <= bc.rb && lds_form(M, K, N, bc.gx, bc.P, false).rd > 0) {
        *slices = 1;
        q4g128::GemvArgs a = gemv_args(x, M, K, W, scale, min, N, dst, 1);
        hipError_t e = launch_balanced(a, bc.gx, bc.P, stream);
        if (e != hipSuccess) {
            set_error("gemv launch", e);
            return Q4G128_EHIP;
        }
        return Q4G128_OK;
    }
    *slices = S;
    return run_gemv(x, M, K, W, scale, min, N, ws, S, stream);
}

// The fused gate/up product with bf16 silu(gate) * up written to act: one
// launch of the balanced kernel when the shape allows it, else the product's
// partial sums into the workspace and sum_swiglu over them.  The per-column
// sums are the plain product's in both cases, so both give the same bits.
// K parts of the fused gate/up plan (1 if it has none or the shape takes the
// per-tile kernel): the split count its fallback must use.
int swiglu_parts(int K, int N)
{
    const int ncu = device_cus();
    if (K % 1024 != 0 || ncu < 1) return 1;
    const int P = plain_grid(K, N, ncu).P;
    return P > 1 && bal_fits(1, K, N, bal_gx(N, true, ncu), P, true) ? P : 1;
}

q4g128_status run_swiglu(const void *x, int M, int K, const uint32_t *W, const void *scale, const void *min,
                         int N, uint16_t *act, float *ws, hipStream_t stream)
{
    clear_pending_error();
    const BalChoice bc = plan_bal(M, K, N, scale, min, true);
    if (bc.gx > 0 && (bc.P == 1 || M <= bc.rb)) {
        q4g128::GemvArgs a = gemv_args(x, M, K, W, scale, min, N, nullptr, 1);
        a.act = act;
        hipError_t e = launch_balanced(a, bc.gx, bc.P, stream);
        if (e != hipSuccess) {
            set_error("gemv+swiglu launch", e);
            return Q4G128_EHIP;
        }
        return Q4G128_OK;
    }
    // A K-part shape too wide for one launch runs as exactly P K splits (the
    // same bits as its one-launch form); any other shape as the default split.
    const int S = bc.gx > 0 && bc.P > 1 ? bc.P : q4g128_splitk_default_splits(K, N);
    int slices = 0;
    q4g128_status rc = run_split(x, M, K, W, scale, min, N, S, ws, ws, &slices, stream);
    if (rc != Q4G128_OK) return rc;
    hipError_t e = q4g128::launch_sum_swiglu(ws, slices, M, N, act, stream);
    if (e != hipSuccess) {
        set_error("swiglu launch", e);
        return Q4G128_EHIP;
    }
    return Q4G128_OK;
}

// Stream-K workspace: partial-sum slots first, then one counter per tile.
constexpr size_t kSkPartBytes = (size_t)2 * q4g128::kSkMaxWaves * 128 * sizeof(float);

size_t streamk_ws_bytes(int N)
{
    const size_t tiles = ((size_t)N + 15) / 16;
    return (kSkPartBytes + tiles * 4 + 255) / 256 * 256;
}

// Split-K partial sums into `workspace` (validated, large enough), then their
// sum in ascending split order into y; one launch when the balanced kernel's
// K parts are these splits.
q4g128_status run_splitk(const void *x, int M, int K, const uint32_t *W, const void *scale, const void *min, int N,
                         float *y, int splits, float *workspace, hipStream_t st)
{
    int slices = 0;
    q4g128_status rc = run_split(x, M, K, W, scale, min, N, splits, workspace, y, &slices, st);
    if (rc != Q4G128_OK || slices == 1) return rc;               // one launch wrote y
    hipError_t e = q4g128::launch_splitk_sum(workspace, splits, (size_t)M * (size_t)N, y, st);
    if (e != hipSuccess) {
        set_error("split-K sum launch", e);
        return Q4G128_EHIP;
    }
    return Q4G128_OK;
}

}  // namespace

extern "C" {

int q4g128_abi_version(void) { return Q4G128_ABI_VERSION; }

const char *q4g128_status_string(q4g128_status s)
{
    switch (s) {
    case Q4G128_OK: return "ok";
    case Q4G128_EINVAL: return "invalid argument";
    case Q4G128_EWORKSPACE: return "workspace too small";
    case Q4G128_EHIP: return "HIP error";
    }
    return "unknown status";
}

const char *q4g128_last_error(void) { return g_last_error; }

size_t q4g128_splitk_workspace_bytes(int M, int N, int splits)
{
    if (M < 1 || M > Q4G128_MAX_M || N < 1 || splits < 1) return 0;
    return (size_t)splits * (size_t)M * (size_t)N * sizeof(float);
}

int q4g128_splitk_default_splits(int K, int N)
{
    if (K <= 0 || K % Q4G128_GROUP != 0 || N <= 0 || K > kMaxK || N > kMaxN) return 0;
    // Where the balanced kernels take the shape in one launch for one row:
    // no splits when it does not cut K (wider M falls back to the per-tile
    // kernel, which then has enough tiles); when it cuts K into parts, that
    // many splits, so that the split-K call runs the one LDS-fed launch for
    // the rows it holds (the 17408 -> 5120 down projection: 6 parts, one row)
    // and the per-tile kernel with the same splits and a reduce beyond, which
    // streams the weights once for any M (same bits either way).
    const int ncu = device_cus();
    if (K % 1024 == 0 && ncu > 0) {
        const BalGrid g = plain_grid(K, N, ncu);
        if (bal_fits(1, K, N, g.gx, g.P, false)) return g.P;
    }
    const long nb = k_blocks(K);
    const long tpw = plan_tiles_per_wave(K, N);
    const long waves = ((long)N + 16 * tpw - 1) / (16 * tpw);
    if (waves >= kTargetWaves) return 1;
    // Enough waves to fill the machine, then the fewest splits that keep the
    // widest split as short as the most even division allows.
    long s = (kTargetWaves + waves - 1) / waves;
    if (s > nb) s = nb;
    const long widest = (nb + s - 1) / s;
    while (s > 1 && (nb + s - 2) / (s - 1) == widest) --s;
    return (int)s;
}

int q4g128_gemm_parts(int K, int N)
{
    if (K <= 0 || K % Q4G128_GROUP != 0 || N <= 0 || K > kMaxK || N > kMaxN) return 0;
    const int ncu = device_cus();
    if (K % 1024 != 0 || ncu < 1) return 1;
    const BalGrid g = plain_grid(K, N, ncu);
    return g.P > 1 && bal_fits(1, K, N, g.gx, g.P, false) ? g.P : 1;
}

q4g128_status q4g128_gemm(const void *x, int M, int K, const uint32_t *W, const void *scale,
                          const void *min, int N, float *y, void *stream)
{
    if (!shape_ok(M, K, N) || !operands_ok(x, W, scale, min, y)) return Q4G128_EINVAL;
    return run_gemv(x, M, K, W, scale, min, N, y, 1, static_cast<hipStream_t>(stream));
}

q4g128_status q4g128_gemm_splitk(const void *x, int M, int K, const uint32_t *W, const void *scale,
                                 const void *min, int N, float *y, int splits, float *workspace,
                                 size_t workspace_bytes, void *stream)
{
    if (!shape_ok(M, K, N) || !operands_ok(x, W, scale, min, y)) return Q4G128_EINVAL;
    if (splits < 1 || splits > max_splits(K) || splits > kMaxSplits) return Q4G128_EINVAL;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (splits == 1) return run_gemv(x, M, K, W, scale, min, N, y, 1, st);
    if (!workspace || !aligned(workspace, 4)) return Q4G128_EINVAL;
    if (workspace_bytes < q4g128_splitk_workspace_bytes(M, N, splits)) return Q4G128_EWORKSPACE;
    return run_splitk(x, M, K, W, scale, min, N, y, splits, workspace, st);
}

q4g128_status q4g128_gemm_splitk_noalloc(const void *x, int M, int K, const uint32_t *W, const void *scale,
                                         const void *min, int N, float *y, int splits, void *stream)
{
    if (!shape_ok(M, K, N) || !operands_ok(x, W, scale, min, y)) return Q4G128_EINVAL;
    if (splits < 1 || splits > max_splits(K) || splits > kMaxSplits) return Q4G128_EINVAL;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (splits == 1) return run_gemv(x, M, K, W, scale, min, N, y, 1, st);
    if (q4g128_splitk_workspace_bytes(M, N, splits) > q4g128::kScratchBytes) {
        snprintf(g_last_error, sizeof g_last_error,
                 "q4g128_gemm_splitk_noalloc: splits*M*N*4 = %zu bytes exceeds the library scratch of %zu bytes",
                 q4g128_splitk_workspace_bytes(M, N, splits), q4g128::kScratchBytes);
        return Q4G128_EWORKSPACE;
    }
    float *ws = nullptr;
    const hipError_t e = q4g128::scratch_pointer(&ws);
    if (e != hipSuccess) {
        set_error("scratch address lookup", e);
        return Q4G128_EHIP;
    }
    return run_splitk(x, M, K, W, scale, min, N, y, splits, ws, st);
}

size_t q4g128_streamk_workspace_bytes(int K, int N)
{
    if (K <= 0 || K % 1024 != 0 || K > kMaxK || N < 1 || N > kMaxN) return 0;
    return streamk_ws_bytes(N);
}

q4g128_status q4g128_gemm_streamk(const void *x, int M, int K, const uint32_t *W, const void *scale,
                                  const void *min, int N, float *y, void *workspace, size_t workspace_bytes,
                                  void *stream)
{
    if (!shape_ok(M, K, N) || !operands_ok(x, W, scale, min, y)) return Q4G128_EINVAL;
    if (M > q4g128::kSkMaxM) return Q4G128_EINVAL;
    if (K % 1024 != 0 || !aligned(scale, 16) || !aligned(min, 16)) return Q4G128_EINVAL;
    if (!workspace || !aligned(workspace, 256)) return Q4G128_EINVAL;
    if (workspace_bytes < streamk_ws_bytes(N)) return Q4G128_EWORKSPACE;
    const int ncu = device_cus();
    if (ncu < 0) {
        set_error("device query", hipGetLastError());
        return Q4G128_EHIP;
    }
    q4g128::SkShape plan;
    if (!q4g128::streamk_plan(K, N, ncu, &plan)) return Q4G128_EINVAL;
    q4g128::GemvArgs a;
    a.x = static_cast<const uint16_t *>(x);
    a.M = M;
    a.K = K;
    a.W = W;
    a.scale = static_cast<const uint16_t *>(scale);
    a.mn = static_cast<const uint16_t *>(min);
    a.N = N;
    a.out = y;
    a.S = 1;
    float *parts = static_cast<float *>(workspace);
    uint32_t *cnt = reinterpret_cast<uint32_t *>(static_cast<char *>(workspace) + kSkPartBytes);
    clear_pending_error();
    hipError_t e = q4g128::launch_gemv_streamk(a, plan, parts, cnt, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) {
        set_error("stream-K launch", e);
        return Q4G128_EHIP;
    }
    return Q4G128_OK;
}

q4g128_status q4g128_dequant(const uint32_t *W, const void *scale, const void *min, int K, int N,
                             float *w_out, void *stream)
{
    if (!shape_ok(1, K, N) || !W || !scale || !min || !w_out) return Q4G128_EINVAL;
    if (!aligned(W, 16) || !aligned(scale, 2) || !aligned(min, 2) || !aligned(w_out, 16))
        return Q4G128_EINVAL;
    clear_pending_error();
    hipError_t e = q4g128::launch_dequant(W, static_cast<const uint16_t *>(scale),
                                          static_cast<const uint16_t *>(min), K, N, w_out,
                                          static_cast<hipStream_t>(stream));
    if (e != hipSuccess) {
        set_error("dequant launch", e);
        return Q4G128_EHIP;
    }
    return Q4G128_OK;
}

q4g128_status q4g128_quantize(const void *w, int K, int N, int ncand, uint32_t *W, void *scale, void *min,
                              double *err, void *stream)
{
    if (!shape_ok(1, K, N) || !w || !W || !scale || !min || ncand < 1 || ncand > Q4G128_QUANT_MAX_CAND)
        return Q4G128_EINVAL;
    if (!aligned(w, 16) || !aligned(W, 16) || !aligned(scale, 2) || !aligned(min, 2) || (err && !aligned(err, 8)))
        return Q4G128_EINVAL;
    const long ngroups = (long)N * (K / Q4G128_GROUP);
    const int gpw = q4g128::quantize_groups_per_block(ncand);
    if ((ngroups + gpw - 1) / gpw > 0x7FFFFFFFL) return Q4G128_EINVAL;
    clear_pending_error();
    hipError_t e = q4g128::launch_quantize(static_cast<const uint16_t *>(w), ngroups, ncand, W,
                                           static_cast<uint16_t *>(scale), static_cast<uint16_t *>(min), err,
                                           static_cast<hipStream_t>(stream));
    if (e != hipSuccess) {
        set_error("quantize launch", e);
        return Q4G128_EHIP;
    }
    return Q4G128_OK;
}

size_t q4g128_swiglu_workspace_bytes(int M, int K, int N)
{
    if (M < 1 || M > Q4G128_MAX_M || N < 2 || N % 2) return 0;
    int S = q4g128_splitk_default_splits(K, N);
    const int P = swiglu_parts(K, N);
    if (P > S) S = P;
    if (S < 1) return 0;
    return (size_t)S * (size_t)M * (size_t)N * sizeof(float);
}

q4g128_status q4g128_gemm_swiglu(const void *x, int M, int K, const uint32_t *W, const void *scale, const void *min,
                                 int N, void *act, float *workspace, size_t workspace_bytes, void *stream)
{
    if (!shape_ok(M, K, N) || N % 2 || !act || !aligned(act, 2)) return Q4G128_EINVAL;
    if (!x || !W || !scale || !min || !aligned(x, 16) || !aligned(W, 16) || !aligned(scale, 2) || !aligned(min, 2))
        return Q4G128_EINVAL;
    if (!workspace || !aligned(workspace, 4)) return Q4G128_EINVAL;
    if (workspace_bytes < q4g128_swiglu_workspace_bytes(M, K, N)) return Q4G128_EWORKSPACE;
    return run_swiglu(x, M, K, W, scale, min, N, static_cast<uint16_t *>(act), workspace,
                      static_cast<hipStream_t>(stream));
}

size_t q4g128_rmsnorm_workspace_bytes(int M, int N, int splits)
{
    const size_t b = q4g128_splitk_workspace_bytes(M, N, splits);
    return b ? b + kNormCtlBytes : 0;
}

q4g128_status q4g128_gemm_rmsnorm(const void *x, int M, int K, const uint32_t *W, const void *scale, const void *min,
                                  int N, const float *residual, const void *gamma, float eps, float *h, void *x_out,
                                  int splits, float *workspace, size_t workspace_bytes, void *stream)
{
    if (!shape_ok(M, K, N) || !operands_ok(x, W, scale, min, h)) return Q4G128_EINVAL;
    if (!residual || !aligned(residual, 4)) return Q4G128_EINVAL;
    const bool norm = x_out != nullptr;          // else the residual add alone
    if (norm && (!gamma || !aligned(gamma, 2) || !aligned(x_out, 2))) return Q4G128_EINVAL;
    if (norm && (!(eps >= 0.0f) || eps > 3.0e38f)) return Q4G128_EINVAL;
    if (splits < 1 || splits > max_splits(K) || splits > kMaxSplits) return Q4G128_EINVAL;
    if (!workspace || !aligned(workspace, 4)) return Q4G128_EINVAL;
    if (workspace_bytes < q4g128_rmsnorm_workspace_bytes(M, N, splits)) return Q4G128_EWORKSPACE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    clear_pending_error();
    // One launch when the splits are the balanced kernel's K parts and the
    // rows fit it: each workgroup adds the residual to its own columns (and
    // with the norm, the last one to finish normalises the rows).  Same bits
    // as below.
    if (splits > 1) {
        const int epi = norm ? 2 : 1;
        const BalChoice bc = plan_bal(M, K, N, scale, min);
        if (bc.gx > 0 && bc.P == splits && M <= bc.rb && q4g128::lds_epi_fits(M, K, N, bc.gx, bc.P, epi)) {
            const q4g128::GemvArgs a = gemv_args(x, M, K, W, scale, min, N, h, 1);
            const q4g128::NormArgs na = {residual, static_cast<const uint16_t *>(gamma), eps,
                                         static_cast<uint16_t *>(x_out), reinterpret_cast<uint32_t *>(workspace)};
            const hipError_t e = q4g128::launch_gemv_lds_epi(a, bc.gx, bc.P, epi, na, st);
            if (e != hipSuccess) {
                set_error(norm ? "gemv+rmsnorm launch" : "gemv+residual launch", e);
                return Q4G128_EHIP;
            }
            return Q4G128_OK;
        }
    }
    float *ws = workspace + kNormCtlBytes / sizeof(float);   // the control block stays untouched
    int slices = 0;
    q4g128_status rc = run_split(x, M, K, W, scale, min, N, splits, ws, ws, &slices, st);
    if (rc != Q4G128_OK) return rc;
    hipError_t e = q4g128::launch_sum_residual_rmsnorm(ws, slices, M, N, residual,
                                                       static_cast<const uint16_t *>(gamma), eps, h,
                                                       static_cast<uint16_t *>(x_out), st);
    if (e != hipSuccess) {
        set_error(norm ? "rmsnorm launch" : "residual launch", e);
        return Q4G128_EHIP;
    }
    return Q4G128_OK;
}

size_t q4g128_prenorm_workspace_bytes(int M, int K, int N, int swiglu)
{
    if (M < 1 || M > Q4G128_MAX_M || K <= 0 || K % Q4G128_GROUP != 0 || K > kMaxK || N < 1 || N > kMaxN) return 0;
    if (swiglu && (N < 2 || N % 2)) return 0;
    const size_t xb = ((size_t)M * (size_t)K * 2 + 255) / 256 * 256;
    return xb + (swiglu ? q4g128_swiglu_workspace_bytes(M, K, N) : 0);
}

// Rows up to which the product of a normalised input runs in one launch: from
// 7 rows a norm launch and the product on its x are the faster pair (gate/up
// + SwiGLU at M = 5 / 7 / 8: 23.23 / 24.28 / 25.14 us in one launch, 23.64 /
// 24.10 / 24.37 in two; plain gate/up M = 8 25.10 against 24.11, q/k/v M = 7
// 15.11 against 14.94; one box, interleaved): every workgroup of the one
// launch reads all M rows of fp32 h, twice x's bytes, before its norm.
constexpr int kXnMaxRows = 6;

// The product of x = RMSNorm(h) * gamma: in one launch when the shape's
// balanced plan takes the normalising staging (whole rows, M <= kXnMaxRows,
// operands 16-byte aligned), else x into the workspace and the product on
// it.  The same bits either way, and those of the product called on that x.
q4g128_status run_prenorm(const float *h, const void *gamma, float eps, int M, int K, const uint32_t *W,
                          const void *scale, const void *min, int N, float *y, uint16_t *act, float *workspace,
                          hipStream_t st)
{
    clear_pending_error();
    const bool sw = act != nullptr;
    const BalChoice bc = plan_bal(M, K, N, scale, min, sw);
    if (bc.gx > 0 && M <= kXnMaxRows && (bc.P == 1 || M <= bc.rb) && aligned(h, 16) && aligned(gamma, 16)) {
        const int mode = balanced_mode(N, sw, bc.gx, bc.P);
        bool lds = mode > 0;
        if (!q4g128::xn_fits(M, K, N, bc.gx, bc.P, sw, lds)) lds = !lds;
        if (q4g128::xn_fits(M, K, N, bc.gx, bc.P, sw, lds)) {
            q4g128::GemvArgs a = gemv_args(h, M, K, W, scale, min, N, y, 1);
            a.act = act;
            const q4g128::NormArgs na = {nullptr, static_cast<const uint16_t *>(gamma), eps, nullptr, nullptr};
            const hipError_t e = q4g128::launch_gemv_xn(a, bc.gx, bc.P, lds, na, st);
            if (e != hipSuccess) {
                set_error("rmsnorm+gemv launch", e);
                return Q4G128_EHIP;
            }
            return Q4G128_OK;
        }
    }
    uint16_t *xb = reinterpret_cast<uint16_t *>(workspace);
    hipError_t e = q4g128::launch_rmsnorm(h, M, K, static_cast<const uint16_t *>(gamma), eps, xb, st);
    if (e != hipSuccess) {
        set_error("rmsnorm launch", e);
        return Q4G128_EHIP;
    }
    float *rest = workspace + ((size_t)M * (size_t)K * 2 + 255) / 256 * 64;
    return sw ? run_swiglu(xb, M, K, W, scale, min, N, act, rest, st) : run_gemv(xb, M, K, W, scale, min, N, y, 1, st);
}

q4g128_status q4g128_gemm_prenorm(const float *h, const void *gamma, float eps, int M, int K, const uint32_t *W,
                                  const void *scale, const void *min, int N, float *y, float *workspace,
                                  size_t workspace_bytes, void *stream)
{
    if (!shape_ok(M, K, N) || !h || !gamma || !aligned(h, 4) || !aligned(gamma, 2)) return Q4G128_EINVAL;
    if (!W || !scale || !min || !y || !aligned(W, 16) || !aligned(scale, 2) || !aligned(min, 2) || !aligned(y, 4))
        return Q4G128_EINVAL;
    if (!(eps >= 0.0f) || eps > 3.0e38f) return Q4G128_EINVAL;
    if (!workspace || !aligned(workspace, 256)) return Q4G128_EINVAL;
    if (workspace_bytes < q4g128_prenorm_workspace_bytes(M, K, N, 0)) return Q4G128_EWORKSPACE;
    return run_prenorm(h, gamma, eps, M, K, W, scale, min, N, y, nullptr, workspace, static_cast<hipStream_t>(stream));
}

q4g128_status q4g128_gemm_swiglu_prenorm(const float *h, const void *gamma, float eps, int M, int K,
                                         const uint32_t *W, const void *scale, const void *min, int N, void *act,
                                         float *workspace, size_t workspace_bytes, void *stream)
{
    if (!shape_ok(M, K, N) || N % 2 || !h || !gamma || !aligned(h, 4) || !aligned(gamma, 2)) return Q4G128_EINVAL;
    if (!W || !scale || !min || !act || !aligned(W, 16) || !aligned(scale, 2) || !aligned(min, 2) || !aligned(act, 2))
        return Q4G128_EINVAL;
    if (!(eps >= 0.0f) || eps > 3.0e38f) return Q4G128_EINVAL;
    if (!workspace || !aligned(workspace, 256)) return Q4G128_EINVAL;
    if (workspace_bytes < q4g128_prenorm_workspace_bytes(M, K, N, 1)) return Q4G128_EWORKSPACE;
    return run_prenorm(h, gamma, eps, M, K, W, scale, min, N, nullptr, static_cast<uint16_t *>(act), workspace,
                       static_cast<hipStream_t>(stream));
}

}  // extern "C"
