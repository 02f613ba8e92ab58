// HIP kernels for the int4-g128 weight-streaming product on gfx950.
//
//   y[m][n] = sum_k x[m][k] * (q[n][k] * s[n][k/128] + mn[n][k/128])
//
// Decode streams every weight byte once per step (Token Rush README,
// bandwidth paragraph); an M-row verify step does the same with M activation
// rows (steps table rows 13-14, 28).  One kernel serves every M in 1..16
// (the MFMA's 16 rows).
//
// Per 128-group the sum is factored as
//   sum_k x*(q*s + mn) = s * sum_k x*(128 + q) + (mn - 128*s) * sum_k x
// The codes enter a bf16 MFMA as the exact bf16 values 128 + q (a mask and an
// OR per pair, no conversion); the x rows are the A operand (A rows >= M
// repeat a real row and are never stored); the group row sums sum_k x are
// formed once per workgroup while x is staged (dot2 with ones, then a fixed
// 16-lane tree).  Every output element is its own dot product inside the
// MFMA, and the schedule of instructions depends on (K, N) only, so row m of
// an M-row call is bit-identical to the one-row call (bw24 article,
// exactness paragraph).
//
// Work layout: a workgroup of WAVES waves (2 for M <= 2, 4 above) owns
// 16*WAVES*TPW output columns and one contiguous range of 128-groups (the K
// split).  Each wave owns TPW tiles of 16 columns.  Lane (i = l%16, h = l/16)
// feeds column i's 16-byte code piece h of every group (words
// 16g+4h .. 16g+4h+3) to the MFMA; the loads themselves are issued with each
// run of four neighbouring lanes reading one column's 64 contiguous bytes, and
// a lane permute moves every piece to its MFMA lane.  The workgroup stages x
// for up to CG groups at a time in LDS (all of its K range unless M*K is
// large), reordered into the pair order of the codes; lanes whose A row is
// >= M read a real row, and their D rows are never stored.  The main loop
// has no branches that depend on data: groups past the end of a range are
// processed with scale and minimum forced to zero.  Which wave or workgroup
// owns a column never changes the instructions that compute it, so the
// choice of WAVES by M keeps rows bit-identical across M.
#include <algorithm>

#include "q4g128_device.h"
#include "q4g128_launch.h"
#include "q4g128_stage.h"

namespace q4g128 {

// One wave's share: TPW tiles of 16 columns, the groups [gs, ge) of one K
// split.  x for the groups [cs, ce) being processed is in LDS (see swz),
// followed by the x row sums of those groups, Xs[g - cs][row] (fp32).
//
// Loads: the codes of a group come from a ring of RING slots (slot = group
// index mod RING, refilled RING groups ahead).  With VSM the scales and
// minimums of 8 groups arrive in one 16-byte load per array; blocks of 8
// groups alternate between two register sets (the loop body covers two
// blocks, so the roles are static).  Without VSM, each group's scale and
// minimum ride in the code ring, and a range may end inside a block: the
// groups past its end are processed with scale and minimum zero (exact zeros)
// on a copy of its last group's x.
//
// PAIR (TPW = 1, VSM, no PAD; ranges of whole 8-group blocks at even group
// offsets): the codes of two consecutive groups, 128 contiguous bytes of each
// column, arrive in two loads, columns 0-7 and 8-15 of the tile: lane l reads
// column l/8 (+8) at bytes 16*(l%8) (columns 0-7) or 16*((l%8)^4) (columns
// 8-15, halves mirrored).  Every load then covers whole 128-byte lines, which
// lets them carry the non-temporal hint (the weights are read once per
// call); a load covering half lines with the hint reads slower than without
// it.  A ring slot holds one pair; the MFMA pieces of the pair's first and
// second group come out of the two loads by a per-lane select and one lane
// permute each, so every MFMA sees the same operands as with one group per
// load.
// RL: D rows per lane that are accumulated, ceil(M/4) (x rows 0..3 sit in
// the first D row of each lane, rows 4..7 in the second, ..., see rowpos).
// A row's instructions do not depend on RL, so its bits do not either.
// CP: cache policy of the one-group-per-load code loads (the paired ones
// always carry the non-temporal hint).
template <int TPW, bool VSM, int RING, bool SML = false, bool PAD = false, bool PAIR = false, int RL = 4,
          int CP = 0>
struct Tile {
    // PAD (with VSM): the range may end inside an 8-group block; groups past
    // its end are processed with scale and minimum zero, as without VSM.
    static constexpr bool kClamp = !VSM || PAD;
    static_assert(!PAIR || (TPW == 1 && VSM && !PAD && RING % 2 == 0), "paired loads: one tile, whole blocks");
    int i, h, M, K, G, gs, ge;
    int src;                                      // lane holding this lane's code piece (one group per load)
    int src_e, src_o;                             // PAIR: lanes holding the first / second group's piece
    uint32_t vw2;                                 // PAIR: lane offset of the columns 8-15 load
    u32x4 cb2[RING];                              // PAIR: columns 8-15 of pair slot q (cb[q][0]: columns 0-7)
    // SML: scales and minimums of the wave's tile sit in LDS ([scale, min]
    // [column][block of 8 groups from smg0], nbl blocks per column row).
    const uint16_t *sml;
    int nbl, smg0;
    size_t K8;
    __amdgpu_buffer_rsrc_t rw, rs, rm;
    uint32_t vw[TPW], vs[TPW];
    u32x4 cb[RING][TPW];
    uint32_t sb[RING][TPW], mb[RING][TPW];       // !VSM
    u32x4 sm[2][2][TPW];                          // VSM: [block set][scale, min][tile]
    float acc[TPW][4];

    __device__ __forceinline__ void fetch(int q, int g)
    {
        if (PAIR) {                               // pair slot q: groups g, g + 1 (g even)
            cb[q][0] = __builtin_amdgcn_raw_buffer_load_b128(rw, vw[0], 64 * g, kPairCpol);
            cb2[q] = __builtin_amdgcn_raw_buffer_load_b128(rw, vw2, 64 * g, kPairCpol);
            return;
        }
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
            cb[q][u] = __builtin_amdgcn_raw_buffer_load_b128(rw, vw[u], 64 * g, CP);
            if (!VSM) {
                sb[q][u] = __builtin_amdgcn_raw_buffer_load_b16(rs, vs[u], 2 * g, 0);
                mb[q][u] = __builtin_amdgcn_raw_buffer_load_b16(rm, vs[u], 2 * g, 0);
            }
        }
    }

    __device__ __forceinline__ void fetch_sm(int set, int g8)
    {
        if (SML) {
            const int b = (g8 - smg0) >> 3;
            sm[set][0][0] = *reinterpret_cast<const u32x4 *>(sml + (i * nbl + b) * 8);
            sm[set][1][0] = *reinterpret_cast<const u32x4 *>(sml + ((16 + i) * nbl + b) * 8);
            return;
        }
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
            sm[set][0][u] = __builtin_amdgcn_raw_buffer_load_b128(rs, vs[u], 2 * g8, 0);
            sm[set][1][u] = __builtin_amdgcn_raw_buffer_load_b128(rm, vs[u], 2 * g8, 0);
        }
    }

    // Fill the ring with the first RING groups of [cs, ce) (clamped to ce - 1)
    // and, with VSM, the first block's scales and minimums.
    __device__ __forceinline__ void prime(int cs, int ce)
    {
        // Scales and minimums first: the loop's first wait for them then
        // leaves the code loads in flight.
        if (VSM && !SML) fetch_sm(0, cs);        // SML: read from LDS once it is written
        if (PAIR) {
#pragma unroll
            for (int q = 0; q < RING / 2; ++q) fetch(q, min(cs + 2 * q, ce - 2));
            return;
        }
#pragma unroll
        for (int q = 0; q < RING; ++q) fetch(q, min(cs + q, ce - 1));
    }

    // The x rows (A operand) and x row sums of LDS group lg.
    __device__ __forceinline__ void xread(const uint16_t *rbase, const int (&aoff)[4], const float *xrow, int lg,
                                          u32x4 (&a)[4], f32x4 &xsum) const
    {
        const uint16_t *gp = rbase + lg * 128;
#pragma unroll
        for (int t = 0; t < 4; ++t) a[t] = *reinterpret_cast<const u32x4 *>(gp + aoff[t]);
        xsum = *reinterpret_cast<const f32x4 *>(xrow + lg * kXsRows);
    }

    // Group g's arithmetic once its code pieces c are in the MFMA lanes.
    __device__ __forceinline__ void arith(const u32x4 (&a)[4], const f32x4 &xsum, const u32x4 (&c)[TPW],
                                          float (&s)[TPW], float (&m)[TPW], int ce, int g, int set, int j,
                                          UnpackConsts uc)
    {
        u32x4 bq[TPW][4];
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
            bq[u][0] = unpack_biased(c[u].x, uc);
            bq[u][1] = unpack_biased(c[u].y, uc);
            bq[u][2] = unpack_biased(c[u].z, uc);
            bq[u][3] = unpack_biased(c[u].w, uc);
            if (VSM && !SML && j == 0) {          // first group of a block: gather its scales/minimums
                sm[set][0][u] = lane_gather(sm[set][0][u], src);
                sm[set][1][u] = lane_gather(sm[set][1][u], src);
            }
            if (VSM) {
                s[u] = bf16_at(sm[set][0][u], j);
                m[u] = bf16_at(sm[set][1][u], j);
            }
        }
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
            f32x4 d = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int t = 0; t < 4; ++t) d = mfma_16x16x32(a[t], bq[u][t], d);
            float sc = s[u];
            float m_adj = fmaf(-kBias, s[u], m[u]);      // mn - 128*s, one rounding
            if (kClamp && g >= ce) {                      // wave-uniform padding group
                sc = 0.0f;
                m_adj = 0.0f;
            }
#pragma unroll
            for (int r = 0; r < RL; ++r) {
                acc[u][r] = fmaf(sc, d[r], acc[u][r]);
                acc[u][r] = fmaf(m_adj, xsum[r], acc[u][r]);
            }
        }
    }

    // Group g (LDS group index lg) from ring slot q; `set`/`j` locate its
    // scale and minimum (VSM).  PAIR: the call for the first group of a pair
    // (q even) does both groups; the call for the second does nothing.
    __device__ __forceinline__ void group(const uint16_t *rbase, const int (&aoff)[4], const float *xrow,
                                          int ce, int q, int g, int lg, int set, int j, UnpackConsts uc)
    {
        if (PAIR && (q & 1)) return;
        u32x4 a[4];
        f32x4 xsum;
        xread(rbase, aoff, xrow, lg, a, xsum);
        // Take the ring slot out (the gather reads it), then refill it at once
        // so RING groups stay in flight; the scheduling barrier keeps the
        // compiler from sinking the refill below the arithmetic.
        u32x4 c[TPW];
        float s[TPW], m[TPW];
        if (PAIR) {
            // q = (g - cs) % RING with cs and RING even: pair slot q / 2.
            const int pq = q >> 1;
            u32x4 c2[TPW];
            // The columns 8-15 load holds the pair's second group in lanes
            // 8c..8c+3 and its first in 8c+4..8c+7 (the mirror of the columns
            // 0-7 load), so each group's pieces are a per-lane choice between
            // the two loads, then one permute.
            const bool lo = (i & 4) == 0;
            c[0] = lane_gather(pick(lo, cb[pq][0], cb2[pq]), src_e);
            c2[0] = lane_gather(pick(lo, cb2[pq], cb[pq][0]), src_o);
            fetch(pq, min(g + RING, ce - 2));
            __builtin_amdgcn_sched_barrier(0);
            arith(a, xsum, c, s, m, ce, g, set, j, uc);
            __builtin_amdgcn_sched_barrier(0);              // keeps the second group's x reads here (registers)
            xread(rbase, aoff, xrow, lg + 1, a, xsum);     // the pair's second group: g + 1, slot j + 1
            arith(a, xsum, c2, s, m, ce, g + 1, set, j + 1, uc);
            return;
        }
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
            c[u] = lane_gather(cb[q][u], src);
            if (!VSM) {                           // scale and minimum ride in the same slot
                s[u] = bf16_lo(sb[q][u]);
                m[u] = bf16_lo(mb[q][u]);
            }
        }
        fetch(q, min(g + RING, ce - 1));
        __builtin_amdgcn_sched_barrier(0);
        arith(a, xsum, c, s, m, ce, g, set, j, uc);
    }

    // Groups [cs, ce) of x staged in LDS for the groups [xg0, xg0 + xng)
    // (row stride xng * 128).  With VSM and !PAD, ce - cs is a multiple of 8.
    // The ring is refilled up to ce - 1.
    __device__ __forceinline__ void run(const uint16_t *xs, int xg0, int xng, int cs, int ce)
    {
        const UnpackConsts uc = unpack_consts();
        const int ng = ce - cs;
        const int arow = min(kRowPerm ? rowof(i) : i, M - 1);   // rows >= M read a real row; never stored
        const uint16_t *rbase = xs + arow * xng * 128;
        const float *xrow = reinterpret_cast<const float *>(xs + M * xng * 128) + 4 * h;
        const int lg0 = cs - xg0;                // LDS group index of cs
        int aoff[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) aoff[t] = swz(4 * h + t, arow) * 8;
        const int nblk = (ng + 7) / 8;                   // blocks of 8 groups (last may be short, !VSM)
        const int last8 = cs + (nblk - 1) * 8;           // first group of the last block
        // Two blocks per iteration with no branch inside, so the scale/minimum
        // prefetch of the second block stays ahead of the first block's work.
        // Ring slot of group g: (g - cs) % RING, a constant per unrolled step.
        int b = 0;
        for (; b + 2 <= nblk; b += 2) {
            const int g0 = cs + 8 * b;
            if (VSM) fetch_sm(1, g0 + 8);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int g = g0 + j;
                group(rbase, aoff, xrow, ce, j % RING, g, lg0 + g - cs, 0, j, uc);
            }
            if (VSM) fetch_sm(0, min(g0 + 16, last8));
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int g = g0 + 8 + j;
                const int lg = lg0 + (kClamp ? min(g - cs, ng - 1) : g - cs);
                group(rbase, aoff, xrow, ce, (8 + j) % RING, g, lg, 1, j, uc);
            }
        }
        if (b < nblk) {                                  // odd block count: the last block
            const int g0 = cs + 8 * b;                   // 16 * (b / 2) groups past cs: slot j % RING
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int g = g0 + j;
                const int lg = lg0 + (kClamp ? min(g - cs, ng - 1) : g - cs);
                group(rbase, aoff, xrow, ce, j % RING, g, lg, 0, j, uc);
            }
        }
    }
};

// CHUNKED = false: the workgroup's whole K range fits in LDS; x is staged
// once.  CHUNKED = true: the range is processed CG groups at a time (CG a
// multiple of 16), each chunk staged, primed and drained on its own.  Both
// accumulate the same groups in the same order with the same instructions, so
// they give identical bits.
// A chunk of 16 groups of x must fit the staging registers: for M <= kSmallM
// rows with the small workgroups, for 16 rows with the large ones.
static_assert(kStageMax * 64 * kWavesSmall >= kSmallM * 16 * 16, "x staging cannot hold one 16-group chunk");
static_assert(kStageMax * 64 * kWavesLarge >= kMaxM * 16 * 16, "x staging cannot hold one 16-group chunk at M = 16");

template <int TPW, bool CHUNKED, bool VSM, int RING, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void gemv_q4g128(
    const uint16_t *__restrict__ x, int M, int K, const uint32_t *__restrict__ W,
    const uint16_t *__restrict__ scale, const uint16_t *__restrict__ mn, int N,
    float *__restrict__ out, int S, int CG)
{
    extern __shared__ __attribute__((aligned(16))) uint16_t xs[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    // One tile per wave with whole 8-group blocks: codes loaded two groups at
    // a time (see Tile).
    constexpr bool PR = kTilePair && TPW == 1 && VSM;
    Tile<TPW, VSM, RING, false, false, PR> T;
    T.i = lane & 15;    // column within a tile; A row
    T.h = lane >> 4;    // 16-byte code piece within a group; D row block
    T.M = M;
    T.K = K;
    T.G = K >> 7;
    T.K8 = (size_t)(K >> 3);
    const int G = T.G;

    // K split: with S <= nb, split s covers 8-group blocks [s*nb/S, (s+1)*nb/S);
    // with more splits than blocks (S <= G), groups [s*G/S, (s+1)*G/S), each
    // at least one group (the launcher then takes the 2-byte scale/minimum
    // loads, which handle ranges ending inside a block).
    const int nb = (G + kRing - 1) / kRing;
    const int split = blockIdx.y;
    if (S <= nb) {
        T.gs = (split * nb / S) * kRing;
        T.ge = min(((split + 1) * nb / S) * kRing, G);
    } else {
        T.gs = (int)((long)split * G / S);
        T.ge = (int)((long)(split + 1) * G / S);
    }

    // Columns: waves past N alias the last column and store nothing.
    const int col0 = (blockIdx.x * WAVES + wave) * TPW * 16;
    const int cbase = __builtin_amdgcn_readfirstlane(min(col0, N - 1));
    const int ncols = __builtin_amdgcn_readfirstlane(max(1, min(16 * TPW, N - cbase)));
    T.rw = make_rsrc(W + (size_t)cbase * T.K8, (uint32_t)((size_t)ncols * T.K8 * 4));
    T.rs = make_rsrc(scale + (size_t)cbase * G, (uint32_t)(ncols * G * 2));
    T.rm = make_rsrc(mn + (size_t)cbase * G, (uint32_t)(ncols * G * 2));
    // Code loads: lane 4a + b reads piece b of column a, so each run of four
    // consecutive lanes covers 64 contiguous bytes (the memory pipeline only
    // merges neighbouring lanes); the MFMA wants piece h of column i in lane
    // i + 16h, which fetches it from lane 4i + h when it is consumed.
    const int la = lane >> 2, lb = lane & 3;
    T.src = 4 * T.i + T.h;
    T.src_e = 8 * (T.i & 7) + 4 * (T.i >> 3) + T.h;   // paired loads (see the balanced kernel)
    T.src_o = 8 * (T.i & 7) + 4 * (1 - (T.i >> 3)) + T.h;
    if (PR) {                                     // columns lane / 8 and 8 + lane / 8 (halves mirrored)
        T.vw2 = (uint32_t)((size_t)min(8 + (lane >> 3), ncols - 1) * T.K8 * 4 + 16 * ((lane ^ 4) & 7));
    }
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        const int cl = min(16 * u + la, ncols - 1);   // ragged tail: read a real column
        T.vw[u] = PR ? (uint32_t)((size_t)min(lane >> 3, ncols - 1) * T.K8 * 4 + 16 * (lane & 7))
                     : (uint32_t)((size_t)cl * T.K8 * 4 + 16 * lb);
        // 16-byte scale/minimum loads (VSM) follow the same quad order and are
        // gathered once per block; 2-byte ones are read by the lane using them.
        const int c = min(16 * u + (VSM ? la : T.i), ncols - 1);
        T.vs[u] = (uint32_t)(c * G * 2);
#pragma unroll
        for (int r = 0; r < 4; ++r) T.acc[u][r] = 0.0f;
    }

    if (!CHUNKED) {
        XStage<64 * WAVES, kStageMax, kRowPerm> xst;
        xst.load(x, M, K, T.gs, T.ge);
        T.prime(T.gs, T.ge);
        xst.store(xs, M, T.gs, T.ge);
        lds_barrier();
        T.run(xs, T.gs, T.ge - T.gs, T.gs, T.ge);
    } else {
        for (int cs = T.gs; cs < T.ge; cs += CG) {
            const int ce = min(cs + CG, T.ge);
            XStage<64 * WAVES, kStageMax, kRowPerm> xst;
            xst.load(x, M, K, cs, ce);
            T.prime(cs, ce);
            xst.store(xs, M, cs, ce);
            lds_barrier();
            T.run(xs, cs, ce - cs, cs, ce);
            __builtin_amdgcn_s_waitcnt(0);      // chunk drained: ring and LDS reads done
            lds_barrier();
        }
    }

    float *o = out + (size_t)split * (size_t)M * (size_t)N;
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        const int n = col0 + 16 * u + T.i;
        if (n < N) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = kRowPerm ? rowof(4 * T.h + r) : 4 * T.h + r;
                if (row < M) o[(size_t)row * N + n] = T.acc[u][r];
            }
        }
    }
}

// SwiGLU of a fused gate/up pair, rounded to bf16 (nearest even).  The
// fused product's gate and up halves are its columns n and I + n (Token Rush
// README, steps table row 3: projections fused side by side); the activation
// is the gated MLP's silu(gate) * up.  Shared by every path that applies it,
// so they give the same bits for the same fp32 gate and up values.
__device__ __forceinline__ uint16_t swiglu_bf16(float g, float u)
{
    const float a = g / (1.0f + expf(-g)) * u;
    const uint32_t b = __float_as_uint(a);
    if ((b & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;        // NaN stays NaN
    return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

// ---- balanced kernel: one workgroup per compute unit ---------------------------
//
// A stream only reaches full rate when every compute unit moves about the
// same number of bytes (Token Rush README, bandwidth paragraph: decode is
// bound by streaming the weights).  Here the grid is gx workgroups per K split,
// at most one per CU (the LDS request is sized so two never share a CU), and
// workgroup c owns an equal share of the columns, dealt in units of 8 (136
// for N = 34816 on 256 CUs), cut into the fewest tiles of at most 16 columns,
// all of (nearly) equal width.  Each of 12 waves takes one tile at a time.
// x is staged once per workgroup; each wave copies
// its tile's scales and minimums into its own LDS area with 16-byte loads of
// consecutive pieces, so the main loop streams nothing but codes.  The
// per-column instructions are those of gemv_q4g128, so results are the same
// bits.  Needs K/128 a multiple of 8 and 16-byte aligned scale/min.

// One group per load (workgroups of few tiles, where pairing streamed
// slower) with the non-temporal hint: 5120 -> 12288 10.54 -> 10.28 us.
template <int RING, bool SML, bool PAD, bool ACT = false, int RL = 4, bool PAIR = true>
struct BalTile : Tile<1, true, RING, SML, PAD, PAIR, RL, kPairCpol> {
    typedef Tile<1, true, RING, SML, PAD, PAIR, RL, kPairCpol> Base;
    int la, lb, nblk, ncols, wact, NC;

    // Column of W that tile column c (0..15) reads, relative to the tile's
    // base: plain, c itself (clamped to the tile's width); ACT, a tile holds
    // `wact` <= 8 gate/up pairs: columns 0..7 the gate columns base + c and
    // 8..15 the up columns NC + base + c - 8, each half clamped to its width.
    __device__ __forceinline__ int colmap(int c) const
    {
        if (ACT) return c < 8 ? min(c, wact - 1) : NC + min(c - 8, wact - 1);
        return min(c, ncols - 1);
    }

    // Descriptors and lane offsets for the tile of `width` columns (ACT:
    // pairs, 1..8; else 1..16) from cbase; lanes past the width read its last
    // column.
    __device__ __forceinline__ void setup(const uint32_t *W, const uint16_t *scale, const uint16_t *mn, int cbase_,
                                          int width, int nc)
    {
        const int cbase = __builtin_amdgcn_readfirstlane(cbase_);
        const int w = __builtin_amdgcn_readfirstlane(width);
        NC = nc;
        wact = w;
        ncols = ACT ? 16 : w;                              // tile columns staged and computed
        const size_t span = ACT ? (size_t)NC + w : (size_t)w;   // columns the descriptors cover
        this->rw = make_rsrc(W + (size_t)cbase * this->K8, (uint32_t)(span * this->K8 * 4));
        this->rs = make_rsrc(scale + (size_t)cbase * this->G, (uint32_t)(span * this->G * 2));
        this->rm = make_rsrc(mn + (size_t)cbase * this->G, (uint32_t)(span * this->G * 2));
        if (PAIR) {                                        // columns lane / 8 and 8 + lane / 8 (halves mirrored)
            this->vw[0] = (uint32_t)((size_t)colmap(la >> 1) * this->K8 * 4 + 16 * (4 * (la & 1) + lb));
            this->vw2 = (uint32_t)((size_t)colmap(8 + (la >> 1)) * this->K8 * 4 + 16 * ((lane_id() ^ 4) & 7));
        } else {
            this->vw[0] = (uint32_t)((size_t)colmap(la) * this->K8 * 4 + 16 * lb);
        }
        this->vs[0] = (uint32_t)((size_t)colmap(la) * this->G * 2);   // !SML: per-block loads, quad order
#pragma unroll
        for (int r = 0; r < 4; ++r) this->acc[0][r] = 0.0f;
    }

    // Scale/minimum pieces (16 bytes = 8 groups of one column) of the tile's
    // K range: slot q = lane + 64r holds column q >> sh, block q & (2^sh - 1),
    // 2^sh the least power of two >= nblk (slots past nblk idle), so no lane
    // divides by nblk.
    __device__ __forceinline__ int sm_shift() const { return nblk <= 1 ? 0 : nblk <= 2 ? 1 : nblk <= 4 ? 2 : 3; }

    __device__ __forceinline__ void sm_load(u32x4 (&sr)[kBalSmRounds], u32x4 (&mr)[kBalSmRounds], int lane) const
    {
        const int sh = sm_shift();
#pragma unroll
        for (int r = 0; r < kBalSmRounds; ++r) {
            if (64 * r < (ncols << sh)) {                  // wave-uniform
                const int q = lane + 64 * r;
                const int col = min(q >> sh, ncols - 1), b = min(q & ((1 << sh) - 1), nblk - 1);   // idle: a real piece
                const uint32_t off = (uint32_t)(((size_t)colmap(col) * this->G + this->gs + 8 * b) * 2);
                sr[r] = __builtin_amdgcn_raw_buffer_load_b128(this->rs, off, 0, 0);
                mr[r] = __builtin_amdgcn_raw_buffer_load_b128(this->rm, off, 0, 0);
            }
        }
    }

    __device__ __forceinline__ void sm_store(const u32x4 (&sr)[kBalSmRounds], const u32x4 (&mr)[kBalSmRounds],
                                             int lane) const
    {
        uint16_t *dst = const_cast<uint16_t *>(this->sml);
        const int sh = sm_shift();
#pragma unroll
        for (int r = 0; r < kBalSmRounds; ++r) {
            const int q = lane + 64 * r;
            const int col = q >> sh, b = q & ((1 << sh) - 1);
            if (64 * r < (ncols << sh) && col < ncols && b < nblk) {
                *reinterpret_cast<u32x4 *>(dst + (col * this->nbl + b) * 8) = sr[r];
                *reinterpret_cast<u32x4 *>(dst + ((16 + col) * this->nbl + b) * 8) = mr[r];
            }
        }
    }

    // y rows < M of the tile's columns through a descriptor over [M][N] fp32
    // (M*N*4 < 2^31): 32-bit offsets, no 64-bit addresses live across tiles.
    __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t ry, int N, int cbase) const
    {
        const int n = cbase + this->i;
        if (this->i < ncols) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = kRowPerm ? rowof(4 * this->h + r) : 4 * this->h + r;
                if (row < this->M)
                    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, this->acc[0][r]), ry,
                                                          (uint32_t)(row * N + n) * 4, 0, 0);
            }
        }
    }

    // ACT: tile column i < 8 holds gate column base + i and column i + 8 the
    // matching up column; lane i + 16h takes the up sums from lane i + 8 + 16h
    // and writes rows 4h..4h+3 of act [M][NC].
    __device__ __forceinline__ void store_act(uint16_t *act, int cbase) const
    {
        float u[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) u[r] = __shfl_down(this->acc[0][r], 8);
        if (this->i < wact) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = kRowPerm ? rowof(4 * this->h + r) : 4 * this->h + r;
                if (row < this->M) act[(size_t)row * NC + cbase + this->i] = swiglu_bf16(this->acc[0][r], u[r]);
            }
        }
    }
};

// PARTS: a workgroup with few tiles cuts each tile's K range into P parts
// (one wave each) at the block boundaries a K split into P splits uses; the
// parts' fp32 sums go to LDS and, after a barrier, are added in part order.
// The result depends on (K, N, P) only (P comes from (K, N) and the CU count,
// never from M), and it is the bits the per-tile kernel gives with P K
// splits and the split-order reduce: the same groups in the same order per
// part, the same additions afterwards.
// ACT: N = 2I is a fused gate/up product.  The workgroup owns pair-columns
// [n0, n1) of I, cut in units of 4 (the same bytes per CU as the plain cut);
// a tile holds 8 pairs, gate columns in its first 8 MFMA columns and the
// matching up columns in the last 8, so a pair meets in one wave's
// registers and bf16 silu(gate) * up goes straight to act [M][I].  The
// per-column sums are those of the plain product.
// PAIR: codes loaded two groups at a time (see Tile); the plan takes it for
// workgroups of 4 or more units, where it streams faster, and leaves it off
// for 3 or fewer tiles per CU, where it streamed slower.  It never changes a
// bit.
// XN: x is the RMSNorm of fp32 rows h (x points to h) times na.gamma, made
// while staging (S == 1: whole rows).
template <int RING, bool SML, bool PARTS, bool ACT, int RL, bool PAIR, bool XN>
__global__ __launch_bounds__(kBalThreads) void gemv_q4g128_bal(
    const uint16_t *__restrict__ x, int M, int K, const uint32_t *__restrict__ W,
    const uint16_t *__restrict__ scale, const uint16_t *__restrict__ mn, int N,
    float *__restrict__ out, uint16_t *__restrict__ act, int S, int nblp, int P, int nps, NormArgs na)
{
    extern __shared__ __attribute__((aligned(16))) uint16_t xs[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int G = K >> 7;
    const int nb = G >> 3;
    const int split = blockIdx.y;
    const int gs = (split * nb / S) * 8;
    const int ge = ((split + 1) * nb / S) * 8;
    const int ng = ge - gs;
    // x first, and alone: every wave's code and scale/minimum loads wait until
    // the workgroup's x is in LDS.  Issued together, its few kilobytes queue
    // behind megabytes of weight requests from all CUs, and the barrier waits
    // for the slowest wave's x.  Its loads go out before any other set-up.
    XStage<kBalThreads, kBalStage, kRowPerm, XN> xst;
    if constexpr (XN)
        xst.load_norm(reinterpret_cast<const float *>(x), na.gamma, M, K);
    else
        xst.load(x, M, K, gs, ge);
    const int gx = gridDim.x;
    // Workgroups are dealt to the 8 XCDs in turn (c -> XCD c % 8); numbering
    // them XCD by XCD before cutting the column range gives every XCD the same
    // mix of larger and smaller shares.
    const int c = (gx % 8 == 0) ? (int)(blockIdx.x % 8) * (gx / 8) + (int)(blockIdx.x / 8) : (int)blockIdx.x;
    // Columns [n0, n1), cut in units of 4 so every CU streams the same bytes to
    // within 4 columns (N = 34816 on 256 CUs: 136 each, 9 tiles of 15-16;
    // N = 5120: 20 each); ACT: pair-columns of I = N/2, likewise (68 pairs).
    const int NC = ACT ? (N >> 1) : N;
    const int NU = (NC + 3) >> 2;
    // (32-bit division where c * NU cannot overflow: a 64-bit one costs the
    // set-up some hundred instructions.)
    const bool n32 = NU < (1 << 22) && gx <= 1024;
    const int n0 = n32 ? (int)((unsigned)c * (unsigned)NU / (unsigned)gx) * 4 : (int)((long)c * NU / gx) * 4;
    const int n1 = min(n32 ? (int)((unsigned)(c + 1) * (unsigned)NU / (unsigned)gx) * 4
                           : (int)((long)(c + 1) * NU / gx) * 4,
                       NC);
    // Tiles of at most TW columns (ACT: pairs), as few as that allows, of
    // equal widths: tile k covers [n0 + k*width/nchunk, n0 + (k+1)*width/nchunk).
    // (136 columns make 9 tiles of 15-16 columns rather than 8 of 16 and one
    // of 8: every wave then streams the same bytes.)
    const int TW = ACT ? 8 : 16;
    const int width = n1 - n0;
    const int nchunk = (width + TW - 1) / TW;
    auto tile = [&](int k, int &cb, int &cw) {
        cb = n0 + (k * width) / nchunk;
        cw = n0 + ((k + 1) * width) / nchunk - cb;
    };
    const int nunit = PARTS ? nchunk * P : nchunk;        // (tile, part) units
    const bool active = wave < nunit;                     // wave-uniform

    BalTile<RING, SML, false, ACT, RL, PAIR> B;
    B.i = lane & 15;
    B.h = lane >> 4;
    B.la = lane >> 2;
    B.lb = lane & 3;
    B.src = 4 * B.i + B.h;
    // Paired loads: piece h of column i < 8 sits in lane 8i + h (first group)
    // and 8i + 4 + h (second group) of the columns 0-7 load; piece h of column
    // i >= 8 in lane 8(i-8) + 4 + h (first) and 8(i-8) + h (second) of the
    // mirrored columns 8-15 load.
    B.src_e = 8 * (B.i & 7) + 4 * (B.i >> 3) + B.h;
    B.src_o = 8 * (B.i & 7) + 4 * (1 - (B.i >> 3)) + B.h;
    B.M = M;
    B.K = K;
    B.G = G;
    B.K8 = (size_t)(K >> 3);
    B.nbl = nblp;
    B.NC = NC;
    // LDS: x [M][ng*128] bf16, row sums [ng][16] fp32, nps part slots of 256
    // fp32 (PARTS), then one scale/minimum area of 2*16*nblp*8 bf16 per wave.
    float *slots = reinterpret_cast<float *>(xs + M * ng * 128 + ng * kXsRows * 2);
    B.sml = xs + M * ng * 128 + ng * kXsRows * 2 + nps * 512 + wave * (2 * 16 * nblp * 8);

    // A unit's column base and group range.
    auto unit = [&](int u, int &cb, int &cw, int &cs, int &ce) {
        const int k = PARTS ? u / P : u;
        const int p = PARTS ? u - k * P : 0;
        tile(k, cb, cw);
        // Part p: 8-group blocks [p*nbs/P, (p+1)*nbs/P) of the split's nbs,
        // the same cut as a K split of the per-tile kernel into P splits.
        cs = PARTS ? gs + ((p * (ng >> 3)) / P) * 8 : gs;
        ce = PARTS ? gs + (((p + 1) * (ng >> 3)) / P) * 8 : ge;
    };
    if constexpr (XN) xst.norm(xs, M, K, na.eps);
    xst.store(xs, M, gs, ge);
    lds_barrier();
    if (!PARTS && !active) return;

    const __amdgpu_buffer_rsrc_t ry = make_rsrc(out + (size_t)split * (size_t)M * (size_t)N, (uint32_t)(M * N * 4));
    if (active) {
        u32x4 sr[kBalSmRounds], mr[kBalSmRounds];
        for (int u = wave; u < nunit; u += kBalWaves) {   // this wave's units
            int cb, cw, cs, ce;
            unit(u, cb, cw, cs, ce);
            B.gs = cs;
            B.ge = ce;
            B.nblk = (ce - cs + 7) >> 3;
            B.smg0 = cs;
            B.setup(W, scale, mn, cb, cw, NC);
            if (SML) B.sm_load(sr, mr, lane);             // before the codes: waiting for them leaves the codes in flight
            B.prime(cs, ce);
            if (SML) B.sm_store(sr, mr, lane);            // the wave's own LDS area; its LDS ops stay in order
            if (SML) B.fetch_sm(0, cs);                   // (!SML: the prime loaded it)
            B.run(xs, gs, ng, cs, ce);
            if (!PARTS) {
                if (ACT) B.store_act(act, cb);
                else B.store(ry, N, cb);
            } else {                                      // the unit's 16 columns x 16 rows
                *reinterpret_cast<f32x4 *>(slots + u * 256 + lane * 4) =
                    f32x4{B.acc[0][0], B.acc[0][1], B.acc[0][2], B.acc[0][3]};
            }
        }
    }
    if (PARTS) {
        lds_barrier();                                    // every wave, with or without a unit
        for (int k = wave; k < nchunk; k += kBalWaves) {
            int cb, cw;
            tile(k, cb, cw);
            f32x4 v = *reinterpret_cast<const f32x4 *>(slots + (k * P) * 256 + lane * 4);
            for (int p = 1; p < P; ++p) v += *reinterpret_cast<const f32x4 *>(slots + (k * P + p) * 256 + lane * 4);
#pragma unroll
            for (int r = 0; r < 4; ++r) B.acc[0][r] = v[r];
            if (ACT) {                                    // all lanes: the pair exchange is a shuffle
                B.wact = cw;
                B.store_act(act, cb);
            } else {
                B.ncols = cw;
                B.store(ry, N, cb);
            }
        }
    }
}

// ---- LDS-fed balanced kernel ----------------------------------------------------
//
// The balanced kernel's work split (one workgroup per CU, equal column shares,
// (tile, K part) units, one unit per wave at a time) and its per-group
// arithmetic, with the weights brought in by the buffer unit's direct-to-LDS
// loads: no register holds a load in flight, and the codes land already in
// the order the MFMA lanes read them.
//
// Codes: each wave owns a ring of RD slots in LDS, one group pair per slot:
// two 1 KB loads, columns 0-7 and 8-15 of its tile, 128 contiguous bytes
// (two groups) of each column per load.  Lane 8c + j of a load reads 16-byte
// piece j ^ c of column c's line (every run of four lanes still covers one
// aligned 64-byte half, and the XOR spreads the MFMA lanes' later reads of
// one piece index over all eight 16-byte bank groups), so MFMA lane i + 16h
// finds piece h of group e of column i at 16-byte position
// 64 [i >= 8] + 8 (i & 7) + ((4e + h) ^ (i & 7)) of its slot: one LDS read per
// group and lane replaces the register ring's lane permutes and selects.
// Slots are refilled RD pairs ahead (no refill past the unit's end); before
// a slot is read the wave waits, by an explicit count, for the loads that
// filled it (the compiler's own tracking of direct-to-LDS loads is not relied
// on), and before a slot or area is refilled, for its earlier LDS reads.
//
// Scales and minimums: the unit's pieces (8 groups of one column, 16 bytes)
// are loaded straight into the wave's LDS area, [column][block] order; one
// 4-byte LDS read per lane gives a pair's two scales (two minimums).
//
// BURST: the first unit's scales, minimums and ring are requested before x,
// so the weights stream from the first microsecond; for short shapes whose
// units fit their ring this is the whole unit.  Otherwise x is staged first
// (alone, it is back in ~1.2 us; behind the weight requests of every CU it
// would wait ~2.5 us).
//
// Bits: the same groups in the same order with the same instructions per
// column as gemv_q4g128_bal and gemv_q4g128 (group_fma below is their
// per-group arithmetic), the same K parts and part-order sum; the choice
// between the kernels never changes a bit.

constexpr int kLdsSlotU4 = 128;            // u32x4 per wave and ring slot: one group pair of a 16-column tile
constexpr int kLdsBurstBlocks = 5;         // BURST: blocks of 8 groups per unit, at most (whole K = 5120 too)
// NR launches: tile waves with a ring slot and a burst area of their own; the
// waves without a tile share one more (their empty loads write only zeros,
// which nothing reads).
constexpr int kNarrowRingWaves = 9;
constexpr int kDeepRing = 8;                // pairs in flight for the youngest tile wave (its slots + 3 idle waves')
// Cache-policy bits of a buffer access: system coherence (sc0 | sc1): loads
// miss every cache, stores write through to memory.
constexpr int kSysCoherent = 17;

// LDS counters shared by the waves of a workgroup, read and added to in
// inline asm: the compiler takes any LDS access it sees as possibly aliasing
// the direct-to-LDS loads in flight and would wait for all of them first
// (draining the weight ring).  The read waits for its own result in the same
// asm block.  f is an LDS address.
__device__ __forceinline__ uint32_t lds_counter(const uint32_t *f)
{
    const uint32_t a = (uint32_t)(size_t)(const __attribute__((address_space(3))) uint32_t *)f;
    uint32_t v;
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(a) : "memory");
    return v;
}

// Sets the LDS counter *f (one writer per counter) to v.
__device__ __forceinline__ void lds_put(uint32_t *f, uint32_t v)
{
    const uint32_t a = (uint32_t)(size_t)(__attribute__((address_space(3))) uint32_t *)f;
    asm volatile("ds_write_b32 %0, %1" : : "v"(a), "v"(v) : "memory");
}

// Wait until every one of the n (1..64) LDS counters f[0..n) has reached v;
// lane j reads f[j].  Each counter has one writer and only grows, so once
// all have been seen at v or above they stay there.  Bounded (about a
// millisecond): every wave leaves the kernel even if a count never arrives.
__device__ __forceinline__ void lds_wait_all_geq(const uint32_t *f, int n, uint32_t v)
{
    const uint32_t *g = f + min((int)(threadIdx.x & 63), n - 1);
    for (int it = 0; it < (1 << 14); ++it) {
        if (__builtin_amdgcn_ballot_w64(lds_counter(g) < v) == 0) break;
        __builtin_amdgcn_s_sleep(2);
    }
}

// Waits until the loads of a ring slot have landed, given how many later
// pairs (two loads each) this wave has requested since (0 .. 3).  Vector
// memory loads complete in order, so "at most 2n outstanding" covers the
// slot and everything requested before it (the unit's scale/minimum pieces).
__device__ __forceinline__ void wait_ring(int newer)
{
    if (newer >= 3) asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
    else if (newer == 2) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else if (newer == 1) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// A ring slot's two code pieces and the pair's scale/minimum words from the
// burst form's area (the minima kLdsBurstBlocks * 256 bytes after the
// scales), read and waited for in one block.  The compiler then adds no wait
// of its own for direct-to-LDS loads it cannot tell apart from these
// addresses (slots of other waves included); the outputs are early-clobber,
// so no later read of the block can take its address from a register an
// earlier read is still writing.
__device__ __forceinline__ void pair_reads(const u32x4 *a0, const u32x4 *a1, const uint8_t *sp, u32x4 &c0, u32x4 &c1,
                                           uint32_t &sw, uint32_t &mw)
{
    static_assert(kLdsBurstBlocks == 5, "the minima are read 5 * 256 bytes after the scales");
    const uint32_t x0 = (uint32_t)(size_t)(const __attribute__((address_space(3))) u32x4 *)a0;
    const uint32_t x1 = (uint32_t)(size_t)(const __attribute__((address_space(3))) u32x4 *)a1;
    const uint32_t xq = (uint32_t)(size_t)(const __attribute__((address_space(3))) uint8_t *)sp;
    uint32_t __attribute__((ext_vector_type(2))) r;
    asm volatile("ds_read_b128 %0, %3\n\tds_read_b128 %1, %4\n\tds_read2st64_b32 %2, %5 offset1:5\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(c0), "=&v"(c1), "=&v"(r) : "v"(x0), "v"(x1), "v"(xq) : "memory");
    sw = r.x;
    mw = r.y;
}

// Per-group arithmetic shared by the LDS-fed kernel: D = x . (128 + q) by
// four MFMAs, then acc = fma(s, D, acc), acc = fma(m - 128 s, X, acc) for
// the RL accumulated D rows.  Identical to Tile::arith for one tile.
template <int RL>
__device__ __forceinline__ void group_fma(const u32x4 (&a)[4], const f32x4 &xsum, const u32x4 &c, float s, float m,
                                          float (&acc)[4], UnpackConsts uc)
{
    u32x4 bq[4];
    bq[0] = unpack_biased(c.x, uc);
    bq[1] = unpack_biased(c.y, uc);
    bq[2] = unpack_biased(c.z, uc);
    bq[3] = unpack_biased(c.w, uc);
    f32x4 d = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int t = 0; t < 4; ++t) d = mfma_16x16x32(a[t], bq[t], d);
    const float m_adj = fmaf(-kBias, s, m);           // mn - 128*s, one rounding
#pragma unroll
    for (int r = 0; r < RL; ++r) {
        acc[r] = fmaf(s, d[r], acc[r]);
        acc[r] = fmaf(m_adj, xsum[r], acc[r]);
    }
}

// EPI (K parts, plain product): 1 stores h = r + y instead of y (out is h);
// 2 also normalises the rows in the workgroup that finishes last.  XN: x is
// the RMSNorm of fp32 rows h (x points to h) times gamma, made while staging.
// XCH (rows that do not fit the LDS whole, every tile one wave's, at least
// one wave without a tile): x is staged in chunks of xcg groups into two
// buffers.  The waves without a tile load chunk c + 1 while the others run
// chunk c; per-wave progress counters in LDS hand the buffers over.
// Every tile's sums run in the same order as with x staged whole.  NR (whole
// K, at most kNarrowRingWaves tiles): ring slots and burst areas for the tile
// waves plus one the others share, 13 KB less static LDS, which leaves x room
// for M = 8 and 9 at K = 5120 in the burst form.
template <int RD, bool PARTS, bool ACT, int RL, bool BURST, int EPI, bool XN, bool XCH = false, bool NR = false>
__global__ __launch_bounds__(kBalThreads) void gemv_q4g128_lds(
    const uint16_t *__restrict__ x, int M, int K, const uint32_t *__restrict__ W,
    const uint16_t *__restrict__ scale, const uint16_t *__restrict__ mn, int N,
    float *__restrict__ out, uint16_t *__restrict__ act, int P, int nps, int nblm, NormArgs na, int xcg)
{
    static_assert(RD == 2 || RD == 4, "ring depth: units are whole blocks of 4 pairs");
    static_assert(EPI == 0 || (PARTS && !ACT), "the residual epilogue follows the K-part reduce of the plain product");
    static_assert(!XCH || (!PARTS && !BURST && !XN && EPI == 0), "chunked x: whole-K tiles, x loaded as is");
    constexpr bool burst = BURST;
    constexpr bool NORM = EPI == 2;
    static_assert(!NR || (RD == 2 && !PARTS && !XCH), "shared spare slot: whole-K tiles, x staged whole");
    constexpr bool DEEP = RD == 2 && BURST && !PARTS && !XCH && RL == 1 && !NR;
    constexpr int RW = NR ? kNarrowRingWaves + 1 : kBalWaves;    // ring slots and burst areas
    __shared__ uint32_t last_wg;
    __shared__ uint32_t xprog[XCH ? kBalWaves : 1];       // XCH, per wave: chunks run (tile) or last staged (loader)
    __shared__ __attribute__((aligned(16))) u32x4 ring0[RW * kLdsSlotU4];
    __shared__ __attribute__((aligned(16))) u32x4 ring1[RW * kLdsSlotU4];
    __shared__ __attribute__((aligned(16))) u32x4 ring2[RD > 2 ? kBalWaves * kLdsSlotU4 : 1];
    __shared__ __attribute__((aligned(16))) u32x4 ring3[RD > 2 ? kBalWaves * kLdsSlotU4 : 1];
    // BURST: the scale/minimum areas in an array of their own (units of at
    // most kLdsBurstBlocks blocks), so that x, staged while every load of the
    // burst is in flight, provably shares no LDS with them and its staging
    // waits for the x loads alone.
    __shared__ __attribute__((aligned(16))) uint8_t smst[BURST ? RW * 512 * kLdsBurstBlocks : 16];
    extern __shared__ __attribute__((aligned(16))) uint16_t xs[];
    u32x4 *const rings[4] = {ring0, ring1, ring2, ring3};
    if (BURST) nblm = kLdsBurstBlocks;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int G = K >> 7;
    const size_t K8 = (size_t)(K >> 3);
    const int gx = gridDim.x;
    const int c = (gx % 8 == 0) ? (int)(blockIdx.x % 8) * (gx / 8) + (int)(blockIdx.x / 8) : (int)blockIdx.x;
    const int NC = ACT ? (N >> 1) : N;
    const int NU = (NC + 3) >> 2;
    const bool n32 = NU < (1 << 22) && gx <= 1024;
    const int n0 = n32 ? (int)((unsigned)c * (unsigned)NU / (unsigned)gx) * 4 : (int)((long)c * NU / gx) * 4;
    const int n1 = min(n32 ? (int)((unsigned)(c + 1) * (unsigned)NU / (unsigned)gx) * 4
                           : (int)((long)(c + 1) * NU / gx) * 4,
                       NC);
    const int TW = ACT ? 8 : 16;
    const int width = n1 - n0;
    const int nchunk = (width + TW - 1) / TW;
    auto tile = [&](int k, int &cb, int &cw) {
        cb = n0 + (k * width) / nchunk;
        cw = n0 + ((k + 1) * width) / nchunk - cb;
    };
    const int nunit = PARTS ? nchunk * P : nchunk;
    const bool active = wave < nunit;                     // wave-uniform
    const int nb = G >> 3;
    auto unit = [&](int u, int &cb, int &cw, int &cs, int &ce) {
        const int k = PARTS ? u / P : u;
        const int p = PARTS ? u - k * P : 0;
        tile(k, cb, cw);
        cs = PARTS ? ((p * nb) / P) * 8 : 0;
        ce = PARTS ? (((p + 1) * nb) / P) * 8 : G;
    };

    // LDS: x [M][G*128] bf16, row sums [G][16] fp32, nps part slots of 256
    // fp32, then one scale/minimum area per wave: [scale, min][16 columns][nblm
    // blocks] of 16 bytes.
    const int xg = XCH ? xcg : G;                          // groups of x staged at once
    const int xstride = M * xg * 128 + xg * kXsRows * 2;  // one x buffer (bf16 units)
    float *slots = reinterpret_cast<float *>(xs + (XCH ? 2 : 1) * xstride);
    // Ring slot and burst area index: the wave's own, or NR's shared spare.
    const int slotw = NR && !active ? kNarrowRingWaves : wave;
    uint8_t *smarea = BURST ? smst + slotw * (512 * kLdsBurstBlocks)
                            : reinterpret_cast<uint8_t *>(slots + nps * 256) + (size_t)slotw * (512 * nblm);

    const int i = lane & 15, h = lane >> 4;
    const int cq = lane >> 3, jq = lane & 7;
    // MFMA lane (i, h): piece h of the pair's first group, piece 4 + h of its second.
    const int boff0 = ((i & 8) ? 64 : 0) + 8 * (i & 7) + (h ^ (i & 7));
    const int boff1 = ((i & 8) ? 64 : 0) + 8 * (i & 7) + ((4 + h) ^ (i & 7));

    // Per-unit load state (wave-uniform descriptors, per-lane offsets).
    __amdgpu_buffer_rsrc_t rw, rs, rm;
    uint32_t voffA = 0, voffB = 0;
    int ucs = 0, unp = 0, unblk = 1, ucw = 1, ucb = 0;
    auto colmap = [&](int cc, int cw) -> int {
        if (ACT) return cc < 8 ? min(cc, cw - 1) : NC + min(cc - 8, cw - 1);
        return min(cc, cw - 1);
    };
    // Loads of ring slot r <- pair p of the current unit (two 1 KB loads).
    // Pair p of the unit into ring slot r.  live == false: the same two loads
    // from an empty descriptor (they read nothing and write zeros into the
    // slot, which is not read again): the main loop refills unconditionally,
    // so every pass issues the same loads and the compiler's count of loads
    // in flight stays exact (a refill under a branch made it wait for every
    // load before reading the second slot).
    const __amdgpu_buffer_rsrc_t rnone = make_rsrc(W, 0u);
    auto fill_at = [&](u32x4 *dst, int p, bool live) {
        // The slot's earlier reads are complete before the load may write it.
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        const uint32_t so = (uint32_t)(64 * ucs + 128 * p);
        const __amdgpu_buffer_rsrc_t src = live ? rw : rnone;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (__attribute__((address_space(3))) void *)dst, 16, voffA, so, 0,
                                                 kPairCpol);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (__attribute__((address_space(3))) void *)(dst + 64), 16, voffB,
                                                 so, 0, kPairCpol);
    };
    auto fill = [&](int r, int p, bool live = true) { fill_at(rings[r] + slotw * kLdsSlotU4, p, live); };
    // Unit u: descriptors and its scale/minimum pieces into the wave's area.
    // live == false (a wave without a unit, burst only): unit 0's geometry
    // with empty descriptors, so its loads read nothing and only fill its own
    // slots with zeros; every wave then issues the same sequence of loads,
    // which lets the compiler count exactly the loads x's staging waits for.
    auto setup_unit = [&](int u, bool live) {
        // The area's earlier reads are complete before new pieces may land.
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        int cb, cw, cs, ce;
        unit(live ? u : 0, cb, cw, cs, ce);
        cb = __builtin_amdgcn_readfirstlane(cb);
        cw = __builtin_amdgcn_readfirstlane(cw);
        ucs = __builtin_amdgcn_readfirstlane(cs);
        unp = __builtin_amdgcn_readfirstlane((ce - cs) >> 1);
        unblk = __builtin_amdgcn_readfirstlane((ce - cs) >> 3);
        ucw = cw;
        ucb = cb;
        const size_t span = live ? (ACT ? (size_t)NC + cw : (size_t)cw) : 0;
        rw = make_rsrc(W + (size_t)cb * K8, (uint32_t)(span * K8 * 4));
        rs = make_rsrc(scale + (size_t)cb * G, (uint32_t)(span * G * 2));
        rm = make_rsrc(mn + (size_t)cb * G, (uint32_t)(span * G * 2));
        voffA = (uint32_t)((size_t)colmap(cq, cw) * K8 * 4 + 16 * (jq ^ cq));
        voffB = (uint32_t)((size_t)colmap(8 + cq, cw) * K8 * 4 + 16 * (jq ^ cq));
        // pieces q = column * nblk + block, 64 per load; lanes past the last idle
        const float rcp = 1.0f / (float)unblk;
        for (int q0 = 0; q0 < 16 * unblk; q0 += 64) {
            const int q = q0 + lane;
            if (q < 16 * unblk) {
                const int col = (int)(((float)q + 0.5f) * rcp);
                const int b = q - col * unblk;
                const uint32_t off = (uint32_t)(((size_t)colmap(col, cw) * G + cs + 8 * b) * 2);
                uint8_t *ds = smarea + 16 * q0;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void *)ds, 16, off, 0,
                                                         0, 0);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rm, (__attribute__((address_space(3))) void *)(ds + 256 * nblm),
                                                         16, off, 0, 0, 0);
            }
        }
    };
    // The ring primed with the unit's first RD pairs.
    auto prime = [&]() {
#pragma unroll
        for (int r = 0; r < RD; ++r) fill(r, min(r, unp - 1));
    };

    // Burst: the first tile's scale/minimum requests, x, then the ring's
    // first pairs; with K parts x goes first (its store then also waits for
    // the scale/minimum loads: 17408 -> 5120 12.88 -> 12.59 us, 6144 -> 5120
    // 7.53 -> 7.47; on whole-K shapes even or slower).
    constexpr bool xfirst = BURST && PARTS;
    XStage<kBalThreads, kBalStage, kRowPerm, XN> xst;
    if (burst && !xfirst) setup_unit(wave, active);
    if constexpr (XN)
        xst.load_norm(reinterpret_cast<const float *>(x), na.gamma, M, K);
    else
        xst.load(x, M, K, 0, xg);
    if (burst && xfirst) setup_unit(wave, active);
    if (burst) prime();                           // after x: x's loads stay older than the ring's
    if constexpr (XN) xst.norm(xs, M, K, na.eps);
    xst.store(xs, M, 0, xg);
    if (XCH && tid < kBalWaves) xprog[tid] = 0u;
    // Deep ring (whole-K burst form, one accumulated row): where at least
    // three waves have no tile, the youngest tile wave (the last to end its
    // loop) also takes the ring slots of the three after it and keeps
    // kDeepRing pairs in flight.  Back-to-back gate/up launches at M = 1-4
    // run 2-4% faster with it on most boxes (e.g. 18.01 -> 17.34 us) and up
    // to 1% slower on some; M = 5-8 gain nothing, so they do not take it.
    // The idle waves' empty primes land before the barrier; the deep wave's
    // pairs 2..7 are requested after it.
    const bool deep_wg = DEEP && kBalWaves - nunit >= 3 && (G >> 1) >= kDeepRing;
    const bool deep = deep_wg && wave == nunit - 1;
    auto dslot = [&](int k) -> u32x4 * { return ((k & 1) ? ring1 : ring0) + (wave + (k >> 1)) * kLdsSlotU4; };
    if (deep_wg && !active) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();
    if (deep) {
#pragma unroll
        for (int k = 2; k < kDeepRing; ++k) fill_at(dslot(k), k, true);
    }
    if (XCH && !active) {
        // Loader: its share of chunk c (>= 1) into buffer c % 2 once every
        // tile wave's counter says it has run chunk c - 2, then c into its
        // own counter.  The tile waves do not wait for one another, only for
        // every loader's counter to reach the chunk they need next: a
        // workgroup barrier at each chunk end would hold every wave to the
        // slowest one while its ring runs dry.  (One counter per wave: a sum
        // of counts cannot tell a wave that is ahead from one that is
        // behind.)
        const int nchk = (G + xg - 1) / xg;
        for (int c = 1; c < nchk; ++c) {
            if (c >= 2) lds_wait_all_geq(xprog, nunit, (uint32_t)(c - 1));
            // Rounds of 8 pieces per thread where a chunk is more than 12
            // per loader thread (M = 16 at 5120 -> 34816: 24.2 against
            // 25.2 us), else of 4 (M = 9, 13: 0.3-0.6 us faster than 8).
            const int cs = c * xg, ce = min((c + 1) * xg, G), lt = tid - 64 * nunit, nlt = 64 * (kBalWaves - nunit);
            if (M * (ce - cs) * 16 > 12 * nlt)
                stage_rounds<8, kRowPerm>(xs + (c & 1) * xstride, x, M, K, cs, ce, lt, nlt);
            else
                stage_rounds<4, kRowPerm>(xs + (c & 1) * xstride, x, M, K, cs, ce, lt, nlt);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");      // this wave's writes have landed
            if (lane == 0) lds_put(&xprog[wave], (uint32_t)c);
        }
        return;
    }
    if (!PARTS && !active) return;

    const UnpackConsts uc = unpack_consts();
    const int arow = min(kRowPerm ? rowof(i) : i, M - 1);
    // x of the current chunk [ccs, cce) (the whole of K without XCH): offsets
    // of the row and of the row sums from xs, indexed by group - ccs.  (Kept
    // as offsets from xs: a pointer that changes inside the loop hides from
    // the compiler that x is not where the direct-to-LDS loads land, and it
    // then waits for all of them before each read of x.)
    int ccs = 0, cce = xg, chk = 0;
    int rofs = arow * xg * 128;                           // bf16 units
    int sofs = (M * xg * 128) / 2 + 4 * h;                // fp32 units
    const float *xsf = reinterpret_cast<const float *>(xs);
    int aoff[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) aoff[t] = swz(4 * h + t, arow) * 8;
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(out, (uint32_t)(M * N * 4));

    if (active) {
        for (int u = wave; u < nunit; u += kBalWaves) {
            if (!(burst && u == wave)) {
                setup_unit(u, true);
                prime();
            }
            float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            const uint8_t *sbase = smarea + i * unblk * 16;
            // Pair p from `slot`; the slot is refilled with pair p + ahead.
            auto pair = [&](int p, u32x4 *slot, int ahead) {
                u32x4 c0, c1;
                uint32_t sw, mw;
                if constexpr (DEEP) {
                    pair_reads(slot + boff0, slot + boff1, sbase + 4 * p, c0, c1, sw, mw);
                } else {
                    c0 = slot[boff0];
                    c1 = slot[boff1];
                    sw = *reinterpret_cast<const uint32_t *>(sbase + 4 * p);
                    mw = *reinterpret_cast<const uint32_t *>(sbase + 256 * nblm + 4 * p);
                }
                fill_at(slot, p + ahead, p + ahead < unp);
                __builtin_amdgcn_sched_barrier(0);
                const int g = ucs + 2 * p - ccs;                  // group within the staged x
                u32x4 a[4];
                f32x4 xsum;
#pragma unroll
                for (int t = 0; t < 4; ++t) a[t] = *reinterpret_cast<const u32x4 *>(xs + rofs + g * 128 + aoff[t]);
                xsum = *reinterpret_cast<const f32x4 *>(xsf + sofs + g * kXsRows);
                group_fma<RL>(a, xsum, c0, bf16_lo(sw), bf16_lo(mw), acc, uc);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    a[t] = *reinterpret_cast<const u32x4 *>(xs + rofs + (g + 1) * 128 + aoff[t]);
                xsum = *reinterpret_cast<const f32x4 *>(xsf + sofs + (g + 1) * kXsRows);
                group_fma<RL>(a, xsum, c1, bf16_hi(sw), bf16_hi(mw), acc, uc);
            };
            if (DEEP && deep) {
                // Slot k: own slots 0, 1, then the lent waves' (k / 2 - 1 past this one).
                for (int p0 = 0; p0 < unp; p0 += kDeepRing) {
#pragma unroll
                    for (int r = 0; r < kDeepRing; ++r) {
                        const int p = p0 + r;
                        if (p < unp) {
                            static_assert(kDeepRing == 8, "vmcnt(14): the 7 later pairs, two loads each");
                            asm volatile("s_waitcnt vmcnt(14)" ::: "memory");
                            pair(p, dslot(r), kDeepRing);
                        }
                    }
                }
            } else {
                for (int p0 = 0; p0 < unp; p0 += RD) {
#pragma unroll
                    for (int r = 0; r < RD; ++r) {
                        const int p = p0 + r;
                        if (XCH && ucs + 2 * p == cce) {
                            // Chunk end: this wave is done with the buffer; wait
                            // until every loader has staged its share of the next.
                            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                            ++chk;
                            if (lane == 0) lds_put(&xprog[wave], (uint32_t)chk);
                            lds_wait_all_geq(xprog + nunit, kBalWaves - nunit, (uint32_t)chk);
                            ccs = cce;
                            cce = min(ccs + xg, G);
                            const int bo = (chk & 1) * xstride;
                            rofs = bo + arow * (cce - ccs) * 128;
                            sofs = (bo + M * (cce - ccs) * 128) / 2 + 4 * h;
                        }
                        // Requested after pair p: RD - 1 pairs (refills past the
                        // last pair included).
                        wait_ring(RD - 1);
                        pair(p, rings[r] + slotw * kLdsSlotU4, RD);
                    }
                }
            }
            if (!PARTS) {
                if (ACT) {
                    float up[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) up[r] = __shfl_down(acc[r], 8);
                    if (i < ucw) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int row = kRowPerm ? rowof(4 * h + r) : 4 * h + r;
                            if (row < M) act[(size_t)row * NC + ucb + i] = swiglu_bf16(acc[r], up[r]);
                        }
                    }
                } else if (i < ucw) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int row = kRowPerm ? rowof(4 * h + r) : 4 * h + r;
                        if (row < M)
                            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, acc[r]), ry,
                                                                  (uint32_t)(row * N + ucb + i) * 4, 0, 0);
                    }
                }
            } else {
                *reinterpret_cast<f32x4 *>(slots + u * 256 + lane * 4) = f32x4{acc[0], acc[1], acc[2], acc[3]};
            }
        }
        // No load into this workgroup's LDS may still be in flight when its
        // waves end (the last refills were skipped, but make it explicit).
        __builtin_amdgcn_s_waitcnt(0);
    }
    if (PARTS) {
        lds_barrier();
        for (int k = wave; k < nchunk; k += kBalWaves) {
            int cb, cw;
            tile(k, cb, cw);
            f32x4 vs = *reinterpret_cast<const f32x4 *>(slots + (k * P) * 256 + lane * 4);
            for (int p = 1; p < P; ++p) vs += *reinterpret_cast<const f32x4 *>(slots + (k * P + p) * 256 + lane * 4);
            // (elements copied out one by one: this compiler bit-casts a vector
            // element expression as element 0)
            float v[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = vs[r];
            if (ACT) {
                float up[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) up[r] = __shfl_down(v[r], 8);
                if (i < cw) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int row = kRowPerm ? rowof(4 * h + r) : 4 * h + r;
                        if (row < M) act[(size_t)row * NC + cb + i] = swiglu_bf16(v[r], up[r]);
                    }
                }
            } else if (i < cw) {
                // EPI: out is h, and this workgroup's columns of h =
                // residual + y are stored at once (EPI 2: written through);
                // the residual loads go out before any store.
                float rv[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = kRowPerm ? rowof(4 * h + r) : 4 * h + r;
                    rv[r] = EPI && row < M ? na.r[(size_t)row * N + cb + i] : 0.0f;
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = kRowPerm ? rowof(4 * h + r) : 4 * h + r;
                    if (row < M) {
                        const float hv = EPI ? rv[r] + v[r] : v[r];
                        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, hv), ry,
                                                              (uint32_t)(row * N + cb + i) * 4, 0,
                                                              NORM ? kSysCoherent : 0);
                    }
                }
            }
        }
    }
    if (NORM) {
        // RMSNorm of the whole rows, done by the workgroup that finishes last.
        // Ordering: h was stored system-coherent (written through to memory,
        // acknowledged only once there); each workgroup waits for its stores'
        // acknowledgements before it counts itself in a system-scope atomic;
        // the atomics are ordered at memory, so the workgroup that reads the
        // count gx - 1 is the last and every h store is complete.  Its h loads
        // are issued only after that count has come back (a branch on it) and
        // bypass the caches (system-coherent), so they read the stored values.
        // The counter is left at zero for the next call.
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (tid == 0) {
            const uint32_t old = __hip_atomic_fetch_add(na.cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
            last_wg = old == (uint32_t)gx - 1 ? 1u : 0u;
        }
        __syncthreads();
        if (!last_wg) return;
        // Loads in batches of 8 per thread, all issued before the first is
        // used (one memory round trip per batch, not per element).
        constexpr int kB = 8;
        float *hl = reinterpret_cast<float *>(xs);        // one row of h, then its group sums (x is done)
        // gamma of the thread's first batch of columns, requested before h
        // (indexes clamped into [0, N), so every load is issued unconditionally)
        uint32_t g0[kB];
#pragma unroll
        for (int j = 0; j < kB; ++j) g0[j] = na.gamma[min(tid + j * kBalThreads, N - 1)];
        for (int m = 0; m < M; ++m) {
            const uint32_t row = (uint32_t)(m * N);
            for (int n0 = tid; n0 < N; n0 += kB * kBalThreads) {
                float t[kB];
#pragma unroll
                for (int j = 0; j < kB; ++j) {
                    const int n = n0 + j * kBalThreads;
                    t[j] = n < N ? __uint_as_float(
                                       __builtin_amdgcn_raw_buffer_load_b32(ry, (row + n) * 4, 0, kSysCoherent))
                                 : 0.0f;
                }
#pragma unroll
                for (int j = 0; j < kB; ++j)
                    if (n0 + j * kBalThreads < N) hl[n0 + j * kBalThreads] = t[j];
            }
            __syncthreads();
            const float tot = row_total<kBalThreads>([&](int n) { return hl[n]; }, N, hl + N);
            const float inv = rms_inv(tot, N, na.eps);
            for (int n0 = tid; n0 < N; n0 += kB * kBalThreads) {
                uint32_t g[kB];
#pragma unroll
                for (int j = 0; j < kB; ++j)
                    g[j] = n0 == tid ? g0[j] : na.gamma[min(n0 + j * kBalThreads, N - 1)];
#pragma unroll
                for (int j = 0; j < kB; ++j) {
                    const int n = n0 + j * kBalThreads;
                    if (n < N) na.xo[row + n] = bf16_rne((hl[n] * inv) * __uint_as_float(g[j] << 16));
                }
            }
            __syncthreads();                              // hl is reused by the next row
        }
        if (tid == 0) __hip_atomic_store(na.cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
}

// Partial sums of R elements e[j] (valid where ok[j]) over S splits,
// t[j] = P[0][e] + P[1][e] + ... + P[S-1][e] in ascending s.  The loads of up
// to BATCH splits are all issued before any is added, so a thread waits
// for ceil(S / BATCH) memory round trips, not S.
#ifndef Q4G128_SUM_BATCH
#define Q4G128_SUM_BATCH 4
#endif
constexpr int kSumBatch = Q4G128_SUM_BATCH;
// The one- and two-element reductions (splitk_sum, sum_swiglu) issue up to 8
// splits' loads before adding: the down projection's 6 splits then cost one
// memory round trip (13.46 -> 13.22 us per down call, same box).
constexpr int kSumBatchOne = 8;

template <int R, int BATCH = kSumBatch>
__device__ __forceinline__ void sum_partials(const float *__restrict__ P, int S, size_t MN, const size_t (&e)[R],
                                             const bool (&ok)[R], float (&t)[R])
{
#pragma unroll
    for (int j = 0; j < R; ++j) t[j] = 0.0f;
    for (int s0 = 0; s0 < S; s0 += BATCH) {
        float v[BATCH][R];
#pragma unroll
        for (int q = 0; q < BATCH; ++q)
#pragma unroll
            for (int j = 0; j < R; ++j)
                v[q][j] = (s0 + q < S && ok[j]) ? P[(size_t)(s0 + q) * MN + e[j]] : 0.0f;
#pragma unroll
        for (int q = 0; q < BATCH; ++q)
#pragma unroll
            for (int j = 0; j < R; ++j)
                if (s0 + q < S) t[j] = (s0 + q == 0) ? v[q][j] : t[j] + v[q][j];
    }
}

// y[e] = P[0][e] + P[1][e] + ... + P[S-1][e], in ascending s.
__global__ __launch_bounds__(256) void splitk_sum(const float *__restrict__ P, int S, size_t MN,
                                                  float *__restrict__ y)
{
    const size_t e0 = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t e[1] = {e0};
    const bool ok[1] = {e0 < MN};
    float t[1];
    sum_partials<1, kSumBatchOne>(P, S, MN, e, ok, t);
    if (ok[0]) y[e0] = t[0];
}

// act[m][i] = swiglu_bf16(sum_s P[s][m][i], sum_s P[s][m][I + i]), N = 2I,
// partials added in ascending s (as splitk_sum adds them).
__global__ __launch_bounds__(256) void sum_swiglu(const float *__restrict__ P, int S, int M, int N,
                                                  uint16_t *__restrict__ act)
{
    const int I = N >> 1;
    const size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= (size_t)M * I) return;
    const size_t m = e / I, i = e - m * I;
    const size_t MN = (size_t)M * N, eg = m * N + i;
    const size_t ee[2] = {eg, eg + I};
    const bool ok[2] = {true, true};
    float t[2];
    sum_partials<2, kSumBatchOne>(P, S, MN, ee, ok, t);
    act[e] = swiglu_bf16(t[0], t[1]);
}

// Residual add + RMSNorm with the split-K partial sums added inside the norm
// (Token Rush README, steps table rows 8-9).  One workgroup of 1024 threads
// per row m: thread t takes n = t, t + 1024, ...; y = sum_s P[s] in ascending
// s, h = r + y (written to h, which may be r itself); the row's sum of squares
// in the shared order (row_total), inv = 1 / sqrt(ss / N + eps) (correctly
// rounded), x_out = bf16((h * inv) * gamma).
//   MODE 0: h and x_out.  MODE 1: h only (gamma, xo unused).  MODE 2: no
//   product: h is r itself (read only, P and S unused), x_out only.
// PT > 0: the thread's h values stay in registers (N <= 1024 PT) and the row
// is also put in LDS for the sum of squares; PT == 0: it is read back from h
// (r for MODE 2).  Dynamic LDS: (PT > 0 ? N : 0) + ceil(N/128) floats.
#ifndef Q4G128_NORM_THREADS
#define Q4G128_NORM_THREADS 1024
#endif
constexpr int kNormThreads = Q4G128_NORM_THREADS;

template <int MODE, int PT>
__global__ __launch_bounds__(kNormThreads) void sum_residual_rmsnorm(const float *__restrict__ P, int S, int M,
                                                                     int N, const float *r,
                                                                     const uint16_t *__restrict__ gamma, float eps,
                                                                     float *h, uint16_t *__restrict__ xo)
{
    extern __shared__ float hl[];
    const int m = blockIdx.x;
    const int tid = threadIdx.x;
    const size_t MN = (size_t)M * N;
    const size_t row = (size_t)m * N;
    constexpr int R = PT > 0 ? PT : 1;
    float hv[R];
    const int passes = PT > 0 ? PT : (N + kNormThreads - 1) / kNormThreads;
    if (PT > 0) {
        // Every load first (r and h may be the same array, so a store to h
        // would otherwise hold back the next element's loads), then h.
        float rv[R];
        size_t e[R];
        bool ok[R];
#pragma unroll
        for (int j = 0; j < R; ++j) {
            const int n = tid + j * kNormThreads;
            e[j] = row + n;
            ok[j] = n < N;
            rv[j] = ok[j] ? r[e[j]] : 0.0f;
        }
        if (MODE != 2) sum_partials<R>(P, S, MN, e, ok, hv);
#pragma unroll
        for (int j = 0; j < R; ++j) {
            const int n = tid + j * kNormThreads;
            const float v = MODE == 2 ? rv[j] : rv[j] + hv[j];
            if (n < N) {
                if (MODE != 2) h[row + n] = v;
                if (MODE != 1) hl[n] = v;
            }
            hv[j] = v;
        }
    } else if (MODE != 2) {
        // Wide rows: the same steps on chunks of 8 of the thread's elements
        // (loads of a chunk batched), h read back afterwards.
        for (int j0 = 0; j0 < passes; j0 += 8) {
            size_t e[8];
            bool ok[8];
            float t[8], rv[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int n = tid + (j0 + j) * kNormThreads;
                e[j] = row + n;
                ok[j] = j0 + j < passes && n < N;
                rv[j] = ok[j] ? r[e[j]] : 0.0f;
            }
            sum_partials<8>(P, S, MN, e, ok, t);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float v = rv[j] + t[j];
                if (ok[j]) h[e[j]] = v;
            }
        }
    }
    if (MODE == 1) return;
    // The row's sum of squares in the shared order: from LDS, or (PT == 0)
    // read back from h, just written by this workgroup (the barrier makes the
    // writes visible), or from r (MODE 2).
    __syncthreads();
    const float *hr = (MODE == 2 ? r : h) + row;
    float *gsum = hl + (PT > 0 ? N : 0);
    const float tot = PT > 0 ? row_total<kNormThreads>([&](int n) { return hl[n]; }, N, gsum)
                             : row_total<kNormThreads>([&](int n) { return hr[n]; }, N, gsum);
    const float inv = rms_inv(tot, N, eps);
    for (int j = 0; j < passes; ++j) {
        const int n = tid + j * kNormThreads;
        if (n < N) {
            const float v = PT > 0 ? hv[PT > 0 ? j : 0] : hr[n];   // PT == 0: this thread's own h
            const float gm = __uint_as_float((uint32_t)gamma[n] << 16);
            xo[row + n] = bf16_rne((v * inv) * gm);
        }
    }
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

// ---- library-owned scratch ---------------------------------------------------

// Split-K partial sums of q4g128_gemm_splitk_noalloc.  Every call on a GPU
// shares that GPU's copy; calls that overlap on one GPU race on it.
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

hipError_t scratch_pointer(float **p)
{
    static std::atomic<float *> ptr[kMaxDevices];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    float *v = ptr[dev].load(std::memory_order_relaxed);
    if (!v) {
        void *addr = nullptr;
        e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));   // this device's copy, with it current
        if (e != hipSuccess) return e;
        v = static_cast<float *>(addr);
        ptr[dev].store(v, std::memory_order_relaxed);         // every thread stores the same address
    }
    *p = v;
    return hipSuccess;
}

// ---- launchers ---------------------------------------------------------------

int waves_for(int M) { return M <= kSmallM ? kWavesSmall : kWavesLarge; }

int columns_per_block(int tpw, int M) { return waves_for(M) * 16 * tpw; }

int chunk_groups(int M)
{
    int cg = kStageMax * 64 * waves_for(M) / 16 / M;   // pieces per thread <= kStageMax
    cg = cg / 16 * 16;
    return cg < 16 ? 16 : cg;
}

template <int TPW, bool CHUNKED, bool VSM, int WAVES>
static hipError_t launch_one(const GemvArgs &a, dim3 grid, int cg, hipStream_t stream)
{
    // x for up to 16 rows of a chunk can pass 64 KiB (66.5 KiB at M = 16).
    static LdsRoom room;
    const size_t lds = (size_t)a.M * (size_t)cg * 128 * 2 + (size_t)cg * kXsRows * 4;
    const hipError_t attr = lds_launch_ok(
        reinterpret_cast<const void *>(&gemv_q4g128<TPW, CHUNKED, VSM, kRingDepth, WAVES>), lds, room);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((gemv_q4g128<TPW, CHUNKED, VSM, kRingDepth, WAVES>), grid, dim3(64 * WAVES, 1, 1), lds,
                       stream, a.x, a.M, a.K, a.W, a.scale, a.mn, a.N, a.out, a.S, cg);
    return hipGetLastError();
}

template <int WAVES>
static hipError_t launch_waves(const GemvArgs &a, dim3 grid, bool chunked, bool vsm, int cg, int span,
                               hipStream_t stream)
{
    if (vsm) {
        if (chunked) return launch_one<1, true, true, WAVES>(a, grid, cg, stream);
        return launch_one<1, false, true, WAVES>(a, grid, span, stream);
    }
    if (chunked) return launch_one<1, true, false, WAVES>(a, grid, cg, stream);
    return launch_one<1, false, false, WAVES>(a, grid, span, stream);
}

hipError_t launch_gemv(const GemvArgs &a, int tpw, hipStream_t stream)
{
    if (tpw != 1) return hipErrorInvalidValue;
    const int waves = waves_for(a.M);
    const int cpb = columns_per_block(tpw, a.M);
    // The widest split spans ceil(nb/S) blocks of 8 groups, or ceil(G/S)
    // groups when there are more splits than blocks.
    const int G = a.K / 128;
    const int nb = (G + kRing - 1) / kRing;
    const bool fine = a.S > nb;
    const int span = fine ? (G + a.S - 1) / a.S : (nb + a.S - 1) / a.S * kRing;
    const int cg = chunk_groups(a.M);
    const bool chunked = span > cg;
    // 16-byte scale/minimum loads need K/128 a multiple of 8, aligned bases
    // and ranges of whole blocks.
    const bool vsm = !fine && G % 8 == 0 && (reinterpret_cast<uintptr_t>(a.scale) & 15) == 0 &&
                     (reinterpret_cast<uintptr_t>(a.mn) & 15) == 0;
    dim3 grid((unsigned)((a.N + cpb - 1) / cpb), (unsigned)a.S, 1);
    if (waves == kWavesSmall) return launch_waves<kWavesSmall>(a, grid, chunked, vsm, cg, span, stream);
    return launch_waves<kWavesLarge>(a, grid, chunked, vsm, cg, span, stream);
}

BalPlan bal_plan(int M, int K, int N, int S, int gx, int P, bool act)
{
    BalPlan bp;
    const int nb = K / 1024;
    const int ngmax = (nb + S - 1) / S * 8;
    int tiles;                                                  // most tiles of one workgroup
    if (act) {
        const int NU = (N / 2 + 3) / 4;
        tiles = ((NU + gx - 1) / gx * 4 + 7) / 8;               // tiles of at most 8 gate/up pairs
    } else {
        const int N4 = (N + 3) / 4;
        tiles = ((N4 + gx - 1) / gx * 4 + 15) / 16;
    }
    const int units = tiles * P;
    const int nw = units < kBalWaves ? units : kBalWaves;
    bp.pair = kBalPair && units >= kBalPairUnits;
    const int pg = P > 1 ? (ngmax / 8 + P - 1) / P * 8 : ngmax;        // longest part, in groups
    bp.nblp = ((pg + 7) / 8) | 1;
    bp.nps = P > 1 ? units : 0;
    bp.lds = (size_t)M * ngmax * 256 + (size_t)ngmax * kXsRows * 4 + (size_t)bp.nps * 1024 +
             (size_t)(kBalSml ? nw : 0) * 2 * 16 * bp.nblp * 16;
    if (bp.lds < kBalOwnCu) bp.lds = kBalOwnCu;
    return bp;
}

template <bool PARTS, bool ACT, int RL, bool PAIR, bool XN>
static hipError_t launch_bal_v(const GemvArgs &a, int gx, int P, const BalPlan &bp, const NormArgs &na,
                               hipStream_t stream)
{
    static LdsRoom room;
    const hipError_t attr = lds_launch_ok(
        reinterpret_cast<const void *>(&gemv_q4g128_bal<kBalRing, kBalSml, PARTS, ACT, RL, PAIR, XN>), bp.lds, room);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((gemv_q4g128_bal<kBalRing, kBalSml, PARTS, ACT, RL, PAIR, XN>),
                       dim3((unsigned)gx, (unsigned)a.S, 1), dim3(kBalThreads, 1, 1), bp.lds, stream, a.x, a.M, a.K,
                       a.W, a.scale, a.mn, a.N, a.out, a.act, a.S, bp.nblp, P, bp.nps, na);
    return hipGetLastError();
}

template <bool PARTS, bool ACT, int RL, bool XN = false>
static hipError_t launch_bal_rl(const GemvArgs &a, int gx, int P, const NormArgs &na, hipStream_t stream)
{
    const BalPlan bp = bal_plan(a.M, a.K, a.N, a.S, gx, P, ACT);
    return bp.pair ? launch_bal_v<PARTS, ACT, RL, true, XN>(a, gx, P, bp, na, stream)
                   : launch_bal_v<PARTS, ACT, RL, false, XN>(a, gx, P, bp, na, stream);
}

// Rows accumulate ceil(M/4) D rows per lane (rowpos).
template <bool PARTS, bool ACT>
static hipError_t launch_bal(const GemvArgs &a, int gx, int P, hipStream_t stream)
{
    const NormArgs na{};
    if (kBalOneRow && (a.M == 1 || (kRowPerm && a.M <= 4))) return launch_bal_rl<PARTS, ACT, 1>(a, gx, P, na, stream);
    if (kRowPerm && a.M <= 8) return launch_bal_rl<PARTS, ACT, 2>(a, gx, P, na, stream);
    if (kRowPerm && a.M <= 12) return launch_bal_rl<PARTS, ACT, 3>(a, gx, P, na, stream);
    return launch_bal_rl<PARTS, ACT, 4>(a, gx, P, na, stream);
}

// XN on the register-ring kernel: S == 1, M <= 8.
template <bool PARTS, bool ACT>
static hipError_t launch_bal_xn(const GemvArgs &a, int gx, int P, const NormArgs &na, hipStream_t stream)
{
    if (a.S != 1 || a.M > 8 || !kRowPerm || !kBalOneRow) return hipErrorInvalidValue;
    return a.M <= 4 ? launch_bal_rl<PARTS, ACT, 1, true>(a, gx, P, na, stream)
                    : launch_bal_rl<PARTS, ACT, 2, true>(a, gx, P, na, stream);
}

LdsPlan lds_plan(int M, int K, int N, int gx, int P, bool act, int rd, bool burst, bool nr)
{
    LdsPlan lp;
    const int G = K / 128, nb = G / 8;
    int tiles;
    if (act) {
        const int NU = (N / 2 + 3) / 4;
        tiles = ((NU + gx - 1) / gx * 4 + 7) / 8;
    } else {
        const int N4 = (N + 3) / 4;
        tiles = ((N4 + gx - 1) / gx * 4 + 15) / 16;
    }
    const int units = tiles * P;
    const int nact = units < kBalWaves ? units : kBalWaves;
    lp.nblm = P > 1 ? (nb + P - 1) / P : nb;
    lp.nps = P > 1 ? units : 0;
    // Static LDS: the rings, the burst area, and 256 bytes for the kernel's
    // small arrays (counters, the 1/rms table); the launcher checks the
    // kernel's actual static size too.
    const size_t rw = nr ? kNarrowRingWaves + 1 : kBalWaves;
    const size_t stat = (size_t)(rd > 2 ? 4 : 2) * rw * kLdsSlotU4 * 16 + (rd > 2 ? 0 : 32) +
                        (burst ? rw * 512 * kLdsBurstBlocks : 16) + 256;
    lp.fits = !burst || lp.nblm <= kLdsBurstBlocks;
    // x staged whole passes through kBalStage registers per thread.
    lp.fits = lp.fits && (long)M * G * 16 <= (long)kBalThreads * kBalStage;
    if (nr) lp.fits = lp.fits && P == 1 && rd == 2 && tiles <= kNarrowRingWaves;
    lp.lds = (size_t)M * G * 256 + (size_t)G * kXsRows * 4 + (size_t)lp.nps * 1024 +
             (burst ? 0 : (size_t)nact * 512 * lp.nblm);
    if (lp.lds + stat < kBalOwnCu) lp.lds = kBalOwnCu - stat;
    lp.total = lp.lds + stat;
    lp.fits = lp.fits && lp.total <= kBalMaxLds;
    return lp;
}

template <int RD, bool PARTS, bool ACT, int RL, bool BURST, int EPI = 0, bool XN = false, bool XCH = false,
          bool NR = false>
static hipError_t launch_lds_v(const GemvArgs &a, int gx, int P, const LdsPlan &lp, const NormArgs &na,
                               hipStream_t stream)
{
    static LdsRoom room;
    const void *k = reinterpret_cast<const void *>(&gemv_q4g128_lds<RD, PARTS, ACT, RL, BURST, EPI, XN, XCH, NR>);
    const hipError_t attr = lds_launch_ok(k, lp.lds, room);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((gemv_q4g128_lds<RD, PARTS, ACT, RL, BURST, EPI, XN, XCH, NR>), dim3((unsigned)gx, 1, 1),
                       dim3(kBalThreads, 1, 1), lp.lds, stream, a.x, a.M, a.K, a.W, a.scale, a.mn, a.N, a.out, a.act,
                       P, lp.nps, lp.nblm, na, lp.xcg);
    return hipGetLastError();
}

LdsPlan lds_plan_xch(int M, int K, int N, int gx, bool act)
{
    LdsPlan lp = lds_plan(M, K, N, gx, 1, act, 2, false);
    lp.fits = false;
    const int G = K / 128;
    int tiles;
    if (act) {
        const int NU = (N / 2 + 3) / 4;
        tiles = ((NU + gx - 1) / gx * 4 + 7) / 8;
    } else {
        const int N4 = (N + 3) / 4;
        tiles = ((N4 + gx - 1) / gx * 4 + 15) / 16;
    }
    if (M > 16 || tiles >= kBalWaves || G < 4) return lp;
    const size_t stat = lp.total - lp.lds;
    const size_t sm = (size_t)tiles * 512 * lp.nblm;          // the tile waves' scale/minimum areas
    // The largest even chunk whose two buffers fit, then the most even cut
    // into that many chunks; chunk 0 is staged by every thread (kBalStage
    // pieces each at most).
    int cg = 0;
    for (int c = 2; c <= G && M * c * 16 <= kBalThreads * kBalStage; c += 2)
        if (stat + 2 * ((size_t)M * c * 256 + (size_t)c * kXsRows * 4) + sm <= kBalMaxLds) cg = c;
    if (cg == 0) return lp;
    const int nch = (G + cg - 1) / cg;
    if (nch < 2) return lp;                                    // fits whole: no chunks needed
    cg = ((G + nch - 1) / nch + 1) & ~1;
    lp.xcg = cg;
    lp.nps = 0;
    lp.lds = 2 * ((size_t)M * cg * 256 + (size_t)cg * kXsRows * 4) + sm;
    if (lp.lds + stat < kBalOwnCu) lp.lds = kBalOwnCu - stat;
    lp.total = lp.lds + stat;
    lp.fits = lp.total <= kBalMaxLds;
    return lp;
}

// Chunked x, x staged first (the burst order, each wave's first tile
// requested before chunk 0, was slower here: M = 12 23.8 against 22.1 us,
// M = 16 25.5 against 25.1 us, one box).
hipError_t launch_gemv_xch(const GemvArgs &a, int gx, hipStream_t stream)
{
    const LdsPlan lp = lds_plan_xch(a.M, a.K, a.N, gx, a.act != nullptr);
    if (!lp.fits || a.S != 1 || a.M <= 8) return hipErrorInvalidValue;
    const NormArgs na{};
    if (a.act)
        return a.M <= 12 ? launch_lds_v<2, false, true, 3, false, 0, false, true>(a, gx, 1, lp, na, stream)
                         : launch_lds_v<2, false, true, 4, false, 0, false, true>(a, gx, 1, lp, na, stream);
    return a.M <= 12 ? launch_lds_v<2, false, false, 3, false, 0, false, true>(a, gx, 1, lp, na, stream)
                     : launch_lds_v<2, false, false, 4, false, 0, false, true>(a, gx, 1, lp, na, stream);
}

template <int RD, bool PARTS, bool ACT, bool BURST>
static hipError_t launch_lds_rl(const GemvArgs &a, int gx, int P, hipStream_t stream)
{
    const LdsPlan lp = lds_plan(a.M, a.K, a.N, gx, P, ACT, RD, BURST);
    if (!lp.fits) return hipErrorInvalidValue;
    const NormArgs na{};
    if (a.M <= 4) return launch_lds_v<RD, PARTS, ACT, 1, BURST>(a, gx, P, lp, na, stream);
    if (a.M <= 8) return launch_lds_v<RD, PARTS, ACT, 2, BURST>(a, gx, P, lp, na, stream);
    if (a.M <= 12) return launch_lds_v<RD, PARTS, ACT, 3, BURST>(a, gx, P, lp, na, stream);
    return launch_lds_v<RD, PARTS, ACT, 4, BURST>(a, gx, P, lp, na, stream);
}

bool lds_epi_fits(int M, int K, int N, int gx, int P, int epi)
{
    const LdsPlan lp = lds_plan(M, K, N, gx, P, false, 2, true);
    const size_t tail = epi == 2 ? (size_t)(N + (N + 127) / 128) * sizeof(float) : 0;
    return P > 1 && M <= 8 && lp.fits && lp.lds >= tail;
}

hipError_t launch_gemv_lds_epi(const GemvArgs &a, int gx, int P, int epi, const NormArgs &na, hipStream_t stream)
{
    if (a.S != 1 || a.act || (epi != 1 && epi != 2) || !lds_epi_fits(a.M, a.K, a.N, gx, P, epi))
        return hipErrorInvalidValue;
    const LdsPlan lp = lds_plan(a.M, a.K, a.N, gx, P, false, 2, true);
    if (epi == 1)
        return a.M <= 4 ? launch_lds_v<2, true, false, 1, true, 1>(a, gx, P, lp, na, stream)
                        : launch_lds_v<2, true, false, 2, true, 1>(a, gx, P, lp, na, stream);
    return a.M <= 4 ? launch_lds_v<2, true, false, 1, true, 2>(a, gx, P, lp, na, stream)
                    : launch_lds_v<2, true, false, 2, true, 2>(a, gx, P, lp, na, stream);
}

// XN on the LDS-fed kernel, ring 2: burst (each wave's first tile requested
// before h and gamma, its ring primed before the norm) where it fits, else
// x made first.
template <bool PARTS, bool ACT>
static hipError_t launch_lds_xn(const GemvArgs &a, int gx, int P, const NormArgs &na, hipStream_t stream)
{
    if (a.M > 8) return hipErrorInvalidValue;
    const LdsPlan lb = lds_plan(a.M, a.K, a.N, gx, P, ACT, 2, true);
    if (lb.fits)
        return a.M <= 4 ? launch_lds_v<2, PARTS, ACT, 1, true, 0, true>(a, gx, P, lb, na, stream)
                        : launch_lds_v<2, PARTS, ACT, 2, true, 0, true>(a, gx, P, lb, na, stream);
    const LdsPlan lp = lds_plan(a.M, a.K, a.N, gx, P, ACT, 2, false);
    if (!lp.fits) return hipErrorInvalidValue;
    return a.M <= 4 ? launch_lds_v<2, PARTS, ACT, 1, false, 0, true>(a, gx, P, lp, na, stream)
                    : launch_lds_v<2, PARTS, ACT, 2, false, 0, true>(a, gx, P, lp, na, stream);
}

hipError_t launch_gemv_xn(const GemvArgs &a, int gx, int P, bool lds, const NormArgs &na, hipStream_t stream)
{
    if (a.S != 1 || a.M > 8) return hipErrorInvalidValue;
    if (lds) {
        if (P > 1) return a.act ? hipErrorInvalidValue : launch_lds_xn<true, false>(a, gx, P, na, stream);
        return a.act ? launch_lds_xn<false, true>(a, gx, 1, na, stream) : launch_lds_xn<false, false>(a, gx, 1, na, stream);
    }
    if (P > 1) return hipErrorInvalidValue;
    return a.act ? launch_bal_xn<false, true>(a, gx, 1, na, stream) : launch_bal_xn<false, false>(a, gx, 1, na, stream);
}

bool xn_fits(int M, int K, int N, int gx, int P, bool act, bool lds)
{
    if (M > 8) return false;
    if (lds) return (P == 1 || !act) && lds_plan(M, K, N, gx, P, act, 2, false).fits;
    return P == 1;
}

// NR: burst form, ring 2, whole K, M = 5-16 (2 to 4 accumulated rows; the
// plan admits it where x leaves the 12-wave burst form too little LDS: M = 8,
// 9 at K = 5120, 10, 11 at 4096, 14, 15 at 3072).
template <bool ACT>
static hipError_t launch_lds_nr(const GemvArgs &a, int gx, hipStream_t stream)
{
    const LdsPlan lp = lds_plan(a.M, a.K, a.N, gx, 1, ACT, 2, true, true);
    if (!lp.fits || a.M < 5 || a.M > 16) return hipErrorInvalidValue;
    const NormArgs na{};
    if (a.M <= 8) return launch_lds_v<2, false, ACT, 2, true, 0, false, false, true>(a, gx, 1, lp, na, stream);
    if (a.M <= 12) return launch_lds_v<2, false, ACT, 3, true, 0, false, false, true>(a, gx, 1, lp, na, stream);
    return launch_lds_v<2, false, ACT, 4, true, 0, false, false, true>(a, gx, 1, lp, na, stream);
}

hipError_t launch_gemv_lds(const GemvArgs &a, int gx, int P, int rd, bool burst, bool nr, hipStream_t stream)
{
    if (a.S != 1) return hipErrorInvalidValue;
    if (nr) {
        if (rd != 2 || !burst || P != 1) return hipErrorInvalidValue;
        return a.act ? launch_lds_nr<true>(a, gx, stream) : launch_lds_nr<false>(a, gx, stream);
    }
    if (a.act) {
        if (rd != 2 || (burst && P > 1)) return hipErrorInvalidValue;
        if (burst) return launch_lds_rl<2, false, true, true>(a, gx, 1, stream);
        return P > 1 ? launch_lds_rl<2, true, true, false>(a, gx, P, stream)
                     : launch_lds_rl<2, false, true, false>(a, gx, 1, stream);
    }
    if (!burst) {
        if (rd != 2) return hipErrorInvalidValue;
        return P > 1 ? launch_lds_rl<2, true, false, false>(a, gx, P, stream)
                     : launch_lds_rl<2, false, false, false>(a, gx, 1, stream);
    }
    if (rd > 2)
        return P > 1 ? launch_lds_rl<4, true, false, true>(a, gx, P, stream)
                     : launch_lds_rl<4, false, false, true>(a, gx, 1, stream);
    return P > 1 ? launch_lds_rl<2, true, false, true>(a, gx, P, stream)
                 : launch_lds_rl<2, false, false, true>(a, gx, 1, stream);
}

hipError_t launch_gemv_bal(const GemvArgs &a, int gx, int P, hipStream_t stream)
{
    if (a.act) return P > 1 ? launch_bal<true, true>(a, gx, P, stream) : launch_bal<false, true>(a, gx, 1, stream);
    return P > 1 ? launch_bal<true, false>(a, gx, P, stream) : launch_bal<false, false>(a, gx, 1, stream);
}

hipError_t launch_splitk_sum(const float *P, int S, size_t MN, float *y, hipStream_t stream)
{
    dim3 grid((unsigned)((MN + 255) / 256), 1, 1);
    hipLaunchKernelGGL(splitk_sum, grid, dim3(256, 1, 1), 0, stream, P, S, MN, y);
    return hipGetLastError();
}

hipError_t launch_sum_swiglu(const float *P, int S, int M, int N, uint16_t *act, hipStream_t stream)
{
    const size_t MI = (size_t)M * (size_t)(N / 2);
    hipLaunchKernelGGL(sum_swiglu, dim3((unsigned)((MI + 255) / 256), 1, 1), dim3(256, 1, 1), 0, stream, P, S, M, N,
                       act);
    return hipGetLastError();
}

// 16 elements per thread in registers only while the batched loads fit too.
constexpr bool kNormPt16 = kSumBatch * 16 <= 64;

template <int MODE>
static hipError_t launch_srn(const float *P, int S, int M, int N, const float *r, const uint16_t *gamma, float eps,
                             float *h, uint16_t *xo, hipStream_t stream)
{
    const dim3 grid((unsigned)M, 1, 1), block(kNormThreads, 1, 1);
    const int pt = (N + kNormThreads - 1) / kNormThreads;
    const size_t gl = (size_t)((N + 127) / 128) * sizeof(float);
    const size_t lds = (size_t)N * sizeof(float) + gl;
    if (lds > 64 * 1024)                                       // the row does not fit the default LDS limit
        hipLaunchKernelGGL((sum_residual_rmsnorm<MODE, 0>), grid, block, gl, stream, P, S, M, N, r, gamma, eps, h, xo);
    else if (pt <= 2)
        hipLaunchKernelGGL((sum_residual_rmsnorm<MODE, 2>), grid, block, lds, stream, P, S, M, N, r, gamma, eps, h, xo);
    else if (pt <= 8)
        hipLaunchKernelGGL((sum_residual_rmsnorm<MODE, 8>), grid, block, lds, stream, P, S, M, N, r, gamma, eps, h, xo);
    else if (pt <= 16 && kNormPt16)
        hipLaunchKernelGGL((sum_residual_rmsnorm<MODE, kNormPt16 ? 16 : 8>), grid, block, lds, stream, P, S, M, N, r,
                           gamma, eps, h, xo);
    else
        hipLaunchKernelGGL((sum_residual_rmsnorm<MODE, 0>), grid, block, gl, stream, P, S, M, N, r, gamma, eps, h, xo);
    return hipGetLastError();
}

hipError_t launch_sum_residual_rmsnorm(const float *P, int S, int M, int N, const float *r, const uint16_t *gamma,
                                       float eps, float *h, uint16_t *xo, hipStream_t stream)
{
    if (!xo) return launch_srn<1>(P, S, M, N, r, nullptr, 0.0f, h, nullptr, stream);
    return launch_srn<0>(P, S, M, N, r, gamma, eps, h, xo, stream);
}

hipError_t launch_rmsnorm(const float *h, int M, int N, const uint16_t *gamma, float eps, uint16_t *xo,
                          hipStream_t stream)
{
    return launch_srn<2>(nullptr, 0, M, N, h, gamma, eps, nullptr, xo, stream);
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
