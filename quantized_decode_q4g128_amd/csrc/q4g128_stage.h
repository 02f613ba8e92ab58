// Device helpers shared by the product kernels: workgroup barrier, x staging
// in LDS (with the per-group row sums) and small bit utilities.  Both kernels
// stage x with exactly this code, so they feed identical operands and row
// sums to their MFMAs.
#pragma once

#include "q4g128_device.h"

namespace q4g128 {

// All outstanding LDS operations of this wave complete, then a workgroup
// barrier.  Outstanding global loads (the code prefetch) stay in flight.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// bf16 number j (0..7, a compile-time constant) of eight packed in a u32x4.
__device__ __forceinline__ float bf16_at(const u32x4 &v, int j)
{
    const uint32_t w = j < 2 ? v.x : j < 4 ? v.y : j < 6 ? v.z : v.w;
    return (j & 1) ? bf16_hi(w) : bf16_lo(w);
}

// x in LDS: row r of the staged range holds its 16-byte blocks (8 bf16 in
// pair order) with block index b stored at b ^ (r & 15) (the XOR stays
// inside the group's 16 blocks).  The 16 lanes of one row block read up to
// 16 different rows at the same block index; the XOR spreads them over 16
// different 16-byte bank groups, without padding rows.
__device__ __forceinline__ int swz(int blk, int row) { return blk ^ (row & 15); }

// Row-sum slots per staged group: Xs[g][row], one per MFMA row (M <= 16);
// rows >= M are never written and their results never stored.
constexpr int kXsRows = 16;

// Sum of a float over each row of 16 lanes, by a fixed tree; lane 15 of the
// row ends with the total.
__device__ __forceinline__ float row16_sum(float v)
{
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x111, 0xf, 0xf, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x112, 0xf, 0xf, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x114, 0xf, 0xf, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x118, 0xf, 0xf, false));
    return v;
}

// ---- RMSNorm: one sum-of-squares order for every kernel that normalises ----
//
// A row h[0..n) is cut into blocks of 8 consecutive elements.  Block partial:
// the fmaf chain v*v over the block's elements in ascending order, from 0.
// 128-group sum: row16_sum's tree over the group's 16 block partials (a
// balanced pairwise tree; absent blocks of a short last group are 0).  Row
// total: 64 lane partials, lane l the sum of the group sums g = l, l + 64,
// ... in ascending g (from 0), then a butterfly over the 64 lanes (every lane
// adds the same pairs, so every lane ends with the same total).  Every path
// that normalises a row (the product's x staging, the norm after the product,
// the one-launch norm) takes these steps, so a row's x does not depend on
// which path served it.  1/rms = 1 / sqrt(total / n + eps), both correctly
// rounded (RMSNorm as the gated-MLP decoder family defines it).

__device__ __forceinline__ uint16_t bf16_rne(float a)
{
    const uint32_t b = __float_as_uint(a);
    if ((b & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;
    return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

// Block partial of the first nv (<= 8) of v.
__device__ __forceinline__ float block_sumsq(const float (&v)[8], int nv)
{
    float s = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e)
        if (e < nv) s = fmaf(v[e], v[e], s);
    return s;
}

// Row total from the group sums gs(g), g < ng, read by every lane of the
// calling wave (all 64 lanes active); every lane returns the total.
template <class GS>
__device__ __forceinline__ float groups_total(const GS &gs, int ng)
{
    const int lane = (int)(threadIdx.x & 63);
    float q = 0.0f;
    for (int g = lane; g < ng; g += 64) q += gs(g);
    for (int off = 32; off > 0; off >>= 1) q += __shfl_xor(q, off);
    return q;
}

__device__ __forceinline__ float rms_inv(float total, int n, float eps)
{
    return 1.0f / sqrtf(total / (float)n + eps);
}

// Row total of h[0..n), h(i) yielding element i, by a workgroup of NT
// threads (a multiple of 16; all of them call it): thread t takes blocks
// t, t + NT, ... so a 16-lane row holds 16 consecutive blocks; gsum:
// ceil(n/128) floats of LDS.  Every thread returns the total.
template <int NT, class H>
__device__ __forceinline__ float row_total(const H &h, int n, float *gsum)
{
    const int tid = threadIdx.x;
    const int nblk = (n + 7) >> 3, ng = (n + 127) >> 7;
    const int rounds = (nblk + NT - 1) / NT;
    for (int j = 0; j < rounds; ++j) {
        const int b = tid + j * NT;
        const int nv = b < nblk ? min(8, n - 8 * b) : 0;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = e < nv ? h(8 * b + e) : 0.0f;
        const float t = row16_sum(block_sumsq(v, nv));
        if ((tid & 15) == 15 && (b >> 4) < ng) gsum[b >> 4] = t;
    }
    __syncthreads();
    const float tot = groups_total([&](int g) { return gsum[g]; }, ng);
    __syncthreads();                                      // gsum may be reused
    return tot;
}

// x = bf16((h * inv) * gamma) for the 8 elements of a block, packed two to a
// word, lower element in the low half (the layout of x in memory).
__device__ __forceinline__ u32x4 norm_pack(const f32x4 &ha, const f32x4 &hb, const u32x4 &g, float inv)
{
    // (elements copied to scalars first: this compiler bit-casts a vector
    // element expression as element 0)
    const float h[8] = {ha.x, ha.y, ha.z, ha.w, hb.x, hb.y, hb.z, hb.w};
    const uint32_t gw[4] = {g.x, g.y, g.z, g.w};
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t lo = bf16_rne((h[2 * i] * inv) * bf16_lo(gw[i]));
        const uint32_t hi = bf16_rne((h[2 * i + 1] * inv) * bf16_hi(gw[i]));
        w[i] = lo | (hi << 16);
    }
    return u32x4{w[0], w[1], w[2], w[3]};
}

// MFMA row of x row m (0..15) and its inverse: x row m = 4r + h sits in MFMA
// row 4h + r.  Lane i + 16h holds D rows 4h..4h+3, so x rows 0..3 land in the
// first D row of the four lane groups, rows 4..7 in the second, and so on:
// an M-row product accumulates ceil(M/4) D rows per lane, not four.  Every
// x row sits in the same MFMA row for every M.
__device__ __forceinline__ int rowpos(int m) { return 4 * (m & 3) + (m >> 2); }
__device__ __forceinline__ int rowof(int j) { return 4 * (j & 3) + (j >> 2); }

// Stage x[0..M)[cs*128 .. ce*128) into LDS (swizzled, pair order) and the
// row sums Xs[g - cs][row] of each 128-group.  Piece p is 16 bytes: row
// p / pr, block p % pr, pr = 16 * (ce - cs); the 16 pieces of one (row,
// group) sit in one 16-lane row of a wave, whose lanes add their pieces'
// sums by a fixed tree.  NT threads take at most SMAX pieces each.
//
// load() issues the global reads; store() waits for them and writes LDS.
// Loads issued between the two (the first code loads) stay in flight: the
// wait only covers memory operations older than them.
// RP: row m's sums go to MFMA row rowpos(m) (the product kernels place x row
// m there); else to row m.
//
// NORM: x is not read but made from fp32 rows h (x = the RMSNorm of h, in
// the order above, times gamma, rounded to bf16): load_norm() issues the
// loads of h and gamma for whole rows (cs = 0, ce = K/128), norm() forms the
// rows' 1/rms (it uses the row-sum area Xs as scratch and ends with a
// barrier), then store() packs x and proceeds as for loaded x.
template <int NT, int SMAX, bool RP = false, bool NORM = false>
struct XStage {
    u32x4 st[SMAX];                              // x pieces; NORM: gamma pieces
    f32x4 ha[NORM ? SMAX : 1], hb[NORM ? SMAX : 1];   // NORM: h elements 0-3, 4-7
    float inv_l;                                 // NORM: lane r (< M) holds row r's 1/rms
    int pieces, pr;

    // Piece tid + NT*j lies at (row0 + j*dq + carries, blk0 + j*dr - carries*pr):
    // one division per thread, then an add and a compare per round.
    int row0, blk0, dq, dr;

    __device__ __forceinline__ void load(const uint16_t *__restrict__ x, int M, int K, int cs, int ce)
    {
        const int tid = threadIdx.x;
        pr = (ce - cs) * 16;
        pieces = M * pr;
        row0 = tid / pr;
        blk0 = tid - row0 * pr;
        dq = NT / pr;
        dr = NT - dq * pr;
        int row = row0, blk = blk0;
#pragma unroll
        for (int j = 0; j < SMAX; ++j) {
            if (NT * j >= pieces) break;      // workgroup-uniform
            {
                int r = row, b = blk;
                if (tid + NT * j >= pieces) {   // past the end: the last piece
                    r = M - 1;
                    b = pr - 1;
                }
                st[j] = *reinterpret_cast<const u32x4 *>(x + (size_t)r * K + (size_t)cs * 128 + b * 8);
            }
            row += dq;
            blk += dr;
            if (blk >= pr) {
                blk -= pr;
                ++row;
            }
        }
    }

    __device__ __forceinline__ void load_norm(const float *__restrict__ h, const uint16_t *__restrict__ gamma, int M,
                                              int K)
    {
        const int tid = threadIdx.x;
        pr = (K >> 7) * 16;
        pieces = M * pr;
        row0 = tid / pr;
        blk0 = tid - row0 * pr;
        dq = NT / pr;
        dr = NT - dq * pr;
        int row = row0, blk = blk0;
#pragma unroll
        for (int j = 0; j < SMAX; ++j) {
            if (NT * j >= pieces) break;      // workgroup-uniform
            {
                int r = row, b = blk;
                if (tid + NT * j >= pieces) {
                    r = M - 1;
                    b = pr - 1;
                }
                const f32x4 *hp = reinterpret_cast<const f32x4 *>(h + (size_t)r * K + b * 8);
                ha[j] = hp[0];
                hb[j] = hp[1];
                st[j] = *reinterpret_cast<const u32x4 *>(gamma + b * 8);
            }
            row += dq;
            blk += dr;
            if (blk >= pr) {
                blk -= pr;
                ++row;
            }
        }
    }

    // After load_norm: group sums of squares of every (row, group) into
    // Xs[g][row] (the 16 pieces of a (row, group) are one 16-lane row of a
    // wave), a barrier, then wave r forms row r's total (all rows at once,
    // M <= NT/64) into an LDS slot; a barrier again, and every lane r takes
    // row r's 1/rms from it before store() reuses Xs.
    __device__ __forceinline__ void norm(uint16_t *xs, int M, int K, float eps)
    {
        const int tid = threadIdx.x;
        const int G = K >> 7;
        float *Xs = reinterpret_cast<float *>(xs + M * G * 128);
        int prow = row0, pblk = blk0;
#pragma unroll
        for (int j = 0; j < SMAX; ++j) {
            if (NT * j >= pieces) break;      // workgroup-uniform
            {
                const int pu = tid + NT * j;
                const float v[8] = {ha[j].x, ha[j].y, ha[j].z, ha[j].w, hb[j].x, hb[j].y, hb[j].z, hb[j].w};
                const float tot = row16_sum(block_sumsq(v, 8));
                if ((tid & 15) == 15 && pu < pieces) Xs[(pblk >> 4) * kXsRows + prow] = tot;
            }
            prow += dq;
            pblk += dr;
            if (pblk >= pr) {
                pblk -= pr;
                ++prow;
            }
        }
        lds_barrier();
        __shared__ float invs[kXsRows];
        const int lane = tid & 63;
        const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
        if (w < M) {
            const float t = groups_total([&](int g) { return Xs[g * kXsRows + w]; }, G);
            if (lane == 0) invs[w] = rms_inv(t, K, eps);
        }
        lds_barrier();
        inv_l = lane < M ? invs[lane] : 0.0f;
    }

    __device__ __forceinline__ void store(uint16_t *xs, int M, int cs, int ce)
    {
        typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
        const int tid = threadIdx.x;
        const int ng = ce - cs;
        float *Xs = reinterpret_cast<float *>(xs + M * ng * 128);
        const bf16x2 ones = __builtin_bit_cast(bf16x2, kOnePair);
        int prow = row0, pblk = blk0;
#pragma unroll
        for (int j = 0; j < SMAX; ++j) {
            if (NT * j >= pieces) break;      // workgroup-uniform
            {
                const int pu = tid + NT * j;
                const int row = pu < pieces ? prow : M - 1, blk = pu < pieces ? pblk : pr - 1;
                if (NORM) st[j] = norm_pack(ha[j], hb[j], st[j], __shfl(inv_l, row));
                *reinterpret_cast<u32x4 *>(&xs[(row * pr + swz(blk, row)) * 8]) = pair_order(st[j]);
                // Each element goes through a scalar before the bit cast: this
                // compiler bit-casts a vector element expression as element 0.
                const uint32_t w0 = st[j].x, w1 = st[j].y, w2 = st[j].z, w3 = st[j].w;
                float part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w0), ones, 0.0f, false);
                part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w1), ones, part, false);
                part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w2), ones, part, false);
                part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w3), ones, part, false);
                const float tot = row16_sum(part);
                if ((tid & 15) == 15 && pu < pieces) Xs[(blk >> 4) * kXsRows + (RP ? rowpos(row) : row)] = tot;
            }
            prow += dq;
            pblk += dr;
            if (pblk >= pr) {
                pblk -= pr;
                ++prow;
            }
        }
    }
};

// Stage x[0..M)[cs*128 .. ce*128) into buf in XStage's layout (x rows of
// (ce - cs)*16 swizzled 16-byte pieces in pair order, then the row sums), by
// nt threads (a multiple of 64; this thread is number t) in rounds of R
// pieces per thread, the loads of a round issued together.  Piece p = base +
// t + j*nt of a round, so the 16 pieces of one (row, group) are one 16-lane
// row, as in XStage, and the row sums come out bit for bit the same.
template <int R, bool RP>
__device__ __forceinline__ void stage_rounds(uint16_t *buf, const uint16_t *__restrict__ x, int M, int K, int cs,
                                             int ce, int t, int nt)
{
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
    const int pr = (ce - cs) * 16;
    const int pieces = M * pr;
    float *Xs = reinterpret_cast<float *>(buf + M * (ce - cs) * 128);
    const bf16x2 ones = __builtin_bit_cast(bf16x2, kOnePair);
    const int lane = (int)(threadIdx.x & 63);
    for (int base = 0; base < pieces; base += R * nt) {
        u32x4 st[R];
        int rw[R], bk[R];
#pragma unroll
        for (int j = 0; j < R; ++j) {
            const int pu = min(base + t + j * nt, pieces - 1);   // past the end: the last piece again
            rw[j] = pu / pr;
            bk[j] = pu - rw[j] * pr;
            st[j] = *reinterpret_cast<const u32x4 *>(x + (size_t)rw[j] * K + (size_t)cs * 128 + bk[j] * 8);
        }
#pragma unroll
        for (int j = 0; j < R; ++j) {
            const int row = rw[j], blk = bk[j];
            *reinterpret_cast<u32x4 *>(&buf[(row * pr + swz(blk, row)) * 8]) = pair_order(st[j]);
            const uint32_t w0 = st[j].x, w1 = st[j].y, w2 = st[j].z, w3 = st[j].w;
            float part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w0), ones, 0.0f, false);
            part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w1), ones, part, false);
            part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w2), ones, part, false);
            part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w3), ones, part, false);
            const float tot = row16_sum(part);
            if ((lane & 15) == 15 && base + t + j * nt < pieces) Xs[(blk >> 4) * kXsRows + (RP ? rowpos(row) : row)] = tot;
        }
    }
}

template <int NT, int SMAX>
__device__ __forceinline__ void stage_x(uint16_t *xs, const uint16_t *__restrict__ x, int M, int K, int cs,
                                        int ce)
{
    XStage<NT, SMAX> xst;
    xst.load(x, M, K, cs, ce);
    xst.store(xs, M, cs, ce);
}

}  // namespace q4g128
