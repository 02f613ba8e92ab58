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
template <int NT, int SMAX, bool RP = false>
struct XStage {
    u32x4 st[SMAX];
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

template <int NT, int SMAX>
__device__ __forceinline__ void stage_x(uint16_t *xs, const uint16_t *__restrict__ x, int M, int K, int cs,
                                        int ce)
{
    XStage<NT, SMAX> xst;
    xst.load(x, M, K, cs, ce);
    xst.store(xs, M, cs, ce);
}

}  // namespace q4g128
