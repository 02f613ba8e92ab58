// Quantizer: bf16 weights w[N][K] -> int4-g128 codes, scale and minimum.
//
// The format is the one the product streams (Token Rush README, weight format
// paragraph): per group of 128 consecutive k of one column n, a bf16 scale s
// and bf16 minimum m, codes q in 0..15, w ~ q*s + m.  Codes are chosen by a
// per-group search over clipped ranges scored by squared error (Token Rush
// README, quantization section: narrowing a group's range past its extreme
// values trades their error for a finer step on all the others;
// round-to-nearest over the full range is the first candidate).
//
// Candidates (i, j), i, j = 0 .. ncand-1, taken in the order i*ncand + j:
//   lo, hi = min, max of the group;  c = (lo + hi) / 2
//   l = lo + (i/20)(c - lo),  h = hi - (j/20)(hi - c),  s = (h - l)/15
//   s_b = bf16(fp32(s)), m_b = bf16(fp32(l))           (nearest even, twice)
//   q_k = 0 if s_b == 0, else clamp(rint((v_k - m_b)/s_b), 0, 15)
//   e   = sum over k ascending of ((q_k s_b + m_b) - v_k)^2
// and the first candidate with the smallest e wins.  Every step is one IEEE
// fp64 operation in that order (no contraction into fused multiply-adds), so
// the choice is reproducible bit for bit by any fp64 implementation of the
// same steps.
//
// Mapping: one thread per (group, candidate), so each e is summed in the
// order above by one thread; a workgroup holds `gpw` consecutive groups,
// widened to fp64 once into LDS (the groups of a row-major [N][K] tensor are
// consecutive 256-byte pieces of memory, group index n*G + g), and each
// group's min and max found once, by 16 lanes.  The first thread of each
// group scans the candidates' errors in order, then writes 16 code words,
// scale, minimum and the error.  The work is fp64 ALU bound
// (per code per candidate: a subtract, a multiply by the reciprocal of the
// scale and the rounding, with a correctly rounded divide only next to a
// half-integer).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q4g128_launch.h"

namespace q4g128 {
namespace {

constexpr int kQThreads = 256;     // threads per workgroup
constexpr int kQMaxGroups = 16;    // groups per workgroup, 4 or more candidates (16 KiB of fp64 in LDS)
constexpr int kQMaxNarrow = 64;    // groups per workgroup, 1-3 candidates (16 KiB of bf16 in LDS)
constexpr int kQWideFrom = 4;      // candidates per range end from which a group's range is scanned once

__device__ __forceinline__ double f64_of_bf16(uint16_t b)
{
    return (double)__uint_as_float((uint32_t)b << 16);
}

// fp32 -> bf16 bits, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint16_t bf16_of_f32(float f)
{
    const uint32_t u = __float_as_uint(f);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ bool finite_bf16(uint16_t b) { return (b & 0x7F80u) != 0x7F80u; }

struct Cand {
    uint16_t s16, m16;
};

// Scale and minimum bits of candidate (bi, bj) of a group with range [lo, hi].
__device__ Cand candidate(double lo, double hi, int bi, int bj)
{
#pragma clang fp contract(off)
    const double c = (lo + hi) * 0.5;
    const double bl = (double)bi / 20.0;
    const double bh = (double)bj / 20.0;
    const double l = lo + bl * (c - lo);
    const double h = hi - bh * (hi - c);
    const double sv = (h - l) / 15.0;
    Cand r;
    r.s16 = bf16_of_f32((float)sv);
    r.m16 = bf16_of_f32((float)l);
    return r;
}

// clamp(rint((v - md) / sd), 0, 15), 0 if sd == 0, with the quotient
// rounded exactly as a correctly rounded fp64 divide would give it.  The
// quotient is first formed as (v - md) * rs with rs = fl(1 / sd): two
// roundings, so it lies within 1.5 * 2^-52 |t| of the divided one, whose
// own error is 2^-53 |t|.  rint of the two can differ only if a half-integer
// lies within that distance; when the product is within 2^-50 |t| of one,
// the divide itself decides.  (t - rint(t) is exact for |t| < 2^52; larger
// quotients clamp to 0 or 15 either way.)
// sd != 0 (the caller takes sd == 0 apart).  The clamp by fmax/fmin may
// give -0 where the comparisons gave +0 (a quotient in (-0.5, 0)): the code
// is 0 either way and the error term below squares a value whose sign of
// zero it does not change.
__device__ __forceinline__ double code_of(double v, double sd, double md, double rs)
{
#pragma clang fp contract(off)
    const double d = v - md;
    const double t = d * rs;
    double q = __builtin_rint(t);
    const double near_half = __builtin_fabs(__builtin_fabs(t - q) - 0.5);
    if (near_half <= 0x1p-50 * __builtin_fabs(t)) q = __builtin_rint(d / sd);
    return __builtin_fmin(__builtin_fmax(q, 0.0), 15.0);
}

// The first candidate with the smallest error (strict <: ties keep the
// earlier) of group gi, from its nc2 errors e[] and scale/minimum bits sm[];
// the group's codes from its values val(k), written with the scale, minimum
// and error.  No finite error (a NaN or infinity in the group): zero codes,
// scale and minimum, error NaN.
template <typename Val>
__device__ void write_group(long gi, const double *e, const uint32_t *sm, int nc2, Val val, uint32_t *__restrict__ W,
                            uint16_t *__restrict__ S, uint16_t *__restrict__ Mn, double *__restrict__ err)
{
#pragma clang fp contract(off)
    double best = __builtin_inf();
    int bi = -1;
    for (int c = 0; c < nc2; ++c) {
        if (e[c] < best) {
            best = e[c];
            bi = c;
        }
    }
    uint4 *dst = reinterpret_cast<uint4 *>(W + gi * 16);
    if (bi < 0) {
        for (int j = 0; j < 4; ++j) dst[j] = make_uint4(0, 0, 0, 0);
        S[gi] = 0;
        Mn[gi] = 0;
        if (err) err[gi] = __builtin_nan("");
        return;
    }
    const uint16_t s16 = (uint16_t)(sm[bi] & 0xFFFFu), m16 = (uint16_t)(sm[bi] >> 16);
    const double sd = f64_of_bf16(s16), md = f64_of_bf16(m16);
    const double rs = sd != 0.0 ? 1.0 / sd : 0.0;
    for (int j = 0; j < 4; ++j) {
        uint32_t word[4];
        for (int t = 0; t < 4; ++t) {
            uint32_t wd = 0;
            for (int i = 0; i < 8; ++i) {
                const int k = 32 * j + 8 * t + i;
                if (sd != 0.0) wd |= (uint32_t)code_of(val(k), sd, md, rs) << (4 * i);
            }
            word[t] = wd;
        }
        dst[j] = make_uint4(word[0], word[1], word[2], word[3]);
    }
    S[gi] = s16;
    Mn[gi] = m16;
    if (err) err[gi] = best;
}

// Error of candidate (bi, bj) of a group with range [lo, hi] and values
// val(k), with the candidate's scale/minimum bits.
template <typename Val>
__device__ __forceinline__ double candidate_error(double lo, double hi, int bi, int bj, Val val, Cand &cd)
{
#pragma clang fp contract(off)
    cd = candidate(lo, hi, bi, bj);
    const double sd = f64_of_bf16(cd.s16), md = f64_of_bf16(cd.m16);
    double e = 0.0;
    if (sd == 0.0) {                      // every code 0: the same terms with q = 0
        for (int k = 0; k < 128; ++k) {
            const double x = val(k);
            const double r = (0.0 * sd + md) - x;
            e = e + r * r;
        }
        return e;
    }
    const double rs = 1.0 / sd;
#pragma unroll 8
    for (int k = 0; k < 128; ++k) {
        const double x = val(k);
        const double r = (code_of(x, sd, md, rs) * sd + md) - x;
        e = e + r * r;
    }
    return e;
}

// WIDE (4 or more candidates per range end): the workgroup's groups widened
// to fp64 in LDS once, and each group's min and max found once by 16 lanes
// (8 consecutive values each, then lane pairs, quads, ... combine ranges
// that stay contiguous, the earlier kept on ties, so lo and hi are the
// values a scan in k order keeps, -0 and +0 included).  Otherwise (1-3
// candidates, up to 64 groups per workgroup) each thread scans its group's
// bf16 values itself.
template <bool WIDE>
__global__ __launch_bounds__(kQThreads) void quantize_q4g128(const uint16_t *__restrict__ w, long ngroups,
                                                             int ncand, int gpw, uint32_t *__restrict__ W,
                                                             uint16_t *__restrict__ S, uint16_t *__restrict__ Mn,
                                                             double *__restrict__ err)
{
#pragma clang fp contract(off)
    __shared__ __attribute__((aligned(16))) uint8_t vals[WIDE ? kQMaxGroups * 128 * 8 : kQMaxNarrow * 128 * 2];
    __shared__ double glo[WIDE ? kQMaxGroups : 1], ghi[WIDE ? kQMaxGroups : 1];
    __shared__ int gbad[WIDE ? kQMaxGroups : 1];
    __shared__ double es[kQThreads];
    __shared__ uint32_t sms[kQThreads];
    double *const vd = reinterpret_cast<double *>(vals);
    uint4 *const vs4 = reinterpret_cast<uint4 *>(vals);
    const uint16_t *const vs = reinterpret_cast<const uint16_t *>(vals);

    const int nc2 = ncand * ncand;
    const long g0 = (long)blockIdx.x * gpw;
    const int ng = (int)min((long)gpw, ngroups - g0);
    const int tid = threadIdx.x;
    const uint4 *src = reinterpret_cast<const uint4 *>(w + g0 * 128);   // ng * 256 contiguous bytes

    if constexpr (WIDE) {
        for (int p = tid; p < ng * 16; p += blockDim.x) {
            const uint4 u = src[p];
            const uint32_t e4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                vd[8 * p + 2 * t] = f64_of_bf16((uint16_t)(e4[t] & 0xFFFFu));
                vd[8 * p + 2 * t + 1] = f64_of_bf16((uint16_t)(e4[t] >> 16));
            }
        }
        const int gq = tid >> 4, sl = tid & 15;
        const bool on = gq < ng;                 // all 16 lanes of a group alike
        double lo = 0.0, hi = 0.0;
        int bad = 0;
        if (on) {
            const uint4 u = src[gq * 16 + sl];
            const uint32_t e4[4] = {u.x, u.y, u.z, u.w};
            lo = hi = f64_of_bf16((uint16_t)(e4[0] & 0xFFFFu));
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const uint16_t b = (uint16_t)((t & 1) ? (e4[t >> 1] >> 16) : (e4[t >> 1] & 0xFFFFu));
                bad |= !finite_bf16(b);
                const double x = f64_of_bf16(b);
                lo = x < lo ? x : lo;
                hi = x > hi ? x : hi;
            }
        }
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) {
            const double rlo = __shfl_down(lo, off, 16), rhi = __shfl_down(hi, off, 16);
            const int rbad = __shfl_down(bad, off, 16);
            if ((sl & (2 * off - 1)) == 0) {
                lo = rlo < lo ? rlo : lo;
                hi = rhi > hi ? rhi : hi;
                bad |= rbad;
            }
        }
        if (on && sl == 0) {
            glo[gq] = lo;
            ghi[gq] = hi;
            gbad[gq] = bad;
        }
    } else {
        for (int p = tid; p < ng * 16; p += blockDim.x) vs4[p] = src[p];
    }
    __syncthreads();

    const int gl = tid / nc2;
    const int cand = tid - gl * nc2;
    const bool active = gl < ng;
    auto val = [&](int k) -> double {
        if constexpr (WIDE) return vd[gl * 128 + k];
        else return f64_of_bf16(vs[gl * 128 + k]);
    };
    if (active) {
        double lo, hi;
        bool bad;
        if constexpr (WIDE) {
            lo = glo[gl];
            hi = ghi[gl];
            bad = gbad[gl] != 0;
        } else {
            lo = hi = val(0);
            bad = false;
            for (int k = 0; k < 128; ++k) {
                const uint16_t b = vs[gl * 128 + k];
                bad |= !finite_bf16(b);
                const double x = f64_of_bf16(b);
                lo = x < lo ? x : lo;
                hi = x > hi ? x : hi;
            }
        }
        double e = __builtin_nan("");
        Cand cd = {0, 0};
        if (!bad) e = candidate_error(lo, hi, cand / ncand, cand % ncand, val, cd);
        es[tid] = e;
        sms[tid] = (uint32_t)cd.s16 | ((uint32_t)cd.m16 << 16);
    }
    __syncthreads();
    if (active && cand == 0) write_group(g0 + gl, es + gl * nc2, sms + gl * nc2, nc2, val, W, S, Mn, err);
}

}  // namespace

int quantize_groups_per_block(int ncand)
{
    const int nc2 = ncand * ncand;
    const int cap = ncand >= kQWideFrom ? kQMaxGroups : kQMaxNarrow;
    const int gpw = kQThreads / nc2;
    return gpw > cap ? cap : gpw;
}

hipError_t launch_quantize(const uint16_t *w, long ngroups, int ncand, uint32_t *W, uint16_t *S, uint16_t *Mn,
                           double *err, hipStream_t stream)
{
    const int gpw = quantize_groups_per_block(ncand);
    const int used = gpw * ncand * ncand;
    const long blocks = (ngroups + gpw - 1) / gpw;
    if (ncand >= kQWideFrom) {
        // one thread per (group, candidate), and 16 per group for the range scan
        const int threads = (max(used, 16 * gpw) + 63) / 64 * 64;
        hipLaunchKernelGGL(quantize_q4g128<true>, dim3((unsigned)blocks, 1, 1), dim3(threads, 1, 1), 0, stream, w,
                           ngroups, ncand, gpw, W, S, Mn, err);
    } else {
        const int threads = (used + 63) / 64 * 64;
        hipLaunchKernelGGL(quantize_q4g128<false>, dim3((unsigned)blocks, 1, 1), dim3(threads, 1, 1), 0, stream, w,
                           ngroups, ncand, gpw, W, S, Mn, err);
    }
    return hipGetLastError();
}

}  // namespace q4g128
