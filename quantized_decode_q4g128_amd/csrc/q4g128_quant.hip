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
// staged once into LDS as bf16 (the groups of a row-major [N][K] tensor are
// consecutive 256-byte pieces of memory, group index n*G + g).  The first
// thread of each group scans the candidates' errors in order, then writes
// 16 code words, scale, minimum and the error.  The work is fp64 ALU bound
// (per code per candidate: a subtract, a multiply by the reciprocal of the
// scale and the rounding, with a correctly rounded divide only next to a
// half-integer).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q4g128_launch.h"

namespace q4g128 {
namespace {

constexpr int kQThreads = 256;     // threads per workgroup
constexpr int kQMaxGroups = 64;    // groups staged per workgroup (16 KiB of LDS)

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
__device__ __forceinline__ double code_of(double v, double sd, double md, double rs)
{
#pragma clang fp contract(off)
    if (sd == 0.0) return 0.0;
    const double d = v - md;
    const double t = d * rs;
    double q = __builtin_rint(t);
    const double near_half = __builtin_fabs(__builtin_fabs(t - q) - 0.5);
    if (near_half <= 0x1p-50 * __builtin_fabs(t)) q = __builtin_rint(d / sd);
    q = q < 0.0 ? 0.0 : q;
    return q > 15.0 ? 15.0 : q;
}

__global__ __launch_bounds__(kQThreads) void quantize_q4g128(const uint16_t *__restrict__ w, long ngroups,
                                                             int ncand, int gpw, uint32_t *__restrict__ W,
                                                             uint16_t *__restrict__ S, uint16_t *__restrict__ Mn,
                                                             double *__restrict__ err)
{
#pragma clang fp contract(off)
    __shared__ uint4 vs4[kQMaxGroups * 16];
    __shared__ double es[kQThreads];
    __shared__ uint32_t sms[kQThreads];
    const uint16_t *vs = reinterpret_cast<const uint16_t *>(vs4);

    const int nc2 = ncand * ncand;
    const long g0 = (long)blockIdx.x * gpw;
    const int ng = (int)min((long)gpw, ngroups - g0);
    const int tid = threadIdx.x;

    // Stage the workgroup's groups: ng * 256 contiguous bytes.
    const uint4 *src = reinterpret_cast<const uint4 *>(w + g0 * 128);
    for (int p = tid; p < ng * 16; p += blockDim.x) vs4[p] = src[p];
    __syncthreads();

    const int gl = tid / nc2;
    const int cand = tid - gl * nc2;
    const bool active = gl < ng;
    const uint16_t *v = vs + gl * 128;
    double lo = 0.0, hi = 0.0;
    bool bad = false;
    if (active) {
        lo = hi = f64_of_bf16(v[0]);
        for (int k = 0; k < 128; ++k) {
            const uint16_t b = v[k];
            bad |= !finite_bf16(b);
            const double x = f64_of_bf16(b);
            lo = x < lo ? x : lo;
            hi = x > hi ? x : hi;
        }
        double e = __builtin_nan("");
        Cand cd = {0, 0};
        if (!bad) {
            cd = candidate(lo, hi, cand / ncand, cand % ncand);
            const double sd = f64_of_bf16(cd.s16), md = f64_of_bf16(cd.m16);
            const double rs = sd != 0.0 ? 1.0 / sd : 0.0;
            e = 0.0;
            for (int k = 0; k < 128; ++k) {
                const double x = f64_of_bf16(v[k]);
                const double r = (code_of(x, sd, md, rs) * sd + md) - x;
                e = e + r * r;
            }
        }
        es[tid] = e;
        sms[tid] = (uint32_t)cd.s16 | ((uint32_t)cd.m16 << 16);
    }
    __syncthreads();
    if (!active || cand != 0) return;

    // First candidate with the smallest error (strict <: ties keep the earlier).
    double best = __builtin_inf();
    int bi = -1;
    for (int c = 0; c < nc2; ++c) {
        const double e = es[gl * nc2 + c];
        if (e < best) {
            best = e;
            bi = c;
        }
    }
    const long gi = g0 + gl;
    uint4 *dst = reinterpret_cast<uint4 *>(W + gi * 16);
    if (bi < 0) {   // the group holds a NaN or infinity
        for (int j = 0; j < 4; ++j) dst[j] = make_uint4(0, 0, 0, 0);
        S[gi] = 0;
        Mn[gi] = 0;
        if (err) err[gi] = __builtin_nan("");
        return;
    }
    const uint32_t sm = sms[gl * nc2 + bi];
    const uint16_t s16 = (uint16_t)(sm & 0xFFFFu), m16 = (uint16_t)(sm >> 16);
    const double sd = f64_of_bf16(s16), md = f64_of_bf16(m16);
    const double rs = sd != 0.0 ? 1.0 / sd : 0.0;
    for (int j = 0; j < 4; ++j) {
        uint32_t word[4];
        for (int t = 0; t < 4; ++t) {
            uint32_t wd = 0;
            for (int i = 0; i < 8; ++i) {
                const int k = 32 * j + 8 * t + i;
                wd |= (uint32_t)code_of(f64_of_bf16(v[k]), sd, md, rs) << (4 * i);
            }
            word[t] = wd;
        }
        dst[j] = make_uint4(word[0], word[1], word[2], word[3]);
    }
    S[gi] = s16;
    Mn[gi] = m16;
    if (err) err[gi] = best;
}

}  // namespace

int quantize_groups_per_block(int ncand)
{
    const int nc2 = ncand * ncand;
    int gpw = kQThreads / nc2;
    return gpw > kQMaxGroups ? kQMaxGroups : gpw;
}

hipError_t launch_quantize(const uint16_t *w, long ngroups, int ncand, uint32_t *W, uint16_t *S, uint16_t *Mn,
                           double *err, hipStream_t stream)
{
    const int gpw = quantize_groups_per_block(ncand);
    const int used = gpw * ncand * ncand;
    const int threads = (used + 63) / 64 * 64;
    const long blocks = (ngroups + gpw - 1) / gpw;
    hipLaunchKernelGGL(quantize_q4g128, dim3((unsigned)blocks, 1, 1), dim3(threads, 1, 1), 0, stream, w, ngroups,
                       ncand, gpw, W, S, Mn, err);
    return hipGetLastError();
}

}  // namespace q4g128
