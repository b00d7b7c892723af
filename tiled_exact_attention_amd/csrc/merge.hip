// Merge of partial softmax states (m, l, O) in a tree, with no atomics.
//
// The pairwise combine ("The Online Softmax" (curionode), One pass, exactly:
// the rescaling identity written for pairs of partial results is associative)
//     m = max(m1, m2),  a_i = exp(m_i - m),  l = a1 l1 + a2 l2,  O = a1 O1 + a2 O2
// has the empty state (-inf, 0, 0) as its identity.  Split-KV decode uses it
// to merge partial softmaxes computed by different workgroups, as the Apple
// decode kernels do for their simdgroups ("Online Softmax" (metalworking),
// Recognition guide).
//
// One wave merges the S partials of one row for one slice of 8 output
// dimensions.  Lane j takes the contiguous partials [j*G, j*G + G),
// G = ceil(S / 64), folds them left to right, and the 64 lane states are then
// combined by a butterfly: at level k lanes j and j ^ 2^k both compute
// combine(lower lane's state, upper lane's state), so after six levels every
// lane holds the root of a balanced binary tree over the lanes (for S <= 64,
// a balanced tree over the partial index, padded with the identity).  Each
// combine takes its operands in the same order in both lanes, so the result
// is bitwise deterministic.
#include "common.hpp"
#include "launch.hpp"

namespace tea {

namespace {

constexpr int kDV = 8;  // output dimensions per wave

// Combine (m1, l1, O1) <- combine((m1, l1, O1), (m2, l2, O2)).  BASE2: the
// maxima are already in base-two units.
template <bool BASE2>
__device__ __forceinline__ void combine_into(float& m1, float& l1, float* O1, float m2, float l2, const float* O2)
{
    const float m = fmaxf(m1, m2);
    const float mu = guard_max(m);
    float a1, a2;
    if constexpr (BASE2) {
        a1 = exp2_hw(m1 - mu);
        a2 = exp2_hw(m2 - mu);
    } else {
        a1 = exp2_hw((m1 - mu) * kLog2eHi);
        a2 = exp2_hw((m2 - mu) * kLog2eHi);
    }
    l1 = fmaf(a1, l1, a2 * l2);
#pragma unroll
    for (int d = 0; d < kDV; ++d) O1[d] = fmaf(a1, O1[d], a2 * O2[d]);
    m1 = m;
}

template <bool BASE2, bool OUT_BF16, bool NORMALIZE>
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ pm, const float* __restrict__ pl,
                                                    const float* __restrict__ pO, int64_t N, int S, int D,
                                                    float* __restrict__ m_out, float* __restrict__ l_out,
                                                    void* __restrict__ O_out, float* __restrict__ lse_out)
{
    const int lane = threadIdx.x & 63;
    const int nslices = (D + kDV - 1) / kDV;
    const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (wid >= N * nslices) return;  // whole wave
    const int64_t n = wid / nslices;
    const int d0 = (int)(wid % nslices) * kDV;
    const int G = (S + 63) / 64;

    float m = kNegInf, l = 0.0f, O[kDV];
#pragma unroll
    for (int d = 0; d < kDV; ++d) O[d] = 0.0f;
    for (int g = 0; g < G; ++g) {
        const int s = lane * G + g;
        if (s >= S) break;
        const int64_t ps = n * S + s;
        float Ot[kDV];
#pragma unroll
        for (int d = 0; d < kDV; ++d) Ot[d] = (d0 + d < D) ? pO[ps * D + d0 + d] : 0.0f;
        combine_into<BASE2>(m, l, O, pm[ps], pl[ps], Ot);
    }

#pragma unroll
    for (int k = 1; k < 64; k <<= 1) {
        float mp = __shfl_xor(m, k), lp = __shfl_xor(l, k), Op[kDV];
#pragma unroll
        for (int d = 0; d < kDV; ++d) Op[d] = __shfl_xor(O[d], k);
        if (lane & k) {  // partner is the lower lane: combine(partner, mine)
            float Om[kDV];
#pragma unroll
            for (int d = 0; d < kDV; ++d) Om[d] = O[d];
            float mm = m, lm = l;
            m = mp;
            l = lp;
#pragma unroll
            for (int d = 0; d < kDV; ++d) O[d] = Op[d];
            combine_into<BASE2>(m, l, O, mm, lm, Om);
        } else {
            combine_into<BASE2>(m, l, O, mp, lp, Op);
        }
    }

    if (lane == 0) {
        if (d0 == 0) {
            const float mn = BASE2 ? m * kLn2 : m;
            if (m_out) m_out[n] = mn;
            if (l_out) l_out[n] = l;
            if (lse_out) lse_out[n] = l > 0.0f ? mn + __logf(l) : kNegInf;
        }
        const float inv = (NORMALIZE && l > 0.0f) ? 1.0f / l : (NORMALIZE ? 0.0f : 1.0f);
#pragma unroll
        for (int d = 0; d < kDV; ++d) {
            if (d0 + d < D) {
                const float v = O[d] * inv;
                if constexpr (OUT_BF16) {
                    bf16x2_t p = {(__bf16)v, (__bf16)0.0f};
                    static_cast<uint16_t*>(O_out)[n * D + d0 + d] = (uint16_t)(__builtin_bit_cast(unsigned, p) & 0xffffu);
                } else {
                    static_cast<float*>(O_out)[n * D + d0 + d] = v;
                }
            }
        }
    }
}

template <bool BASE2>
hipError_t launch_merge_t(const MergeArgs& a)
{
    if (a.N == 0) return hipSuccess;
    const int64_t waves = a.N * ((a.D + kDV - 1) / kDV);
    const dim3 grid((unsigned)((waves + 3) / 4)), block(256);
    if (a.out_bf16) {
        if (a.normalize)
            hipLaunchKernelGGL((merge_kernel<BASE2, true, true>), grid, block, 0, a.stream, a.m, a.l, a.O, a.N, a.S,
                               a.D, a.m_out, a.l_out, a.O_out, a.lse_out);
        else
            hipLaunchKernelGGL((merge_kernel<BASE2, true, false>), grid, block, 0, a.stream, a.m, a.l, a.O, a.N, a.S,
                               a.D, a.m_out, a.l_out, a.O_out, a.lse_out);
    } else {
        if (a.normalize)
            hipLaunchKernelGGL((merge_kernel<BASE2, false, true>), grid, block, 0, a.stream, a.m, a.l, a.O, a.N, a.S,
                               a.D, a.m_out, a.l_out, a.O_out, a.lse_out);
        else
            hipLaunchKernelGGL((merge_kernel<BASE2, false, false>), grid, block, 0, a.stream, a.m, a.l, a.O, a.N,
                               a.S, a.D, a.m_out, a.l_out, a.O_out, a.lse_out);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a) { return launch_merge_t<false>(a); }

// Used by split-KV decode, whose workspace keeps maxima in base-two units.
hipError_t launch_merge_base2(const MergeArgs& a) { return launch_merge_t<true>(a); }

}  // namespace tea
