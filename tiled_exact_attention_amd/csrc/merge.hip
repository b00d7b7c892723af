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
#include <utility>

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

// One level of the balanced tree across the wave: lanes X apart exchange
// their states and both compute combine(lower lane, upper lane), so both
// hold the same bits; then the next level.
template <bool BASE2, int X>
__device__ __forceinline__ void lane_butterfly(int lane, float& m, float& l, float* O)
{
    if constexpr (X < 64) {
        float mp = lane_xor<X>(m), lp = lane_xor<X>(l), Op[kDV];
#pragma unroll
        for (int d = 0; d < kDV; ++d) Op[d] = lane_xor<X>(O[d]);
        if (lane & X) {  // partner is the lower lane: combine(partner, mine)
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
        lane_butterfly<BASE2, X * 2>(lane, m, l, O);
    }
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
    // a partial's kDV dimensions as two 16-byte loads when every row start
    // is 16-byte aligned (D a multiple of 8 and an aligned base, as the
    // decode's workspace is), else one by one
    const bool vec = D % kDV == 0 && ((uintptr_t)pO % 16) == 0;
    for (int g = 0; g < G; ++g) {
        const int s = lane * G + g;
        if (s >= S) break;
        const int64_t ps = n * S + s;
        float Ot[kDV];
        if (vec) {
            const f32x4v_t a = *reinterpret_cast<const f32x4v_t*>(pO + ps * D + d0);
            const f32x4v_t b = *reinterpret_cast<const f32x4v_t*>(pO + ps * D + d0 + 4);
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                Ot[d] = a[d];
                Ot[d + 4] = b[d];
            }
        } else {
#pragma unroll
            for (int d = 0; d < kDV; ++d) Ot[d] = (d0 + d < D) ? pO[ps * D + d0 + d] : 0.0f;
        }
        combine_into<BASE2>(m, l, O, pm[ps], pl[ps], Ot);
    }

    // the balanced tree over the 64 lanes' states: lane distances 1 .. 32,
    // exchanged by DPP and permlane swaps
    lane_butterfly<BASE2, 1>(lane, m, l, O);

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

// Few partials per row (S <= kRowsMaxS, D <= 256): one wave per row, lane
// j owning output dimensions j, j + 64, ... (DPL of them), so each partial's
// O row is read by the whole wave in one coalesced pass.  The partials are
// combined in the same balanced tree over the partial index as above, built
// by a binary counter: leaf s is pushed on a stack whose level-k entry holds
// a complete subtree of 2^k leaves, merging (older entry, newer one) while
// bit k of s is set; the entries left after the last leaf (the set bits of
// S) are then folded from the lowest level up.  That equals the tree padded
// with the identity, whose combines are exact no-ops.
constexpr int kRowsMaxS = 32;

constexpr int trailing_ones(int s) { return (s & 1) ? 1 + trailing_ones(s >> 1) : 0; }

// f(integral_constant<int, I>) for each I of the sequence, in order
template <class F, int... I>
__device__ __forceinline__ void each_index(F&& f, std::integer_sequence<int, I...>)
{
    (f(std::integral_constant<int, I>{}), ...);
}

template <bool BASE2, bool OUT_BF16, bool NORMALIZE, int DPL>
__global__ __launch_bounds__(256) void merge_rows_kernel(const float* __restrict__ pm, const float* __restrict__ pl,
                                                         const float* __restrict__ pO, int64_t N, int S, int D,
                                                         float* __restrict__ m_out, float* __restrict__ l_out,
                                                         void* __restrict__ O_out, float* __restrict__ lse_out)
{
    constexpr int LEV = 6;  // stack levels: 2^5 = kRowsMaxS leaves
    static_assert((1 << (LEV - 1)) == kRowsMaxS, "stack depth");
    const int lane = threadIdx.x & 63;
    const int64_t n = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (n >= N) return;  // whole wave

    auto combine = [](float& m1, float& l1, float* O1, float m2, float l2, const float* O2) {
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
        for (int k = 0; k < DPL; ++k) O1[k] = fmaf(a1, O1[k], a2 * O2[k]);
        m1 = m;
    };

    float sm[LEV], sl[LEV], sO[LEV][DPL];
    // leaf s: merge with the stack entries of its trailing one bits, then
    // push; every index is a compile-time constant (one step per s)
    auto step = [&](auto s_c) {
        constexpr int s = decltype(s_c)::value;
        constexpr int T = trailing_ones(s);
        if (s >= S) return;
        const int64_t ps = n * S + s;
        float m = pm[ps], l = pl[ps], O[DPL];
#pragma unroll
        for (int k = 0; k < DPL; ++k) {
            const int d = lane + 64 * k;
            O[k] = d < D ? pO[ps * D + d] : 0.0f;
        }
#pragma unroll
        for (int lev = 0; lev < T; ++lev) {
            // left operand: the older subtree on the stack
            float mo = sm[lev], lo = sl[lev], Oo[DPL];
#pragma unroll
            for (int k = 0; k < DPL; ++k) Oo[k] = sO[lev][k];
            combine(mo, lo, Oo, m, l, O);
            m = mo;
            l = lo;
#pragma unroll
            for (int k = 0; k < DPL; ++k) O[k] = Oo[k];
        }
        sm[T] = m;
        sl[T] = l;
#pragma unroll
        for (int k = 0; k < DPL; ++k) sO[T][k] = O[k];
    };
    each_index(step, std::make_integer_sequence<int, kRowsMaxS>{});
    // fold the subtrees of the set bits of S, lowest level first, each as
    // the right operand of the next higher one
    float m = kNegInf, l = 0.0f, O[DPL];
#pragma unroll
    for (int k = 0; k < DPL; ++k) O[k] = 0.0f;
    bool have = false;
#pragma unroll
    for (int lev = 0; lev < LEV; ++lev) {
        if (((S >> lev) & 1) == 0) continue;
        if (!have) {
            m = sm[lev];
            l = sl[lev];
#pragma unroll
            for (int k = 0; k < DPL; ++k) O[k] = sO[lev][k];
            have = true;
        } else {
            float mo = sm[lev], lo = sl[lev], Oo[DPL];
#pragma unroll
            for (int k = 0; k < DPL; ++k) Oo[k] = sO[lev][k];
            combine(mo, lo, Oo, m, l, O);
            m = mo;
            l = lo;
#pragma unroll
            for (int k = 0; k < DPL; ++k) O[k] = Oo[k];
        }
    }

    if (lane == 0) {
        const float mn = BASE2 ? m * kLn2 : m;
        if (m_out) m_out[n] = mn;
        if (l_out) l_out[n] = l;
        if (lse_out) lse_out[n] = l > 0.0f ? mn + __logf(l) : kNegInf;
    }
    const float inv = (NORMALIZE && l > 0.0f) ? 1.0f / l : (NORMALIZE ? 0.0f : 1.0f);
#pragma unroll
    for (int k = 0; k < DPL; ++k) {
        const int d = lane + 64 * k;
        if (d < D) {
            const float v = O[k] * inv;
            if constexpr (OUT_BF16) {
                bf16x2_t p = {(__bf16)v, (__bf16)0.0f};
                static_cast<uint16_t*>(O_out)[n * D + d] = (uint16_t)(__builtin_bit_cast(unsigned, p) & 0xffffu);
            } else {
                static_cast<float*>(O_out)[n * D + d] = v;
            }
        }
    }
}

template <bool BASE2, int DPL>
hipError_t launch_merge_rows(const MergeArgs& a)
{
    const dim3 grid((unsigned)((a.N + 3) / 4)), block(256);
    if (a.out_bf16) {
        if (a.normalize)
            hipLaunchKernelGGL((merge_rows_kernel<BASE2, true, true, DPL>), grid, block, 0, a.stream, a.m, a.l, a.O, a.N,
                               a.S, a.D, a.m_out, a.l_out, a.O_out, a.lse_out);
        else
            hipLaunchKernelGGL((merge_rows_kernel<BASE2, true, false, DPL>), grid, block, 0, a.stream, a.m, a.l, a.O,
                               a.N, a.S, a.D, a.m_out, a.l_out, a.O_out, a.lse_out);
    } else {
        if (a.normalize)
            hipLaunchKernelGGL((merge_rows_kernel<BASE2, false, true, DPL>), grid, block, 0, a.stream, a.m, a.l, a.O,
                               a.N, a.S, a.D, a.m_out, a.l_out, a.O_out, a.lse_out);
        else
            hipLaunchKernelGGL((merge_rows_kernel<BASE2, false, false, DPL>), grid, block, 0, a.stream, a.m, a.l, a.O,
                               a.N, a.S, a.D, a.m_out, a.l_out, a.O_out, a.lse_out);
    }
    return hipGetLastError();
}

template <bool BASE2>
hipError_t launch_merge_t(const MergeArgs& a)
{
    if (a.N == 0) return hipSuccess;
    if (a.S <= kRowsMaxS) {
        if (a.D <= 64) return launch_merge_rows<BASE2, 1>(a);
        if (a.D <= 128) return launch_merge_rows<BASE2, 2>(a);
        if (a.D <= 256) return launch_merge_rows<BASE2, 4>(a);
    }
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
