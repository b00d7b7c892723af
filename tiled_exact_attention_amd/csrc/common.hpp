// Device helpers shared by the gfx950 kernels: wave64 reductions, the
// pairwise combine of partial softmax states, bf16 packing, exponentials.
//
// The online-softmax state of a set of logits is (m, l[, O]): m the running
// maximum, l the sum of exp(x - m), O the exp(x - m)-weighted sum of values
// ("Online softmax" (roadmapper), The recurrence; "Online Softmax"
// (metalworking), The problem).  Inside kernels every exponential is base two
// (v_exp_f32); the conversion factor log2(e) is applied once, in one place
// per kernel, never mixed with a base-e factor ("Online softmax", Things that
// break).  Maxima handed across the C ABI are in natural-log units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tea {

// log2(e) split into a float head and tail: head + tail equals log2(e) to
// about 2^-49, so x*head + x*tail carries the product beyond fp32 precision.
constexpr float kLog2eHi = 1.44269502162933349609375f;
constexpr float kLog2eLo = 1.925963033500011079e-08f;
constexpr float kLn2 = 0.693147180559945309417f;
constexpr float kNegInf = -__builtin_inff();

typedef short bf16x8_t __attribute__((__vector_size__(8 * sizeof(short))));
typedef float f32x16_t __attribute__((__vector_size__(16 * sizeof(float))));
typedef float f32x4_t __attribute__((__vector_size__(4 * sizeof(float))));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4v_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Hardware base-two exponential (v_exp_f32): exp2(-inf) = 0, exp2(0) = 1.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// bf16 <-> fp32.  Widening is exact; narrowing rounds to nearest even
// (v_cvt_pk_bf16_f32).
__device__ __forceinline__ float bf16_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ unsigned pack_bf16x2(float a, float b)
{
    bf16x2_t v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(unsigned, v);
}

// ---- wave64 reductions -----------------------------------------------------
// Four DPP steps reduce within each row of 16 lanes (quad swaps, then the
// half-row and row mirrors), then permlane16/permlane32 swaps fold rows
// together.  Every lane ends with the full-wave result.  The swaps return
// (lower-lane value, upper-lane value) in every lane, so op(r[0], r[1]) is
// the same ordered combine in both halves.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

struct MaxOp {
    __device__ __forceinline__ float operator()(float a, float b) const { return fmaxf(a, b); }
};
struct AddOp {
    __device__ __forceinline__ float operator()(float a, float b) const { return a + b; }
};

template <class Op>
__device__ __forceinline__ float row16_reduce(float v, Op op)
{
    v = op(v, dpp_f<0xB1>(v));   // quad_perm [1,0,3,2]
    v = op(v, dpp_f<0x4E>(v));   // quad_perm [2,3,0,1]
    v = op(v, dpp_f<0x141>(v));  // row_half_mirror
    v = op(v, dpp_f<0x140>(v));  // row_mirror
    return v;
}

template <class Op>
__device__ __forceinline__ float swap16_reduce(float v, Op op)
{
    unsigned u = __float_as_uint(v);
    auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

template <class Op>
__device__ __forceinline__ float swap32_reduce(float v, Op op)
{
    unsigned u = __float_as_uint(v);
    auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

template <class Op>
__device__ __forceinline__ float wave_reduce(float v, Op op)
{
    v = row16_reduce(v, op);
    v = swap16_reduce(v, op);
    return swap32_reduce(v, op);
}

// Value held by lane (lane ^ 32).
__device__ __forceinline__ float xor32(float v)
{
    unsigned u = __float_as_uint(v);
    auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(__lane_id() < 32 ? r[1] : r[0]);
}

// Value held by lane (lane ^ 16).
__device__ __forceinline__ float xor16(float v)
{
    unsigned u = __float_as_uint(v);
    auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return __uint_as_float((__lane_id() & 16) ? r[0] : r[1]);
}

// Value held by lane (lane ^ X), X a power of two below 64, with no LDS
// traffic: DPP inside each row of 16 lanes (quad permutes for 1 and 2, row
// rotations for 4 and 8; row_ror:n hands lane i the value of lane
// (i - n) mod 16), permlane swaps across rows for 16 and 32.
template <int X>
__device__ __forceinline__ float lane_xor(float v)
{
    static_assert(X == 1 || X == 2 || X == 4 || X == 8 || X == 16 || X == 32, "lane distance");
    if constexpr (X == 1) return dpp_f<0xB1>(v);  // quad_perm [1,0,3,2]
    else if constexpr (X == 2) return dpp_f<0x4E>(v);  // quad_perm [2,3,0,1]
    else if constexpr (X == 4) {
        const float down = dpp_f<0x124>(v);  // row_ror:4:  lane i - 4 (mod 16)
        const float up = dpp_f<0x12C>(v);    // row_ror:12: lane i + 4 (mod 16)
        return (__lane_id() & 4) ? down : up;
    } else if constexpr (X == 8) return dpp_f<0x128>(v);  // row_ror:8
    else if constexpr (X == 16) return xor16(v);
    else return xor32(v);
}

// ---- the guard and the correction -----------------------------------------
// While a running maximum is still -inf (nothing seen yet, or only masked
// logits) the exponent is taken relative to 0 instead, so exp2(-inf - -inf)
// never produces NaN: the stale state (0) is multiplied by exp2(-inf) = 0 and
// the new terms exp2(-inf) = 0 as well ("Online softmax", Initialise
// honestly).
__device__ __forceinline__ float guard_max(float m) { return m == kNegInf ? 0.0f : m; }

// Weights of two partial states (natural-unit maxima m1, m2) relative to
// their common maximum: the pairwise combine identity ("The Online Softmax"
// (curionode), One pass, exactly).  Returns the combined maximum.
__device__ __forceinline__ float combine_weights(float m1, float m2, float& a1, float& a2)
{
    float m = fmaxf(m1, m2);
    float mu = guard_max(m);
    a1 = exp2_hw((m1 - mu) * kLog2eHi);
    a2 = exp2_hw((m2 - mu) * kLog2eHi);
    return m;
}

}  // namespace tea
