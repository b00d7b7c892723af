// Row softmax in one HBM read and one HBM write per row, by the online
// normaliser recurrence ("Online softmax" (roadmapper), The recurrence;
// "The Online Softmax" (curionode), intro and Workshop).
//
// A row is split across TPR lanes (one wave, or several waves of one
// workgroup).  Each lane holds its N logits in registers (128-bit loads when
// the row is 16-byte aligned), folds them in blocks of BLOCK values with the
// recurrence
//     m' = max(m, max block);  l = l * exp(m - m') + sum exp(x - m');  m = m'
// starting from m = -inf, l = 0, then the lanes' (m, l) states are merged
// with the pairwise identity ("The Online Softmax", One pass, exactly):
// a wave max-reduce gives the row maximum M, each lane rescales its l by
// exp(m - M), and a wave sum-reduce (then an LDS step across waves) gives the
// row normaliser L.  Finally y = exp(x - M) / L is written once.
//
// Exponentials: base two inside, with the difference taken first,
// exp2((x - m) * log2 e), so large logits do not lose the difference to
// rounding.  The fp32 output uses a compensated exponent: x*log2(e) - M*log2(e)
// is carried as a head (one rounding) plus a tail (the parts below fp32
// precision), and exp2(head + tail) = exp2(head) * (1 + tail * ln 2).
#include "common.hpp"
#include "launch.hpp"

namespace tea {

// One step of the per-lane fold: the state (m, l) absorbs a block of B
// logits.  RS picks how the accumulated l is put on the new scale; all three
// give the same bits:
//   kRescaleAlways  multiply by c = exp(m - m') every block, as the MLX kernel
//                   does ("Online Softmax" (metalworking), Recognition guide);
//   kRescaleIfRise  compute c and multiply only when the maximum rose, the
//                   guard of metal-flash-attention (same passage).  Lanes run
//                   in lock step, so the work is skipped when no lane of the
//                   wave saw a rise; for a lane without a rise c is exactly
//                   exp2(0) = 1 and fma(l, 1, s) = l + s;
//   kRescaleL0One   start from l = 1 instead of 0, as the attention tutorial
//                   does ("Online softmax" (roadmapper), Initialise honestly):
//                   the first non-empty block has c = exp(-inf) = 0, which
//                   removes the 1 (fma(1, 0, s) = s).
template <int RS, int B>
__device__ __forceinline__ void fold_block(const float* x, float& m, float& l)
{
    float bm = x[0];
#pragma unroll
    for (int e = 1; e < B; ++e) bm = fmaxf(bm, x[e]);
    const float mn = fmaxf(m, bm);
    const float mu = guard_max(mn);
    float s = 0.0f;
#pragma unroll
    for (int e = 0; e < B; ++e) s += exp2_hw((x[e] - mu) * kLog2eHi);
    if constexpr (RS == kRescaleIfRise) {
        if (__builtin_amdgcn_ballot_w64(mn > m)) l = fmaf(l, exp2_hw((m - mu) * kLog2eHi), s);
        else l = l + s;
    } else {
        l = fmaf(l, exp2_hw((m - mu) * kLog2eHi), s);  // c = 0 on the first non-empty block
    }
    m = mn;
}

template <bool BF16, int TPR, int N, bool VEC, int BLOCK, int WG, int RS>
__global__ __launch_bounds__(WG) void row_softmax_kernel(const void* xv, void* yv, int64_t rows, int64_t cols,
                                                         float* __restrict__ m_out, float* __restrict__ l_out)
{
    constexpr int W = VEC ? (BF16 ? 8 : 4) : 1;  // elements per load
    constexpr int NV = N / W;                     // loads per lane
    constexpr int RPW = WG / TPR;                 // rows per workgroup
    constexpr int NWAVE = TPR / 64;               // waves per row
    static_assert(N % W == 0 && N % BLOCK == 0 && TPR % 64 == 0 && WG % TPR == 0, "bad config");

    const int tid = threadIdx.x;
    const int t = tid % TPR;
    const int64_t row = (int64_t)blockIdx.x * RPW + tid / TPR;
    if (RPW > 1 && row >= rows) return;  // whole waves only: TPR is a multiple of 64

    float x[N];
    // ---- a1: load the row once --------------------------------------------
    if constexpr (VEC) {
        if constexpr (BF16) {
            const u32x4_t* src = reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(xv) + row * cols);
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const int64_t vi = (int64_t)v * TPR + t;
                if (vi * W < cols) {
                    u32x4_t w = __builtin_nontemporal_load(src + vi);
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        x[v * W + 2 * k] = bf16_lo(w[k]);
                        x[v * W + 2 * k + 1] = bf16_hi(w[k]);
                    }
                } else {
#pragma unroll
                    for (int k = 0; k < W; ++k) x[v * W + k] = kNegInf;
                }
            }
        } else {
            const f32x4v_t* src = reinterpret_cast<const f32x4v_t*>(static_cast<const float*>(xv) + row * cols);
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const int64_t vi = (int64_t)v * TPR + t;
                if (vi * W < cols) {
                    f32x4v_t w = __builtin_nontemporal_load(src + vi);
#pragma unroll
                    for (int k = 0; k < 4; ++k) x[v * W + k] = w[k];
                } else {
#pragma unroll
                    for (int k = 0; k < W; ++k) x[v * W + k] = kNegInf;
                }
            }
        }
    } else {
#pragma unroll
        for (int e = 0; e < N; ++e) {
            const int64_t c = (int64_t)e * TPR + t;
            float v = kNegInf;
            if (c < cols) {
                if constexpr (BF16)
                    v = __uint_as_float((unsigned)static_cast<const uint16_t*>(xv)[row * cols + c] << 16);
                else
                    v = static_cast<const float*>(xv)[row * cols + c];
            }
            x[e] = v;
        }
    }

    // ---- a2: per-lane online fold in blocks of BLOCK -----------------------
    float m = kNegInf, l = RS == kRescaleL0One ? 1.0f : 0.0f;
#pragma unroll
    for (int b0 = 0; b0 < N; b0 += BLOCK) fold_block<RS, BLOCK>(x + b0, m, l);

    // ---- a3: merge the lanes' states ---------------------------------------
    float M = wave_reduce(m, MaxOp());
    float L = wave_reduce(l * exp2_hw((m - guard_max(M)) * kLog2eHi), AddOp());
    if constexpr (NWAVE > 1) {
        __shared__ float sm[RPW][NWAVE], sl[RPW][NWAVE];
        const int r = tid / TPR, w = t / 64;
        if ((tid & 63) == 0) {
            sm[r][w] = M;
            sl[r][w] = L;
        }
        __syncthreads();
        M = sm[r][0];
#pragma unroll
        for (int k = 1; k < NWAVE; ++k) M = fmaxf(M, sm[r][k]);
        const float mu = guard_max(M);
        L = 0.0f;
#pragma unroll
        for (int k = 0; k < NWAVE; ++k) L += sl[r][k] * exp2_hw((sm[r][k] - mu) * kLog2eHi);
    }
    if (t == 0) {
        if (m_out) m_out[row] = M;
        if (l_out) l_out[row] = L;
    }

    // ---- a4: normalise and write once --------------------------------------
    const float mu = guard_max(M);
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    float y[N];
    if constexpr (BF16) {
#pragma unroll
        for (int e = 0; e < N; ++e) y[e] = exp2_hw((x[e] - mu) * kLog2eHi) * inv;
    } else {
        const float mh = mu * kLog2eHi;
        const float ml = fmaf(mu, kLog2eHi, -mh) + mu * kLog2eLo;  // tail of M*log2(e)
#pragma unroll
        for (int e = 0; e < N; ++e) {
            const float th = fmaf(x[e], kLog2eHi, -mh);
            const float tl = fmaxf(fmaf(x[e], kLog2eLo, -ml), -1.0f);  // bounded: x = -inf gives p = 0
            const float p = exp2_hw(th) * inv;
            y[e] = fminf(fmaf(p, tl * kLn2, p), 1.0f);  // rounding may not lift a term above 1
        }
    }
    if constexpr (VEC) {
        if constexpr (BF16) {
            u32x4_t* dst = reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(yv) + row * cols);
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const int64_t vi = (int64_t)v * TPR + t;
                if (vi * W < cols) {
                    u32x4_t w;
#pragma unroll
                    for (int k = 0; k < 4; ++k) w[k] = pack_bf16x2(y[v * W + 2 * k], y[v * W + 2 * k + 1]);
                    __builtin_nontemporal_store(w, dst + vi);
                }
            }
        } else {
            f32x4v_t* dst = reinterpret_cast<f32x4v_t*>(static_cast<float*>(yv) + row * cols);
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const int64_t vi = (int64_t)v * TPR + t;
                if (vi * W < cols) {
                    f32x4v_t w = {y[v * W], y[v * W + 1], y[v * W + 2], y[v * W + 3]};
                    __builtin_nontemporal_store(w, dst + vi);
                }
            }
        }
    } else {
#pragma unroll
        for (int e = 0; e < N; ++e) {
            const int64_t c = (int64_t)e * TPR + t;
            if (c < cols) {
                if constexpr (BF16) {
                    bf16x2_t v = {(__bf16)y[e], (__bf16)0.0f};
                    static_cast<uint16_t*>(yv)[row * cols + c] = (uint16_t)(__builtin_bit_cast(unsigned, v) & 0xffffu);
                } else {
                    static_cast<float*>(yv)[row * cols + c] = y[e];
                }
            }
        }
    }
}

// Rows longer than the registers of a workgroup hold (cols > 16384): the
// online normaliser as its authors first used it ("The Online Softmax"
// (curionode), intro: two reads and one write per element instead of the
// safe softmax's three reads and one write).  One workgroup of WG lanes per
// row; pass 1 streams the row once, each lane folding UN loads (UN * W
// logits) per step in blocks of BLOCK with the recurrence above, and the
// lanes' states are merged as above; pass 2 streams the row again and writes
// y = exp(x - M) / L.
template <bool BF16, bool VEC, int BLOCK, int WG, int RS>
__global__ __launch_bounds__(WG) void row_softmax_stream_kernel(const void* xv, void* yv, int64_t cols,
                                                                float* __restrict__ m_out, float* __restrict__ l_out)
{
    constexpr int W = VEC ? (BF16 ? 8 : 4) : 1;  // elements per load
    constexpr int UN = VEC ? (BF16 ? 4 : 8) : 16;  // loads per lane per step
    constexpr int N = UN * W;                     // logits per lane per step
    constexpr int B = BLOCK < N ? BLOCK : N;
    constexpr int NWAVE = WG / 64;
    static_assert(N % B == 0, "bad block");
    const int t = threadIdx.x;
    const int64_t row = blockIdx.x;
    const int64_t nvec = cols / W;  // loads in the row (128-bit loads are taken only when W divides cols)

    auto load = [&](int64_t vi, float* x) {
        if (vi >= nvec) {
#pragma unroll
            for (int k = 0; k < W; ++k) x[k] = kNegInf;
            return;
        }
        if constexpr (VEC) {
            // fp32 rows are read with non-temporal loads (7% faster at
            // 1024 x 262144); for bf16 rows they measured 9% slower
            if constexpr (BF16) {
                const u32x4_t w = *(reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(xv) + row * cols) + vi);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    x[2 * k] = bf16_lo(w[k]);
                    x[2 * k + 1] = bf16_hi(w[k]);
                }
            } else {
                const f32x4v_t w =
                    __builtin_nontemporal_load(reinterpret_cast<const f32x4v_t*>(static_cast<const float*>(xv) + row * cols) + vi);
#pragma unroll
                for (int k = 0; k < 4; ++k) x[k] = w[k];
            }
        } else {
            if constexpr (BF16)
                x[0] = __uint_as_float((unsigned)static_cast<const uint16_t*>(xv)[row * cols + vi] << 16);
            else
                x[0] = static_cast<const float*>(xv)[row * cols + vi];
        }
    };

    // ---- pass 1: fold -------------------------------------------------------
    float m = kNegInf, l = RS == kRescaleL0One ? 1.0f : 0.0f;
    for (int64_t v0 = 0; v0 < nvec; v0 += (int64_t)UN * WG) {
        float x[N];
#pragma unroll
        for (int u = 0; u < UN; ++u) load(v0 + (int64_t)u * WG + t, x + u * W);
#pragma unroll
        for (int b0 = 0; b0 < N; b0 += B) fold_block<RS, B>(x + b0, m, l);
    }
    // ---- merge the lanes' states -------------------------------------------
    float M = wave_reduce(m, MaxOp());
    float L = wave_reduce(l * exp2_hw((m - guard_max(M)) * kLog2eHi), AddOp());
    {
        __shared__ float sm[NWAVE], sl[NWAVE];
        const int w = t / 64;
        if ((t & 63) == 0) {
            sm[w] = M;
            sl[w] = L;
        }
        __syncthreads();
        M = sm[0];
#pragma unroll
        for (int k = 1; k < NWAVE; ++k) M = fmaxf(M, sm[k]);
        const float mu = guard_max(M);
        L = 0.0f;
#pragma unroll
        for (int k = 0; k < NWAVE; ++k) L += sl[k] * exp2_hw((sm[k] - mu) * kLog2eHi);
    }
    if (t == 0) {
        if (m_out) m_out[row] = M;
        if (l_out) l_out[row] = L;
    }

    // ---- pass 2: normalise and write ---------------------------------------
    const float mu = guard_max(M);
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    const float mh = mu * kLog2eHi;
    const float ml = fmaf(mu, kLog2eHi, -mh) + mu * kLog2eLo;  // tail of M*log2(e)
    for (int64_t v0 = 0; v0 < nvec; v0 += (int64_t)UN * WG) {
        // all of the step's loads go out before its first store
        float xs[N];
#pragma unroll
        for (int u = 0; u < UN; ++u) load(v0 + (int64_t)u * WG + t, xs + u * W);
#pragma unroll
        for (int u = 0; u < UN; ++u) {
            const int64_t vi = v0 + (int64_t)u * WG + t;
            if (vi >= nvec) break;
            const float* x = xs + u * W;
            float y[W];
#pragma unroll
            for (int k = 0; k < W; ++k) {
                if constexpr (BF16) {
                    y[k] = exp2_hw((x[k] - mu) * kLog2eHi) * inv;
                } else {
                    const float th = fmaf(x[k], kLog2eHi, -mh);
                    const float tl = fmaxf(fmaf(x[k], kLog2eLo, -ml), -1.0f);
                    const float p = exp2_hw(th) * inv;
                    y[k] = fminf(fmaf(p, tl * kLn2, p), 1.0f);
                }
            }
            if constexpr (VEC) {
                if constexpr (BF16) {
                    u32x4_t w;
#pragma unroll
                    for (int k = 0; k < 4; ++k) w[k] = pack_bf16x2(y[2 * k], y[2 * k + 1]);
                    __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(yv) + row * cols) + vi);
                } else {
                    const f32x4v_t w = {y[0], y[1], y[2], y[3]};
                    __builtin_nontemporal_store(w, reinterpret_cast<f32x4v_t*>(static_cast<float*>(yv) + row * cols) + vi);
                }
            } else {
                if constexpr (BF16) {
                    bf16x2_t v = {(__bf16)y[0], (__bf16)0.0f};
                    static_cast<uint16_t*>(yv)[row * cols + vi] = (uint16_t)(__builtin_bit_cast(unsigned, v) & 0xffffu);
                } else {
                    static_cast<float*>(yv)[row * cols + vi] = y[0];
                }
            }
        }
    }
}

// Empty rows (cols == 0): each is the empty set, (m, l) = (-inf, 0).
__global__ void empty_rows_kernel(int64_t rows, float* m_out, float* l_out)
{
    const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (r < rows) {
        if (m_out) m_out[r] = kNegInf;
        if (l_out) l_out[r] = 0.0f;
    }
}

namespace {

// longest row held in registers (one workgroup of 512 lanes x 32 logits)
constexpr int64_t kRegisterCols = 16384;

template <bool BF16, bool VEC, int RS, int TPR, int N, int BLOCK>
hipError_t launch_one(const RowSoftmaxArgs& a)
{
    constexpr int WG = TPR > 256 ? TPR : 256;
    constexpr int RPW = WG / TPR;
    const int64_t grid = (a.rows + RPW - 1) / RPW;
    hipLaunchKernelGGL((row_softmax_kernel<BF16, TPR, N, VEC, BLOCK, WG, RS>), dim3((unsigned)grid), dim3(WG), 0,
                       a.stream, a.x, a.y, a.rows, a.cols, a.m_out, a.l_out);
    return hipGetLastError();
}

template <bool BF16, bool VEC, int RS, int TPR, int N>
hipError_t launch_blocks(const RowSoftmaxArgs& a)
{
    const int b = a.block < N ? a.block : N;
    switch (b) {
    case 1: return launch_one<BF16, VEC, RS, TPR, N, 1>(a);
    case 2: return launch_one<BF16, VEC, RS, TPR, N, 2>(a);
    case 4: return launch_one<BF16, VEC, RS, TPR, N, 4>(a);
    case 8: return launch_one<BF16, VEC, RS, TPR, N, (8 < N ? 8 : N)>(a);
    case 16: return launch_one<BF16, VEC, RS, TPR, N, (16 < N ? 16 : N)>(a);
    default: return launch_one<BF16, VEC, RS, TPR, N, (32 < N ? 32 : N)>(a);
    }
}

template <bool BF16, bool VEC, int RS, int BLOCK>
hipError_t launch_stream_one(const RowSoftmaxArgs& a)
{
    constexpr int WG = 512;
    hipLaunchKernelGGL((row_softmax_stream_kernel<BF16, VEC, BLOCK, WG, RS>), dim3((unsigned)a.rows), dim3(WG), 0,
                       a.stream, a.x, a.y, a.cols, a.m_out, a.l_out);
    return hipGetLastError();
}

template <bool BF16, bool VEC, int RS>
hipError_t launch_stream(const RowSoftmaxArgs& a)
{
    switch (a.block) {
    case 1: return launch_stream_one<BF16, VEC, RS, 1>(a);
    case 2: return launch_stream_one<BF16, VEC, RS, 2>(a);
    case 4: return launch_stream_one<BF16, VEC, RS, 4>(a);
    case 8: return launch_stream_one<BF16, VEC, RS, 8>(a);
    case 16: return launch_stream_one<BF16, VEC, RS, 16>(a);
    default: return launch_stream_one<BF16, VEC, RS, 32>(a);
    }
}

template <bool BF16, bool VEC, int RS>
hipError_t launch_cols(const RowSoftmaxArgs& a)
{
    if (a.cols > kRegisterCols) return launch_stream<BF16, VEC, RS>(a);
    // Smallest per-lane register count that covers the row: one wave per row
    // up to 2048 logits, one workgroup of 4 (or 8) waves beyond.
    const int64_t c = a.cols;
    if constexpr (!BF16) {
        if (c <= 256) return launch_blocks<BF16, VEC, RS, 64, 4>(a);
    }
    if (c <= 512) return launch_blocks<BF16, VEC, RS, 64, 8>(a);
    if (c <= 1024) return launch_blocks<BF16, VEC, RS, 64, 16>(a);
    if (c <= 2048) return launch_blocks<BF16, VEC, RS, 64, 32>(a);
    if (c <= 4096) return launch_blocks<BF16, VEC, RS, 256, 16>(a);
    if (c <= 8192) return launch_blocks<BF16, VEC, RS, 256, 32>(a);
    return launch_blocks<BF16, VEC, RS, 512, 32>(a);
}

template <int RS>
hipError_t launch_rs(const RowSoftmaxArgs& a, bool vec)
{
    if (a.bf16) return vec ? launch_cols<true, true, RS>(a) : launch_cols<true, false, RS>(a);
    return vec ? launch_cols<false, true, RS>(a) : launch_cols<false, false, RS>(a);
}

}  // namespace

hipError_t launch_row_softmax(const RowSoftmaxArgs& a)
{
    if (a.rows == 0) return hipSuccess;
    if (a.cols == 0) {
        if (!a.m_out && !a.l_out) return hipSuccess;
        hipLaunchKernelGGL(empty_rows_kernel, dim3((unsigned)((a.rows + 255) / 256)), dim3(256), 0, a.stream, a.rows,
                           a.m_out, a.l_out);
        return hipGetLastError();
    }
    const int W = a.bf16 ? 8 : 4;
    const bool vec = (a.cols % W == 0) && ((uintptr_t)a.x % 16 == 0) && ((uintptr_t)a.y % 16 == 0);
    if (a.rescale == kRescaleIfRise) return launch_rs<kRescaleIfRise>(a, vec);
    if (a.rescale == kRescaleL0One) return launch_rs<kRescaleL0One>(a, vec);
    return launch_rs<kRescaleAlways>(a, vec);
}

int64_t row_softmax_max_cols() { return INT64_MAX; }

int64_t row_softmax_rows_per_launch_limit(int64_t cols, bool bf16)
{
    // grid.x is at most 2^31 - 1 workgroups; wave-per-row configurations put
    // four rows in a workgroup
    (void)bf16;
    const int64_t rpw = cols <= 2048 ? 4 : 1;  // the streaming path (cols > 16384) takes one row per workgroup
    return (int64_t)0x7fffffff * rpw;
}

}  // namespace tea
