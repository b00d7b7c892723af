// Tiled attention forward, O = softmax(Q K^T * scale) V, with the online
// softmax over KV tiles ("Online softmax" (roadmapper), The recurrence;
// "Online Softmax" (metalworking), The problem; "The Online Softmax"
// (curionode), One pass, exactly: blocks stream through fast memory and no
// row of scores is ever stored).
//
// Workgroup: 4 waves, 128 queries (32 per wave); KV tiles of BN keys (64 for
// D = 128, 128 for D = 64) double-buffered in LDS.  Both products run on v_mfma_f32_32x32x16_bf16 in transposed form:
//     S^T = K Q^T   (A = K tile from LDS, B = Q^T held in registers)
//     O^T = V^T P^T (A = V^T tile from LDS, B = P^T straight from the S^T
//                    accumulators)
// so a lane of the 32x32 result owns one query (lane % 32) and half of the
// keys or dimensions (lane / 32).  The per-query state m, l and the
// correction alpha are lane-local; the row maximum needs one permlane32 swap,
// and l is kept as two half sums (one per lane half) added at the end.
//
// The MFMA contraction index need not follow key order as long as both
// operands agree: P^T is used in the order its accumulator registers hold
// keys, and the V^T tile is written to LDS in that same order.
//
// Base-two exponentials throughout with scale * log2(e) folded in once (the
// correction alpha too); m starts at -inf and l at 0; a row whose keys in a
// tile are all masked keeps -inf out of every exponent through the guard
// ("Online softmax", Initialise honestly and Things that break).
#include "common.hpp"
#include "launch.hpp"

namespace tea {

namespace {

constexpr int kBM = 128;  // queries per workgroup (4 waves x 32)

// Position of key (4*kg .. 4*kg+3) inside its 16-key chunk of the V^T tile:
// keys 16c + 4a + r sit at 16c + {0, 8, 4, 12}[a] + r, which is the order in
// which the S^T accumulator registers of one lane half hold them.
__device__ __forceinline__ int vt_pos(int kg) { return 16 * (kg >> 2) + ((kg & 1) << 3) + ((kg & 2) << 1); }

// D: head dimension; BN: keys per KV tile.  Two waves per SIMD (at most 256
// registers each) so that one wave's exponentials overlap the other's MFMAs.
template <int D, int BN, bool CAUSAL, bool OUT_BF16>
__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(const uint16_t* __restrict__ q,
                                                          const uint16_t* __restrict__ k,
                                                          const uint16_t* __restrict__ v, void* __restrict__ o,
                                                          float* __restrict__ lse, int Sq, int Sk, float c, int nqb)
{
    constexpr int KST = D + 8;             // K tile row stride (elements), padded against bank conflicts
    constexpr int VST = BN + 8;            // V^T tile row stride
    constexpr int KCH = D / 8;             // 16-byte chunks per K/V row
    constexpr int KPT = BN * KCH / 256;    // K chunks staged per thread
    constexpr int NKB = BN / 32;           // 32-key blocks of S^T
    constexpr int NC4 = BN / 16;           // 16-key chunks of P^T
    constexpr int NDB = D / 32;            // 32-wide dimension blocks of O^T
    constexpr int NQC = D / 16;            // 16-wide contraction chunks of Q K^T
    constexpr int VKG = BN / 4;            // key groups of 4 in a tile
    static_assert(VKG * KCH == 256, "one 4-key x 8-dim V block per thread");
    __shared__ __attribute__((aligned(16))) uint16_t sK[2][BN * KST];
    __shared__ __attribute__((aligned(16))) uint16_t sV[2][D * VST];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int lq = lane & 31, h = lane >> 5;

    // Workgroups are dealt to the 8 XCDs round robin; regroup them so the
    // query blocks of one (b, h) run on one XCD and share its L2 copy of K, V.
    const int T = gridDim.x;
    const int bid = blockIdx.x;
    const int logical = (T % 8 == 0) ? (bid % 8) * (T / 8) + bid / 8 : bid;
    int qb = logical % nqb;
    const int64_t bh = logical / nqb;
    if (CAUSAL) qb = nqb - 1 - qb;  // longest rows first
    const int q0 = qb * kBM;
    const int qrow = q0 + w * 32 + lq;

    const uint16_t* qp = q + bh * (int64_t)Sq * D;
    const uint16_t* kp = k + bh * (int64_t)Sk * D;
    const uint16_t* vp = v + bh * (int64_t)Sk * D;

    // Q^T operand: lane (query lq, half h) holds Q[q][16c + 8h .. +8)
    bf16x8_t qop[NQC];
    {
        const bool ok = qrow < Sq;
        const int qr = ok ? qrow : Sq - 1;
#pragma unroll
        for (int cc = 0; cc < NQC; ++cc) {
            u32x4_t t4 = *reinterpret_cast<const u32x4_t*>(qp + (int64_t)qr * D + 16 * cc + 8 * h);
            if (!ok) t4 = u32x4_t{0u, 0u, 0u, 0u};
            qop[cc] = __builtin_bit_cast(bf16x8_t, t4);
        }
    }

    f32x16_t oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] = 0.0f;
    float m = kNegInf, l = 0.0f;

    const int kend = CAUSAL ? (Sk < q0 + kBM ? Sk : q0 + kBM) : Sk;
    const int ntiles = (kend + BN - 1) / BN;

    // staging registers: the next tile's K chunks and one 4-key x 8-dim V block
    u32x4_t kreg[KPT], vreg[4];
    const int vkg = tid % VKG, vdc = tid / VKG;  // V: keys 4*vkg.., dims 8*vdc..

    // per-thread element offsets of the staged chunks inside a tile
    int koff[KPT], voff[4];
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        const int i = tid + 256 * j;
        koff[j] = (i / KCH) * D + (i % KCH) * 8;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) voff[r] = (4 * vkg + r) * D + vdc * 8;

    auto gload = [&](int t) {
        const int key0 = t * BN;
        const uint16_t* kt = kp + (int64_t)key0 * D;
        const uint16_t* vt = vp + (int64_t)key0 * D;
        if (key0 + BN <= Sk) {  // full tile: no per-chunk test (uniform branch)
#pragma unroll
            for (int j = 0; j < KPT; ++j) kreg[j] = *reinterpret_cast<const u32x4_t*>(kt + koff[j]);
#pragma unroll
            for (int r = 0; r < 4; ++r) vreg[r] = *reinterpret_cast<const u32x4_t*>(vt + voff[r]);
        } else {  // ragged last tile: rows past Sk read row Sk - 1 and are zeroed
            const int nvalid = Sk - key0;
#pragma unroll
            for (int j = 0; j < KPT; ++j) {
                const int row = (tid + 256 * j) / KCH;
                const int off = row < nvalid ? koff[j] : koff[j] - (row - nvalid + 1) * D;
                const u32x4_t x = *reinterpret_cast<const u32x4_t*>(kt + off);
                kreg[j] = row < nvalid ? x : u32x4_t{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 4 * vkg + r;
                const int off = row < nvalid ? voff[r] : voff[r] - (row - nvalid + 1) * D;
                const u32x4_t x = *reinterpret_cast<const u32x4_t*>(vt + off);
                vreg[r] = row < nvalid ? x : u32x4_t{0u, 0u, 0u, 0u};
            }
        }
    };
    auto lds_store = [&](int buf) {
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const int i = tid + 256 * j;
            *reinterpret_cast<u32x4_t*>(&sK[buf][(i / KCH) * KST + (i % KCH) * 8]) = kreg[j];
        }
        // transpose the 4 x 8 block: row d of V^T gets the 4 keys' values
        const int pos = vt_pos(vkg);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {  // dims 8*vdc + 2jj (lo halves) and + 2jj + 1 (hi halves)
            const unsigned a0 = __builtin_amdgcn_perm(vreg[1][jj], vreg[0][jj], 0x05040100u);
            const unsigned a1 = __builtin_amdgcn_perm(vreg[3][jj], vreg[2][jj], 0x05040100u);
            const unsigned b0 = __builtin_amdgcn_perm(vreg[1][jj], vreg[0][jj], 0x07060302u);
            const unsigned b1 = __builtin_amdgcn_perm(vreg[3][jj], vreg[2][jj], 0x07060302u);
            const int d = 8 * vdc + 2 * jj;
            *reinterpret_cast<u32x2_t*>(&sV[buf][d * VST + pos]) = u32x2_t{a0, a1};
            *reinterpret_cast<u32x2_t*>(&sV[buf][(d + 1) * VST + pos]) = u32x2_t{b0, b1};
        }
    };

    // Two LDS buffers: tile t is read from buffer t % 2 while tile t + 1 is
    // written to the other one and tile t + 2 is in flight from HBM/L2.
    if (ntiles > 0) {
        gload(0);
        lds_store(0);
        if (ntiles > 1) gload(1);
    }
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
        const int cur = t & 1;
        const int key0 = t * BN;
        // a wave skips tiles entirely above its diagonal
        if (!(CAUSAL && key0 > q0 + w * 32 + 31)) {
            // ---- S^T = K Q^T ---------------------------------------------
            f32x16_t sacc[NKB];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.0f;
#pragma unroll
                for (int cc = 0; cc < NQC; ++cc) {
                    const bf16x8_t a =
                        *reinterpret_cast<const bf16x8_t*>(&sK[cur][(kb * 32 + lq) * KST + 16 * cc + 8 * h]);
                    sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qop[cc], sacc[kb], 0, 0, 0);
                }
            }

            // ---- mask: sequence tail and the causal diagonal --------------
            if ((key0 + BN > Sk) || (CAUSAL && key0 + BN - 1 > q0 + w * 32)) {
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = key0 + kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                        if (key >= Sk || (CAUSAL && key > qrow)) sacc[kb][r] = kNegInf;
                    }
            }

            // ---- online update (base two, scale folded into c) -------------
            float mx = kNegInf;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
            mx = fmaxf(mx, xor32(mx));
            const float mn = fmaxf(m, mx * c);
            const float mu = guard_max(mn);
            const float alpha = exp2_hw(m - mu);
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) sacc[kb][r] = exp2_hw(fmaf(sacc[kb][r], c, -mu));
            // The correction is exactly 1 for rows whose maximum did not rise;
            // when that holds for the whole wave the rescale is skipped (the
            // conditional form of "Online Softmax" (metalworking),
            // Recognition guide), which changes no bit of the result.
            if (__any(alpha != 1.0f)) {
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
            }

            // ---- P to bf16; l sums the same rounded P that multiplies V ----
            bf16x8_t pop[NC4];
            float rs = 0.0f;
            const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
            for (int c4 = 0; c4 < NC4; ++c4) {
                const int kb = c4 >> 1, g0 = 2 * (c4 & 1);
                u32x4_t t4;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    // The dot2 operand is the freshly rounded pair itself: hipcc
                    // (ROCm 7.2) feeds v_dot2c the wrong register when it is
                    // given a bit-cast element of t4 instead.
                    const bf16x2_t pv = {(__bf16)sacc[kb][4 * g0 + 2 * j], (__bf16)sacc[kb][4 * g0 + 2 * j + 1]};
                    t4[j] = __builtin_bit_cast(unsigned, pv);
                    rs = __builtin_amdgcn_fdot2_f32_bf16(pv, ones, rs, false);
                }
                pop[c4] = __builtin_bit_cast(bf16x8_t, t4);
            }
            l = fmaf(l, alpha, rs);
            m = mn;

            // ---- O^T += V^T P^T -------------------------------------------
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int c4 = 0; c4 < NC4; ++c4) {
                    const bf16x8_t a =
                        *reinterpret_cast<const bf16x8_t*>(&sV[cur][(db * 32 + lq) * VST + 16 * c4 + 8 * h]);
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pop[c4], oacc[db], 0, 0, 0);
                }
        }
        if (t + 1 < ntiles) lds_store(cur ^ 1);  // buffer cur ^ 1 was last read before the previous barrier
        if (t + 2 < ntiles) gload(t + 2);
        __syncthreads();
    }

    // ---- epilogue: O /= l, store, log-sum-exp -----------------------------
    const float lt = l + xor32(l);
    const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
    if (qrow < Sq) {
        const int64_t orow = (bh * Sq + qrow) * (int64_t)D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = db * 32 + 8 * g + 4 * h;
                const float y0 = oacc[db][4 * g] * inv, y1 = oacc[db][4 * g + 1] * inv;
                const float y2 = oacc[db][4 * g + 2] * inv, y3 = oacc[db][4 * g + 3] * inv;
                if constexpr (OUT_BF16) {
                    *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(o) + orow + d) =
                        u32x2_t{pack_bf16x2(y0, y1), pack_bf16x2(y2, y3)};
                } else {
                    *reinterpret_cast<f32x4v_t*>(static_cast<float*>(o) + orow + d) = f32x4v_t{y0, y1, y2, y3};
                }
            }
        if (lse && h == 0) lse[bh * Sq + qrow] = lt > 0.0f ? m * kLn2 + __logf(lt) : kNegInf;
    }
}

template <int D, int BN, bool CAUSAL>
hipError_t launch_d(const AttnArgs& a)
{
    const int nqb = (a.Sq + kBM - 1) / kBM;
    const int64_t grid = (int64_t)nqb * a.H * a.B;
    const float c = a.scale * kLog2eHi;
    if (a.out_bf16)
        hipLaunchKernelGGL((attn_fwd_kernel<D, BN, CAUSAL, true>), dim3((unsigned)grid), dim3(256), 0, a.stream,
                           (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, a.o, a.lse, a.Sq, a.Sk, c,
                           nqb);
    else
        hipLaunchKernelGGL((attn_fwd_kernel<D, BN, CAUSAL, false>), dim3((unsigned)grid), dim3(256), 0, a.stream,
                           (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, a.o, a.lse, a.Sq, a.Sk, c,
                           nqb);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd(const AttnArgs& a)
{
    if ((int64_t)a.B * a.H * a.Sq == 0) return hipSuccess;
    if (a.D == 128) return a.causal ? launch_d<128, 64, true>(a) : launch_d<128, 64, false>(a);
    return a.causal ? launch_d<64, 128, true>(a) : launch_d<64, 128, false>(a);
}

}  // namespace tea
