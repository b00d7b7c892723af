// Split-KV decode: one query token per (batch, head) against a ragged KV
// cache, split into num_splits contiguous chunks whose partial softmax states
// (m, l, O) are merged by the associative combine ("The Online Softmax"
// (curionode), One pass, exactly; "Online Softmax" (metalworking),
// Recognition guide: split-KV decode kernels merge partials with the same
// correction, with no float atomics).
//
// Launch 1 (this file): one wave per (b, h, chunk).  Chunk c of a sequence of
// L keys covers keys [floor(c L / S), floor((c+1) L / S)), so chunks are empty
// when L < S.  Each lane group of D/8 lanes owns one key slot and a slice of 8
// dimensions; per step a slot takes U keys, computes their scores (DPP
// reduction across the group), and folds them into its running (m, l, O) with
// the online recurrence.  The slots' states are merged inside the wave by a
// butterfly and the chunk's state is written to the workspace (maxima in
// base-two units, O unnormalised).  K and V are read from HBM exactly once,
// with non-temporal loads.
// Launch 2 (merge.hip): a tree merge of the num_splits partials per (b, h).
#include <atomic>
#include <mutex>

#include "common.hpp"
#include "launch.hpp"

namespace tea {

hipError_t launch_merge_base2(const MergeArgs& a);

// Partial states of the allocation-free decode (attn_decode_splitkv_noalloc):
// a file-scope device array, one copy on every GPU the library runs on, held
// until the process ends.  In host code `scratch` names a host-side stand-in,
// not the device memory: its device address is looked up once per device
// (hipGetSymbolAddress, with that device current) and only that address is
// handed to kernels.  Every call on a GPU shares the GPU's copy and leaves its
// partials in it; each call writes every partial it reads, so nothing needs
// clearing, and calls that overlap on one GPU race.
static __device__ __align__(256) char scratch[kDecodeScratchBytes];

namespace {

template <int D>
__device__ __forceinline__ float group_sum(float v)
{
    // sum over the D/8 lanes of one key slot
    v += dpp_f<0xB1>(v);
    v += dpp_f<0x4E>(v);
    v += dpp_f<0x141>(v);
    if constexpr (D == 128) v += dpp_f<0x140>(v);
    return v;
}

// (m1, l1, O1) <- combine((m1, l1, O1), (m2, l2, O2)), base-two maxima.
__device__ __forceinline__ void combine8(float& m1, float& l1, float* O1, float m2, float l2, const float* O2)
{
    const float m = fmaxf(m1, m2);
    const float mu = guard_max(m);
    const float a1 = exp2_hw(m1 - mu), a2 = exp2_hw(m2 - mu);
    l1 = fmaf(a1, l1, a2 * l2);
#pragma unroll
    for (int d = 0; d < 8; ++d) O1[d] = fmaf(a1, O1[d], a2 * O2[d]);
    m1 = m;
}

// the same combine for one dimension
__device__ __forceinline__ void combine8_1(float& m1, float& l1, float& O1, float m2, float l2, float O2)
{
    const float m = fmaxf(m1, m2);
    const float mu = guard_max(m);
    const float a1 = exp2_hw(m1 - mu), a2 = exp2_hw(m2 - mu);
    l1 = fmaf(a1, l1, a2 * l2);
    O1 = fmaf(a1, O1, a2 * O2);
    m1 = m;
}

// The partial state of one chunk [k0, k1) of one (b, h): each group of D/8
// lanes owns a key slot and 8 dimensions; per step a slot takes U keys,
// computes their scores (DPP reduction across the group) and folds them into
// its running (m, l, O) with the online recurrence; the slots' states are then
// merged by a butterfly over lane groups (both partners combine (lower slot,
// upper slot) in that order).  On return every lane group holds the chunk's
// state for its 8 dimensions; maxima are in base-two units.
// One level of the butterfly that merges the key slots' states: lanes X
// apart exchange (m, l, O) and both compute combine(lower, upper), so both
// hold the same bits; then the next level.
template <int X>
__device__ __forceinline__ void slot_butterfly(int lane, float& m, float& l, float* O)
{
    if constexpr (X < 64) {
        float mp = lane_xor<X>(m), lp = lane_xor<X>(l), Op[8];
#pragma unroll
        for (int d = 0; d < 8; ++d) Op[d] = lane_xor<X>(O[d]);
        if (lane & X) {
            float Om[8], mm = m, lm = l;
#pragma unroll
            for (int d = 0; d < 8; ++d) {
                Om[d] = O[d];
                O[d] = Op[d];
            }
            m = mp;
            l = lp;
            combine8(m, l, O, mm, lm, Om);
        } else {
            combine8(m, l, O, mp, lp, Op);
        }
        slot_butterfly<X * 2>(lane, m, l, O);
    }
}

template <int D, int U>
__device__ __forceinline__ void chunk_state(const float* qs, const u32x4_t* kb, const u32x4_t* vb, int64_t k0,
                                            int64_t k1, int lane, float& m, float& l, float* O)
{
    constexpr int LPK = D / 8;     // lanes per key
    constexpr int KPW = 64 / LPK;  // key slots per wave
    constexpr int RS = D / 8;      // row stride in 16-byte units
    const int slot = lane / LPK;
    m = kNegInf;
    l = 0.0f;
#pragma unroll
    for (int d = 0; d < 8; ++d) O[d] = 0.0f;

    // each step: U keys per slot, KPW slots -> U * KPW consecutive keys
    for (int64_t base = k0; base < k1; base += U * KPW) {
        u32x4_t kr[U], vr[U];
        bool ok[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            int64_t key = base + u * KPW + slot;
            ok[u] = key < k1;
            key = ok[u] ? key : k1 - 1;  // in bounds; its score is masked below
            kr[u] = __builtin_nontemporal_load(kb + key * RS);
            vr[u] = __builtin_nontemporal_load(vb + key * RS);
        }
        float s[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float acc = 0.0f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                acc = fmaf(qs[2 * j], bf16_lo(kr[u][j]), acc);
                acc = fmaf(qs[2 * j + 1], bf16_hi(kr[u][j]), acc);
            }
            acc = group_sum<D>(acc);
            s[u] = ok[u] ? acc : kNegInf;
        }
        float bm = s[0];
#pragma unroll
        for (int u = 1; u < U; ++u) bm = fmaxf(bm, s[u]);
        const float mn = fmaxf(m, bm);
        const float mu = guard_max(mn);
        const float corr = exp2_hw(m - mu);
        float ps = 0.0f;
#pragma unroll
        for (int d = 0; d < 8; ++d) O[d] *= corr;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float p = exp2_hw(s[u] - mu);
            ps += p;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                O[2 * j] = fmaf(p, bf16_lo(vr[u][j]), O[2 * j]);
                O[2 * j + 1] = fmaf(p, bf16_hi(vr[u][j]), O[2 * j + 1]);
            }
        }
        l = fmaf(l, corr, ps);
        m = mn;
    }

    // butterfly over the key slots of the wave (lane distances LPK .. 32),
    // the exchanges by DPP and permlane swaps
    slot_butterfly<LPK>(lane, m, l, O);
}

// q of (b, h) with scale * log2(e) folded in once (scores come out in base
// two): lane group member dl holds dimensions 8 dl .. 8 dl + 8
// The sequence that the r-th sequence slot of the grid takes: sequences in
// descending kv_len (ties by index), so the chunks of the longest sequences
// are dispatched first and the last to finish are short ones (longest
// processing time first; about 3% at a uniform length mix of 16 sequences).
// Each lane ranks one sequence; with more than 64 sequences the grid order
// is kept.  The chunks and the merge do not depend on this order.
__device__ __forceinline__ int seq_by_length(const int32_t* __restrict__ kv_len, int B, int Lmax, int r)
{
    if (B > 64) return r;
    const int lane = threadIdx.x & 63;
    auto clamp_len = [Lmax](int x) { return x < 0 ? 0 : (x > Lmax ? Lmax : x); };
    const int Li = lane < B ? clamp_len(kv_len[lane]) : -1;
    int rank = 0;
    for (int j = 0; j < B; ++j) {
        const int Lj = clamp_len(kv_len[j]);
        rank += (Lj > Li || (Lj == Li && j < lane)) ? 1 : 0;
    }
    const uint64_t hit = __builtin_amdgcn_ballot_w64(lane < B && rank == r);
    return hit ? (int)__builtin_ctzll(hit) : r;
}

template <int D>
__device__ __forceinline__ void load_q(const uint16_t* q, int64_t bh, int dl, float scale_log2, float* qs)
{
    const u32x4_t w4 = *reinterpret_cast<const u32x4_t*>(q + bh * D + dl * 8);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        qs[2 * j] = bf16_lo(w4[j]) * scale_log2;
        qs[2 * j + 1] = bf16_hi(w4[j]) * scale_log2;
    }
}

// Launch 1 of the two-launch form: one wave per (b, h, chunk).  A wave streams
// its chunk's keys on its own, so there is no LDS and no barrier, and many
// chunks are in flight per CU.
template <int D, int U>
__global__ __launch_bounds__(256) void decode_partial_kernel(const uint16_t* __restrict__ q,
                                                             const uint16_t* __restrict__ k,
                                                             const uint16_t* __restrict__ v,
                                                             const int32_t* __restrict__ kv_len, int64_t nchunks, int H,
                                                             int Lmax, int S, float scale_log2, float* __restrict__ ws_m,
                                                             float* __restrict__ ws_l, float* __restrict__ ws_O)
{
    constexpr int LPK = D / 8;
    const int lane = threadIdx.x & 63;
    const int64_t gw = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // chunk handled by this wave
    if (gw >= nchunks) return;  // whole wave
    const int dl = lane % LPK;
    const int c = (int)(gw % S);
    const int64_t slot = gw / S;  // (sequence slot, head)
    const int h = (int)(slot % H);
    const int b = seq_by_length(kv_len, (int)(nchunks / ((int64_t)S * H)), Lmax, (int)(slot / H));
    const int64_t bh = (int64_t)b * H + h;
    int L = kv_len[b];
    L = L < 0 ? 0 : (L > Lmax ? Lmax : L);
    const int64_t k0 = (int64_t)c * L / S, k1 = (int64_t)(c + 1) * L / S;

    float qs[8];
    load_q<D>(q, bh, dl, scale_log2, qs);
    const u32x4_t* kb = reinterpret_cast<const u32x4_t*>(k + bh * (int64_t)Lmax * D + dl * 8);
    const u32x4_t* vb = reinterpret_cast<const u32x4_t*>(v + bh * (int64_t)Lmax * D + dl * 8);
    float m, l, O[8];
    chunk_state<D, U>(qs, kb, vb, k0, k1, lane, m, l, O);
    if (lane < LPK) {
        const int64_t p = bh * S + c;
        if (lane == 0) {
            ws_m[p] = m;
            ws_l[p] = l;
        }
        f32x4v_t* dst = reinterpret_cast<f32x4v_t*>(ws_O + p * D + dl * 8);
        dst[0] = f32x4v_t{O[0], O[1], O[2], O[3]};
        dst[1] = f32x4v_t{O[4], O[5], O[6], O[7]};
    }
}

// Single-launch form: one workgroup of kFW waves per (b, h); the chunks are
// the leaves 0 .. 4 kFW - 1 of a balanced binary tree (leaves at or past
// num_splits are empty), wave w takes leaves 4w .. 4w + 3 and combines them
// as the tree's two lowest levels, and the waves' states are combined through
// LDS as its upper levels.  The tree and the combine are those of the
// two-launch form (whose merge is the same balanced tree over the partial
// index); within a chunk a slot takes 4 keys per step instead of 8, to fit
// 16 waves' registers, so the two agree up to rounding.  This form needs no
// workspace and one launch, as the Apple decode kernels merge their
// simdgroups ("Online Softmax" (metalworking), Recognition guide), but all
// of a (b, h) runs on one CU.
constexpr int kFW = 16;  // waves per workgroup: 64 leaves

template <int D, int U, bool OUT_BF16>
__global__ __launch_bounds__(64 * kFW) void decode_fused_kernel(const uint16_t* __restrict__ q,
                                                                const uint16_t* __restrict__ k,
                                                                const uint16_t* __restrict__ v,
                                                                const int32_t* __restrict__ kv_len, int H, int Lmax,
                                                                int S, float scale_log2, void* __restrict__ o)
{
    constexpr int LPK = D / 8;
    __shared__ float sm[kFW], sl[kFW], sO[kFW][D];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int dl = lane % LPK;
    const int h = (int)(blockIdx.x % H);
    const int b = seq_by_length(kv_len, (int)(gridDim.x / H), Lmax, (int)(blockIdx.x / H));
    const int64_t bh = (int64_t)b * H + h;
    int L = kv_len[b];
    L = L < 0 ? 0 : (L > Lmax ? Lmax : L);

    float qs[8];
    load_q<D>(q, bh, dl, scale_log2, qs);
    const u32x4_t* kb = reinterpret_cast<const u32x4_t*>(k + bh * (int64_t)Lmax * D + dl * 8);
    const u32x4_t* vb = reinterpret_cast<const u32x4_t*>(v + bh * (int64_t)Lmax * D + dl * 8);

    // leaves 4w .. 4w+3: ((4w, 4w+1), (4w+2, 4w+3))
    float m2[2], l2[2], O2[2][8];
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {
        float ma = kNegInf, la = 0.0f, Oa[8];
#pragma unroll
        for (int d = 0; d < 8; ++d) Oa[d] = 0.0f;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int c = 4 * w + 2 * pr + e;
            float mc = kNegInf, lc = 0.0f, Oc[8];
#pragma unroll
            for (int d = 0; d < 8; ++d) Oc[d] = 0.0f;
            if (c < S) {
                const int64_t k0 = (int64_t)c * L / S, k1 = (int64_t)(c + 1) * L / S;
                chunk_state<D, U>(qs, kb, vb, k0, k1, lane, mc, lc, Oc);
            }
            if (e == 0) {
                ma = mc;
                la = lc;
#pragma unroll
                for (int d = 0; d < 8; ++d) Oa[d] = Oc[d];
            } else {
                combine8(ma, la, Oa, mc, lc, Oc);
            }
        }
        m2[pr] = ma;
        l2[pr] = la;
#pragma unroll
        for (int d = 0; d < 8; ++d) O2[pr][d] = Oa[d];
    }
    combine8(m2[0], l2[0], O2[0], m2[1], l2[1], O2[1]);
    if (lane < LPK) {
        if (lane == 0) {
            sm[w] = m2[0];
            sl[w] = l2[0];
        }
#pragma unroll
        for (int d = 0; d < 8; ++d) sO[w][dl * 8 + d] = O2[0][d];
    }
    __syncthreads();

    // upper levels: thread d < D combines the kFW wave states for dimension d
    const int d = threadIdx.x;
    if (d < D) {
        float mw[kFW], lw[kFW], Ow[kFW];
#pragma unroll
        for (int i = 0; i < kFW; ++i) {
            mw[i] = sm[i];
            lw[i] = sl[i];
            Ow[i] = sO[i][d];
        }
#pragma unroll
        for (int span = 1; span < kFW; span <<= 1)
#pragma unroll
            for (int i = 0; i < kFW; i += 2 * span) combine8_1(mw[i], lw[i], Ow[i], mw[i + span], lw[i + span], Ow[i + span]);
        const float inv = lw[0] > 0.0f ? 1.0f / lw[0] : 0.0f;
        const float val = Ow[0] * inv;
        if constexpr (OUT_BF16) {
            bf16x2_t pk = {(__bf16)val, (__bf16)0.0f};
            static_cast<uint16_t*>(o)[bh * D + d] = (uint16_t)(__builtin_bit_cast(unsigned, pk) & 0xffffu);
        } else {
            static_cast<float*>(o)[bh * D + d] = val;
        }
    }
}

}  // namespace

size_t decode_workspace_bytes(int B, int H, int D, int num_splits)
{
    const size_t n = (size_t)B * H * num_splits;
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    return 2 * up(n * sizeof(float)) + up(n * D * sizeof(float));
}

void decode_bind_workspace(DecodeArgs& a, void* workspace)
{
    // m [B H S], l [B H S], O [B H S, D] fp32, each 256-byte aligned
    const size_t n = (size_t)a.B * a.H * a.num_splits;
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    char* ws = static_cast<char*>(workspace);
    a.ws_m = reinterpret_cast<float*>(ws);
    a.ws_l = reinterpret_cast<float*>(ws + up(n * 4));
    a.ws_O = reinterpret_cast<float*>(ws + 2 * up(n * 4));
}

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// device address of the current device's copy of `scratch`
hipError_t scratch_address(void** out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (!p) return hipErrorInvalidSymbol;
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return hipSuccess;
}
}  // namespace

hipError_t launch_decode_noalloc(DecodeArgs a)
{
    void* base = nullptr;
    hipError_t e = scratch_address(&base);
    if (e != hipSuccess) return e;
    decode_bind_workspace(a, base);
    return launch_decode(a);
}

hipError_t launch_decode(const DecodeArgs& a)
{
    const int64_t nchunks = (int64_t)a.B * a.H * a.num_splits;
    const int64_t grid = (nchunks + 3) / 4;
    const float scale_log2 = a.scale * kLog2eHi;
    if (a.D == 128)
        hipLaunchKernelGGL((decode_partial_kernel<128, 8>), dim3((unsigned)grid), dim3(256), 0, a.stream,
                           (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, a.kv_len, nchunks, a.H,
                           a.Lmax, a.num_splits, scale_log2, a.ws_m, a.ws_l, a.ws_O);
    else
        hipLaunchKernelGGL((decode_partial_kernel<64, 8>), dim3((unsigned)grid), dim3(256), 0, a.stream,
                           (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, a.kv_len, nchunks, a.H,
                           a.Lmax, a.num_splits, scale_log2, a.ws_m, a.ws_l, a.ws_O);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    MergeArgs m{a.ws_m, a.ws_l, a.ws_O, (int64_t)a.B * a.H, a.num_splits, a.D, nullptr, nullptr, a.o, a.out_bf16,
                true, a.stream};
    return launch_merge_base2(m);
}

hipError_t launch_decode_fused(const DecodeArgs& a)
{
    const dim3 grid((unsigned)((int64_t)a.B * a.H)), block(64 * kFW);
    const float scale_log2 = a.scale * kLog2eHi;
    const uint16_t *q = (const uint16_t*)a.q, *k = (const uint16_t*)a.k, *v = (const uint16_t*)a.v;
    if (a.D == 128) {
        if (a.out_bf16)
            hipLaunchKernelGGL((decode_fused_kernel<128, 4, true>), grid, block, 0, a.stream, q, k, v, a.kv_len, a.H,
                               a.Lmax, a.num_splits, scale_log2, a.o);
        else
            hipLaunchKernelGGL((decode_fused_kernel<128, 4, false>), grid, block, 0, a.stream, q, k, v, a.kv_len, a.H,
                               a.Lmax, a.num_splits, scale_log2, a.o);
    } else {
        if (a.out_bf16)
            hipLaunchKernelGGL((decode_fused_kernel<64, 4, true>), grid, block, 0, a.stream, q, k, v, a.kv_len, a.H,
                               a.Lmax, a.num_splits, scale_log2, a.o);
        else
            hipLaunchKernelGGL((decode_fused_kernel<64, 4, false>), grid, block, 0, a.stream, q, k, v, a.kv_len, a.H,
                               a.Lmax, a.num_splits, scale_log2, a.o);
    }
    return hipGetLastError();
}

int decode_fused_max_splits() { return 4 * kFW; }

}  // namespace tea
