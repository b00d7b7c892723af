// Tiled attention forward, O = softmax(Q K^T * scale) V, with the online
// softmax over KV tiles ("Online softmax" (roadmapper), The recurrence;
// "Online Softmax" (metalworking), The problem; "The Online Softmax"
// (curionode), One pass, exactly: blocks stream through fast memory and no
// row of scores is ever stored).
//
// Workgroup: 32 queries per wave; 8 waves (256 queries) for head dimension
// 128, 16 waves (512 queries) for 64, so each K/V tile staged in LDS serves
// that many queries; KV tiles of 64 keys, double-buffered.  Both products
// run on v_mfma_f32_32x32x16_bf16 in transposed form:
//     S^T = K Q^T   (A = K tile from LDS, B = Q^T held in registers)
//     O^T = V^T P^T (A = V^T tile from LDS, B = P^T straight from the S^T
//                    accumulators)
// so a lane of the 32x32 result owns one query (lane % 32) and half of the
// keys or dimensions (lane / 32).  The per-query state m, l and the
// correction alpha are lane-local; the row maximum needs one permlane32 swap.
// l sums the same bf16-rounded P that multiplies V, on the matrix core
// (v_mfma_f32_16x16x32_bf16 against a 0/1 selector, the full sum in every
// lane), in the matrix phase; at head dimension 64 the tile's sum also
// checks the reference (below), before that P meets V.
//
// The MFMA contraction index need not follow key order as long as both
// operands agree: P^T is used in the order its accumulator registers hold
// keys, and the V^T tile is written to LDS in that same order.
//
// Base-two exponentials throughout with scale * log2(e) folded in once (the
// correction alpha too); m starts at -inf and l at 0; a row whose keys in a
// tile are all masked keeps -inf out of every exponent through the guard
// ("Online softmax", Initialise honestly and Things that break).
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace tea {

namespace {


typedef __attribute__((address_space(1))) const void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t* lds_s16x4_p;

// Tiles live in LDS row-major (one key per row, D contiguous bf16), without
// padding, because they are filled by direct HBM->LDS loads that write 1 KiB
// contiguously per wave.  Bank conflicts are avoided instead by XOR-swizzling
// the 16-byte chunks of each row:
//   K rows are read 16 bytes per lane, 16 lanes (16 consecutive rows) per
//   LDS cycle: chunk ^ (row % 16) (D = 128) or chunk ^ ((row / 2) % 8)
//   (D = 64, two rows share the 64 banks) puts those 16 reads on distinct
//   banks;
//   V rows are read by the transposing ds_read_b64_tr_b16, 32 lanes covering
//   4 rows x 8 half-chunks: chunk ^ 4 * (row % 4) (D = 128) or
//   chunk ^ 4 * ((row / 2) % 2) (D = 64) spreads them over all 64 banks.
template <int D>
__device__ __forceinline__ int k_swz(int row)
{
    if constexpr (D == 128) return row & 15;
    else return (row >> 1) & 7;
}
template <int D>
__device__ __forceinline__ int v_swz(int row)
{
    if constexpr (D == 128) return (row & 3) << 2;
    else return ((row >> 1) & 1) << 2;
}

// how far (base two) a score may exceed its row's reference before the
// reference has to move: P <= 2^kLag.  At head dimension 64 it is checked
// through the row's sum of P for the tile (64 keys), at most
// kMaxTileSum = 2^kLag.
constexpr float kLag = 8.0f;
constexpr float kMaxTileSum = 256.0f;

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// One wave-wide 16-byte-per-lane load from HBM straight into LDS: lane i's
// 16 bytes from `base` + `off` (base the same in every lane, off the lane's
// byte offset) land at LDS byte address `dst` + 16 i (dst the same in every
// lane).  The wave-uniform base sits in scalar registers and each lane keeps
// a 32-bit offset, not a 64-bit address.  Issued as inline assembly so that
// the compiler does not treat every later LDS read as a possible reader of
// this write and wait for the load right away (it cannot tell the buffers
// apart); the kernel instead waits for such loads (s_waitcnt vmcnt) before
// the barrier that hands the buffer to its readers.
__device__ __forceinline__ void lds_dma16(const void* base, unsigned off, const void* dst)
{
    const unsigned lds = (unsigned)(uintptr_t)dst;  // low 32 bits of a flat LDS address: the LDS offset
    asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(__builtin_amdgcn_readfirstlane(lds))
                 : "memory");
}

// D: head dimension; BN: keys per KV tile; NW: waves, 8 or 16 (two or four
// per SIMD).
//
// Two groups of NW / 2 waves per workgroup, NW / 8 waves of each group on
// every SIMD, take turns ("ping-pong"): while one group runs the matrix
// phase of a tile (M: O += V(t)^T P(t) and S(t+1) = K(t+1) Q^T, MFMAs fed
// from LDS) the other runs the softmax phase (X: reference, exponentials,
// P), which is vector work only.  A SIMD then overlaps one group's MFMAs
// with the other group's vector instructions; with 16 waves two waves of a
// group share a SIMD, which raises the vector issue rate of the softmax
// phase (a single wave issues a vector instruction only every few cycles).
// Each wave alternates X(t), M(t), X(t+1), ...; group 1 runs one phase
// behind group 0, and every phase ends at a workgroup barrier:
//   slot 2t  : group 0 X(t)        group 1 M(t-1)
//   slot 2t+1: group 0 M(t)        group 1 X(t)      + loads of V(t+1), K(t+2)
// M(t) reads V(t) and K(t+1) (slots 2t+1 and 2t+2); the loads issued in slot
// 2t+1 overwrite V(t-1) and K(t), last read in slot 2t, and are waited for at
// the end of slot 2t+2, before their first reader.
//
// Lagged reference.  The recurrence subtracts the running maximum so that no
// exponential overflows ("Online softmax" (roadmapper), The recurrence and
// Things that break); any reference r with every score - r small enough
// serves as well, since O and l are taken relative to the same r and only
// their ratio is used (and LSE = r + log l).  The reference moves only when
// a score of the tile exceeds it by more than 2^kLag (and on a row's first
// tile): then it moves to the running maximum and O and l are multiplied by
// 2^(m_old - m_new), a conditional correction as the pages attribute to
// Metal FlashAttention ("Online Softmax" (metalworking), Recognition guide),
// taken one step further.  At head dimension 128 the softmax phase checks
// this with the lane's tile maximum before the exponentials.  At 64 it
// takes P against the current reference without the maximum, and the
// matrix phase checks that P before its first product with V: if every
// row's sum of P for the tile is at most kMaxTileSum (so no single P
// exceeds it) that P stands, otherwise P is taken again after the move.  The
// reference is always a past running maximum, so some key of the row has
// P >= 1 and nothing underflows that the exact recurrence keeps; P <= 2^8
// and l <= Sk 2^8 stay far inside fp32 and bf16 range, and rounding is
// relative, so the result equals that of the exact running maximum up to
// rounding.
template <int D, int BN, int NW, bool OUT_BF16>
__global__ __launch_bounds__(64 * NW, NW / 4) void attn_fwd_kernel(const uint16_t* __restrict__ q,
                                                          const uint16_t* __restrict__ k,
                                                          const uint16_t* __restrict__ v, void* __restrict__ o,
                                                          float* __restrict__ lse, int Sq, int Sk, float c, int nqb, int causal,
                                                          int nsplit, float* __restrict__ pm, float* __restrict__ pl,
                                                          float* __restrict__ pO)
{
    static_assert(NW == 8 || NW == 16, "two groups of NW / 2 waves, NW / 8 waves of each group per SIMD");
    // causal is a runtime flag: as a template parameter it made hipcc spill
    // the non-causal instantiation
    const bool CAUSAL = causal != 0;
    constexpr int TILE = BN * D;                  // elements per K or V tile (16 KiB at D = 128, 8 KiB at 64)
    constexpr int NCH = D / 8;                    // 16-byte chunks per row
    constexpr int RPI = 1024 / (2 * D);           // rows one wave-wide 16-byte-per-lane load fills
    constexpr int kBM = 32 * NW;                  // queries per workgroup
    constexpr int NL = TILE * 2 / 1024;           // such loads per tile
    constexpr int DPW = NL >= NW ? NL / NW : 1;   // loads per wave per tile
    constexpr int NKB = BN / 32;                  // 32-key blocks of S^T
    constexpr int NC4 = BN / 16;                  // 16-key chunks of P^T
    constexpr int NDB = D / 32;                   // 32-wide dimension blocks of O^T
    constexpr int NQC = D / 16;                   // 16-wide contraction chunks of Q K^T
    static_assert((NL >= NW && DPW * NW == NL) || (NL < NW && 2 * NL <= NW), "tile loads must split evenly");
    static_assert(NL * RPI == BN, "tile rows");
    __shared__ __attribute__((aligned(1024))) uint16_t sK[2][TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t sV[2][TILE];
    // Staging of each wave's 32 rows of Q (in the prologue) and of O (bf16,
    // in the epilogue).  In the operand and accumulator layouts a lane holds
    // a few dimensions of one query, so a wave's direct loads and stores
    // would touch all 32 of its rows per instruction; through LDS the wave
    // reads Q and writes O (32 rows, contiguous in HBM) 1 KiB per
    // instruction instead.  One region per wave, rows padded by 16 bytes so
    // that 16-byte accesses stay aligned.
    constexpr int ORS = D + 8;
    __shared__ __attribute__((aligned(16))) uint16_t sO[NW][32 * ORS];

    // the wave index is uniform: keep it (and all that derives from it) in
    // scalar registers
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lq = lane & 31, h = lane >> 5;
    const int grp = w / (NW / 2);  // wave w runs on SIMD w % 4

    // Workgroups are dealt to the 8 XCDs round robin; regroup them so the
    // query blocks of one (b, h) run on one XCD and share its L2 copy of K, V.
    const int G = gridDim.x;
    const int bid = blockIdx.x;
    const int logical = (G % 8 == 0) ? (bid % 8) * (G / 8) + bid / 8 : bid;
    // split-K (nsplit > 1): workgroup `split` of a query block takes its
    // share of the KV tiles and writes a partial state
    const int split = logical % nsplit;
    const int lq_block = logical / nsplit;
    int qb = lq_block % nqb;
    int64_t bh = lq_block / nqb;
    if (CAUSAL) qb = nqb - 1 - qb;  // longest rows first
    const int nbh = G / (nqb * nsplit);
    if (CAUSAL && nsplit == 1 && G % 8 == 0 && nbh % 8 == 0) {
        // each XCD owns nbh / 8 heads and takes them two at a time; within a
        // pair the query blocks go longest first across both heads (the
        // pair's longest block, then the next longest, ...).  Longest first
        // shortens the tail of uneven causal blocks; keeping to two heads
        // keeps the blocks that run at the same time close in their walk
        // over K and V, so a K/V tile fetched into the XCD's L2 is still
        // there for the other blocks of its head.
        const int x = bid % 8, local = bid / 8, bhx = nbh / 8;
        const int gh = bhx % 2 == 0 ? 2 : 1;
        const int per = gh * nqb, gi = local / per, in = local % per;
        qb = nqb - 1 - in / gh;
        bh = (int64_t)x * bhx + gi * gh + in % gh;
    }
    const int q0 = qb * kBM;
    const int qrow = q0 + w * 32 + lq;
    const int qlast = q0 + w * 32 + 31;  // last query of this wave

    const uint16_t* qp = q + bh * (int64_t)Sq * D;
    const char* kp = reinterpret_cast<const char*>(k + bh * (int64_t)Sk * D);
    const char* vp = reinterpret_cast<const char*>(v + bh * (int64_t)Sk * D);

    // Q^T operand: lane (query lq, half h) holds Q[q][16c + 8h .. +8)
    // Q: the wave's 32 rows are contiguous, so lane i of load j takes 16-byte
    // chunk j * 64 + i of them (1 KiB per instruction); the rows go through
    // the wave's LDS staging region into the operand layout after the
    // prologue's wait.  Rows past the sequence read its last row and are
    // zeroed.
    constexpr int QCPR = D / 8;               // 16-byte chunks per row
    constexpr int NQL = 32 * QCPR / 64;       // such loads per lane
    u32x4_t qld[NQL];
#pragma unroll
    for (int j = 0; j < NQL; ++j) {
        const int ci = j * 64 + lane, r = ci / QCPR, u = ci % QCPR;
        const int row = q0 + w * 32 + r;
        qld[j] = *reinterpret_cast<const u32x4_t*>(qp + (int64_t)(row < Sq ? row : Sq - 1) * D + 8 * u);
        if (row >= Sq) qld[j] = u32x4_t{0u, 0u, 0u, 0u};
    }
    bf16x8_t qop[NQC];

    f32x16_t oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] = 0.0f;
    float m = kNegInf;

    const int kend = CAUSAL ? (Sk < q0 + kBM ? Sk : q0 + kBM) : Sk;
    const int nall = (kend + BN - 1) / BN;
    // this workgroup's tiles: [t0, t0 + ntiles) of the query block's nall;
    // t below is the index within that range and key0 = kbase + t * BN
    const int t0 = (int)((int64_t)split * nall / nsplit);
    const int ntiles = (int)((int64_t)(split + 1) * nall / nsplit) - t0;
    const int kbase = t0 * BN;
    // tiles after tlast hold no key visible to any query of this wave
    const int tlast = !CAUSAL ? ntiles - 1 : (qlast < kbase ? -1 : min(ntiles - 1, (qlast - kbase) / BN));

    // ---- HBM -> LDS: lane `lane` of load L fills 16 bytes at byte
    // L * 1024 + 16 * lane of the tile, i.e. row L * RPI + lane / NCH,
    // physical chunk lane % NCH, which holds logical chunk
    // (lane % NCH) ^ swizzle(row).  Rows past the sequence end repeat the
    // last valid row (their scores are masked, their values meet P = 0).
    // With fewer loads than waves (NL < NW), K is loaded by waves
    // 0 .. NL - 1 and V by waves NL .. 2 NL - 1, one load each, so a wave
    // keeps one row and one chunk offset per lane.
    const bool wv = NL < NW && w >= NL;
    const int wrow = (wv ? w - NL : w) * RPI + lane / NCH;
    const int wchunk = ((lane % NCH) ^ (wv ? v_swz<D>(wrow) : k_swz<D>(wrow))) << 4;
    auto dma = [&](const char* src, uint16_t* tile, bool is_v, int key0) {
        const char* g = src + (int64_t)key0 * 2 * D;
        const int nvalid = Sk - key0;  // >= 1 for every tile loaded
        if constexpr (NL < NW) {
            if (is_v != wv || w >= 2 * NL) return;
            const int srow = wrow < nvalid ? wrow : nvalid - 1;
            lds_dma16(g, (unsigned)(srow * 2 * D + wchunk), tile + (w - (is_v ? NL : 0)) * 512);
        } else {
#pragma unroll
            for (int j = 0; j < DPW; ++j) {
                const int L = w * DPW + j;
                const int row = L * RPI + lane / NCH;
                const int chunk = (lane % NCH) ^ (is_v ? v_swz<D>(row) : k_swz<D>(row));
                const int srow = row < nvalid ? row : nvalid - 1;
                lds_dma16(g, (unsigned)(srow * 2 * D + (chunk << 4)), tile + L * 512);
            }
        }
    };

    // ---- LDS -> registers ---------------------------------------------------
    // K operand: row kb*32 + lq, logical chunk 2cc + h.  The swizzle depends
    // on the row only through lq, so each lane keeps one byte offset per cc
    // and kb adds a constant.
    const int kswz = k_swz<D>(lq);
    int kro[NQC];
#pragma unroll
    for (int cc = 0; cc < NQC; ++cc) kro[cc] = (lq * D + (((2 * cc + h) ^ kswz) << 3)) * 2;
    // V^T operand via ds_read_b64_tr_b16: in each 16-lane group g, lane
    // s = a + 4 kk points at row 16 c4 + 8 r + 4 h + kk, dims
    // 32 db + 16 (g % 2) + 4 a .. +4; the transposing read then hands lane
    // 16 g + j the values of dim 32 db + 16 (g % 2) + j for those four rows,
    // which are the keys P^T holds at contraction positions 8 h + 4 r .. +4.
    // The swizzle bits depend on the row only through 4 h + kk, so each lane
    // keeps one byte offset per db and (c4, r) add constants.
    int vro[NDB];
    {
        const int g16 = lane >> 4, sl = lane & 15;
        const int vk = sl >> 2, va = sl & 3;
        const int vrow0 = 4 * h + vk;
        const int vchunk = 2 * (g16 & 1) + (va >> 1);
        const int vswz = v_swz<D>(vrow0);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
            vro[db] = (vrow0 * D + (((4 * db + vchunk) ^ vswz) << 3) + ((va & 1) << 2)) * 2;
    }
    // A operand of the j-th MFMA of the matrix phase: first the P V MFMAs
    // (db = j % NDB, c4 = j / NDB), then the Q K MFMAs (kb = i % NKB,
    // cc = i / NKB with i = j - NPV): consecutive MFMAs go to different
    // accumulators, since back-to-back dependent MFMAs issue at about two
    // thirds of the rate of independent ones when one wave has the SIMD's
    // matrix core to itself
    auto vread = [&](const char* vt8, int i) -> bf16x8_t {
        const int db = i % NDB, c4 = i / NDB;
        const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_p)(vt8 + vro[db] + 16 * c4 * D * 2));
        const s16x4_t hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_p)(vt8 + vro[db] + (16 * c4 + 8) * D * 2));
        return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    auto kread = [&](const char* kt8, int i) -> bf16x8_t {
        const int kb = i % NKB, cc = i / NKB;
        return *reinterpret_cast<const bf16x8_t*>(kt8 + kro[cc] + kb * 32 * D * 2);
    };

    f32x16_t sacc[NKB];
    constexpr int NPAIR = NKB * 8;  // pairs of S^T values per lane

    // l, the row sum of P, always sums the same bf16-rounded P that
    // multiplies V, so O = sum p v / sum p is a convex combination of the
    // values ("Online softmax" (roadmapper), The recurrence: one p feeds
    // both).  It is taken on the matrix core (below), so the vector units
    // spend no instruction on it; where depends on the head dimension:
    //  - D = 128: in the matrix phase, one v_mfma_f32_16x16x32_bf16 per
    //    16-key chunk accumulated into lacc across tiles, with P stored in
    //    place in the score accumulators (kPInPlace);
    //  - D = 64: at the start of the matrix phase, the four chunks' MFMAs
    //    into a fresh accumulator.  That tile sum is the check of the
    //    lagged reference (below) and is then added to l.  P goes to
    //    separate registers, since the check may need the scores again
    //    after P is taken.  (Taken at the end of the softmax phase instead,
    //    these MFMAs wait there for a matrix core that the other group
    //    keeps busy, and that phase ends the slot.)
    // (A vector sum, v_dot2c_f32_bf16 of each rounded pair with (1, 1), waits
    // for a busy matrix core and issues 16 more vector instructions per
    // tile.)
    constexpr bool kPInPlace = NW == 8;
    // In place, P^T chunk c4 (16 keys) sits in registers 4 (c4 % 2) .. +3 of
    // sacc[c4 / 2] and is made from registers 8 (c4 % 2) .. +7, which are
    // read before they are overwritten when the pairs go in order.  The
    // matrix phase reads every chunk of P before it starts the next tile's
    // scores in sacc.
    u32x4_t pprev[kPInPlace ? 1 : NC4];
    // P for one pair of S^T values: exponentials and rounding to bf16
    auto exp_pair = [&](int pp, float mu) {
        const int c4 = pp / 4, j = pp % 4;
        const int kb = c4 >> 1, hc = c4 & 1;
        const float p0 = exp2_hw(fmaf(sacc[kb][8 * hc + 2 * j], c, -mu));
        const float p1 = exp2_hw(fmaf(sacc[kb][8 * hc + 2 * j + 1], c, -mu));
        const bf16x2_t pv2 = {(__bf16)p0, (__bf16)p1};
        if constexpr (kPInPlace) sacc[kb][4 * hc + j] = __builtin_bit_cast(float, pv2);
        else pprev[c4][j] = __builtin_bit_cast(unsigned, pv2);
    };
    // P^T chunk c4 as the B operand of an MFMA
    auto pchunk = [&](int c4) -> bf16x8_t {
        if constexpr (kPInPlace) {
            const int kb = c4 >> 1, b = 4 * (c4 & 1);
            const f32x4_t w = {sacc[kb][b], sacc[kb][b + 1], sacc[kb][b + 2], sacc[kb][b + 3]};
            return __builtin_bit_cast(bf16x8_t, w);
        } else {
            return __builtin_bit_cast(bf16x8_t, pprev[c4]);
        }
    };

    // The sum on the matrix core: one
    // v_mfma_f32_16x16x32_bf16 per 16-key chunk takes the P^T operand as its
    // B operand (lane i: column i % 16, the 8 keys of k-block i / 16) against
    // a constant A of ones and zeros.  Lane i of the P^T operand holds query
    // i % 32 and key half i / 32, so k-block g belongs to query column
    // n + 16 (g % 2); result row r (held by lanes 16 (r / 4) + n) sums the
    // k-blocks with g % 2 == (r / 4) % 2, i.e. both key halves of exactly the
    // query that lane owns.  Every lane thus accumulates its query's full
    // sum of the same bf16-rounded P that multiplies V, and the vector units
    // spend no instruction on it.
    const bool lsel_on = ((lane >> 4) & 1) == ((lane >> 2) & 1);
    const short sel1 = lsel_on ? (short)0x3F80 : (short)0;  // bf16 1.0 or 0
    const bf16x8_t lsel = {sel1, sel1, sel1, sel1, sel1, sel1, sel1, sel1};
    f32x4_t lacc = {0.0f, 0.0f, 0.0f, 0.0f};  // D = 128: the row sum, accumulated in the matrix phase
    float l = 0.0f;                          // D = 64: the row sum, from the tile sums
    // D = 64: the row's sum of this tile's P (all four chunks)
    auto tile_sum = [&]() -> float {
        f32x4_t ts = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int c4 = 0; c4 < NC4; ++c4) ts = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lsel, pchunk(c4), ts, 0, 0, 0);
        return ts[0];
    };

    // ---- matrix phase M(t): O += V(t)^T P(t) (DO_PV), S(t+1) = K(t+1) Q^T
    // (DO_S).  MFMAs only, with their operands read from LDS through a ring of
    // R registers, R - 1 MFMAs ahead.
    constexpr int NPV = NDB * NC4, NS = NKB * NQC;
    auto mphase = [&](auto pv_c, auto s_c, const char* vt8, const char* kt8) {
        constexpr bool DO_PV = decltype(pv_c)::value, DO_S = decltype(s_c)::value;
        // the row sum of chunk c4 goes just before its first P V MFMA
        constexpr int N0 = DO_PV ? NPV : 0;
        constexpr int N = N0 + (DO_S ? NS : 0);
        // four waves per SIMD leave room for a ring of two only
        constexpr int R = NW == 8 ? 4 : 2;
        auto rd = [&](int j) -> bf16x8_t { return j < N0 ? vread(vt8, j) : kread(kt8, j - N0); };
        bf16x8_t op[R];
#pragma unroll
        for (int j = 0; j < R - 1; ++j)
            if (j < N) op[j] = rd(j);
#pragma unroll
        for (int j = 0; j < N; ++j) {
            if (j + R - 1 < N) op[(j + R - 1) % R] = rd(j + R - 1);
            if (j < N0) {
                if (kPInPlace && j % NDB == 0) {
                    lacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lsel, pchunk(j / NDB), lacc, 0, 0, 0);
                    __builtin_amdgcn_sched_barrier(0);
                }
                oacc[j % NDB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[j % R], pchunk(j / NDB), oacc[j % NDB], 0, 0, 0);
            } else {
                const int i = j - N0, kb = i % NKB, cc = i / NKB;
                if (cc == 0) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.0f;
                }
                sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[j % R], qop[cc], sacc[kb], 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // ---- softmax phase X(t) on S(t) (in sacc): vector work only ----------
    auto xphase = [&](int t) __attribute__((always_inline)) {
        const int key0 = kbase + t * BN;
        const bool mask = (key0 + BN > Sk) || (CAUSAL && key0 + BN - 1 > q0 + w * 32);
        if (mask) {
            // key = key0 + 4h + off with off = kb*32 + 8*(r/4) + r%4 a constant;
            // masked when key >= Sk or (causal) key > qrow
            int lim = Sk - key0 - 4 * h;
            if (CAUSAL) lim = min(lim, qrow + 1 - key0 - 4 * h);
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (kb * 32 + 8 * (r >> 2) + (r & 3) >= lim) sacc[kb][r] = kNegInf;
        }
        if constexpr (kPInPlace) {
            // the lane's tile maximum first (a chain of three-input maxima).
            // The reference stands while every score of the tile is within
            // 2^kLag of it, i.e. no P exceeds 2^kLag.
            float mx = kNegInf;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
            // no reference yet (m = -inf) with a visible key, a rise beyond
            // the lag, or a NaN: move the reference to the running maximum
            // (the same for both key halves of a query) and rescale O and l
            // by 2^(m_old - m_new), exactly 1 where the reference stays
            if (__builtin_amdgcn_ballot_w64(!(mx * c <= m + kLag))) {
                mx = fmaxf(mx, xor32(mx));
                const float ms = mx * c;
                const bool up = ms > m;                   // m = -inf: any finite score moves it
                const float mn = up ? ms : m;
                const float alpha = exp2_hw(m - guard_max(mn));
                m = mn;
#pragma unroll
                for (int r = 0; r < 4; ++r) lacc[r] *= alpha;
                if (__builtin_amdgcn_ballot_w64(up)) {
#pragma unroll
                    for (int db = 0; db < NDB; ++db)
#pragma unroll
                        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
                }
            }
            const float mu = guard_max(m);
#pragma unroll
            for (int pp = 0; pp < NPAIR; ++pp) exp_pair(pp, mu);
        } else {
            // P against the row's current reference, without the tile
            // maximum; the matrix phase checks it (check below)
            const float mu = guard_max(m);
#pragma unroll
            for (int pp = 0; pp < NPAIR; ++pp) exp_pair(pp, mu);
        }
    };
    // D = 64, at the start of the matrix phase M(t), before P(t) meets V:
    // the P of the softmax phase stands when the row's sum of it for the
    // tile is at most 2^kLag (so no single P exceeds it) and the row has a
    // reference
    auto check = [&]() __attribute__((always_inline)) {
        float rs = tile_sum();
        const bool redo = m == kNegInf || !(rs <= kMaxTileSum);
        if (__builtin_amdgcn_ballot_w64(redo)) {
            // slow path (the first tile of a row, a large rise, or a
            // NaN): the reference moves to the running maximum, O and l
            // follow it, and P is taken again against it
            float mx = kNegInf;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
            mx = fmaxf(mx, xor32(mx));
            const float ms = mx * c;
            const bool up = ms > m;                   // m = -inf: any finite score moves it
            const float mn = up ? ms : m;
            const float mu = guard_max(mn);
            const float alpha = exp2_hw(m - mu);      // exactly 1 where the reference stays
#pragma unroll
            for (int pp = 0; pp < NPAIR; ++pp) exp_pair(pp, mu);
            rs = tile_sum();
            l *= alpha;
            m = mn;
            if (__builtin_amdgcn_ballot_w64(up)) {
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
            }
        }
        l += rs;
    };

    // ---- prologue: K(0), V(0), K(1) into LDS; each wave's rows of Q, loaded
    // at the start, go through its staging region into the operand layout;
    // every wave computes its S(0) ------------------------------------------
    if (ntiles > 0) {
        dma(kp, sK[0], false, kbase);
        dma(vp, sV[0], true, kbase);
        if (ntiles > 1) dma(kp, sK[1], false, kbase + BN);
    }
    wait_vmem();
    {
        uint16_t* sq = sO[w];
#pragma unroll
        for (int j = 0; j < NQL; ++j) {
            const int ci = j * 64 + lane, r = ci / QCPR, u = ci % QCPR;
            *reinterpret_cast<u32x4_t*>(sq + r * ORS + 8 * u) = qld[j];
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's Q rows are in LDS
#pragma unroll
        for (int cc = 0; cc < NQC; ++cc)
            qop[cc] = *reinterpret_cast<const bf16x8_t*>(sq + lq * ORS + 8 * (2 * cc + h));
    }
    __syncthreads();
    if (ntiles > 0) mphase(std::false_type{}, std::true_type{}, nullptr, reinterpret_cast<const char*>(sK[0]));
    if (grp == 1) __syncthreads();  // group 1 runs one slot behind group 0

    // loads of V(t+1) and K(t+2), issued in slot 2t+1 into the buffers of
    // V(t-1) and K(t), whose last reader ran in slot 2t
    auto loads = [&](int t, auto par) {
        constexpr int P = decltype(par)::value;
        if (t + 1 < ntiles) dma(vp, sV[P ^ 1], true, kbase + (t + 1) * BN);
        if (t + 2 < ntiles) dma(kp, sK[P], false, kbase + (t + 2) * BN);
    };
    // X(t) then M(t) for one tile; P = t & 1 is a constant, so every LDS
    // address is a per-lane offset plus an immediate
    auto tile = [&](int t, auto par) {
        constexpr int P = decltype(par)::value;
        // X(t): slot 2t for group 0, 2t+1 for group 1
        if (grp == 1) loads(t, par);
        if (t <= tlast) xphase(t);
        if (grp == 0) wait_vmem();  // loads issued in slot 2t-1, read from slot 2t+1
        __syncthreads();
        // M(t): slot 2t+1 for group 0, 2t+2 for group 1
        if (grp == 0) loads(t, par);
        if (t <= tlast) {
            __builtin_amdgcn_s_setprio(1);  // this wave's MFMAs go ahead of its partner's vector work
            if constexpr (!kPInPlace) check();
            mphase(std::true_type{}, std::true_type{}, reinterpret_cast<const char*>(sV[P]),
                   reinterpret_cast<const char*>(sK[P ^ 1]));
            __builtin_amdgcn_s_setprio(0);
        }
        if (grp == 1) wait_vmem();  // loads issued in slot 2t+1, read from slot 2t+3
        __syncthreads();
    };
    for (int t = 0; t < ntiles; t += 2) {
        tile(t, std::integral_constant<int, 0>{});
        if (t + 1 < ntiles) tile(t + 1, std::integral_constant<int, 1>{});
    }
    // the rows' output: (m, l, unnormalised O) for merge_partials with KV
    // splits, else O / l and the log-sum-exp
    auto write_out = [&]() __attribute__((always_inline)) {
        const float lt = kPInPlace ? lacc[0] : l;  // the row sum
        if (nsplit > 1) {
            if (qrow >= Sq) return;
            // [row, split] with row = (b, h, query); m in natural units
            const int64_t pr = (bh * Sq + qrow) * nsplit + split;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int d = db * 32 + 8 * g + 4 * h;
                    *reinterpret_cast<f32x4v_t*>(pO + pr * D + d) =
                        f32x4v_t{oacc[db][4 * g], oacc[db][4 * g + 1], oacc[db][4 * g + 2], oacc[db][4 * g + 3]};
                }
            if (h == 0) {
                pm[pr] = lt > 0.0f ? m * kLn2 : kNegInf;
                pl[pr] = lt;
            }
            return;
        }
        const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
        if constexpr (OUT_BF16) {
            // the lane id again (mbcnt), so that nothing lane-derived from
            // before the loop is kept live across it for this
            const int ln = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
            const int lq2 = ln & 31, h2 = ln >> 5;
            uint16_t* so = sO[w];
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int d = db * 32 + 8 * g + 4 * h2;
                    const float y0 = oacc[db][4 * g] * inv, y1 = oacc[db][4 * g + 1] * inv;
                    const float y2 = oacc[db][4 * g + 2] * inv, y3 = oacc[db][4 * g + 3] * inv;
                    *reinterpret_cast<u32x2_t*>(so + lq2 * ORS + d) = u32x2_t{pack_bf16x2(y0, y1), pack_bf16x2(y2, y3)};
                }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's rows are in LDS
            constexpr int CPR = D / 8;  // 16-byte chunks per row
            // this wave's 32 rows are contiguous in O: a uniform base and a
            // 32-bit lane offset per chunk
            char* obase = reinterpret_cast<char*>(static_cast<uint16_t*>(o) + (bh * Sq + q0 + w * 32) * (int64_t)D);
            const int nrow = Sq - q0 - w * 32;  // rows of this wave inside the sequence
#pragma unroll
            for (int j = 0; j < 32 * CPR / 64; ++j) {
                const int ci = j * 64 + ln, r = ci / CPR, u = ci % CPR;
                const u32x4_t val = *reinterpret_cast<const u32x4_t*>(so + r * ORS + 8 * u);
                if (r < nrow) *reinterpret_cast<u32x4_t*>(obase + (unsigned)(r * D + 8 * u) * 2u) = val;
            }
        } else {
            if (qrow < Sq) {
                const int64_t orow = (bh * Sq + qrow) * (int64_t)D;
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int d = db * 32 + 8 * g + 4 * h;
                        const float y0 = oacc[db][4 * g] * inv, y1 = oacc[db][4 * g + 1] * inv;
                        const float y2 = oacc[db][4 * g + 2] * inv, y3 = oacc[db][4 * g + 3] * inv;
                        *reinterpret_cast<f32x4v_t*>(static_cast<float*>(o) + orow + d) = f32x4v_t{y0, y1, y2, y3};
                    }
            }
        }
        if (lse && h == 0 && qrow < Sq) lse[bh * Sq + qrow] = lt > 0.0f ? m * kLn2 + __logf(lt) : kNegInf;
    };
    // ---- epilogue.  Group 0 ran its last matrix phase one slot before group
    // 1, so it writes its rows first, its stores overlapping group 1's last
    // matrix phase, and then meets group 1 at the barrier of that extra slot.
    // After the loop only each wave's own staging region is touched in LDS.
    write_out();
    if (grp == 0) __syncthreads();
}

template <int D, int BN, int NW>
hipError_t launch_d(const AttnArgs& a, int nsplit, float* pm, float* pl, float* pO)
{
    constexpr int BM = 32 * NW;
    const int nqb = (a.Sq + BM - 1) / BM;
    const int64_t grid = (int64_t)nqb * a.H * a.B * nsplit;
    const float c = a.scale * kLog2eHi;
    if (a.out_bf16)
        hipLaunchKernelGGL((attn_fwd_kernel<D, BN, NW, true>), dim3((unsigned)grid), dim3(64 * NW), 0, a.stream,
                           (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, a.o, a.lse, a.Sq, a.Sk, c,
                           nqb, a.causal ? 1 : 0, nsplit, pm, pl, pO);
    else
        hipLaunchKernelGGL((attn_fwd_kernel<D, BN, NW, false>), dim3((unsigned)grid), dim3(64 * NW), 0, a.stream,
                           (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, a.o, a.lse, a.Sq, a.Sk, c,
                           nqb, a.causal ? 1 : 0, nsplit, pm, pl, pO);
    return hipGetLastError();
}

hipError_t launch_any(const AttnArgs& a, int nsplit, float* pm, float* pl, float* pO)
{
    if (a.D == 128) return launch_d<128, 64, 8>(a, nsplit, pm, pl, pO);
    return launch_d<64, 64, 16>(a, nsplit, pm, pl, pO);
}

}  // namespace

hipError_t launch_attn_fwd(const AttnArgs& a)
{
    if ((int64_t)a.B * a.H * a.Sq == 0) return hipSuccess;
    return launch_any(a, 1, nullptr, nullptr, nullptr);
}

size_t attn_splitk_workspace_bytes(int B, int H, int Sq, int D, int nsplit)
{
    const size_t n = (size_t)B * H * Sq * nsplit;
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    return 2 * up(n * sizeof(float)) + up(n * D * sizeof(float));
}

hipError_t launch_attn_fwd_splitk(const AttnArgs& a, int nsplit, void* workspace)
{
    if ((int64_t)a.B * a.H * a.Sq == 0) return hipSuccess;
    if (nsplit == 1) return launch_any(a, 1, nullptr, nullptr, nullptr);  // one range: the plain kernel
    const size_t n = (size_t)a.B * a.H * a.Sq * nsplit;
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    char* ws = static_cast<char*>(workspace);
    float* pm = reinterpret_cast<float*>(ws);
    float* pl = reinterpret_cast<float*>(ws + up(n * 4));
    float* pO = reinterpret_cast<float*>(ws + 2 * up(n * 4));
    hipError_t e = launch_any(a, nsplit, pm, pl, pO);
    if (e != hipSuccess) return e;
    MergeArgs m{pm, pl, pO, (int64_t)a.B * a.H * a.Sq, nsplit, a.D, nullptr, nullptr, a.o, a.out_bf16, true,
                a.stream};
    m.lse_out = a.lse;
    return launch_merge(m);
}

}  // namespace tea
