/*
 * tea.h -- C ABI of libtea.so: the one-pass online softmax on MI355X (gfx950),
 * as a row softmax, a tiled attention forward and a split-KV decode, plus the
 * associative merge of partial softmax states.
 *
 * The method ("Online softmax" (roadmapper-2x4.pages.dev), The recurrence;
 * "The Online Softmax" (llm.curionode.com, Vol. XVI plate 3), intro and One
 * pass, exactly; "Online Softmax" (metalworking.vercel.app), The problem):
 * keep a running maximum m and normaliser l = sum exp(x - m) per row, fold
 * the row in block by block, and whenever the maximum rises multiply the
 * accumulated l (and output O) by exp(m_old - m_new).  The result equals the
 * two-pass safe softmax in exact arithmetic and up to rounding in floating
 * point.
 *
 * Conventions for every entry point:
 *   - Pointers named as tensors are DEVICE pointers owned by the caller;
 *     tensors are row-major and contiguous.  The library never allocates,
 *     keeps no pointer after returning and has no mutable global state
 *     other than the device scratch of attn_decode_splitkv_noalloc.
 *   - `stream` is a hipStream_t (NULL: the default stream).  Every call is
 *     asynchronous on it; results are visible after the stream synchronises.
 *   - Arguments are validated before any HIP call; a failed validation
 *     returns its status and touches nothing.  TEA_EHIP reports a launch
 *     error from the HIP runtime; faults during execution surface at the
 *     caller's synchronisation.  Nothing is printed; nothing aborts.
 *   - Maxima, m_out and lse outputs are in natural-log units of the (scaled)
 *     logits; base two is used only inside the kernels.
 *   - The empty set (no logit, or all -inf) has state (m, l, O) =
 *     (-inf, 0, 0) and output 0, never NaN.
 *   - bf16 values are IEEE binary32 truncated to 16 bits (as torch.bfloat16);
 *     bf16 outputs are rounded to nearest even.
 */
#ifndef TEA_H
#define TEA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum tea_status {
    TEA_OK = 0,
    TEA_EINVAL = 1,       /* bad argument: null pointer, negative size, bad dtype, misalignment, ... */
    TEA_EUNSUPPORTED = 2, /* valid but not implemented: head_dim, row length, block size */
    TEA_EHIP = 3,         /* the HIP runtime reported an error at launch */
    TEA_ENOSPACE = 4      /* attn_decode_splitkv_noalloc: the partials would not fit its scratch */
};

enum tea_dtype { TEA_F32 = 0, TEA_BF16 = 1 };

/*
 * row_softmax -- y[r, :] = softmax(x[r, :]) for every row r, reading each row
 * from HBM once and writing it once ("The Online Softmax" (curionode): n
 * logits processed in blocks of a chosen size, maximum and normaliser found
 * in one pass).
 *   x, y    [rows, cols] of `dtype` (TEA_F32 or TEA_BF16; y has x's dtype).
 *           y == x (in place) is allowed; partial overlap is not.
 *           4-byte (f32) or 2-byte (bf16) aligned; rows whose start is
 *           16-byte aligned take 128-bit loads.
 *   rows    >= 0 (0: nothing to do).
 *   cols    >= 0 (0: every row is the empty set).  Rows of up to 16384 logits
 *           are read once and written once; longer rows are streamed twice
 *           (maximum and normaliser in one read, the output in the second),
 *           one workgroup per row (the original setting of the online
 *           normaliser, "The Online Softmax" (curionode), intro).
 *   block   logits folded per online step in each lane: 1, 2, 4, 8, 16, 32,
 *           or 0 for the default 8; values above a lane's share act as one
 *           block per lane; other values: TEA_EUNSUPPORTED.  The result does
 *           not depend on it beyond rounding.
 *   m_out   nullable [rows] f32: row maximum (-inf for an empty row).
 *   l_out   nullable [rows] f32: sum over the row of exp(x - m_out).
 *           m_out and l_out may overlap neither x, y nor each other
 *           (TEA_EINVAL).
 * Returns TEA_OK, TEA_EINVAL, TEA_EUNSUPPORTED or TEA_EHIP.
 */
int row_softmax(const void* x, void* y, int64_t rows, int64_t cols, int dtype, int block, float* m_out,
                float* l_out, void* stream);

/* Rescale policies of row_softmax_variant (see there). */
enum tea_rescale { TEA_RESCALE_ALWAYS = 0, TEA_RESCALE_IF_RISE = 1, TEA_RESCALE_L0_ONE = 2 };

/*
 * row_softmax_variant -- row_softmax with a choice of how each lane's running
 * normaliser is put on a new scale when a block is folded in.  The pages set
 * two good kernels against each other here ("Online Softmax"
 * (metalworking), Recognition guide: metal-flash-attention multiplies by the
 * correction exp(m - m') only when the maximum rose, MLX multiplies every
 * time), and note that the attention tutorial starts the normaliser at 1
 * instead of 0 ("Online softmax" (roadmapper), Initialise honestly).
 *   rescale  TEA_RESCALE_ALWAYS: multiply every block (what row_softmax does);
 *            TEA_RESCALE_IF_RISE: compute the correction and multiply only
 *              when the maximum rose (a wave skips the work when no lane's
 *              maximum rose);
 *            TEA_RESCALE_L0_ONE: start each lane's normaliser at 1, removed
 *              by the zero correction of its first non-empty block;
 *            anything else: TEA_EINVAL.
 * All three return the same bits in y, m_out and l_out (the correction is
 * exactly 1 when the maximum stays, and exactly 0 against the -inf start).
 * Other arguments, limits and errors as for row_softmax.
 */
int row_softmax_variant(const void* x, void* y, int64_t rows, int64_t cols, int dtype, int block, int rescale,
                        float* m_out, float* l_out, void* stream);

/*
 * attn_fwd -- O = softmax(Q K^T * scale) V per (batch, head), streaming K and
 * V in tiles with the online softmax so no row of scores is stored ("The
 * Online Softmax" (curionode), One pass, exactly; "Online Softmax"
 * (metalworking), The problem: O = O c + P V per tile, O /= l at the end).
 *   q       [B, H, Sq, D] bf16;  k, v [B, H, Sk, D] bf16; 16-byte aligned.
 *   o       [B, H, Sq, D] of out_dtype (TEA_BF16 or TEA_F32); must not
 *           overlap q, k or v.
 *   B, H, Sq >= 0 (any zero: nothing to do);  Sk >= 0 (0: O = 0).
 *   D       64 or 128 (else TEA_EUNSUPPORTED).
 *   scale   finite and > 0 (else TEA_EINVAL).
 *   causal  0: every key visible; 1: key j visible to query i iff j <= i,
 *           which requires Sq == Sk (else TEA_EUNSUPPORTED).
 *   lse_out nullable [B, H, Sq] f32: m + ln(l) of the scaled scores
 *           (-inf for a query with no visible key); must not overlap q, k,
 *           v or o.
 * Returns TEA_OK, TEA_EINVAL, TEA_EUNSUPPORTED or TEA_EHIP.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, int B, int H, int Sq, int Sk, int D,
             float scale, int causal, int out_dtype, float* lse_out, void* stream);

/*
 * attn_fwd_splitk_workspace_bytes -- bytes of workspace attn_fwd_splitk needs
 * for these sizes (0 for invalid sizes).
 */
size_t attn_fwd_splitk_workspace_bytes(int B, int H, int Sq, int D, int num_splits);

/*
 * attn_fwd_splitk -- attn_fwd with each query block's KV tiles split into
 * num_splits contiguous ranges, one workgroup each, for shapes with too few
 * query blocks to fill the GPU.  Each range yields a partial state (m, l, O)
 * per query, and the partials are merged by the associative combine, as
 * merge_partials does ("The Online Softmax" (curionode), One pass, exactly:
 * partial results merge in any order or tree, or across devices).
 *   Arguments as for attn_fwd, plus
 *   num_splits 1 .. 64 (else TEA_EINVAL); tile ranges may be empty (their
 *            partial is the empty state).  The grid has B * H * query
 *            blocks * num_splits workgroups (query blocks of 256 rows at
 *            D = 128, 512 at D = 64), one resident per CU; the fastest
 *            count measured is the one that fills the 256 CUs once;
 *   workspace device memory of at least attn_fwd_splitk_workspace_bytes(),
 *            16-byte aligned, owned by the caller, overlapping no other
 *            argument; concurrent calls need separate workspaces.
 * The result equals attn_fwd's up to rounding.
 * Returns TEA_OK, TEA_EINVAL, TEA_EUNSUPPORTED or TEA_EHIP.
 */
int attn_fwd_splitk(const void* q, const void* k, const void* v, void* o, int B, int H, int Sq, int Sk, int D,
                    float scale, int causal, int num_splits, int out_dtype, float* lse_out, void* workspace,
                    size_t workspace_bytes, void* stream);

/*
 * attn_decode_workspace_bytes -- bytes of workspace attn_decode_splitkv needs
 * for these sizes (0 for invalid sizes).
 */
size_t attn_decode_workspace_bytes(int B, int H, int D, int num_splits);

/*
 * attn_decode_splitkv -- one query token per (batch, head) against a KV cache
 * of per-sequence length kv_len[b], split into num_splits contiguous chunks;
 * each chunk yields a partial state (m, l, O) and the partials are merged by
 * the associative combine in a tree, with no atomics ("The Online Softmax"
 * (curionode), One pass, exactly; "Online Softmax" (metalworking),
 * Recognition guide).  Chunk c of a sequence of L keys is
 * [floor(c L / S), floor((c + 1) L / S)), empty when L < S.
 *   q        [B, H, 1, D] bf16;  k, v [B, H, Lmax, D] bf16; 16-byte aligned.
 *            Positions >= kv_len[b] are never read.
 *   kv_len   [B] int32 device array; values are clamped to [0, Lmax]; a
 *            sequence of length 0 gives O = 0.
 *   o        [B, H, D] of out_dtype (TEA_BF16 or TEA_F32); must not overlap
 *            q, k, v, kv_len or the workspace.
 *   B, H >= 0 (zero: nothing to do); Lmax >= 1; D: 64 or 128 (else
 *            TEA_EUNSUPPORTED); num_splits 1 .. 1024; scale finite, > 0.
 *   workspace device memory of at least attn_decode_workspace_bytes(),
 *            16-byte aligned, owned by the caller, not read before written,
 *            overlapping no input; concurrent calls need separate
 *            workspaces.
 * Returns TEA_OK, TEA_EINVAL, TEA_EUNSUPPORTED or TEA_EHIP.
 */
int attn_decode_splitkv(const void* q, const void* k, const void* v, const int32_t* kv_len, void* o, int B,
                        int H, int Lmax, int D, int num_splits, float scale, int out_dtype, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * attn_decode_splitkv_noalloc -- attn_decode_splitkv for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the caller passes inputs and output only,
 * and the partial states go to a scratch array that the library holds in
 * device memory, TEA_DECODE_NOALLOC_MAX_BYTES bytes on every GPU it runs on,
 * kept until the process ends.  Same kernels, chunks and merge tree as
 * attn_decode_splitkv, so the same bits.
 *   Arguments as for attn_decode_splitkv, without the workspace.
 *   The partials need attn_decode_workspace_bytes(B, H, D, num_splits)
 *   bytes; above TEA_DECODE_NOALLOC_MAX_BYTES the call returns TEA_ENOSPACE
 *   (B16 H32 D128 with 64 splits needs 17 MB).
 *   Allocates nothing: no hipMalloc, hipFree or allocating library call.
 *   The scratch's device address is looked up on the first call on each
 *   device (with that device current) and cached.  Every call on a GPU shares
 *   that GPU's scratch, which keeps the last call's partials; each call
 *   writes every partial before reading it, so nothing needs clearing, but
 *   calls that overlap on one GPU (concurrent streams or threads) race.
 * Returns TEA_OK, TEA_EINVAL, TEA_EUNSUPPORTED, TEA_ENOSPACE or TEA_EHIP.
 */
#define TEA_DECODE_NOALLOC_MAX_BYTES ((size_t)32 << 20)
int attn_decode_splitkv_noalloc(const void* q, const void* k, const void* v, const int32_t* kv_len, void* o, int B,
                                int H, int Lmax, int D, int num_splits, float scale, int out_dtype, void* stream);

/*
 * attn_decode_fused -- the same decode in one launch and with no workspace:
 * one workgroup of 16 waves per (batch, head); the num_splits chunks are the
 * leaves of a balanced binary tree of 64 leaves (those at or past num_splits
 * are empty), each wave computes four of them and combines them, and the
 * waves' states are combined through LDS ("Online Softmax" (metalworking),
 * Recognition guide: the Apple decode kernels merge partial results from
 * different simdgroups).  Same chunk bounds, tree and combine as
 * attn_decode_splitkv; the two agree up to rounding.  All of a (batch,
 * head) runs on one compute unit, so this form fills the GPU only with at
 * least as many (batch, head) pairs as it has compute units (256 on
 * MI355X); below that, attn_decode_splitkv is the faster form.
 *   Arguments as for attn_decode_splitkv, without the workspace (o must
 *   not overlap q, k, v or kv_len); num_splits 1 .. 64 (else TEA_EINVAL).
 * Returns TEA_OK, TEA_EINVAL, TEA_EUNSUPPORTED or TEA_EHIP.
 */
int attn_decode_fused(const void* q, const void* k, const void* v, const int32_t* kv_len, void* o, int B, int H,
                      int Lmax, int D, int num_splits, float scale, int out_dtype, void* stream);

/*
 * merge_partials -- merge S partial softmax states per row into one, by a
 * balanced pairwise tree over the partial index (for S <= 64; for larger S,
 * contiguous groups of ceil(S/64) are folded in order first), with no atomics
 * ("The Online Softmax" (curionode), One pass, exactly: the pairwise
 * rescaling identity is associative, so partials merge in any order or tree).
 *   m, l     [N, S] f32: maxima (natural units; -inf marks an empty partial)
 *            and normalisers (l = sum exp(x - m) of that partial, >= 0).
 *   O        [N, S, D] f32: unnormalised outputs sum exp(x - m) v.
 *   N >= 0 (0: nothing to do); S 1 .. 65536; D 1 .. 4096.
 *   m_out, l_out nullable [N] f32: merged maximum and normaliser; they
 *            overlap no input, O_out or each other.
 *   O_out    [N, D] of out_dtype: O / l when normalize = 1 (0 where l = 0),
 *            or the merged unnormalised O when normalize = 0 (TEA_F32 only).
 * Returns TEA_OK, TEA_EINVAL or TEA_EHIP.
 */
int merge_partials(const float* m, const float* l, const float* O, int64_t N, int S, int D, float* m_out,
                   float* l_out, void* O_out, int out_dtype, int normalize, void* stream);

/* Human-readable name of a status code (static string). */
const char* tea_status_string(int status);

/* Version of this ABI (incremented on incompatible change). */
int tea_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TEA_H */
