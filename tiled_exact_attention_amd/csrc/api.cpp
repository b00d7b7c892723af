// C ABI of libtea.so: argument validation (before any HIP call) and dispatch
// to the kernels.  See include/tea.h for the contract of each entry point.
#include "tea.h"

#include <math.h>

#include "launch.hpp"

static_assert(TEA_DECODE_NOALLOC_MAX_BYTES == tea::kDecodeScratchBytes,
              "the scratch limit stated in tea.h is the size of the device array");

namespace {

inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// [a, a + na) and [b, b + nb) overlap (bytes)
inline bool overlap(const void* a, size_t na, const void* b, size_t nb)
{
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

inline int status_of(hipError_t e) { return e == hipSuccess ? TEA_OK : TEA_EHIP; }

inline bool good_scale(float s) { return isfinite(s) && s > 0.0f; }

// a decode output region [p, p + nb) overlaps one of the decode's inputs: q
// [B, H, D] bf16, k and v [B, H, Lmax, D] bf16, kv_len [B] int32
inline bool decode_outputs_overlap_inputs(const void* q, const void* k, const void* v, const int32_t* kv_len,
                                          int B, int H, int Lmax, int D, const void* p, size_t nb)
{
    const size_t qb = (size_t)B * H * D * 2, kb = (size_t)B * H * Lmax * D * 2, lb = (size_t)B * 4;
    return overlap(p, nb, q, qb) || overlap(p, nb, k, kb) || overlap(p, nb, v, kb) || overlap(p, nb, kv_len, lb);
}

}  // namespace

extern "C" {

int tea_abi_version(void) { return 1; }

const char* tea_status_string(int status)
{
    switch (status) {
    case TEA_OK: return "ok";
    case TEA_EINVAL: return "invalid argument";
    case TEA_EUNSUPPORTED: return "unsupported configuration";
    case TEA_EHIP: return "HIP runtime error";
    case TEA_ENOSPACE: return "request exceeds the scratch memory of the allocation-free entry point";
    default: return "unknown status";
    }
}

int row_softmax_variant(const void* x, void* y, int64_t rows, int64_t cols, int dtype, int block, int rescale,
                        float* m_out, float* l_out, void* stream)
{
    if (rescale != TEA_RESCALE_ALWAYS && rescale != TEA_RESCALE_IF_RISE && rescale != TEA_RESCALE_L0_ONE)
        return TEA_EINVAL;
    if (rows < 0 || cols < 0) return TEA_EINVAL;
    if (dtype != TEA_F32 && dtype != TEA_BF16) return TEA_EINVAL;
    if (block < 0) return TEA_EINVAL;
    if (block == 0) block = 8;
    if (block > 32) block = 32;
    if (block & (block - 1)) return TEA_EUNSUPPORTED;
    if (rows == 0) return TEA_OK;
    if (cols > tea::row_softmax_max_cols()) return TEA_EUNSUPPORTED;
    if (rows > (int64_t)0x7fffffff) return TEA_EUNSUPPORTED;  // grid limit (one row per workgroup at most)
    const size_t es = dtype == TEA_F32 ? 4 : 2;
    if (cols > 0) {
        if (!x || !y) return TEA_EINVAL;
        if (!aligned(x, es) || !aligned(y, es)) return TEA_EINVAL;
        const size_t bytes = (size_t)rows * (size_t)cols * es;
        if (x != y && overlap(x, bytes, y, bytes)) return TEA_EINVAL;
    }
    if ((m_out && !aligned(m_out, 4)) || (l_out && !aligned(l_out, 4))) return TEA_EINVAL;
    // the row statistics are outputs of their own: they may overlap neither
    // each other nor the logits or the softmax
    const size_t sb = (size_t)rows * 4, xb = (size_t)rows * (size_t)cols * es;
    if (m_out && l_out && overlap(m_out, sb, l_out, sb)) return TEA_EINVAL;
    for (const float* st : {m_out, l_out})
        if (st && cols > 0 && (overlap(st, sb, x, xb) || overlap(st, sb, y, xb))) return TEA_EINVAL;
    tea::RowSoftmaxArgs a{x, y, rows, cols, dtype == TEA_BF16, block, m_out, l_out, (hipStream_t)stream};
    a.rescale = rescale == TEA_RESCALE_IF_RISE ? tea::kRescaleIfRise
                : rescale == TEA_RESCALE_L0_ONE ? tea::kRescaleL0One
                                                : tea::kRescaleAlways;
    return status_of(tea::launch_row_softmax(a));
}

int row_softmax(const void* x, void* y, int64_t rows, int64_t cols, int dtype, int block, float* m_out,
                float* l_out, void* stream)
{
    return row_softmax_variant(x, y, rows, cols, dtype, block, TEA_RESCALE_ALWAYS, m_out, l_out, stream);
}

int attn_fwd(const void* q, const void* k, const void* v, void* o, int B, int H, int Sq, int Sk, int D,
             float scale, int causal, int out_dtype, float* lse_out, void* stream)
{
    if (B < 0 || H < 0 || Sq < 0 || Sk < 0 || D <= 0) return TEA_EINVAL;
    if (out_dtype != TEA_F32 && out_dtype != TEA_BF16) return TEA_EINVAL;
    if (causal != 0 && causal != 1) return TEA_EINVAL;
    if (!good_scale(scale)) return TEA_EINVAL;
    if (D != 64 && D != 128) return TEA_EUNSUPPORTED;
    if (causal && Sq != Sk) return TEA_EUNSUPPORTED;
    if ((int64_t)B * H * Sq == 0) return TEA_OK;
    if ((int64_t)B * H * ((Sq + 255) / 256) > (int64_t)0x7fffffff) return TEA_EUNSUPPORTED;
    if (!q || !o || (Sk > 0 && (!k || !v))) return TEA_EINVAL;
    if (!aligned(q, 16) || !aligned(o, 16) || !aligned(k, 16) || !aligned(v, 16)) return TEA_EINVAL;
    if (lse_out && !aligned(lse_out, 4)) return TEA_EINVAL;
    const size_t qb = (size_t)B * H * Sq * D * 2, kb = (size_t)B * H * Sk * D * 2;
    const size_t ob = (size_t)B * H * Sq * D * (out_dtype == TEA_F32 ? 4 : 2);
    if (overlap(o, ob, q, qb) || (Sk > 0 && (overlap(o, ob, k, kb) || overlap(o, ob, v, kb)))) return TEA_EINVAL;
    if (lse_out) {
        const size_t lb = (size_t)B * H * Sq * 4;
        if (overlap(lse_out, lb, o, ob) || overlap(lse_out, lb, q, qb) ||
            (Sk > 0 && (overlap(lse_out, lb, k, kb) || overlap(lse_out, lb, v, kb))))
            return TEA_EINVAL;
    }
    tea::AttnArgs a{q, k, v, o, B, H, Sq, Sk, D, scale, causal == 1, out_dtype == TEA_BF16, lse_out,
                    (hipStream_t)stream};
    return status_of(tea::launch_attn_fwd(a));
}

size_t attn_fwd_splitk_workspace_bytes(int B, int H, int Sq, int D, int num_splits)
{
    if (B < 0 || H < 0 || Sq < 0 || D <= 0 || num_splits < 1 || num_splits > 64) return 0;
    return tea::attn_splitk_workspace_bytes(B, H, Sq, D, num_splits);
}

int attn_fwd_splitk(const void* q, const void* k, const void* v, void* o, int B, int H, int Sq, int Sk, int D,
                    float scale, int causal, int num_splits, int out_dtype, float* lse_out, void* workspace,
                    size_t workspace_bytes, void* stream)
{
    if (B < 0 || H < 0 || Sq < 0 || Sk < 0 || D <= 0) return TEA_EINVAL;
    if (num_splits < 1 || num_splits > 64) return TEA_EINVAL;
    if (out_dtype != TEA_F32 && out_dtype != TEA_BF16) return TEA_EINVAL;
    if (causal != 0 && causal != 1) return TEA_EINVAL;
    if (!good_scale(scale)) return TEA_EINVAL;
    if (D != 64 && D != 128) return TEA_EUNSUPPORTED;
    if (causal && Sq != Sk) return TEA_EUNSUPPORTED;
    if ((int64_t)B * H * Sq == 0) return TEA_OK;
    if ((int64_t)B * H * ((Sq + 255) / 256) * num_splits > (int64_t)0x7fffffff) return TEA_EUNSUPPORTED;
    if (!q || !o || !workspace || (Sk > 0 && (!k || !v))) return TEA_EINVAL;
    if (!aligned(q, 16) || !aligned(o, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(workspace, 16))
        return TEA_EINVAL;
    if (lse_out && !aligned(lse_out, 4)) return TEA_EINVAL;
    const size_t need = tea::attn_splitk_workspace_bytes(B, H, Sq, D, num_splits);
    if (workspace_bytes < need) return TEA_EINVAL;
    const size_t qb = (size_t)B * H * Sq * D * 2, kb = (size_t)B * H * Sk * D * 2;
    const size_t ob = (size_t)B * H * Sq * D * (out_dtype == TEA_F32 ? 4 : 2);
    if (overlap(o, ob, q, qb) || (Sk > 0 && (overlap(o, ob, k, kb) || overlap(o, ob, v, kb)))) return TEA_EINVAL;
    if (overlap(workspace, need, o, ob) || overlap(workspace, need, q, qb) ||
        (Sk > 0 && (overlap(workspace, need, k, kb) || overlap(workspace, need, v, kb))))
        return TEA_EINVAL;
    if (lse_out) {
        const size_t lb = (size_t)B * H * Sq * 4;
        if (overlap(lse_out, lb, o, ob) || overlap(lse_out, lb, workspace, need) || overlap(lse_out, lb, q, qb) ||
            (Sk > 0 && (overlap(lse_out, lb, k, kb) || overlap(lse_out, lb, v, kb))))
            return TEA_EINVAL;
    }
    tea::AttnArgs a{q, k, v, o, B, H, Sq, Sk, D, scale, causal == 1, out_dtype == TEA_BF16, lse_out,
                    (hipStream_t)stream};
    return status_of(tea::launch_attn_fwd_splitk(a, num_splits, workspace));
}

size_t attn_decode_workspace_bytes(int B, int H, int D, int num_splits)
{
    if (B < 0 || H < 0 || D <= 0 || num_splits < 1 || num_splits > 1024) return 0;
    return tea::decode_workspace_bytes(B, H, D, num_splits);
}

int attn_decode_splitkv(const void* q, const void* k, const void* v, const int32_t* kv_len, void* o, int B,
                        int H, int Lmax, int D, int num_splits, float scale, int out_dtype, void* workspace,
                        size_t workspace_bytes, void* stream)
{
    if (B < 0 || H < 0 || Lmax < 1 || D <= 0) return TEA_EINVAL;
    if (num_splits < 1 || num_splits > 1024) return TEA_EINVAL;
    if (out_dtype != TEA_F32 && out_dtype != TEA_BF16) return TEA_EINVAL;
    if (!good_scale(scale)) return TEA_EINVAL;
    if (D != 64 && D != 128) return TEA_EUNSUPPORTED;
    if ((int64_t)B * H == 0) return TEA_OK;
    if ((int64_t)B * H * num_splits > (int64_t)0x7fffffff) return TEA_EUNSUPPORTED;
    if (!q || !k || !v || !kv_len || !o || !workspace) return TEA_EINVAL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(kv_len, 4) || !aligned(o, 4) ||
        !aligned(workspace, 16))
        return TEA_EINVAL;
    const size_t need = tea::decode_workspace_bytes(B, H, D, num_splits);
    if (workspace_bytes < need) return TEA_EINVAL;
    // the output and the workspace are written: neither may overlap an
    // input or the other
    const size_t ob = (size_t)B * H * D * (out_dtype == TEA_F32 ? 4 : 2);
    if (decode_outputs_overlap_inputs(q, k, v, kv_len, B, H, Lmax, D, o, ob)) return TEA_EINVAL;
    if (decode_outputs_overlap_inputs(q, k, v, kv_len, B, H, Lmax, D, workspace, need)) return TEA_EINVAL;
    if (overlap(workspace, need, o, ob)) return TEA_EINVAL;
    tea::DecodeArgs a{q, k, v, kv_len, o, B, H, Lmax, D, num_splits, scale, out_dtype == TEA_BF16, nullptr, nullptr,
                      nullptr, (hipStream_t)stream};
    tea::decode_bind_workspace(a, workspace);
    return status_of(tea::launch_decode(a));
}

int attn_decode_splitkv_noalloc(const void* q, const void* k, const void* v, const int32_t* kv_len, void* o, int B,
                                int H, int Lmax, int D, int num_splits, float scale, int out_dtype, void* stream)
{
    if (B < 0 || H < 0 || Lmax < 1 || D <= 0) return TEA_EINVAL;
    if (num_splits < 1 || num_splits > 1024) return TEA_EINVAL;
    if (out_dtype != TEA_F32 && out_dtype != TEA_BF16) return TEA_EINVAL;
    if (!good_scale(scale)) return TEA_EINVAL;
    if (D != 64 && D != 128) return TEA_EUNSUPPORTED;
    if ((int64_t)B * H == 0) return TEA_OK;
    if ((int64_t)B * H * num_splits > (int64_t)0x7fffffff) return TEA_EUNSUPPORTED;
    if (tea::decode_workspace_bytes(B, H, D, num_splits) > tea::kDecodeScratchBytes) return TEA_ENOSPACE;
    if (!q || !k || !v || !kv_len || !o) return TEA_EINVAL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(kv_len, 4) || !aligned(o, 4))
        return TEA_EINVAL;
    if (decode_outputs_overlap_inputs(q, k, v, kv_len, B, H, Lmax, D, o,
                                      (size_t)B * H * D * (out_dtype == TEA_F32 ? 4 : 2)))
        return TEA_EINVAL;
    tea::DecodeArgs a{q, k, v, kv_len, o, B, H, Lmax, D, num_splits, scale, out_dtype == TEA_BF16, nullptr, nullptr,
                      nullptr, (hipStream_t)stream};
    return status_of(tea::launch_decode_noalloc(a));
}

int attn_decode_fused(const void* q, const void* k, const void* v, const int32_t* kv_len, void* o, int B, int H,
                      int Lmax, int D, int num_splits, float scale, int out_dtype, void* stream)
{
    if (B < 0 || H < 0 || Lmax < 1 || D <= 0) return TEA_EINVAL;
    if (num_splits < 1 || num_splits > tea::decode_fused_max_splits()) return TEA_EINVAL;
    if (out_dtype != TEA_F32 && out_dtype != TEA_BF16) return TEA_EINVAL;
    if (!good_scale(scale)) return TEA_EINVAL;
    if (D != 64 && D != 128) return TEA_EUNSUPPORTED;
    if ((int64_t)B * H == 0) return TEA_OK;
    if ((int64_t)B * H > (int64_t)0x7fffffff) return TEA_EUNSUPPORTED;
    if (!q || !k || !v || !kv_len || !o) return TEA_EINVAL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(kv_len, 4) || !aligned(o, 4))
        return TEA_EINVAL;
    if (decode_outputs_overlap_inputs(q, k, v, kv_len, B, H, Lmax, D, o,
                                      (size_t)B * H * D * (out_dtype == TEA_F32 ? 4 : 2)))
        return TEA_EINVAL;
    tea::DecodeArgs a{q, k, v, kv_len, o, B, H, Lmax, D, num_splits, scale, out_dtype == TEA_BF16, nullptr, nullptr,
                      nullptr, (hipStream_t)stream};
    return status_of(tea::launch_decode_fused(a));
}

int merge_partials(const float* m, const float* l, const float* O, int64_t N, int S, int D, float* m_out,
                   float* l_out, void* O_out, int out_dtype, int normalize, void* stream)
{
    if (N < 0 || S < 1 || S > 65536 || D < 1 || D > 4096) return TEA_EINVAL;
    if (out_dtype != TEA_F32 && out_dtype != TEA_BF16) return TEA_EINVAL;
    if (normalize != 0 && normalize != 1) return TEA_EINVAL;
    if (!normalize && out_dtype != TEA_F32) return TEA_EINVAL;
    if (N == 0) return TEA_OK;
    if (N * ((D + 7) / 8) > (int64_t)0x7fffffff * 4) return TEA_EUNSUPPORTED;
    if (!m || !l || !O || !O_out) return TEA_EINVAL;
    if (!aligned(m, 4) || !aligned(l, 4) || !aligned(O, 4) || !aligned(O_out, out_dtype == TEA_F32 ? 4 : 2))
        return TEA_EINVAL;
    if ((m_out && !aligned(m_out, 4)) || (l_out && !aligned(l_out, 4))) return TEA_EINVAL;
    const size_t ob = (size_t)N * D * (out_dtype == TEA_F32 ? 4 : 2);
    const size_t pb = (size_t)N * S * 4, Ob = (size_t)N * S * D * 4, sb = (size_t)N * 4;
    if (overlap(O_out, ob, O, Ob) || overlap(O_out, ob, m, pb) || overlap(O_out, ob, l, pb)) return TEA_EINVAL;
    // the merged statistics are outputs too: no overlap with an input, the
    // merged O or each other
    if (m_out && l_out && overlap(m_out, sb, l_out, sb)) return TEA_EINVAL;
    for (const float* st : {m_out, l_out})
        if (st && (overlap(st, sb, O, Ob) || overlap(st, sb, m, pb) || overlap(st, sb, l, pb) ||
                   overlap(st, sb, O_out, ob)))
            return TEA_EINVAL;
    tea::MergeArgs a{m, l, O, N, S, D, m_out, l_out, O_out, out_dtype == TEA_BF16, normalize == 1,
                     (hipStream_t)stream};
    return status_of(tea::launch_merge(a));
}

}  // extern "C"
