// Internal launch interface between the C ABI (api.cpp) and the kernels.
// Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tea {

// rescale policy of the online fold (the three give the same bits)
enum : int { kRescaleAlways = 0, kRescaleIfRise = 1, kRescaleL0One = 2 };

struct RowSoftmaxArgs {
    const void* x;
    void* y;
    int64_t rows, cols;
    bool bf16;
    int block;  // power of two >= 1
    float* m_out;
    float* l_out;
    hipStream_t stream;
    int rescale = kRescaleAlways;
};
hipError_t launch_row_softmax(const RowSoftmaxArgs& a);
int64_t row_softmax_max_cols();

struct MergeArgs {
    const float* m;  // [N, S]
    const float* l;  // [N, S]
    const float* O;  // [N, S, D]
    int64_t N;
    int S, D;
    float* m_out;  // [N] nullable
    float* l_out;  // [N] nullable
    void* O_out;   // [N, D]
    bool out_bf16;
    bool normalize;
    hipStream_t stream;
    float* lse_out = nullptr;  // [N] nullable: m + log l (natural units), -inf for an empty state
};
hipError_t launch_merge(const MergeArgs& a);

struct DecodeArgs {
    const void* q;  // [B, H, 1, D] bf16
    const void* k;  // [B, H, Lmax, D] bf16
    const void* v;
    const int32_t* kv_len;  // [B]
    void* o;                // [B, H, D]
    int B, H, Lmax, D, num_splits;
    float scale;
    bool out_bf16;
    float* ws_m;  // [B, H, S]
    float* ws_l;  // [B, H, S]
    float* ws_O;  // [B, H, S, D]
    hipStream_t stream;
};
hipError_t launch_decode(const DecodeArgs& a);
hipError_t launch_decode_fused(const DecodeArgs& a);  // ws_* unused
int decode_fused_max_splits();
size_t decode_workspace_bytes(int B, int H, int D, int num_splits);
// points a.ws_m, a.ws_l and a.ws_O into a workspace of decode_workspace_bytes()
void decode_bind_workspace(DecodeArgs& a, void* workspace);
// bytes of the device-resident scratch of the allocation-free decode
constexpr size_t kDecodeScratchBytes = size_t(32) << 20;
// launch_decode with the partials in that scratch (a.ws_* ignored); the
// caller has checked decode_workspace_bytes() <= kDecodeScratchBytes
hipError_t launch_decode_noalloc(DecodeArgs a);

struct AttnArgs {
    const void* q;  // [B, H, Sq, D] bf16
    const void* k;  // [B, H, Sk, D] bf16
    const void* v;  // [B, H, Sk, D] bf16
    void* o;        // [B, H, Sq, D]
    int B, H, Sq, Sk, D;
    float scale;
    bool causal;
    bool out_bf16;
    float* lse;  // [B, H, Sq] nullable
    hipStream_t stream;
};
hipError_t launch_attn_fwd(const AttnArgs& a);
size_t attn_splitk_workspace_bytes(int B, int H, int Sq, int D, int nsplit);
hipError_t launch_attn_fwd_splitk(const AttnArgs& a, int nsplit, void* workspace);

}  // namespace tea
