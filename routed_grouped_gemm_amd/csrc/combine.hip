// S7: combine. out[t] = BF16(sum over the token's local slots of its BF16 rows),
// summed in fp64 in slot order and rounded once (GC-MoE page, "Approach":
// the finalize role combines the BF16 fragments into token order).
#include "moe_device.h"
#include "moe_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kVec = 8;                 // bf16 per thread per pass (16 bytes)
constexpr int kSlotBatch = 8;           // slots whose rows are requested together
constexpr int kTwoTokenMinT = 1024;     // two tokens per workgroup from this many tokens

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// One workgroup per (TOK tokens, 2048-column block). The tokens' slot rows
// are read first (the same for every lane), then one 16-byte load per slot
// of every token is issued before any is used, each through a resource over
// that slot's row (empty for slots that are not local, which then read zeros
// without a branch); each token's sum runs in slot order in fp64. The rows
// are read once and the output written once: both bypass the caches'
// retention (non-temporal), which took 12 us off the 16K-token prefill's
// combine. TOK = 2 for many tokens (twice the loads in flight per lane:
// the 16K-token prefill layer 2-14 us faster over two runs), 1 otherwise
// (more workgroups for few tokens: with 2, T = 8 took 46.3 -> 47.1 us).
template <int TOK>
__global__ __launch_bounds__(kThreads)
void combine_kernel(const uint16_t* __restrict__ y, const int32_t* __restrict__ slot_row,
                    const float* __restrict__ row_w, int T, int ks, int H, uint16_t* __restrict__ out) {
    const int t0 = blockIdx.x * TOK;
    const int h0 = (blockIdx.y * kThreads + threadIdx.x) * kVec;
    if (h0 >= H) return;
    double acc[TOK][kVec];
    #pragma unroll
    for (int q = 0; q < TOK; ++q)
        #pragma unroll
        for (int i = 0; i < kVec; ++i) acc[q][i] = 0.0;
    for (int j0 = 0; j0 < ks; j0 += kSlotBatch) {
        int r[TOK][kSlotBatch];
        #pragma unroll
        for (int q = 0; q < TOK; ++q)
            #pragma unroll
            for (int j = 0; j < kSlotBatch; ++j)
                r[q][j] = __builtin_amdgcn_readfirstlane(
                    t0 + q < T && j0 + j < ks ? slot_row[(size_t)(t0 + q) * ks + j0 + j] : -1);
        uint4 v[TOK][kSlotBatch];
        #pragma unroll
        for (int q = 0; q < TOK; ++q)
            #pragma unroll
            for (int j = 0; j < kSlotBatch; ++j) {
                const int rr = r[q][j];
                const rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                    const_cast<uint16_t*>(y) + (size_t)(rr < 0 ? 0 : rr) * H, 0, rr < 0 ? 0 : H * 2, 0x00020000);
                const i32x4 d = __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)(h0 * 2), 0, 2);
                v[q][j] = make_uint4((uint32_t)d[0], (uint32_t)d[1], (uint32_t)d[2], (uint32_t)d[3]);
            }
        #pragma unroll
        for (int q = 0; q < TOK; ++q)
            #pragma unroll
            for (int j = 0; j < kSlotBatch; ++j) {
                if (r[q][j] < 0) continue;         // uniform: the same slot for every lane
                const double w = row_w ? (double)row_w[r[q][j]] : 1.0;
                const uint32_t pw[4] = {v[q][j].x, v[q][j].y, v[q][j].z, v[q][j].w};
                #pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc[q][2 * i]     += (double)bf16_to_f32(pw[i] & 0xFFFFu) * w;
                    acc[q][2 * i + 1] += (double)bf16_to_f32(pw[i] >> 16) * w;
                }
            }
    }
    #pragma unroll
    for (int q = 0; q < TOK; ++q) {
        if (t0 + q >= T) break;
        i32x4 ov;
        #pragma unroll
        for (int i = 0; i < 4; ++i)
            ov[i] = (int)(f64_to_bf16(acc[q][2 * i]) | (f64_to_bf16(acc[q][2 * i + 1]) << 16));
        __builtin_nontemporal_store(ov, (i32x4*)(out + (size_t)(t0 + q) * H + h0));
    }
}

}  // namespace

int moe_launch_combine(const uint16_t* y, const int32_t* slot_row, const float* row_w, int T,
                       int ks, int H, uint16_t* out, hipStream_t stream) {
    if (T == 0) return 0;
    const int blocks = (H / kVec + kThreads - 1) / kThreads;
    if (T >= kTwoTokenMinT)
        hipLaunchKernelGGL(combine_kernel<2>, dim3((T + 1) / 2, blocks), dim3(kThreads), 0, stream, y,
                           slot_row, row_w, T, ks, H, out);
    else
        hipLaunchKernelGGL(combine_kernel<1>, dim3(T, blocks), dim3(kThreads), 0, stream, y, slot_row,
                           row_w, T, ks, H, out);
    return (int)hipGetLastError();
}
