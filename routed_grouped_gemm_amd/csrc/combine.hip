// S7: combine. out[t] = BF16(sum over the token's local slots of its BF16 rows),
// summed in fp64 in slot order and rounded once (GC-MoE page, "Approach":
// the finalize role combines the BF16 fragments into token order).
#include "moe_device.h"
#include "moe_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kVec = 8;                 // bf16 per thread per pass (16 bytes)
constexpr int kSlotBatch = 8;           // slots whose rows are requested together

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// One workgroup per (token, 2048-column block). The token's slot rows are
// read first (the same for every lane), then one 16-byte load per slot is
// issued before any is used, each through a resource over that slot's row
// (empty for slots that are not local, which then read zeros without a
// branch); the sum runs in slot order in fp64. The rows are read once and
// the output written once: both bypass the caches' retention (non-temporal),
// which took 12 us off the 16K-token prefill's combine.
__global__ __launch_bounds__(kThreads)
void combine_kernel(const uint16_t* __restrict__ y, const int32_t* __restrict__ slot_row,
                    const float* __restrict__ row_w, int ks, int H, uint16_t* __restrict__ out) {
    const int t = blockIdx.x;
    const int h0 = (blockIdx.y * kThreads + threadIdx.x) * kVec;
    if (h0 >= H) return;
    double acc[kVec];
    #pragma unroll
    for (int i = 0; i < kVec; ++i) acc[i] = 0.0;
    const int32_t* sr = slot_row + (size_t)t * ks;
    for (int j0 = 0; j0 < ks; j0 += kSlotBatch) {
        int r[kSlotBatch];
        #pragma unroll
        for (int j = 0; j < kSlotBatch; ++j)
            r[j] = __builtin_amdgcn_readfirstlane(j0 + j < ks ? sr[j0 + j] : -1);
        uint4 v[kSlotBatch];
        #pragma unroll
        for (int j = 0; j < kSlotBatch; ++j) {
            const rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint16_t*>(y) + (size_t)(r[j] < 0 ? 0 : r[j]) * H, 0, r[j] < 0 ? 0 : H * 2, 0x00020000);
            const i32x4 d = __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)(h0 * 2), 0, 2);
            v[j] = make_uint4((uint32_t)d[0], (uint32_t)d[1], (uint32_t)d[2], (uint32_t)d[3]);
        }
        #pragma unroll
        for (int j = 0; j < kSlotBatch; ++j) {
            if (r[j] < 0) continue;                // uniform: the same slot for every lane
            const double w = row_w ? (double)row_w[r[j]] : 1.0;
            const uint32_t pw[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
            #pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[2 * i]     += (double)bf16_to_f32(pw[i] & 0xFFFFu) * w;
                acc[2 * i + 1] += (double)bf16_to_f32(pw[i] >> 16) * w;
            }
        }
    }
    uint4 o;
    uint32_t q[4];
    #pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = f64_to_bf16(acc[2 * i]) | (f64_to_bf16(acc[2 * i + 1]) << 16);
    o.x = q[0]; o.y = q[1]; o.z = q[2]; o.w = q[3];
    const i32x4 ov = {(int)o.x, (int)o.y, (int)o.z, (int)o.w};
    __builtin_nontemporal_store(ov, (i32x4*)(out + (size_t)t * H + h0));
}

}  // namespace

int moe_launch_combine(const uint16_t* y, const int32_t* slot_row, const float* row_w, int T,
                       int ks, int H, uint16_t* out, hipStream_t stream) {
    if (T == 0) return 0;
    dim3 grid(T, (H / kVec + kThreads - 1) / kThreads), block(kThreads);
    hipLaunchKernelGGL(combine_kernel, grid, block, 0, stream, y, slot_row, row_w, ks, H, out);
    return (int)hipGetLastError();
}
