// A plain streaming read of device memory: the practical HBM read rate that
// the bandwidth-bound kernels are compared with, next to the 8 TB/s of the
// spec. Not a step of the layer.
//
// Every 16-byte chunk of the buffer is read once, with non-temporal buffer
// loads, eight per lane in flight, from a grid of 32 waves per CU. Each
// workgroup reads one contiguous run of the buffer, 32 KiB per pass. The
// chunks are folded with XOR so that no load can be dropped, and each wave
// writes its one word to `sink`.
#include "moe_device.h"
#include "moe_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;              // 16-byte loads in flight per lane

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__global__ __launch_bounds__(kThreads)
void hbm_read_kernel(const uint8_t* __restrict__ src, uint32_t bytes, uint32_t* __restrict__ sink) {
    const rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(src), 0, (int)bytes, 0x00020000);
    constexpr uint32_t kStep = kThreads * kUnroll;          // chunks per workgroup pass (32 KiB)
    const uint32_t n16 = bytes / 16;
    // this workgroup's contiguous run of chunks, in whole passes
    const uint32_t per = (n16 + gridDim.x * kStep - 1) / (gridDim.x * kStep) * kStep;
    const uint32_t lo = blockIdx.x * per, hi = min(n16, lo + per);
    uint32_t acc = 0;
    for (uint32_t i0 = lo + threadIdx.x; i0 < hi; i0 += kStep) {
        i32x4 v[kUnroll];
        #pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            // chunks past the run or the end read zeros: offsets at or past
            // `hi` are sent past the resource's range (bytes <= 2^31 keeps
            // every offset below 2^32)
            const uint32_t i = i0 + u * kThreads;
            v[u] = __builtin_amdgcn_raw_buffer_load_b128(r, i < hi ? i * 16u : bytes, 0, 2);
        }
        #pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= (uint32_t)(v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3]);
    }
    #pragma unroll
    for (int m = 32; m >= 1; m >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, m, 64);
    if ((threadIdx.x & 63) == 0) sink[blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6)] = acc;
}

}  // namespace

int moe_launch_hbm_read_probe(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream) {
    const int grid = MOE_HBM_PROBE_SINK_WORDS / (kThreads / 64);
    hipLaunchKernelGGL(hbm_read_kernel, dim3(grid), dim3(kThreads), 0, stream, (const uint8_t*)src,
                       (uint32_t)bytes, sink);
    return (int)hipGetLastError();
}
