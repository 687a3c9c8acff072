// S1: top-k softmax router: 32 lanes per token (two tokens per wave) up to
// 256 experts and top-16, a whole wave per token beyond.
//
// Selection compares the fp32 logits (ties to the lower expert id), so the
// chosen experts do not depend on how exp() is evaluated; the weights are the
// softmax probabilities exp(l - max) / sum_e exp(l_e - max) in fp32 (GC-MoE
// page, "Approach": routing precedes the token dispatch; the softmax top-k
// reading is this library's, the pages never give the router function).
#include "moe_device.h"
#include "moe_internal.h"

namespace {

constexpr int kWavesPerBlock = 4;

// LPT lanes per token, 64 / LPT tokens per wave.
template <int LPT, int VPL>
__global__ __launch_bounds__(64 * kWavesPerBlock)
void route_kernel(const float* __restrict__ logits, int T, int E, int k, int renorm,
                  int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
    constexpr int TPW = 64 / LPT;
    const int lane = threadIdx.x & 63;
    const int t0 = (blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6)) * TPW;
    if (t0 >= T) return;
    const int t = t0 + lane / LPT;
    float v[VPL];
    if (t < T) load_logits<LPT, VPL>(logits + (size_t)t * E, E, lane, v);
    else {
        #pragma unroll
        for (int i = 0; i < VPL; ++i) v[i] = -INFINITY;
    }
    int e = 0;
    float w = 0.f;
    route_values<LPT, VPL>(v, t < T ? E : 0, k, renorm != 0, lane, e, w);
    const int j = lane & (LPT - 1);
    if (t < T && j < k) {
        topk_idx[(size_t)t * k + j] = e;
        topk_w[(size_t)t * k + j] = w;
    }
}

}  // namespace

int moe_launch_route(const float* logits, int T, int E, int k, uint32_t flags,
                     int32_t* topk_idx, float* topk_w, hipStream_t stream) {
    if (T == 0) return 0;
    const int renorm = (flags & MOE_ROUTE_RENORM) ? 1 : 0;
    const dim3 block(64 * kWavesPerBlock);
    if (E <= 256 && k <= 16) {                       // two tokens per wave, 32 lanes each
        const dim3 grid((T + 2 * kWavesPerBlock - 1) / (2 * kWavesPerBlock));
        const int vpl = (E + 31) / 32;
#define MOE_ROUTE32_CASE(N)                                                                     \
        if (vpl <= N) {                                                                         \
            hipLaunchKernelGGL((route_kernel<32, N>), grid, block, 0, stream, logits, T, E, k,  \
                               renorm, topk_idx, topk_w);                                       \
            return (int)hipGetLastError();                                                      \
        }
        MOE_ROUTE32_CASE(2)
        MOE_ROUTE32_CASE(4)
        MOE_ROUTE32_CASE(8)
#undef MOE_ROUTE32_CASE
    }
    const dim3 grid((T + kWavesPerBlock - 1) / kWavesPerBlock);
    const int vpl = (E + 63) / 64;
#define MOE_ROUTE_CASE(N)                                                                       \
    if (vpl <= N) {                                                                             \
        hipLaunchKernelGGL((route_kernel<64, N>), grid, block, 0, stream, logits, T, E, k,      \
                           renorm, topk_idx, topk_w);                                           \
        return (int)hipGetLastError();                                                          \
    }
    MOE_ROUTE_CASE(1)
    MOE_ROUTE_CASE(2)
    MOE_ROUTE_CASE(4)
    MOE_ROUTE_CASE(8)
    MOE_ROUTE_CASE(16)
    MOE_ROUTE_CASE(32)
#undef MOE_ROUTE_CASE
    return -1;
}
