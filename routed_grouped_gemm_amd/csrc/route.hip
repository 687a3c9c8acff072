// S1: top-k softmax router. One wave64 per token.
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

template <int VPL>
__global__ __launch_bounds__(64 * kWavesPerBlock)
void route_kernel(const float* __restrict__ logits, int T, int E, int k, int renorm,
                  int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
    if (t >= T) return;
    int e = 0;
    float w = 0.f;
    float v[VPL];
    load_logits<VPL>(logits + (size_t)t * E, E, lane, v);
    wave_route_values<VPL>(v, E, k, renorm != 0, lane, e, w);
    if (lane < k) {
        topk_idx[(size_t)t * k + lane] = e;
        topk_w[(size_t)t * k + lane] = w;
    }
}

}  // namespace

int moe_launch_route(const float* logits, int T, int E, int k, uint32_t flags,
                     int32_t* topk_idx, float* topk_w, hipStream_t stream) {
    if (T == 0) return 0;
    dim3 grid((T + kWavesPerBlock - 1) / kWavesPerBlock), block(64 * kWavesPerBlock);
    int renorm = (flags & MOE_ROUTE_RENORM) ? 1 : 0;
    int vpl = (E + 63) / 64;
#define MOE_ROUTE_CASE(N)                                                              \
    if (vpl <= N) {                                                                    \
        hipLaunchKernelGGL(route_kernel<N>, grid, block, 0, stream, logits, T, E, k,   \
                           renorm, topk_idx, topk_w);                                  \
        return (int)hipGetLastError();                                                 \
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
