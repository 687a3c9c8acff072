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

// Lane-strided: lane l holds experts l, l + 64, l + 128, ... (VPL per lane).
template <int VPL>
__global__ __launch_bounds__(64 * kWavesPerBlock)
void route_kernel(const float* __restrict__ logits, int T, int E, int k, int renorm,
                  int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
    if (t >= T) return;
    const float* row = logits + (size_t)t * E;

    float v[VPL];
    #pragma unroll
    for (int i = 0; i < VPL; ++i) {
        int e = lane + 64 * i;
        v[i] = e < E ? row[e] : -INFINITY;
    }
    // global max: the top-1 logit
    float m = v[0];
    #pragma unroll
    for (int i = 1; i < VPL; ++i) m = fmaxf(m, v[i]);
    #pragma unroll
    for (int s = 32; s >= 1; s >>= 1) m = fmaxf(m, __shfl_xor(m, s, 64));
    // softmax denominator, fp32, fixed reduction tree
    float sum = 0.f;
    #pragma unroll
    for (int i = 0; i < VPL; ++i) {
        int e = lane + 64 * i;
        if (e < E) sum += expf(v[i] - m);
    }
    #pragma unroll
    for (int s = 32; s >= 1; s >>= 1) sum += __shfl_xor(sum, s, 64);
    const float inv = 1.0f / sum;

    uint32_t taken = 0;                 // per-lane bitmask over its VPL slots
    float wsum = 0.f;
    int my_j = -1;                      // lane j (< k) stores result j
    int   res_e = 0;
    float res_w = 0.f;
    for (int j = 0; j < k; ++j) {
        // lane-local best among not-taken: larger value, then lower expert id
        float bv = -INFINITY;
        int be = 0x7FFFFFFF;
        #pragma unroll
        for (int i = 0; i < VPL; ++i) {
            int e = lane + 64 * i;
            bool ok = e < E && !((taken >> i) & 1u);
            if (ok && (v[i] > bv || (v[i] == bv && e < be))) { bv = v[i]; be = e; }
        }
        // wave argmax
        #pragma unroll
        for (int s = 32; s >= 1; s >>= 1) {
            float ov = __shfl_xor(bv, s, 64);
            int oe = __shfl_xor(be, s, 64);
            if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
        }
        if ((be & 63) == lane) taken |= 1u << (be >> 6);
        float w = expf(bv - m) * inv;
        wsum += w;
        if (lane == j) { res_e = be; res_w = w; my_j = j; }
    }
    if (my_j >= 0) {
        float w = renorm ? res_w / wsum : res_w;
        topk_idx[(size_t)t * k + my_j] = res_e;
        topk_w[(size_t)t * k + my_j] = w;
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
