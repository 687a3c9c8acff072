// One-time weight preparation: MX quantisation of fp32 rows (a utility) and
// the prepack of logical MX weights into the layout the grouped GEMMs stream.
//
// Prepacked layout, group-major: group g occupies bytes [g*S, (g+1)*S) with
// S = data + scales of one group, so groups can be prepacked one at a time:
//   unit   = 64 output rows: for W2 rows [64u, 64u+64); for W1 the gate rows
//            [32u, 32u+32) followed by the up rows I + [32u, 32u+32), so one
//            workgroup owns gate row n and up row n (the fusion blog's gate/up
//            repack for a fused GLU epilogue, done at load time)
//   tile   = 16 rows x 128 K of a unit (4 tiles per unit per K-tile)
//   data   [g][unit][kt][tile][...], lane l holding row l%16 of the tile and
//          lane group q = l/16 in MFMA operand order:
//            FP4: [lane][16 B], K [kt*128 + 32q, +32), element 2i in the low nibble
//            FP8: [half][lane][16 B], half 0 = K [kt*128 + 16q, +16),
//                 half 1 = K [kt*128 + 64 + 16q, +16)
//          so every 16-byte load of a wave reads 1 KiB contiguous
//   scales [g][unit][kt/4][tile][lane][kt%4]: the E8M0 byte of row l%16,
//          K-block kt*4 + q; one dword per lane covers four K-tiles.
// A 16x128 tile is one contiguous 1 KiB (FP4) / 2 KiB (FP8) burst.
#include "moe_device.h"
#include "moe_internal.h"

PackGeom moe_pack_geom(int G, int N, int K, int fmt) {
    PackGeom p;
    p.units = N / 64;
    p.kt = K / 128;
    p.kt4 = (p.kt + 3) / 4;
    p.bpl = (fmt == MOE_FMT_MXFP4) ? 16 : 32;
    p.data_per_unit = (size_t)p.kt * 4 * 64 * p.bpl;
    p.scale_per_unit = (size_t)p.kt4 * 4 * 64 * 4;
    p.data_per_group = p.data_per_unit * p.units;
    p.scale_per_group = p.scale_per_unit * p.units;
    p.group_stride = p.data_per_group + p.scale_per_group;
    p.total = p.group_stride * G;
    return p;
}

namespace {

// logical row of (unit, tile, row-in-tile)
MOE_DEV int logical_row(int u, int tile, int r, int is_w1, int half) {
    if (!is_w1) return 64 * u + 16 * tile + r;
    int base = (tile >= 2) ? half : 0;          // tiles 0,1 gate; 2,3 up
    return base + 32 * u + 16 * (tile & 1) + r;
}

__global__ void prepack_data_kernel(const uint8_t* __restrict__ q, int G, int N, int K, int fmt,
                                    int is_w1, uint8_t* __restrict__ dst, PackGeom p) {
    const size_t n = (size_t)G * p.units * p.kt * 256;
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const int lane = (int)(i % 64);
    const int tile = (int)((i / 64) % 4);
    const int kt = (int)((i / 256) % p.kt);
    const int u = (int)((i / (256 * (size_t)p.kt)) % p.units);
    const int g = (int)(i / (256 * (size_t)p.kt * p.units));
    const int row = logical_row(u, tile, lane % 16, is_w1, N / 2);
    const int grp = lane / 16;
    uint8_t* out = dst + g * p.group_stride + u * p.data_per_unit +
                   (size_t)(kt * 4 + tile) * 64 * p.bpl + lane * 16;
    if (fmt == MOE_FMT_MXFP4) {
        const size_t rowb = (size_t)K / 2;
        const uint8_t* src = q + ((size_t)g * N + row) * rowb + kt * 64 + 16 * grp;
        *(uint4*)out = *(const uint4*)src;
    } else {
        const uint8_t* src = q + ((size_t)g * N + row) * (size_t)K + kt * 128;
        *(uint4*)out = *(const uint4*)(src + 16 * grp);
        *(uint4*)(out + 1024) = *(const uint4*)(src + 64 + 16 * grp);
    }
}

__global__ void prepack_scale_kernel(const uint8_t* __restrict__ sc, int G, int N, int K,
                                     int is_w1, uint8_t* __restrict__ dst, PackGeom p) {
    const size_t n = (size_t)G * p.units * p.kt4 * 256;
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const int lane = (int)(i % 64);
    const int tile = (int)((i / 64) % 4);
    const int k4 = (int)((i / 256) % p.kt4);
    const int u = (int)((i / (256 * (size_t)p.kt4)) % p.units);
    const int g = (int)(i / (256 * (size_t)p.kt4 * p.units));
    const int row = logical_row(u, tile, lane % 16, is_w1, N / 2);
    const int grp = lane / 16;
    const uint8_t* src = sc + ((size_t)g * N + row) * (size_t)(K / 32);
    uint32_t word = 0;
    for (int j = 0; j < 4; ++j) {
        int kt = k4 * 4 + j;
        uint32_t b = kt < p.kt ? src[kt * 4 + grp] : 127u;
        word |= b << (8 * j);
    }
    uint8_t* out = dst + g * p.group_stride + p.data_per_group + u * p.scale_per_unit +
                   ((size_t)(k4 * 4 + tile) * 64 + lane) * 4;
    *(uint32_t*)out = word;
}

// One thread per 32-element block.
__global__ void quantize_kernel(const float* __restrict__ src, size_t nblocks, int K, int fmt,
                                int ceil_rule, uint8_t* __restrict__ q, uint8_t* __restrict__ s) {
    const size_t b = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= nblocks) return;
    const float4* in = (const float4*)(src + b * 32);
    float v[32];
    #pragma unroll
    for (int i = 0; i < 8; ++i) {
        float4 f = in[i];
        v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
    }
    float amax = 0.f;
    #pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    uint32_t code;
    if (fmt == MOE_FMT_MXFP8) {
        code = e4m3_scale_code(amax, ceil_rule);
        const float inv = inv_scale(code);
        uint32_t w[8];
        #pragma unroll
        for (int i = 0; i < 8; ++i)
            w[i] = f32_to_e4m3(v[4 * i] * inv) | (f32_to_e4m3(v[4 * i + 1] * inv) << 8) |
                   (f32_to_e4m3(v[4 * i + 2] * inv) << 16) | (f32_to_e4m3(v[4 * i + 3] * inv) << 24);
        uint4* o = (uint4*)(q + b * 32);
        o[0] = make_uint4(w[0], w[1], w[2], w[3]);
        o[1] = make_uint4(w[4], w[5], w[6], w[7]);
    } else {
        code = e2m1_scale_code(amax, ceil_rule);
        const float inv = inv_scale(code);
        uint32_t w[4] = {0, 0, 0, 0};
        #pragma unroll
        for (int i = 0; i < 32; ++i) w[i / 8] |= f32_to_e2m1(v[i] * inv) << (4 * (i % 8));
        *(uint4*)(q + b * 16) = make_uint4(w[0], w[1], w[2], w[3]);
    }
    s[b] = (uint8_t)code;
}

}  // namespace

int moe_launch_prepack(const uint8_t* q, const uint8_t* sc, int G, int N, int K, int fmt,
                       int is_w1, uint8_t* dst, hipStream_t stream) {
    PackGeom p = moe_pack_geom(G, N, K, fmt);
    size_t nd = (size_t)G * p.units * p.kt * 256, ns = (size_t)G * p.units * p.kt4 * 256;
    if (nd) hipLaunchKernelGGL(prepack_data_kernel, dim3((unsigned)((nd + 255) / 256)), dim3(256), 0,
                               stream, q, G, N, K, fmt, is_w1, dst, p);
    if (ns) hipLaunchKernelGGL(prepack_scale_kernel, dim3((unsigned)((ns + 255) / 256)), dim3(256), 0,
                               stream, sc, G, N, K, is_w1, dst, p);
    return (int)hipGetLastError();
}

int moe_launch_quantize(const float* src, int rows, int K, int fmt, uint32_t flags, uint8_t* q,
                        uint8_t* s, hipStream_t stream) {
    size_t nb = (size_t)rows * (K / 32);
    if (!nb) return 0;
    hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, stream, src,
                       nb, K, fmt, (flags & MOE_SCALE_RULE_CEIL) ? 1 : 0, q, s);
    return (int)hipGetLastError();
}
