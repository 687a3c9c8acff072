// S4-S6: grouped W1 (with the fused SwiGLU * w + FP8 requantisation epilogue)
// and grouped W2 (BF16 rows) on gfx950 scaled MFMA.
//
// Operand-swapped tiling (the GC-MoE page's Blackwell path puts the weights in
// the MMA's M slot and the few decode tokens in N, "Key contributions"): the
// prepacked weight tile is the A operand (16 rows x 128 K, streamed straight
// from HBM into registers in one 1-2 KiB burst per wave) and 16 grouped token
// rows are the B operand. A workgroup owns one 64-row weight unit of one group
// (for W1: 32 gate + the matching 32 up rows) and a pass of up to 16*NTT rows
// of that group; its 4 waves split K in runs of four 128-wide K-tiles and
// their partial sums are added in LDS in a fixed order, so results do not
// depend on scheduling. Group sizes are read from device memory: workgroups of
// empty groups or of passes past a group's end exit at once (no host sync;
// fusion blog, "Removing host-device synchronisation").
#include "moe_device.h"
#include "moe_internal.h"

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

struct KParams {
    const uint8_t* wbase[2];
    size_t gstride, dpg, dpu, spu;   // group stride; data bytes per group; per unit data / scales
    int E_loc, K, kt, kt4;
    const int32_t* counts;
    const int32_t* offsets;
    const int32_t* offsets32;
    const float* row_w;
    const uint8_t* aq;
    const uint8_t* as;
    const int32_t* row_src;       // null: grouped row r is activation row r
    int N;                        // W1: 2I ; W2: H (y row length)
    int ceil_rule, transpose, use_w;
    uint8_t* hq; uint8_t* hs; uint8_t* hTq; uint8_t* hTs; int ldT;
    uint16_t* y;
};

// Load a 16x128 weight tile operand for this lane (bpl bytes).
template <int WFMT>
MOE_DEV i32x8 load_w(const uint8_t* p) {
    i32x8 r;
    const i32x4 a = *(const i32x4*)p;
    r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
    if (WFMT == MFMA_FMT_FP8) {
        const i32x4 b = *(const i32x4*)(p + 16);
        r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
    } else {
        r[4] = 0; r[5] = 0; r[6] = 0; r[7] = 0;
    }
    return r;
}

// B operand: one grouped FP8 row's 128-wide K-tile in the MFMA FP8 order.
MOE_DEV i32x8 load_x(const uint8_t* row_kt, int grp) {
    const i32x4 a = *(const i32x4*)(row_kt + 16 * grp);
    const i32x4 b = *(const i32x4*)(row_kt + 64 + 16 * grp);
    i32x8 r;
    r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
    r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
    return r;
}

// One K-tile (index kt, scale byte SEL of the packed dword) for all active
// token tiles. xrow[tt] is this lane's activation row for token tile tt, or
// -1 past the end of the pass.
template <int WFMT, int NTT, int SEL>
MOE_DEV void k_step(const KParams& p, const uint8_t* wunit, const int (&sA)[4], int kt, int lane,
                    const long (&xrow)[NTT], int ntt_active, f32x4 (&acc)[NTT][4]) {
    if (kt >= p.kt) return;
    const int grp = lane >> 4;
    i32x8 A[4];
    #pragma unroll
    for (int t = 0; t < 4; ++t)
        A[t] = load_w<WFMT>(wunit + ((size_t)(kt * 4 + t) * 64 + lane) * (WFMT == MFMA_FMT_FP4 ? 16 : 32));
    #pragma unroll
    for (int tt = 0; tt < NTT; ++tt) {
        if (tt < ntt_active) {
            i32x8 B;
            int sB = 127;
            if (xrow[tt] >= 0) {
                const size_t row = (size_t)xrow[tt];
                B = load_x(p.aq + row * p.K + (size_t)kt * 128, grp);
                sB = p.as[row * (p.K / 32) + kt * 4 + grp];
            } else {
                B = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
            }
            #pragma unroll
            for (int t = 0; t < 4; ++t)
                acc[tt][t] = mfma16x16x128<WFMT, MFMA_FMT_FP8, SEL, 0>(A[t], B, acc[tt][t], sA[t], sB);
        }
    }
}

template <int WFMT, bool IS_W1, int NTT>
__global__ __launch_bounds__(kThreads)
void grouped_gemm_kernel(KParams p) {
    const int u = blockIdx.x, g = blockIdx.y;
    const int n_g = p.counts[g];
    const int rows_per_pass = 16 * NTT;
    const int npass = (n_g + rows_per_pass - 1) / rows_per_pass;
    if ((int)blockIdx.z >= npass) return;

    extern __shared__ float lds[];
    float* red = lds;                                   // [2][NTT][4 tiles][4][64 lanes]
    float* hbuf = lds + 2 * NTT * 1024;                 // [16*NTT][33]  (W1)

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int sel = g < p.E_loc ? 0 : 1;
    const int gi = g < p.E_loc ? g : 0;
    const uint8_t* wgrp = p.wbase[sel] + gi * p.gstride;
    const uint8_t* wunit = wgrp + u * p.dpu;
    const uint8_t* sunit = wgrp + p.dpg + u * p.spu;
    const int row0 = p.offsets[g];
    const int kg0 = (w * p.kt4) / kWaves, kg1 = ((w + 1) * p.kt4) / kWaves;

    for (int pass = blockIdx.z; pass < npass; pass += gridDim.z) {
        const int rbase = row0 + pass * rows_per_pass;
        const int nrows = min(rows_per_pass, n_g - pass * rows_per_pass);
        const int ntt_active = (nrows + 15) / 16;

        f32x4 acc[NTT][4];
        long xrow[NTT];
        #pragma unroll
        for (int tt = 0; tt < NTT; ++tt) {
            #pragma unroll
            for (int t = 0; t < 4; ++t) acc[tt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
            const int r = tt * 16 + (lane & 15);
            xrow[tt] = r < nrows ? (p.row_src ? (long)p.row_src[rbase + r] : (long)(rbase + r)) : -1;
        }

        for (int kg = kg0; kg < kg1; ++kg) {
            int sA[4];
            #pragma unroll
            for (int t = 0; t < 4; ++t)
                sA[t] = *(const int*)(sunit + ((size_t)(kg * 4 + t) * 64 + lane) * 4);
            k_step<WFMT, NTT, 0>(p, wunit, sA, kg * 4 + 0, lane, xrow, ntt_active, acc);
            k_step<WFMT, NTT, 1>(p, wunit, sA, kg * 4 + 1, lane, xrow, ntt_active, acc);
            k_step<WFMT, NTT, 2>(p, wunit, sA, kg * 4 + 2, lane, xrow, ntt_active, acc);
            k_step<WFMT, NTT, 3>(p, wunit, sA, kg * 4 + 3, lane, xrow, ntt_active, acc);
        }

        // Sum the four waves' partials in a fixed order, ((w0 + w2) + (w1 + w3)),
        // through two LDS slots; the total ends up in slot 0.
        auto store_acc = [&](int slot) {
            #pragma unroll
            for (int tt = 0; tt < NTT; ++tt)
                #pragma unroll
                for (int t = 0; t < 4; ++t)
                    #pragma unroll
                    for (int v = 0; v < 4; ++v)
                        red[(((slot * NTT + tt) * 4 + t) * 4 + v) * 64 + lane] = acc[tt][t][v];
        };
        auto add_acc = [&](int slot) {
            #pragma unroll
            for (int tt = 0; tt < NTT; ++tt)
                #pragma unroll
                for (int t = 0; t < 4; ++t)
                    #pragma unroll
                    for (int v = 0; v < 4; ++v)
                        acc[tt][t][v] += red[(((slot * NTT + tt) * 4 + t) * 4 + v) * 64 + lane];
        };
        if (w >= 2) store_acc(w - 2);
        __syncthreads();
        if (w < 2) add_acc(w);
        __syncthreads();
        if (w == 1) store_acc(0);
        __syncthreads();
        if (w == 0) { add_acc(0); store_acc(0); }
        __syncthreads();

        if (IS_W1) {
            const int I = p.N / 2;
            // gate/up pairs -> h (fp32) in LDS, [token][feature of this unit]
            for (int e = tid; e < NTT * 512; e += kThreads) {
                const int le = e & 63, v = (e >> 6) & 3, gt = (e >> 8) & 1, tt = e >> 9;
                const int tok = tt * 16 + (le & 15);
                if (tok >= nrows) continue;
                const float gsum = red[((tt * 4 + gt) * 4 + v) * 64 + le];
                const float usum = red[((tt * 4 + gt + 2) * 4 + v) * 64 + le];
                const int f = gt * 16 + 4 * (le >> 4) + v;
                const float wgt = p.use_w ? p.row_w[rbase + tok] : 1.0f;
                hbuf[tok * 33 + f] = silu(gsum) * usum * wgt;
            }
            __syncthreads();
            // row-wise MX-E4M3 quantisation: 32 threads per token (one 32-block)
            for (int t0 = 0; t0 < rows_per_pass; t0 += kThreads / 32) {
                const int tok = t0 + (tid >> 5), f = tid & 31;
                const bool valid = tok < nrows;
                const float h = valid ? hbuf[tok * 33 + f] : 0.f;
                float amax = fabsf(h);
                #pragma unroll
                for (int m = 16; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
                const uint32_t code = e4m3_scale_code(amax, p.ceil_rule);
                const uint32_t qb = f32_to_e4m3(h * inv_scale(code));
                const uint32_t b1 = __shfl_down(qb, 1, 64), b2 = __shfl_down(qb, 2, 64),
                               b3 = __shfl_down(qb, 3, 64);
                if (valid) {
                    const size_t r = (size_t)(rbase + tok);
                    if ((f & 3) == 0)
                        *(uint32_t*)(p.hq + r * I + 32 * u + f) = qb | (b1 << 8) | (b2 << 16) | (b3 << 24);
                    if (f == 0) p.hs[r * (I / 32) + u] = (uint8_t)code;
                }
            }
            if (p.transpose) {
                // columns of this pass: [offsets32[g] + pass*rows_per_pass, ...) ; blocks of 32 tokens
                const int ncols = (nrows + 31) & ~31;
                const int col0 = p.offsets32[g] + pass * rows_per_pass;
                for (int it = 0; it < 32 * (rows_per_pass / 32); it += kThreads / 32) {
                    const int pr = it + (tid >> 5);
                    const int f = pr & 31, tb = pr >> 5;
                    const int tok = tb * 32 + (tid & 31);
                    const float h = tok < nrows ? hbuf[tok * 33 + f] : 0.f;
                    float amax = fabsf(h);
                    #pragma unroll
                    for (int m = 16; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
                    const uint32_t code = e4m3_scale_code(amax, p.ceil_rule);
                    const uint32_t qb = tok < nrows ? f32_to_e4m3(h * inv_scale(code)) : 0u;
                    if (tb * 32 < ncols) {
                        const size_t frow = (size_t)(32 * u + f);
                        p.hTq[frow * p.ldT + col0 + tok] = (uint8_t)qb;
                        if ((tid & 31) == 0) p.hTs[frow * (p.ldT / 32) + (col0 >> 5) + tb] = (uint8_t)code;
                    }
                }
            }
        } else {
            const int H = p.N;
            for (int e = tid; e < NTT * 256; e += kThreads) {
                const int le = e & 63, t = (e >> 6) & 3, tt = e >> 8;
                const int tok = tt * 16 + (le & 15);
                if (tok >= nrows) continue;
                float s[4];
                #pragma unroll
                for (int v = 0; v < 4; ++v) s[v] = red[((tt * 4 + t) * 4 + v) * 64 + le];
                uint2 o;
                o.x = f32_to_bf16(s[0]) | (f32_to_bf16(s[1]) << 16);
                o.y = f32_to_bf16(s[2]) | (f32_to_bf16(s[3]) << 16);
                *(uint2*)(p.y + (size_t)(rbase + tok) * H + 64 * u + 16 * t + 4 * (le >> 4)) = o;
            }
        }
        __syncthreads();
    }
}

KParams make_params(const GemmArgs& a, bool w1) {
    KParams p{};
    PackGeom geo = moe_pack_geom(1, a.N, a.K, a.fmt);
    for (int i = 0; i < 2; ++i) p.wbase[i] = a.w_base[i];
    p.gstride = geo.group_stride; p.dpg = geo.data_per_group;
    p.dpu = geo.data_per_unit;    p.spu = geo.scale_per_unit;
    p.E_loc = a.E_loc; p.K = a.K; p.kt = geo.kt; p.kt4 = geo.kt4;
    p.counts = a.counts; p.offsets = a.offsets; p.offsets32 = a.offsets32;
    p.row_w = a.row_w; p.aq = a.aq; p.as = a.as; p.row_src = a.row_src; p.N = a.N;
    p.ceil_rule = (a.flags & MOE_SCALE_RULE_CEIL) ? 1 : 0;
    p.transpose = (w1 && (a.flags & MOE_W1_WRITE_TRANSPOSE)) ? 1 : 0;
    p.use_w = (w1 && a.row_w && !(a.flags & MOE_WEIGHT_AT_COMBINE)) ? 1 : 0;
    p.hq = a.hq; p.hs = a.hs; p.hTq = a.hTq; p.hTs = a.hTs; p.ldT = a.ldT;
    p.y = a.y;
    return p;
}

// Token tiles per pass, from the expected rows per group (T*k spread over the groups).
int pick_ntt(const GemmArgs& a, bool transpose) {
    const int avg = a.rows_hint > 0 ? a.rows_hint : a.R_max / (a.G > 0 ? a.G : 1);
    int ntt = avg <= 16 ? 1 : (avg <= 32 ? 2 : 4);
    if (transpose && ntt < 2) ntt = 2;       // 32-token blocks must not straddle passes
    return ntt;
}

template <int WFMT, bool IS_W1, int NTT>
int launch(const KParams& p, int units, int G, int passes, hipStream_t stream) {
    size_t lds = (size_t)2 * NTT * 1024 * 4 + (IS_W1 ? (size_t)16 * NTT * 33 * 4 : 0);
    dim3 grid(units, G, passes);
    hipLaunchKernelGGL((grouped_gemm_kernel<WFMT, IS_W1, NTT>), grid, dim3(kThreads), lds, stream, p);
    return (int)hipGetLastError();
}

template <bool IS_W1>
int launch_grouped(const GemmArgs& a, hipStream_t stream) {
    if (a.G == 0 || a.R_max == 0) return 0;
    KParams p = make_params(a, IS_W1);
    const int ntt = pick_ntt(a, p.transpose);
    const int units = a.N / 64;
    const int avg = a.rows_hint > 0 ? a.rows_hint : a.R_max / a.G;
    int passes = 2 * ((avg + 16 * ntt - 1) / (16 * ntt));
    passes = passes < 1 ? 1 : (passes > 16 ? 16 : passes);
    const bool fp4 = a.fmt == MOE_FMT_MXFP4;
#define MOE_GEMM_CASE(N)                                                                      \
    if (ntt == N)                                                                             \
        return fp4 ? launch<MFMA_FMT_FP4, IS_W1, N>(p, units, a.G, passes, stream)            \
                   : launch<MFMA_FMT_FP8, IS_W1, N>(p, units, a.G, passes, stream);
    MOE_GEMM_CASE(1)
    MOE_GEMM_CASE(2)
    MOE_GEMM_CASE(4)
#undef MOE_GEMM_CASE
    return -1;
}

}  // namespace

int moe_launch_grouped_w1(const GemmArgs& a, hipStream_t stream) { return launch_grouped<true>(a, stream); }
int moe_launch_grouped_w2(const GemmArgs& a, hipStream_t stream) { return launch_grouped<false>(a, stream); }
