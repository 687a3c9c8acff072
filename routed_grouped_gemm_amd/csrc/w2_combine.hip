// S6 + S7 in one launch for decode batches of at most 16 tokens: grouped W2
// and the combine, by column ownership. (FlashDMoE page, abstract: dispatch,
// compute and combine in one persistent kernel; GC-MoE page, "Approach": the
// finalize role combines the BF16 fragments into token order.)
//
// Workgroup cb owns output columns [32 cb, 32 cb + 32) (half of a 64-row W2
// weight unit) for every token. It computes those columns of y for every
// active group, stages them in LDS as BF16, and then forms each token's sum
// over its local slots in slot order in fp64 with one rounding, exactly as
// the combine kernel does, and writes `out`. No workgroup reads what another
// wrote, so there is no hand-off between workgroups and nothing to wait for.
//
// Every token selects an expert at most once, so with T <= 16 each group has
// at most 16 rows: one 16-row token tile. When few groups are active their
// K is split across the 8 waves (partials summed in LDS in a fixed order);
// otherwise each wave takes whole groups. y is also written to memory (the
// layer's y rows, as the separate W2 launch writes them).
#include "gemm_common.h"
#include "gemm_stream.h"

namespace {

constexpr int kOWaves = 8;
constexpr int kOThreads = 64 * kOWaves;
constexpr int kOCols = 32;                  // output columns per workgroup

template <int WFMT>
__global__ __launch_bounds__(kOThreads, 1)
void w2_combine_kernel(KParams p, const int32_t* __restrict__ slot_row, const float* __restrict__ comb_w,
                       int T, int ks, uint16_t* __restrict__ out) {
    const int G = p.G, H = p.N, nkt = p.kt;
    const int cb = blockIdx.x;
    const int u = cb >> 1, t0 = (cb & 1) * 2;           // weight unit, its first 16-row tile
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    float* part = (float*)smem;                                     // [8 items][2 tiles][4][64]
    uint16_t* ylds = (uint16_t*)(part + kOWaves * 512);              // [R_max][32] BF16
    int* act = (int*)(ylds + (size_t)p.R_max * kOCols);             // [G] active groups, then their count

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int q = lane >> 4, r = lane & 15;

    // the active groups in group order (wave 0, one ballot per 64 groups)
    if (w == 0) {
        int n = 0;
        for (int g0 = 0; g0 < G; g0 += 64) {
            const int g = g0 + lane;
            const bool a = g < G && p.counts[g] > 0;
            const uint64_t m = __ballot(a);
            if (a) act[n + __popcll(m & ((1ull << lane) - 1ull))] = g;
            n += __popcll(m);
        }
        if (lane == 0) act[G] = n;
    }
    __syncthreads();
    const int n_act = act[G];
    // K split: the largest power of two S with n_act * S <= 8 work items (1
    // from 5 active groups on, when each wave takes whole groups)
    const int S = n_act >= 5 ? 1 : (n_act >= 3 ? 2 : (n_act == 2 ? 4 : 8));

    constexpr int KB = batch_kt<WFMT, 1>();
    const int nbt = (nkt + KB - 1) / KB;
    const rsrc_t rx = make_rsrc(p.aq, p.aq_bytes);
    const rsrc_t rxs = make_rsrc(p.as, p.as_bytes);
    for (int i = w; i < n_act * S; i += kOWaves) {
        const int ai = i / S, kp = i - ai * S;
        const int g = act[ai];
        const int rows = min(16, p.counts[g]), rbase = p.offsets[g];
        // this item's K-tiles: whole batches (batches start at multiples of KB)
        const int kt0 = ((kp * nbt) / S) * KB, kt1 = min(nkt, (((kp + 1) * nbt) / S) * KB);
        const int sel = g < p.E_loc ? 0 : 1;
        const int gi = g < p.E_loc ? g : 0;
        const uint8_t* wgrp = p.wbase[sel] + gi * p.gstride;
        const rsrc_t rw = make_rsrc(wgrp + (size_t)u * p.dpu, (uint32_t)p.dpu);
        const rsrc_t rs = make_rsrc(wgrp + p.dpg + (size_t)u * p.spu, (uint32_t)p.spu);
        const bool v = r < rows;
        uint32_t xoff[1], xsoff[1];
        xoff[0] = v ? (uint32_t)(rbase + r) * (uint32_t)p.K : kInvalid;
        xsoff[0] = v ? (uint32_t)(rbase + r) * (uint32_t)(p.K / 32) : kInvalid;
        f32x4 acc[1][2];
        acc[0][0] = f32x4{0.f, 0.f, 0.f, 0.f};
        acc[0][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        // two batches requested before either is multiplied (past kt1 the
        // loads read zeros and their products add nothing)
        for (int ktb = kt0; ktb < kt1; ktb += 2 * KB) {
            Batch<WFMT, 1, 2> b0, b1;
            load_batch<WFMT, 1, kNonTemporal, 2>(b0, ktb, kt1, lane, rw, rs, rx, rxs, xoff, xsoff, t0);
            load_batch<WFMT, 1, kNonTemporal, 2>(b1, ktb + KB, kt1, lane, rw, rs, rx, rxs, xoff, xsoff, t0);
            mma_batch<WFMT, 1, 2>(b0, 1, acc);
            if (ktb + KB < kt1) mma_batch<WFMT, 1, 2>(b1, 1, acc);
        }
        // acc[0][t][c] is column 16 t + 4 q + c of the block for row r
        if (S == 1) {
            if (v) {
                #pragma unroll
                for (int t = 0; t < 2; ++t) {
                    uint2 o;
                    o.x = bf16x2(acc[0][t][0], acc[0][t][1]);
                    o.y = bf16x2(acc[0][t][2], acc[0][t][3]);
                    *(uint2*)(ylds + (size_t)(rbase + r) * kOCols + 16 * t + 4 * q) = o;
                }
            }
        } else {
            // at most 8 items: item i is this wave's only one
            #pragma unroll
            for (int t = 0; t < 2; ++t)
                #pragma unroll
                for (int c = 0; c < 4; ++c) part[((i * 2 + t) * 4 + c) * 64 + lane] = acc[0][t][c];
        }
    }
    __syncthreads();
    if (S > 1) {
        // the S partials of each group, in K order
        for (int e = tid; e < n_act * 512; e += kOThreads) {
            const int ai = e >> 9, rem = e & 511;
            const int ln = rem & 63, t = rem >> 8, c = (rem >> 6) & 3;
            float s = 0.f;
            for (int kp = 0; kp < S; ++kp) s += part[(((ai * S + kp) * 2 + t) * 4 + c) * 64 + ln];
            const int g = act[ai];
            const int row = ln & 15;
            if (row < min(16, p.counts[g]))
                ylds[(size_t)(p.offsets[g] + row) * kOCols + 16 * t + 4 * (ln >> 4) + c] =
                    (uint16_t)f32_to_bf16(s);
        }
        __syncthreads();
    }

    // y rows (this block's columns of every grouped row)
    const int R = p.offsets[G];
    for (int e = tid; e < R * (kOCols / 2); e += kOThreads) {
        const int row = e / (kOCols / 2), c2 = e - row * (kOCols / 2);
        *(uint32_t*)(p.y + (size_t)row * H + kOCols * cb + 2 * c2) =
            *(const uint32_t*)(ylds + (size_t)row * kOCols + 2 * c2);
    }
    // the combine of this block's columns: slots in order, fp64, one rounding
    for (int e = tid; e < T * (kOCols / 2); e += kOThreads) {
        const int t = e / (kOCols / 2), c2 = e - t * (kOCols / 2);
        double a0 = 0.0, a1 = 0.0;
        for (int j = 0; j < ks; ++j) {
            const int rr = slot_row[t * ks + j];
            if (rr < 0) continue;
            const double wt = comb_w ? (double)comb_w[rr] : 1.0;
            const uint32_t pr = *(const uint32_t*)(ylds + (size_t)rr * kOCols + 2 * c2);
            a0 += (double)bf16_to_f32(pr & 0xFFFFu) * wt;
            a1 += (double)bf16_to_f32(pr >> 16) * wt;
        }
        *(uint32_t*)(out + (size_t)t * H + kOCols * cb + 2 * c2) = f64_to_bf16(a0) | (f64_to_bf16(a1) << 16);
    }
}

}  // namespace

// Whether moe_layer's W2 and combine run as one launch: at most 16 tokens
// (so at most 16 rows per group), the grouped rows staged within the LDS,
// no kernel family or separate launches forced, and either at most 4 active
// groups expected or at most 8 whose W2 weights are small (active * H * I at
// most 2^24 elements). Each workgroup streams its 32 columns of every active
// group's weights plus all their h rows, on H / 32 workgroups, so the cost
// grows with the active groups' weights: on the decode share (H = 7168,
// I = 2048) one token (0.8 active experts) took 3-5 us against 10.3 us for
// W2 and the combine, eight tokens (7.5 active) 2.8 us more per layer; the
// 16-token, 8-expert case (H = 512, I = 256, all 8 active) 14.3 against
// 15.4 us per layer (same-box A/B).
bool moe_w2_combine_ok(int T, int R_max, int G, int H, int I, int active_hint, uint32_t flags) {
    if (T < 1 || T > 16 || R_max > 1024 || G > 4096) return false;
    if (active_hint > 8 || (active_hint > 4 && (int64_t)active_hint * H * I > ((int64_t)1 << 24))) return false;
    return !(flags & (MOE_LAYER_SEPARATE_KERNELS | MOE_GEMM_STREAMED | MOE_GEMM_TILED | MOE_GEMM_PASS));
}

int moe_launch_w2_combine(const GemmArgs& a, const int32_t* slot_row, const float* comb_w, int T, int ks,
                          uint16_t* out, hipStream_t stream) {
    const KParams p = make_params(a, false);
    const size_t lds = (size_t)kOWaves * 512 * 4 + (size_t)a.R_max * kOCols * 2 + (size_t)(a.G + 1) * 4;
    const dim3 grid((unsigned)(a.N / kOCols));
    if (a.fmt == MOE_FMT_MXFP4)
        hipLaunchKernelGGL(w2_combine_kernel<MFMA_FMT_FP4>, grid, dim3(kOThreads), lds, stream, p, slot_row, comb_w,
                           T, ks, out);
    else
        hipLaunchKernelGGL(w2_combine_kernel<MFMA_FMT_FP8>, grid, dim3(kOThreads), lds, stream, p, slot_row, comb_w,
                           T, ks, out);
    return (int)hipGetLastError();
}
