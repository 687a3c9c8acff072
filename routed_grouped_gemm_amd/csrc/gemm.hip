// S4-S6: grouped W1 (with the fused SwiGLU * w + FP8 requantisation epilogue)
// and grouped W2 (BF16 rows) on gfx950 scaled MFMA.
//
// Operand-swapped tiling (the GC-MoE page's Blackwell path puts the weights in
// the MMA's M slot and the few decode tokens in N, "Key contributions"): the
// prepacked weight tile is the A operand (16 rows x 128 K, streamed straight
// from HBM into registers in one 1-2 KiB burst per wave) and 16 grouped token
// rows are the B operand. A workgroup owns one 64-row weight unit of one group
// (for W1: 32 gate + the matching 32 up rows) and a pass of up to 16*NTT rows
// of that group; its KW waves split K into contiguous runs of 128-wide K-tiles
// and their partial sums are added in LDS in a fixed tree order, so results do
// not depend on scheduling. Group sizes are read from device memory:
// workgroups of empty groups or of passes past a group's end exit at once (no
// host sync; fusion blog, "Removing host-device synchronisation").
//
// Memory pipeline: every operand is read with buffer loads whose resource
// bounds the region, so an access marked invalid (past the wave's K run, past
// the pass's rows) returns zeros without a branch and without memory traffic.
// A wave issues the loads of a batch of KB K-tiles (16 KiB of FP4 weights for
// one token tile) before it waits, and the register budget stays at 128 VGPRs
// so four waves per SIMD overlap one another's loads.
#include <algorithm>

#include "moe_device.h"
#include "moe_internal.h"
#include "gemm_common.h"
#include "gemm_stream.h"
#include "permute_block.h"

namespace {

// Persistent grid: each workgroup walks the work items item = pass * units + u
// (every pass of 16*NTT rows of every group, times the 64-row weight units),
// striding by the grid size; empty groups contribute no items. CP is the
// cache policy of the weight loads: non-temporal when groups mostly fit one
// pass (each weight byte is read once), cached when a group's passes re-read
// its units and can find them in L2. RT (W1 at decode shapes): 0, or the
// lanes per token with which every workgroup first routes and groups the
// tokens itself in LDS (one launch fewer per layer); workgroup 0 also writes
// the routing results to device memory for W2 and the combine. TPI (W2
// only): 4, or 2 for items of half a unit (two of its four 16-row weight
// tiles), twice as many items of half the work, which fill the last round of
// items better when the items are few.
template <int WFMT, bool IS_W1, int NTT, int KW, int CP, int RT = 0, int TPI = 4>
__global__ __launch_bounds__(64 * KW, NTT == 1 ? 4 : 2)   // waves per SIMD: 4 (128 VGPRs) for one token tile
void grouped_gemm_kernel(KParams p) {
    static_assert(TPI == 4 || (TPI == 2 && !IS_W1), "W1 items pair gate and up tiles: whole units");
    constexpr int NT = 64 * KW;
    constexpr int IPU = 4 / TPI;                        // items per unit
    const int rows_per_pass = 16 * NTT;
    const int G = p.G, units = p.N / 64;

    extern __shared__ float lds[];
    int* pass_off = (int*)lds;                          // [G + 1]
    float* red = lds + ((G + 4) & ~3);                  // [KW/2][NTT][4 tiles][4][64 lanes]
    float* hbuf = red + (KW / 2) * NTT * 1024;          // [16*NTT][33]  (W1)

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    // group sizes, offsets, source rows and routing weights: the inputs, or
    // the LDS tables this workgroup builds from the logits
    const int32_t* cnt_tab = p.counts;
    const int32_t* off_tab = p.offsets;
    const int32_t* rsrc_tab = p.row_src;
    const float* roww_tab = p.row_w;
    if constexpr (RT != 0) {
        const int Tk = p.T * p.k_top, s_sh = G - p.E_loc, ks = p.k_top + s_sh;
        int* sidx = (int*)(hbuf + (IS_W1 ? 16 * NTT * 33 : 0));    // [T*k]
        float* sw = (float*)(sidx + Tk);                          // [T*k]
        int* cnt_l = (int*)(sw + Tk);                             // [G]
        int* off_l = cnt_l + G;                                   // [G + 1]
        int* off32_l = off_l + G + 1;                             // [G + 1]
        int* rsrc_l = off32_l + G + 1;                            // [R_max]
        float* roww_l = (float*)(rsrc_l + p.R_max);               // [R_max]
        int* slot_l = (int*)(roww_l + p.R_max);                   // [T * (k + s)]
        int* scr = slot_l + p.T * ks;                             // permute scratch
        const bool lead = blockIdx.x == 0;
        route_block<KW, RT, 256 / RT>(p.logits, p.T, p.E_tot, p.k_top, p.renorm != 0, sidx, sw,
                                      lead ? p.topk_idx : nullptr, p.topk_w);
        __syncthreads();
        permute_in_block<KW>([&](int a) { return sidx[a]; }, [&](int a) { return sw[a]; },
                             p.T, p.k_top, p.e0, p.E_loc, s_sh, cnt_l, off_l, off32_l, rsrc_l, roww_l,
                             slot_l, scr);
        __syncthreads();
        if (lead) {
            const int R = off_l[G];
            for (int i = tid; i < G; i += NT) const_cast<int32_t*>(p.counts)[i] = cnt_l[i];
            for (int i = tid; i <= G; i += NT) {
                const_cast<int32_t*>(p.offsets)[i] = off_l[i];
                if (p.offsets32) const_cast<int32_t*>(p.offsets32)[i] = off32_l[i];
            }
            for (int i = tid; i < R; i += NT) {
                const_cast<int32_t*>(p.row_src)[i] = rsrc_l[i];
                const_cast<float*>(p.row_w)[i] = roww_l[i];
            }
            for (int i = tid; i < p.T * ks; i += NT) p.slot_row[i] = slot_l[i];
        }
        cnt_tab = cnt_l; off_tab = off_l; rsrc_tab = rsrc_l; roww_tab = roww_l;
    }
    if (w == 0) pass_prefix(cnt_tab, G, rows_per_pass, lane, pass_off);
    __syncthreads();
    const int n_items = pass_off[G] * units * IPU;

    const rsrc_t rx = make_rsrc(p.aq, p.aq_bytes);
    const rsrc_t rxs = make_rsrc(p.as, p.as_bytes);
    // this wave's contiguous run of K-tiles, in whole batches (batches of KB
    // K-tiles start at multiples of KB, and KB divides 4)
    constexpr int KB = Batch<WFMT, NTT, TPI>::KB;
    const int nbt = (p.kt + KB - 1) / KB;
    const int kt0 = ((w * nbt) / KW) * KB, kt1 = min(p.kt, (((w + 1) * nbt) / KW) * KB);

    for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
        const int pg = item / (units * IPU), ui = item - pg * units * IPU;
        const int u = ui / IPU, t0 = (ui - u * IPU) * TPI;     // unit, its first tile of this item
        // the largest g with pass_off[g] <= pg: the count of such g, less
        // one (pass_off is non-decreasing), one ballot per 64 groups
        int ng = 0;
        for (int g0 = 0; g0 < G; g0 += 64)
            ng += __popcll(__ballot(g0 + lane < G && pass_off[g0 + lane] <= pg));
        const int g = ng - 1, pass = pg - pass_off[g];
        const int n_g = cnt_tab[g];
        const int sel = g < p.E_loc ? 0 : 1;
        const int gi = g < p.E_loc ? g : 0;
        const uint8_t* wgrp = p.wbase[sel] + gi * p.gstride;
        const rsrc_t rw = make_rsrc(wgrp + u * p.dpu, (uint32_t)p.dpu);
        const rsrc_t rs = make_rsrc(wgrp + p.dpg + u * p.spu, (uint32_t)p.spu);
        const int rbase = off_tab[g] + pass * rows_per_pass;
        const int nrows = min(rows_per_pass, n_g - pass * rows_per_pass);
        const int ntt_active = (nrows + 15) / 16;

        f32x4 acc[NTT][TPI];
        uint32_t xoff[NTT], xsoff[NTT];
        #pragma unroll
        for (int tt = 0; tt < NTT; ++tt) {
            #pragma unroll
            for (int t = 0; t < TPI; ++t) acc[tt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
            const int r = tt * 16 + (lane & 15);
            const long xr = r < nrows ? (rsrc_tab ? (long)rsrc_tab[rbase + r] : (long)(rbase + r)) : -1;
            xoff[tt] = xr >= 0 ? (uint32_t)(xr * p.K) : kInvalid;
            xsoff[tt] = xr >= 0 ? (uint32_t)(xr * (p.K / 32)) : kInvalid;
        }

        for (int ktb = kt0; ktb < kt1; ktb += KB) {
            Batch<WFMT, NTT, TPI> b;
            load_batch<WFMT, NTT, CP, TPI>(b, ktb, kt1, lane, rw, rs, rx, rxs, xoff, xsoff, t0);
            mma_batch<WFMT, NTT, TPI>(b, ntt_active, acc);
        }

        // Sum the KW waves' partials in a fixed tree order through KW/2 LDS
        // slots: in the round of half-width h, waves [h, 2h) store, waves
        // [0, h) add; the total ends up in wave 0 and is stored to slot 0.
        auto slot = [&](int s_, int tt, int t, int v) -> float& {
            return red[(((s_ * NTT + tt) * TPI + t) * 4 + v) * 64 + lane];
        };
        #pragma unroll
        for (int h = KW / 2; h >= 1; h >>= 1) {
            if (w >= h && w < 2 * h) {
                #pragma unroll
                for (int tt = 0; tt < NTT; ++tt)
                    #pragma unroll
                    for (int t = 0; t < TPI; ++t)
                        #pragma unroll
                        for (int v = 0; v < 4; ++v) slot(w - h, tt, t, v) = acc[tt][t][v];
            }
            __syncthreads();
            if (w < h) {
                #pragma unroll
                for (int tt = 0; tt < NTT; ++tt)
                    #pragma unroll
                    for (int t = 0; t < TPI; ++t)
                        #pragma unroll
                        for (int v = 0; v < 4; ++v) acc[tt][t][v] += slot(w, tt, t, v);
            }
            __syncthreads();
        }
        if (w == 0) {
            #pragma unroll
            for (int tt = 0; tt < NTT; ++tt)
                #pragma unroll
                for (int t = 0; t < TPI; ++t)
                    #pragma unroll
                    for (int v = 0; v < 4; ++v) slot(0, tt, t, v) = acc[tt][t][v];
        }
        __syncthreads();

        if (IS_W1) {
            const int I = p.N / 2;
            // gate/up pairs -> h (fp32) in LDS, [token][feature of this unit]
            for (int e = tid; e < NTT * 512; e += NT) {
                const int le = e & 63, v = (e >> 6) & 3, gt = (e >> 8) & 1, tt = e >> 9;
                const int tok = tt * 16 + (le & 15);
                if (tok >= nrows) continue;
                const float gsum = red[((tt * 4 + gt) * 4 + v) * 64 + le];
                const float usum = red[((tt * 4 + gt + 2) * 4 + v) * 64 + le];
                const int f = gt * 16 + 4 * (le >> 4) + v;
                const float wgt = p.use_w ? roww_tab[rbase + tok] : 1.0f;
                if (p.generic) {
                    // epilogue variant: bias, BF16 pre-activation copy, clamp, activation
                    const int feat = 32 * u + f;
                    float gz = gsum, uz = usum;
                    if (p.bias) {
                        gz += p.bias[(size_t)g * 2 * I + feat];
                        uz += p.bias[(size_t)g * 2 * I + I + feat];
                    }
                    if (p.save_pre) {
                        uint16_t* pr = p.save_pre + (size_t)(rbase + tok) * 2 * I;
                        pr[feat] = (uint16_t)f32_to_bf16(gz);
                        pr[I + feat] = (uint16_t)f32_to_bf16(uz);
                    }
                    if (p.limit > 0.f) {
                        gz = fminf(fmaxf(gz, -p.limit), p.limit);
                        uz = fminf(fmaxf(uz, -p.limit), p.limit);
                    }
                    hbuf[tok * 33 + f] = act_value(gz, p.act, p.beta) * uz * wgt;
                } else {
                    hbuf[tok * 33 + f] = silu(gsum) * usum * wgt;
                }
            }
            __syncthreads();
            // row-wise MX-E4M3 quantisation: 32 threads per token (one 32-block;
            // the amax over the half wave with DPP and a row swap, the bytes
            // of a quad gathered with quad broadcasts)
            for (int t0 = 0; t0 < rows_per_pass; t0 += NT / 32) {
                const int tok = t0 + (tid >> 5), f = tid & 31;
                const bool valid = tok < nrows;
                const float h = valid ? hbuf[tok * 33 + f] : 0.f;
                uint32_t ab = row16_umax(__float_as_uint(fabsf(h)));
                const auto sw = __builtin_amdgcn_permlane16_swap(ab, ab, false, false);
                ab = max(sw[0], sw[1]);
                const uint32_t code = e4m3_scale_code(__uint_as_float(ab), p.ceil_rule);
                const uint32_t qb = f32_to_e4m3(h * inv_scale(code));
                const uint32_t b1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)qb, 0x55, 0xF, 0xF, true);
                const uint32_t b2 = (uint32_t)__builtin_amdgcn_mov_dpp((int)qb, 0xAA, 0xF, 0xF, true);
                const uint32_t b3 = (uint32_t)__builtin_amdgcn_mov_dpp((int)qb, 0xFF, 0xF, 0xF, true);
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
                for (int it = 0; it < 32 * (rows_per_pass / 32); it += NT / 32) {
                    const int pr = it + (tid >> 5);
                    const int f = pr & 31, tb = pr >> 5;
                    const int tok = tb * 32 + (tid & 31);
                    const float h = tok < nrows ? hbuf[tok * 33 + f] : 0.f;
                    float amax = fabsf(h);
                    #pragma unroll
                    for (int m = 16; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
                    const uint32_t code = e4m3_scale_code(amax, p.ceil_rule);
                    const uint32_t qb = tok < nrows ? f32_to_e4m3(h * inv_scale(code)) : 0u;
                    if (pr < 32 * (rows_per_pass / 32) && tb * 32 < ncols) {
                        const size_t frow = (size_t)(32 * u + f);
                        p.hTq[frow * p.ldT + col0 + tok] = (uint8_t)qb;
                        if ((tid & 31) == 0) p.hTs[frow * (p.ldT / 32) + (col0 >> 5) + tb] = (uint8_t)code;
                    }
                }
            }
        } else {
            const int H = p.N;
            for (int e = tid; e < NTT * 64 * TPI; e += NT) {
                const int le = e & 63, t = (e >> 6) % TPI, tt = e / (64 * TPI);
                const int tok = tt * 16 + (le & 15);
                if (tok >= nrows) continue;
                float s[4];
                #pragma unroll
                for (int v = 0; v < 4; ++v) s[v] = red[((tt * TPI + t) * 4 + v) * 64 + le];
                uint2 o;
                o.x = f32_to_bf16(s[0]) | (f32_to_bf16(s[1]) << 16);
                o.y = f32_to_bf16(s[2]) | (f32_to_bf16(s[3]) << 16);
                *(uint2*)(p.y + (size_t)(rbase + tok) * H + 64 * u + 16 * (t0 + t) + 4 * (le >> 4)) = o;
            }
        }
        __syncthreads();
    }
}

// LDS ints of the routing tables of a W1 launch that routes its own tokens
inline size_t route_lds_ints(const KParams& p, int KW) {
    const int s = p.G - p.E_loc, Tk = p.T * p.k_top;
    return (size_t)2 * Tk + p.G + 2 * (p.G + 1) + 2 * (size_t)p.R_max + (size_t)p.T * (p.k_top + s) +
           block_lds_ints(KW, p.G, p.E_loc);
}

template <int WFMT, bool IS_W1, int NTT, int KW, int CP, int RT = 0, int TPI = 4>
int launch(const KParams& p, long max_items, hipStream_t stream) {
    auto kern = grouped_gemm_kernel<WFMT, IS_W1, NTT, KW, CP, RT, TPI>;
    const size_t lds = (size_t)((p.G + 4) & ~3) * 4 + (size_t)(KW / 2) * NTT * 1024 * 4 +
                       (IS_W1 ? (size_t)16 * NTT * 33 * 4 : 0) + (RT ? route_lds_ints(p, KW) * 4 : 0);
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 64 * KW, lds) != hipSuccess || per_cu < 1)
        per_cu = 1;
    const long grid = std::max<long>(1, std::min<long>(max_items * (4 / TPI), (long)per_cu * device_cu_count()));
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * KW), lds, stream, p);
    return (int)hipGetLastError();
}

// 16 K-split waves only with one token tile: 1024-thread workgroups get 128
// VGPRs, too few for more; 2 only with one token tile as well
template <int WFMT, bool IS_W1, int NTT, int CP, int RT = 0, int TPI = 4>
int launch_kw(const KParams& p, int kw, long max_items, hipStream_t stream) {
    if constexpr (NTT == 1 && TPI == 4)
        if (kw >= 16) return launch<WFMT, IS_W1, NTT, 16, CP, RT>(p, max_items, stream);
    if (kw >= 8) return launch<WFMT, IS_W1, NTT, 8, CP, RT, TPI>(p, max_items, stream);
    if constexpr (NTT == 1)
        if (kw <= 2) return launch<WFMT, IS_W1, NTT, 2, CP, RT, TPI>(p, max_items, stream);
    return launch<WFMT, IS_W1, NTT, 4, CP, RT, TPI>(p, max_items, stream);
}

constexpr int kTiledMinRows = 96;   // expected rows per group from which the tiled kernel runs
// tokens a W1 launch routes itself, at most: every workgroup routes all of
// them, so the saving of a launch turns into a loss from about 32 tokens on
// (measured on the decode share: 12 tokens 58.3 -> 56.5 us, 16 tokens
// unchanged; 16 tokens of the 8-expert case 16.3 -> 15.5 us)
constexpr int kRouteMaxT = 16;

// expected rows per group, as the launch sees them
inline int expected_rows(int rows_hint, int R_max, int G) { return rows_hint > 0 ? rows_hint : R_max / G; }

template <bool IS_W1>
int launch_grouped(const GemmArgs& a, hipStream_t stream) {
    if (a.G == 0 || a.R_max == 0) return 0;
    // token tiles per pass, from the expected rows per group
    const int avg = expected_rows(a.rows_hint, a.R_max, a.G);
    // many rows per group: the weights are reused across many token tiles and
    // the MFMA, not HBM, is the bound -> the LDS-tiled kernel (unless the
    // caller asked for one family)
    const bool tiled = (a.flags & MOE_GEMM_TILED) ||
                       (!(a.flags & MOE_GEMM_STREAMED) && avg >= kTiledMinRows);
    if (tiled) {
        if (IS_W1 && a.route) return (int)hipErrorInvalidValue;      // never routes: see moe_w1_can_route
        return IS_W1 ? moe_launch_tiled_w1(a, stream) : moe_launch_tiled_w2(a, stream);
    }
    KParams p = make_params(a, IS_W1);
    // groups of 16 or more rows: their weight units are read by several
    // passes and every unit reads the pass's rows -> the pass-resident
    // kernel with 32-row passes (measured on the full-expert shape, 16 rows
    // per group expected: 16-row passes 349 us, 32-row 286 us, 64-row 311
    // us per layer)
    if (!a.route && !(a.flags & MOE_GEMM_STREAMED) && ((a.flags & MOE_GEMM_PASS) || avg >= 16)) {
        int nt = avg >= 16 || p.transpose ? 2 : 1;   // 32-token blocks of the transposed copy: whole passes
        if (nt == 2 && !p.transpose && !moe_pass_fits(a.K, a.G, 2, a.fmt)) nt = 1;
        if (moe_pass_fits(a.K, a.G, nt, a.fmt)) return moe_launch_pass(a, IS_W1, nt, stream);
    }
    int ntt = avg <= 16 ? 1 : (avg <= 32 ? 2 : 4);
    if (p.transpose && ntt < 2) ntt = 2;       // 32-token blocks must not straddle passes
    const int units = a.N / 64;
    const int rpp = 16 * ntt;
    // items never exceed units * (R_max / rpp + G): each group adds at most one partial pass
    const long max_items = (long)units * ((long)a.R_max / rpp + a.G);
    // K-split waves per workgroup. W2 (the shorter K = I, where wider splits
    // cost more in the reduction than they gain): enough waves for two per
    // SIMD, but never 16 (slower even with a single token); with one token
    // tile and at least 1024 items, 2 (eight small workgroups per CU, so one
    // item's start and end overlap seven others: T = 32 95.5 -> 94.2 us on
    // the decode share, same-box A/B). W1 with one token tile: 16 waves per
    // CU whatever the split, so a round of items covers cus * 16 / kw of
    // them, each in about 1/kw of the time of a one-wave item; the split with
    // the fewest kw-weighted rounds leaves the least of the last, partly idle
    // round (ties: fewer waves), but from four items per CU on two waves
    // (T = 32 and 128: W1 launch rate 5.48 -> 5.63 TB/s).
    const long active = a.active_hint > 0 ? a.active_hint
                        : std::min<long>(a.G, std::max<long>(1, a.R_max / std::max(avg, 1)));
    const long items = active * units * std::max(1, (avg + rpp - 1) / rpp);
    int kw = !IS_W1 && ntt == 1 && items * 2 >= 2048 ? 2 : (items * 4 >= 2048 ? 4 : (items * 8 >= 2048 || !IS_W1 ? 8 : 16));
    if (IS_W1 && ntt == 1) {
        const long cus = device_cu_count();
        double best = 1e30;
        for (int c : {2, 4, 8, 16}) {
            const long slots = cus * (16 / c);
            const double t = (double)((items + slots - 1) / slots) / c;
            if (t < best - 1e-9) { best = t; kw = c; }
        }
        // from four items per CU on, two-wave workgroups, whatever the
        // rounds say (T = 32 of the decode share: 94.6 -> 93.9 us)
        if (items >= 4 * cus) kw = 2;
    }
    kw = std::min(kw, std::max(ntt == 1 ? 2 : 4, p.kt));     // no more waves than K-tiles
    if (ntt > 1) kw = std::min(kw, 8);          // 1024-thread workgroups get 128 VGPRs: too few
    // weights stay in L2 (cached loads) when a typical group needs more than
    // one pass, so that its other passes re-read them there; otherwise they
    // stream through non-temporally
    const bool reread = ntt > 1 || avg >= rpp;
    const bool fp4 = a.fmt == MOE_FMT_MXFP4;
    // W2 streaming its weights once: items of half a unit, each done in
    // about half the time, when whole units would not fill one round of
    // workgroups or when the halves' rounds take less time than the whole
    // units' rounds, so that the last round leaves less of the chip idle.
    // Measured on the decode share (same-box A/B): one token, W2 7.3 -> 6.4
    // us; eight tokens (about 840 units), layer 45.1 -> 43.8 us; T = 32
    // (2285 units on two-wave workgroups, 2048 slots: 1.5 rounds of halves
    // against 2 of whole units) halves faster; T = 128 (3528 units, 2 rounds
    // either way) whole units 1.0 us faster.
    if constexpr (!IS_W1) if (ntt == 1 && !reread) {
        const long slots = (long)device_cu_count() * (16 / kw);
        const long r_whole = (items + slots - 1) / slots, r_half = (2 * items + slots - 1) / slots;
        if (items <= slots || r_half < 2 * r_whole)
            return fp4 ? launch_kw<MFMA_FMT_FP4, IS_W1, 1, kNonTemporal, 0, 2>(p, kw, max_items, stream)
                       : launch_kw<MFMA_FMT_FP8, IS_W1, 1, kNonTemporal, 0, 2>(p, kw, max_items, stream);
    }
    if constexpr (IS_W1) if (a.route) {
        // the layer skipped its routing launches: moe_w1_can_route held, so
        // ntt == 1 and the weights stream non-temporally
        if (ntt != 1 || reread) return (int)hipErrorInvalidValue;
        const bool wide = a.route->T <= kw;     // one token per wave per round
        if (fp4) return wide ? launch_kw<MFMA_FMT_FP4, IS_W1, 1, kNonTemporal, 64>(p, kw, max_items, stream)
                             : launch_kw<MFMA_FMT_FP4, IS_W1, 1, kNonTemporal, 16>(p, kw, max_items, stream);
        return wide ? launch_kw<MFMA_FMT_FP8, IS_W1, 1, kNonTemporal, 64>(p, kw, max_items, stream)
                    : launch_kw<MFMA_FMT_FP8, IS_W1, 1, kNonTemporal, 16>(p, kw, max_items, stream);
    }
#define MOE_GEMM_CASE(N, CP)                                                                      \
    return fp4 ? launch_kw<MFMA_FMT_FP4, IS_W1, N, CP>(p, kw, max_items, stream)                  \
               : launch_kw<MFMA_FMT_FP8, IS_W1, N, CP>(p, kw, max_items, stream);
    if (ntt == 1) {
        if (reread) { MOE_GEMM_CASE(1, 0) }
        MOE_GEMM_CASE(1, kNonTemporal)
    }
    if (ntt == 2) { MOE_GEMM_CASE(2, 0) }
    MOE_GEMM_CASE(4, 0)
#undef MOE_GEMM_CASE
}

}  // namespace

int moe_launch_grouped_w1(const GemmArgs& a, hipStream_t stream) { return launch_grouped<true>(a, stream); }

// Whether launch_grouped runs these arguments on the LDS-tiled kernel.
bool moe_grouped_uses_tiled(const GemmArgs& a) {
    const int avg = expected_rows(a.rows_hint, a.R_max, a.G);
    return (a.flags & MOE_GEMM_TILED) || (!(a.flags & MOE_GEMM_STREAMED) && avg >= kTiledMinRows);
}

// The conditions under which launch_grouped<true> takes the one-token-tile,
// non-temporal path, plus the limits of the in-workgroup routing (at most
// 256 experts, k <= 16, T <= 16 tokens, at most 513 groups).
bool moe_w1_can_route(int T, int E_tot, int k, int E_loc, int s, int R_max, int H, int I,
                      int rows_hint, uint32_t flags) {
    (void)H; (void)I;
    const int G = E_loc + s;
    if (T < 1 || T > kRouteMaxT || E_tot > 256 || k > 16 || G > 513 || G < 1) return false;
    if (flags & (MOE_W1_WRITE_TRANSPOSE | MOE_GEMM_TILED)) return false;
    const int avg = expected_rows(rows_hint, R_max, G);
    return avg < 16;
}
int moe_launch_grouped_w2(const GemmArgs& a, hipStream_t stream) { return launch_grouped<false>(a, stream); }
