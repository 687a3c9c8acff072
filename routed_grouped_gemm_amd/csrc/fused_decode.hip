// The whole layer in one persistent launch, for decode batches of at most 8
// tokens (the FlashDMoE page's abstract: dispatch, expert computation and
// combine fused into a single persistent kernel, with no launches between
// the phases; the GC-MoE page's "Key contributions": W2 work waits on a
// completion record of W1 rather than on a kernel boundary).
//
// Every workgroup first routes and groups the tokens itself in LDS (the
// in-workgroup router and grouping of the W1 launch of the separate-kernel
// path); workgroup 0 also writes the routing results to the workspace. Then
// the workgroups take work items from a device ticket counter, in this order:
//   W1 items (active group, 64-row W1 unit): h of the group's rows for the
//     unit's 32 features, SwiGLU (or the epilogue variant) and the routing
//     weight fused, requantised to MX-E4M3, stored; then the group's
//     completion count goes up by one;
//   W2 items (active group, 64 output columns): wait until the group's count
//     reaches the number of W1 units, then y = h . W2^T for those columns,
//     BF16, stored; the column block's arrival count goes up by one, and the
//     item that completes the block (the last of the active groups) sums the
//     BF16 rows of every token's slots, in slot order, in fp64, into `out`.
// Tickets are claimed in increasing order, so every W1 item is held by a
// running workgroup before any W2 item is: a wait is always on work that is
// in progress, whatever number of workgroups the GPU runs at once.
//
// Hand-off without L2 write-back: the data passed between workgroups (h and
// its scales, the BF16 rows y) is stored and loaded with the agent-coherent
// cache policy (sc1, as for agent-scope atomics), so it does not sit in one
// XCD's L2; each workgroup waits for its stores before its counter update,
// and the counters are relaxed device-scope atomics. Waits poll with a
// bound: a wait that runs out sets the control block's error word and lets
// the workgroup go on (the results are then wrong, and the word says so).
//
// The control block in the workspace carries a magic value once initialised;
// its counters are back at zero when a launch ends (the last workgroup to
// leave resets them), so the next launch finds them ready. A workspace whose
// block was never initialised is initialised by workgroup 0 at the start
// while the others wait for the magic value.
#include <algorithm>

#include "gemm_common.h"
#include "gemm_stream.h"
#include "permute_block.h"

namespace {

constexpr int kFW = 16;                      // waves per workgroup (K split)
constexpr int kFT = 64 * kFW;
constexpr int kCoherent = 16;                // sc1: agent-coherent loads and stores
constexpr int kWaitMs = 100;                 // a wait gives up after this long (wall clock)
constexpr uint32_t kMagicLo = 0x4D6F4521u, kMagicHi = 0x7C3A9E55u;
constexpr bool kFusedEnabled = false;

// control block words: magic (2), error, ticket, exit count, the word a
// timed-out wait watched and the value it last saw, then per group the W1
// units done, then per 64-column block the W2 arrivals. Error codes: 1 = the
// wait for the block's initialisation, 2 = a W2 item's wait for its group.
enum { kCtlMagicLo = 0, kCtlMagicHi = 1, kCtlErr = 2, kCtlTick = 3, kCtlExit = 4, kCtlWhere = 5,
       kCtlSeen = 6, kCtlDone = 8 };

struct FusedArgs {
    KParams p1, p2;                          // the W1 and W2 parameter blocks (p2.aq/as: h)
    uint32_t* ctrl;
    uint16_t* out;                           // [T, H] bf16
    int units2;                              // H / 64
    int weight_at_combine;
    uint64_t wait_ticks;                     // kWaitMs in wall-clock ticks
};

MOE_DEV uint32_t ld_coherent(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
MOE_DEV void st_coherent(uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until ctrl[idx] >= target (thread 0 of the workgroup), for at most
// `ticks` of the constant-rate wall clock; on a timeout record the error
// code, the word and its last value, and return (so the launch always ends).
MOE_DEV void wait_at_least(uint32_t* ctrl, int idx, uint32_t target, uint64_t ticks, uint32_t code) {
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    for (;;) {
        const uint32_t v = ld_coherent(ctrl + idx);
        if (v >= target || ld_coherent(ctrl + kCtlErr) != 0) return;
        if (__builtin_amdgcn_s_memrealtime() - t0 > ticks) {
            st_coherent(ctrl + kCtlWhere, (uint32_t)idx);
            st_coherent(ctrl + kCtlSeen, v);
            st_coherent(ctrl + kCtlErr, code);
            return;
        }
        __builtin_amdgcn_s_sleep(8);
    }
}

// Sum of the KW waves' partials through KW/2 LDS slots in a fixed tree order;
// the total ends up in slot 0 (as in the decode-shaped GEMM kernel).
template <int KW>
MOE_DEV void reduce_waves(float* red, f32x4 (&acc)[4], int w, int lane) {
    auto slot = [&](int s_, int t, int v) -> float& { return red[((s_ * 4 + t) * 4 + v) * 64 + lane]; };
    #pragma unroll
    for (int h = KW / 2; h >= 1; h >>= 1) {
        if (w >= h && w < 2 * h) {
            #pragma unroll
            for (int t = 0; t < 4; ++t)
                #pragma unroll
                for (int v = 0; v < 4; ++v) slot(w - h, t, v) = acc[t][v];
        }
        __syncthreads();
        if (w < h) {
            #pragma unroll
            for (int t = 0; t < 4; ++t)
                #pragma unroll
                for (int v = 0; v < 4; ++v) acc[t][v] += slot(w, t, v);
        }
        __syncthreads();
    }
    if (w == 0) {
        #pragma unroll
        for (int t = 0; t < 4; ++t)
            #pragma unroll
            for (int v = 0; v < 4; ++v) slot(0, t, v) = acc[t][v];
    }
    __syncthreads();
}

// One wave's share of unit `wu` (prepacked weights at wunit, scales at sunit)
// against the 16-row token tile whose rows start at byte xoff of rx (kInvalid:
// past the rows), K-tiles split evenly over the KW waves in batches of KB.
template <int WFMT, int KB, int XCP>
MOE_DEV void unit_dot(const KParams& p, const uint8_t* wunit, const uint8_t* sunit, rsrc_t rx, rsrc_t rxs,
                      uint32_t xoff, uint32_t xsoff, int w, int lane, f32x4 (&acc)[4]) {
    #pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    const rsrc_t rw = make_rsrc(wunit, (uint32_t)p.dpu);
    const rsrc_t rs = make_rsrc(sunit, (uint32_t)p.spu);
    const int nbt = (p.kt + KB - 1) / KB;
    const int kt0 = ((w * nbt) / kFW) * KB, kt1 = min(p.kt, (((w + 1) * nbt) / kFW) * KB);
    const uint32_t xo[1] = {xoff}, xso[1] = {xsoff};
    f32x4 a2[1][4];
    #pragma unroll
    for (int t = 0; t < 4; ++t) a2[0][t] = acc[t];
    for (int ktb = kt0; ktb < kt1; ktb += KB) {
        Batch<WFMT, 1, 4, KB> b;
        load_batch<WFMT, 1, kNonTemporal, 4, KB, XCP>(b, ktb, kt1, lane, rw, rs, rx, rxs, xo, xso);
        mma_batch<WFMT, 1, 4, KB>(b, 1, a2);
    }
    #pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = a2[0][t];
}

template <int WFMT, int RT>
__global__ __launch_bounds__(kFT, 4)
void fused_decode_kernel(FusedArgs f) {
    const KParams& p = f.p1;
    const int G = p.G, T = p.T, k = p.k_top, s_sh = G - p.E_loc, ks = k + s_sh, Tk = T * k;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int units1 = p.N / 64, units2 = f.units2, I = p.N / 2, H = f.p2.N;
    uint32_t* ctrl = f.ctrl;

    extern __shared__ float lds[];
    float* red = lds;                                         // [8][4 tiles][4][64]
    float* hbuf = red + (kFW / 2) * 1024;                     // [16][33]
    int* misc = (int*)(hbuf + 16 * 33);                       // [8]: ticket, flags, active count
    int* act_l = misc + 8;                                    // [G] active groups
    int* sidx = act_l + G;                                    // [T*k]
    float* sw = (float*)(sidx + Tk);                          // [T*k]
    int* cnt_l = (int*)(sw + Tk);                             // [G]
    int* off_l = cnt_l + G;                                   // [G + 1]
    int* off32_l = off_l + G + 1;                             // [G + 1]
    int* rsrc_l = off32_l + G + 1;                            // [R_max]
    float* roww_l = (float*)(rsrc_l + p.R_max);               // [R_max]
    int* slot_l = (int*)(roww_l + p.R_max);                   // [T * ks]
    int* scr = slot_l + T * ks;                               // grouping scratch

    // ---- routing and grouping, every workgroup on its own
    const bool lead = blockIdx.x == 0;
    route_block<kFW, RT, 256 / RT>(p.logits, T, p.E_tot, k, p.renorm != 0, sidx, sw,
                                   lead ? p.topk_idx : nullptr, p.topk_w);
    __syncthreads();
    permute_in_block<kFW>([&](int a) { return sidx[a]; }, [&](int a) { return sw[a]; }, T, k, p.e0,
                          p.E_loc, s_sh, cnt_l, off_l, off32_l, rsrc_l, roww_l, slot_l, scr);
    __syncthreads();
    if (lead) {
        const int R = off_l[G];
        for (int i = tid; i < G; i += kFT) const_cast<int32_t*>(p.counts)[i] = cnt_l[i];
        for (int i = tid; i <= G; i += kFT) {
            const_cast<int32_t*>(p.offsets)[i] = off_l[i];
            if (p.offsets32) const_cast<int32_t*>(p.offsets32)[i] = off32_l[i];
        }
        for (int i = tid; i < R; i += kFT) {
            const_cast<int32_t*>(p.row_src)[i] = rsrc_l[i];
            const_cast<float*>(p.row_w)[i] = roww_l[i];
        }
        for (int i = tid; i < T * ks; i += kFT) p.slot_row[i] = slot_l[i];
    }
    // the active groups in ascending order (wave 0, 64 groups per ballot)
    if (w == 0) {
        int base = 0;
        for (int g0 = 0; g0 < G; g0 += 64) {
            const int g = g0 + lane;
            const bool has = g < G && cnt_l[g] > 0;
            const uint64_t m = __ballot(has);
            if (has) act_l[base + __popcll(m & lanemask_lt(lane))] = g;
            base += __popcll(m);
        }
        if (lane == 0) misc[2] = base;
    }
    // ---- control block: ready (magic) before any counter is touched; the
    // magic value carries the block's shape, so a block left by a layer of
    // another shape is initialised again
    const uint32_t magic_hi = kMagicHi ^ ((uint32_t)G << 12) ^ (uint32_t)units2;
    if (tid == 0) {
        const bool ready = ld_coherent(ctrl + kCtlMagicLo) == kMagicLo && ld_coherent(ctrl + kCtlMagicHi) == magic_hi;
        if (!ready) {
            if (lead) {
                for (int i = kCtlErr; i < kCtlDone + G + units2; ++i) st_coherent(ctrl + i, 0);
                __builtin_amdgcn_s_waitcnt(0);
                st_coherent(ctrl + kCtlMagicHi, magic_hi);
                __builtin_amdgcn_s_waitcnt(0);
                st_coherent(ctrl + kCtlMagicLo, kMagicLo);
            } else {
                const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
                for (;;) {
                    if (ld_coherent(ctrl + kCtlMagicLo) == kMagicLo && ld_coherent(ctrl + kCtlMagicHi) == magic_hi) break;
                    if (__builtin_amdgcn_s_memrealtime() - t0 > f.wait_ticks) {
                        st_coherent(ctrl + kCtlWhere, kCtlMagicLo);
                        st_coherent(ctrl + kCtlSeen, ld_coherent(ctrl + kCtlMagicLo));
                        st_coherent(ctrl + kCtlErr, 1);
                        break;
                    }
                    __builtin_amdgcn_s_sleep(8);
                }
            }
        }
    }
    __syncthreads();
    const int n_act = misc[2];
    const int n1 = n_act * units1;
    const int n2 = n_act > 0 ? n_act * units2 : units2;      // with no local rows: zero the output

    const KParams& q = f.p2;
    const uint32_t hq_bytes = (uint32_t)((size_t)p.R_max * I), hs_bytes = (uint32_t)((size_t)p.R_max * (I / 32));

    for (;;) {
        if (tid == 0) misc[0] = (int)__hip_atomic_fetch_add(ctrl + kCtlTick, 1u, __ATOMIC_RELAXED,
                                                            __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        // (compared unsigned: a ticket past the items, whatever its value, ends the loop)
        const uint32_t tu = (uint32_t)misc[0];
        __syncthreads();
        if (tu >= (uint32_t)(n1 + n2)) break;
        const int t = (int)tu;
        f32x4 acc[4];
        if (t < n1) {
            // ---- W1 item: active group g, unit u
            const int g = act_l[t / units1], u = t - (t / units1) * units1;
            const int rbase = off_l[g], nrows = cnt_l[g];
            const int sel = g < p.E_loc ? 0 : 1, gi = g < p.E_loc ? g : 0;
            const uint8_t* wgrp = p.wbase[sel] + gi * p.gstride;
            const int r = lane & 15;
            const uint32_t xr = r < nrows ? (uint32_t)rsrc_l[rbase + r] : 0u;
            const rsrc_t rx = make_rsrc(p.aq, p.aq_bytes), rxs = make_rsrc(p.as, p.as_bytes);
            unit_dot<WFMT, WFMT == MFMA_FMT_FP4 ? 4 : 2, 0>(
                p, wgrp + u * p.dpu, wgrp + p.dpg + u * p.spu, rx, rxs,
                r < nrows ? xr * (uint32_t)p.K : kInvalid, r < nrows ? xr * (uint32_t)(p.K / 32) : kInvalid,
                w, lane, acc);
            reduce_waves<kFW>(red, acc, w, lane);
            // gate/up pairs -> h (fp32) in LDS, [token][feature of this unit]
            for (int e = tid; e < 512; e += kFT) {
                const int le = e & 63, v = (e >> 6) & 3, gt = (e >> 8) & 1;
                const int tok = le & 15;
                if (tok >= nrows) continue;
                const float gsum = red[(gt * 4 + v) * 64 + le];
                const float usum = red[((gt + 2) * 4 + v) * 64 + le];
                const int fi = gt * 16 + 4 * (le >> 4) + v;
                const float wgt = p.use_w ? roww_l[rbase + tok] : 1.0f;
                float hv;
                if (p.generic) {
                    const int feat = 32 * u + fi;
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
                    hv = act_value(gz, p.act, p.beta) * uz * wgt;
                } else {
                    hv = silu(gsum) * usum * wgt;
                }
                hbuf[tok * 33 + fi] = hv;
            }
            __syncthreads();
            // row-wise MX-E4M3 quantisation: 32 threads per token (one 32-block),
            // stored with the agent-coherent policy for the W2 items
            if (tid < 16 * 32) {
                const rsrc_t rhw = make_rsrc(p.hq, hq_bytes), rhsw = make_rsrc(p.hs, hs_bytes);
                const int tok = tid >> 5, fi = tid & 31;
                const bool valid = tok < nrows;
                const float h = valid ? hbuf[tok * 33 + fi] : 0.f;
                float amax = fabsf(h);
                #pragma unroll
                for (int m = 16; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
                const uint32_t code = e4m3_scale_code(amax, p.ceil_rule);
                const uint32_t qb = f32_to_e4m3(h * inv_scale(code));
                const uint32_t b1 = __shfl_down(qb, 1, 64), b2 = __shfl_down(qb, 2, 64), b3 = __shfl_down(qb, 3, 64);
                const uint32_t row = (uint32_t)(rbase + tok);
                __builtin_amdgcn_raw_buffer_store_b32(qb | (b1 << 8) | (b2 << 16) | (b3 << 24), rhw,
                                                      valid && (fi & 3) == 0 ? row * I + 32 * u + fi : kInvalid, 0,
                                                      kCoherent);
                __builtin_amdgcn_raw_buffer_store_b8((unsigned char)code, rhsw,
                                                     valid && fi == 0 ? row * (I / 32) + u : kInvalid, 0, kCoherent);
            }
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (tid == 0)
                __hip_atomic_fetch_add(ctrl + kCtlDone + g, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else if (n_act > 0) {
            // ---- W2 item: active group g, 64 output columns c
            const int t2 = t - n1, ai = t2 / units2, c = t2 - ai * units2;
            const int g = act_l[ai];
            const int rbase = off_l[g], nrows = cnt_l[g];
            if (tid == 0) wait_at_least(ctrl, kCtlDone + g, (uint32_t)units1, f.wait_ticks, 2);
            __syncthreads();
            const int sel = g < q.E_loc ? 0 : 1, gi = g < q.E_loc ? g : 0;
            const uint8_t* wgrp = q.wbase[sel] + gi * q.gstride;
            const int r = lane & 15;
            const uint32_t hr = (uint32_t)(rbase + r);
            const rsrc_t rh = make_rsrc(p.hq, hq_bytes), rhs = make_rsrc(p.hs, hs_bytes);
            unit_dot<WFMT, 1, kCoherent>(q, wgrp + c * q.dpu, wgrp + q.dpg + c * q.spu, rh, rhs,
                                         r < nrows ? hr * (uint32_t)I : kInvalid,
                                         r < nrows ? hr * (uint32_t)(I / 32) : kInvalid, w, lane, acc);
            reduce_waves<kFW>(red, acc, w, lane);
            // BF16 rows of y for these columns
            const rsrc_t ry = make_rsrc(q.y, (uint32_t)((size_t)p.R_max * H * 2));
            if (tid < 4 * 64) {
                const int tt = tid >> 6, le = tid & 63, tok = le & 15;
                const float* sl = red + tt * 4 * 64;
                uint2 o;
                o.x = f32_to_bf16(sl[0 * 64 + le]) | (f32_to_bf16(sl[1 * 64 + le]) << 16);
                o.y = f32_to_bf16(sl[2 * 64 + le]) | (f32_to_bf16(sl[3 * 64 + le]) << 16);
                const uint32_t off = (uint32_t)(((rbase + tok) * H + 64 * c + 16 * tt + 4 * (le >> 4)) * 2);
                __builtin_amdgcn_raw_buffer_store_b32(o.x, ry, tok < nrows ? off : kInvalid, 0, kCoherent);
                __builtin_amdgcn_raw_buffer_store_b32(o.y, ry, tok < nrows ? off + 4 : kInvalid, 0, kCoherent);
            }
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (tid == 0) {
                const uint32_t old = __hip_atomic_fetch_add(ctrl + kCtlDone + G + c, 1u, __ATOMIC_RELAXED,
                                                            __HIP_MEMORY_SCOPE_AGENT);
                misc[1] = old == (uint32_t)(n_act - 1);
            }
            __syncthreads();
            if (misc[1]) {
                // the last group of this column block: combine. Each thread
                // takes 4 columns of one token: BF16 rows of its slots, in slot
                // order, summed in fp64, rounded once.
                for (int e = tid; e < T * 16; e += kFT) {
                    const int tok = e >> 4, c4 = (e & 15) * 4;
                    double a4[4] = {0.0, 0.0, 0.0, 0.0};
                    for (int j = 0; j < ks; ++j) {
                        const int rr = slot_l[tok * ks + j];
                        if (rr < 0) continue;
                        const uint32_t off = (uint32_t)((rr * H + 64 * c + c4) * 2);
                        const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b32(ry, off, 0, kCoherent);
                        const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b32(ry, off + 4, 0, kCoherent);
                        const double wj = f.weight_at_combine ? (double)roww_l[rr] : 1.0;
                        a4[0] += (double)bf16_to_f32(lo & 0xFFFFu) * wj;
                        a4[1] += (double)bf16_to_f32(lo >> 16) * wj;
                        a4[2] += (double)bf16_to_f32(hi & 0xFFFFu) * wj;
                        a4[3] += (double)bf16_to_f32(hi >> 16) * wj;
                    }
                    uint2 o;
                    o.x = f64_to_bf16(a4[0]) | (f64_to_bf16(a4[1]) << 16);
                    o.y = f64_to_bf16(a4[2]) | (f64_to_bf16(a4[3]) << 16);
                    *(uint2*)(f.out + (size_t)tok * H + 64 * c + c4) = o;
                }
            }
        } else {
            // ---- no local rows: output columns of block t - n1 are zero
            const int c = t - n1;
            for (int e = tid; e < T * 16; e += kFT) {
                const int tok = e >> 4, c4 = (e & 15) * 4;
                *(uint2*)(f.out + (size_t)tok * H + 64 * c + c4) = make_uint2(0u, 0u);
            }
        }
    }
    // ---- leave; the last workgroup out resets the counters for the next launch
    __syncthreads();
    if (tid == 0) {
        const uint32_t old = __hip_atomic_fetch_add(ctrl + kCtlExit, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        misc[1] = old == gridDim.x - 1;
    }
    __syncthreads();
    if (misc[1]) {
        for (int i = tid; i < G + units2; i += kFT) st_coherent(ctrl + kCtlDone + i, 0);
        if (tid == 0) {
            st_coherent(ctrl + kCtlTick, 0);
            st_coherent(ctrl + kCtlExit, 0);
        }
    }
}

// The device's constant wall-clock rate in kHz (cached per device; 100 MHz if
// the attribute is unavailable).
int wall_clock_khz() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 100000;
    if (!cached[dev]) {
        int r = 0;
        if (hipDeviceGetAttribute(&r, hipDeviceAttributeWallClockRate, dev) != hipSuccess || r <= 0) r = 100000;
        cached[dev] = r;
    }
    return cached[dev];
}

template <int WFMT, int RT>
int launch_fused(const FusedArgs& f, hipStream_t stream) {
    auto kern = fused_decode_kernel<WFMT, RT>;
    const KParams& p = f.p1;
    const int s = p.G - p.E_loc, Tk = p.T * p.k_top;
    const size_t ints = (size_t)(kFW / 2) * 1024 + 16 * 33 + 8 + p.G + 2 * (size_t)Tk + p.G + 2 * (p.G + 1) +
                        2 * (size_t)p.R_max + (size_t)p.T * (p.k_top + s) + block_lds_ints(kFW, p.G, p.E_loc);
    const size_t lds = ints * 4;
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kFT, lds) != hipSuccess || per_cu < 1)
        per_cu = 1;
    const long grid = (long)per_cu * device_cu_count();
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kFT), lds, stream, f);
    return (int)hipGetLastError();
}

}  // namespace

size_t moe_fused_ctrl_words(int G, int H) { return (size_t)kCtlDone + G + H / 64; }

bool moe_fused_decode_ok(int T, int E_tot, int k, int E_loc, int s, uint32_t flags) {
    // Switched off: on the GPU the first launch of this kernel ran for minutes
    // instead of microseconds (twice, the second time with every wait bounded
    // in wall-clock time); the cause is not established (the hand-off's
    // cross-XCD visibility and the wall clock are the candidates), so every
    // layer takes the separate-kernel path.
    if (!kFusedEnabled) return false;
    const int G = E_loc + s;
    if (T < 1 || T > 8 || E_tot > 256 || k > 16 || G > 513 || G < 1) return false;
    return !(flags & (MOE_W1_WRITE_TRANSPOSE | MOE_GEMM_TILED | MOE_LAYER_SEPARATE_KERNELS));
}

int moe_launch_fused_decode(const GemmArgs& a1, const GemmArgs& a2, uint32_t* ctrl, uint16_t* out,
                            hipStream_t stream) {
    FusedArgs f{};
    f.p1 = make_params(a1, true);
    f.p2 = make_params(a2, false);
    f.ctrl = ctrl;
    f.out = out;
    f.units2 = a2.N / 64;
    f.weight_at_combine = (a1.flags & MOE_WEIGHT_AT_COMBINE) ? 1 : 0;
    f.wait_ticks = (uint64_t)wall_clock_khz() * kWaitMs;
    const bool fp4 = a1.fmt == MOE_FMT_MXFP4;
    const bool wide = a1.route->T <= kFW;   // one token per wave per round
    if (fp4) return wide ? launch_fused<MFMA_FMT_FP4, 64>(f, stream) : launch_fused<MFMA_FMT_FP4, 16>(f, stream);
    return wide ? launch_fused<MFMA_FMT_FP8, 64>(f, stream) : launch_fused<MFMA_FMT_FP8, 16>(f, stream);
}
