// S4-S6 for groups of a few tens of rows that span several 16-row passes
// (the full-expert decode shape: every local expert active, 16 rows per
// expert on average and a skewed tail of 50-120): the weights are still
// streamed from HBM, but a unit's weights are read by every pass of its
// group, and every unit reads the pass's token rows.
//
// A workgroup of 8 waves takes work items (group, block of 8 weight units,
// pass of R = 16 NT rows). The pass's token rows and their E8M0 words are
// staged in LDS in chunks of KC K-tiles, double-buffered (the next chunk's
// buffer loads, which write LDS directly, in flight while the current chunk
// is multiplied); each wave multiplies one 64-row weight unit over the whole
// K against them: weights streamed into registers in batches, the next batch
// in flight while the current one is multiplied, token operands read from
// LDS. No wave splits K with another, so there is no cross-wave reduction,
// and each output is summed by one wave in K order (deterministic). Larger
// passes read each weight unit fewer times (a unit is read once per pass of
// its group); K-chunks keep them within the LDS.
//
// Against the K-split decode kernel this moves the token rows out of the
// vector-memory path (they were loaded once per unit: 48 times per pass for
// the W1 of a 6144-wide model, and the address unit was the busiest part of
// the CU), and removes the per-item LDS reduction and its barriers.
//
// Items are ordered (group, unit block, pass), pass fastest, and
// consecutive items go to workgroups of one XCD (blockIdx % 8), so the
// passes of a unit block run together on one XCD and find the unit's
// weights in its L2 after the first.
//
// LDS, per chunk buffer: X[kt][row][8 slots of 16 B] (chunk c of a row's
// K-tile at slot c ^ ((row >> 1) & 7), so the B operand reads of 16 rows hit
// distinct bank groups) and XS[kt][row] (the row's four E8M0 bytes of K-tile
// kt); then the pass prefix over the groups.
#include <algorithm>

#include "gemm_common.h"

namespace {

constexpr int kPWaves = 8;                 // waves per workgroup: one weight unit each
constexpr int kPThreads = 64 * kPWaves;

typedef __attribute__((address_space(3))) void lds_void_t;
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

MOE_DEV int pswz(int row) { return (row >> 1) & 7; }

// K-tiles per weight batch: 16 KiB of weights per wave and batch, 8 KiB with
// four token tiles (whose accumulators take the registers)
template <int WFMT, int NT>
constexpr int pass_kb() { return (WFMT == MFMA_FMT_FP4 ? 4 : 2) / (NT == 4 ? 2 : 1); }

// One wave's batch of a unit's weights: KB K-tiles x 4 tiles of 16 rows.
template <int WFMT, int NT>
struct WBatch {
    static constexpr int KB = pass_kb<WFMT, NT>();
    i32x4 lo[KB][4], hi[KB][4];             // hi: FP8 only
    int s[4];                               // E8M0 words of the batch's group of four K-tiles
};

// Issue the loads of batch b (K-tiles [b KB, b KB + KB)); K-tiles past the
// end (and every batch with ok == false) read zeros with no memory traffic.
template <int WFMT, int NT>
MOE_DEV void wload(WBatch<WFMT, NT>& B, rsrc_t rw, rsrc_t rs, int b, int kt_end, bool ok, int lane) {
    constexpr int KB = WBatch<WFMT, NT>::KB;
    constexpr int BPL = WFMT == MFMA_FMT_FP4 ? 16 : 32;
    const int k0 = b * KB;
    #pragma unroll
    for (int t = 0; t < 4; ++t)
        B.s[t] = (int)__builtin_amdgcn_raw_buffer_load_b32(
            rs, ok && k0 < kt_end ? (uint32_t)((((k0 >> 2) * 4 + t) * 64 + lane) * 4) : kInvalid, 0, 0);
    #pragma unroll
    for (int i = 0; i < KB; ++i) {
        const bool v = ok && k0 + i < kt_end;
        #pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint32_t off = v ? (uint32_t)(((k0 + i) * 4 + t) * 64 * BPL + lane * 16) : kInvalid;
            B.lo[i][t] = __builtin_amdgcn_raw_buffer_load_b128(rw, off, 0, 0);
            if (WFMT == MFMA_FMT_FP8)
                B.hi[i][t] = __builtin_amdgcn_raw_buffer_load_b128(rw, v ? off + 1024u : kInvalid, 0, 0);
        }
    }
}

// MFMAs of batch b against the staged token tiles [0, ntt); the staged
// chunk starts at K-tile k_base.
template <int WFMT, int NT>
MOE_DEV void wmma(const WBatch<WFMT, NT>& B, int b, int kt_end, int ntt, const uint8_t* X, const uint32_t* XS,
                  int k_base, const int (&bo_lo)[NT], const int (&bo_hi)[NT], int q, int r,
                  f32x4 (&acc)[NT][4]) {
    constexpr int KB = WBatch<WFMT, NT>::KB;
    constexpr int R = 16 * NT;
    const int k0 = b * KB;
    #pragma unroll
    for (int i = 0; i < KB; ++i) {
        const int kt = k0 + i;
        if (kt >= kt_end) break;                        // uniform
        const int kr = kt - k_base;                     // K-tile within the staged chunk
        const uint8_t* xk = X + (size_t)kr * R * 128;
        #pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            if (tt >= ntt) break;                       // uniform
            const i32x4 blo = *(const i32x4*)(xk + bo_lo[tt]);
            const i32x4 bhi = *(const i32x4*)(xk + bo_hi[tt]);
            const i32x8 Bop = __builtin_shufflevector(blo, bhi, 0, 1, 2, 3, 4, 5, 6, 7);
            const int sb = (int)(XS[kr * R + 16 * tt + r] >> (8 * q));
            #pragma unroll
            for (int t = 0; t < 4; ++t) {
                i32x8 A;
                A[0] = B.lo[i][t][0]; A[1] = B.lo[i][t][1]; A[2] = B.lo[i][t][2]; A[3] = B.lo[i][t][3];
                if (WFMT == MFMA_FMT_FP8) {
                    A[4] = B.hi[i][t][0]; A[5] = B.hi[i][t][1]; A[6] = B.hi[i][t][2]; A[7] = B.hi[i][t][3];
                } else {
                    A[4] = 0; A[5] = 0; A[6] = 0; A[7] = 0;
                }
                acc[tt][t] = mfma16x16x128<WFMT, MFMA_FMT_FP8, 0, 0>(A, Bop, acc[tt][t],
                                                                   B.s[t] >> (8 * (kt & 3)), sb);
            }
        }
    }
}

// Kernel modes: the epilogue after the K loop.
enum { kPassW2 = 0, kPassW1 = 1, kPassW1Gen = 2 };

template <int WFMT, int MODE, int NT>
__global__ __launch_bounds__(kPThreads, 1)
void pass_gemm_kernel(KParams p) {
    constexpr bool IS_W1 = MODE != kPassW2;
    constexpr int R = 16 * NT;               // token rows per pass
    constexpr int RG = R / 8;                // row groups of 8 (one staging load each)
    const int G = p.G, units = p.N / 64, nkt = p.kt;
    const int nub = (units + kPWaves - 1) / kPWaves;     // unit blocks per pass
    constexpr int KB = WBatch<WFMT, NT>::KB;
    const int nb = (nkt + KB - 1) / KB;                  // weight batches per unit
    const int KC = p.pass_kc;                            // K-tiles per chunk: a multiple of 2 KB, or >= nkt
    const int nchunk = (nkt + KC - 1) / KC;

    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int xs_words = ((KC * R + 63) / 64) * 64;      // scale words per chunk buffer
    uint8_t* X = smem;                                              // [2][KC][R][128]
    uint32_t* XS = (uint32_t*)(smem + (size_t)2 * KC * R * 128);     // [2][xs_words]
    int* pass_off = (int*)(XS + 2 * xs_words);                      // [G + 1]

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int q = lane >> 4, r = lane & 15;
    if (w == 0) pass_prefix(p.counts, G, R, lane, pass_off);
    __syncthreads();
    const int n_items = pass_off[G] * nub;
    const int grid = gridDim.x;
    const int slot = grid % 8 == 0 ? (int)(blockIdx.x % 8) * (grid / 8) + (int)blockIdx.x / 8 : (int)blockIdx.x;

    const rsrc_t rx = make_rsrc(p.aq, p.aq_bytes);
    const rsrc_t rxs = make_rsrc(p.as, p.as_bytes);

    // this lane's B operand offsets within a K-tile block: row 16 tt + r,
    // chunks q (bytes 0-15) and 4 + q (bytes 16-31), swizzled
    int bo_lo[NT], bo_hi[NT];
    #pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
        const int row = 16 * tt + r;
        bo_lo[tt] = row * 128 + 16 * (q ^ pswz(row));
        bo_hi[tt] = row * 128 + 16 * ((4 + q) ^ pswz(row));
    }

    // One work item as this lane sees it: group, pass, rows, this wave's
    // unit and its weight resources, and the source offsets of the rows this
    // lane stages (rows 8 j + l / 8 of the token rows, row l % R of the
    // scale words).
    struct PItem {
        int g, pass, rbase, nrows, ntt, u;
        bool active;
        rsrc_t rw, rs;
        uint32_t xo[RG];
        int ssrc;
    };
    auto decode = [&](int item, PItem& it) {
        int glo = 0, ghi = G;                           // largest g with pass_off[g] * nub <= item
        while (ghi - glo > 1) {
            const int mid = (glo + ghi) >> 1;
            if (pass_off[mid] * nub <= item) glo = mid; else ghi = mid;
        }
        it.g = glo;
        const int np = pass_off[glo + 1] - pass_off[glo];   // passes of the group (>= 1)
        const int local = item - pass_off[glo] * nub;
        const int ub = local / np;
        it.pass = local - ub * np;
        it.rbase = p.offsets[glo] + it.pass * R;
        it.nrows = min(R, p.counts[glo] - it.pass * R);
        it.ntt = (it.nrows + 15) / 16;
        it.u = ub * kPWaves + w;
        it.active = it.u < units;                       // uniform
        const int sel = glo < p.E_loc ? 0 : 1;
        const int gi = glo < p.E_loc ? glo : 0;
        const uint8_t* wgrp = p.wbase[sel] + gi * p.gstride;
        const int uu = it.active ? it.u : 0;
        it.rw = make_rsrc(wgrp + (size_t)uu * p.dpu, it.active ? (uint32_t)p.dpu : 0u);
        it.rs = make_rsrc(wgrp + p.dpg + (size_t)uu * p.spu, it.active ? (uint32_t)p.spu : 0u);
        #pragma unroll
        for (int j = 0; j < RG; ++j) {
            const int row = 8 * j + (lane >> 3);
            const int src = row < it.nrows ? (p.row_src ? p.row_src[it.rbase + row] : it.rbase + row) : -1;
            it.xo[j] = src >= 0 ? (uint32_t)src * (uint32_t)p.K : kInvalid;
        }
        const int srow = lane % R;
        it.ssrc = srow < it.nrows ? (p.row_src ? p.row_src[it.rbase + srow] : it.rbase + srow) : -1;
    };

    // Stage chunk c (K-tiles [c KC, c KC + KC)) of an item into buffer buf:
    // instruction i copies K-tile i / RG of rows 8 (i % RG) + [0, 8) (lane
    // l: row + l / 8, slot l % 8 holding chunk (l % 8) ^ pswz(row)), and scale
    // instruction i the words [64 i, 64 i + 64) of the buffer (K-tile
    // (64 i + l) / R, row l % R); rows past the pass read zeros.
    auto stage = [&](const PItem& it, int c, int buf) {
        const int k0 = c * KC, kc = min(KC, nkt - k0);
        uint8_t* Xb = X + (size_t)buf * KC * R * 128;
        uint32_t* XSb = XS + buf * xs_words;
        for (int i = w; i < kc * RG; i += kPWaves) {
            const int kr = i / RG, j = i - kr * RG;
            const int row = 8 * j + (lane >> 3);
            const int chunk = (lane & 7) ^ pswz(row);
            uint32_t o = kInvalid;
            #pragma unroll
            for (int jj = 0; jj < RG; ++jj)
                if (jj == j && it.xo[jj] != kInvalid) o = it.xo[jj] + (uint32_t)((k0 + kr) * 128 + 16 * chunk);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void_t*)(Xb + ((size_t)kr * R + 8 * j) * 128), 16,
                                                     o, 0, 0, 0);
        }
        for (int i = w; i < (kc * R + 63) / 64; i += kPWaves) {
            const int kr = (64 * i + lane) / R;
            const uint32_t o = it.ssrc >= 0 && kr < kc ? (uint32_t)it.ssrc * (uint32_t)(p.K / 32) + 4u * (k0 + kr)
                                                       : kInvalid;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rxs, (lds_void_t*)(XSb + 64 * i), 4, o, 0, 0, 0);
        }
    };

    const int n_my = slot < n_items ? (n_items - slot + grid - 1) / grid : 0;   // this workgroup's items
    if (n_my == 0) return;
    PItem cur, nxt;
    decode(slot, cur);
    // the first weight batch and the first chunk, then one wait
    WBatch<WFMT, NT> B0, B1;
    wload<WFMT, NT>(B0, cur.rw, cur.rs, 0, nkt, cur.active, lane);
    stage(cur, 0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // The workgroup's chunks form one sequence over its items: while a chunk
    // is multiplied, the next one (of this item, or the first of the next
    // item) is staged into the other buffer; the wait and barrier at a
    // chunk's end make it visible and free the chunk's own buffer. Weights:
    // two register batches, the next one's loads in flight while the current
    // one is multiplied (past the last batch the loads read nothing); a chunk
    // that is not an item's last holds an even number of batches, so B0
    // holds the first batch of every chunk; the next item's first batch is
    // requested before this item's epilogue.
    int s = 0;                               // chunks consumed: buffer s % 2 holds the current one
    for (int it = 0; it < n_my; ++it) {
        const bool more = it + 1 < n_my;
        if (more) decode(slot + (it + 1) * grid, nxt);
        const int g = cur.g, pass = cur.pass, rbase = cur.rbase, nrows = cur.nrows, u = cur.u;
        const bool active = cur.active;

        f32x4 acc[NT][4];
        #pragma unroll
        for (int tt = 0; tt < NT; ++tt)
            #pragma unroll
            for (int t = 0; t < 4; ++t) acc[tt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
        int b = 0;
        for (int c = 0; c < nchunk; ++c, ++s) {
            if (c + 1 < nchunk) stage(cur, c + 1, (s + 1) & 1);
            else if (more) stage(nxt, 0, (s + 1) & 1);
            const uint8_t* Xb = X + (size_t)(s & 1) * KC * R * 128;
            const uint32_t* XSb = XS + (s & 1) * xs_words;
            const int b_end = c + 1 == nchunk ? nb : (c + 1) * KC / KB;
            if (active) {
                for (; b < b_end; b += 2) {
                    wload<WFMT, NT>(B1, cur.rw, cur.rs, b + 1, nkt, b + 1 < nb, lane);
                    wmma<WFMT, NT>(B0, b, nkt, cur.ntt, Xb, XSb, c * KC, bo_lo, bo_hi, q, r, acc);
                    if (b + 1 < b_end) {
                        wload<WFMT, NT>(B0, cur.rw, cur.rs, b + 2, nkt, b + 2 < nb, lane);
                        wmma<WFMT, NT>(B1, b + 1, nkt, cur.ntt, Xb, XSb, c * KC, bo_lo, bo_hi, q, r, acc);
                    }
                }
            }
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
        if (more) wload<WFMT, NT>(B0, nxt.rw, nxt.rs, 0, nkt, nxt.active, lane);

        if (active) {
            // epilogue on the accumulators: acc[tt][t][v] is weight row
            // 16 t + 4 q + v of the unit against token row 16 tt + r
            if constexpr (IS_W1) {
                const int I = p.N / 2;
                const rsrc_t rhq = make_rsrc(p.hq + (size_t)rbase * I, (uint32_t)(nrows * I));
                const rsrc_t rhs = make_rsrc(p.hs + (size_t)rbase * (I / 32), (uint32_t)(nrows * (I / 32)));
                const rsrc_t rww = make_rsrc(p.row_w + rbase, p.use_w ? (uint32_t)(nrows * 4) : 0u);
                // variant epilogue: this lane's gate and up biases (zero
                // without a bias), the BF16 pre-activation rows of 2I
                float bg[2][4] = {}, bu[2][4] = {};
                const bool spre = MODE == kPassW1Gen && p.save_pre;
                const rsrc_t rpre = make_rsrc(spre ? p.save_pre + (size_t)rbase * 2 * I : (uint16_t*)p.hq,
                                              spre ? (uint32_t)(nrows * 2 * I * 2) : 0u);
                if constexpr (MODE == kPassW1Gen) {
                    const rsrc_t rb = make_rsrc(p.bias + (size_t)g * 2 * I, p.bias ? (uint32_t)(2 * I * 4) : 0u);
                    #pragma unroll
                    for (int a = 0; a < 2; ++a)
                        #pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            const uint32_t f = (uint32_t)(32 * u + 16 * a + 4 * q + v);
                            bg[a][v] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rb, 4 * f, 0, 0));
                            bu[a][v] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rb, 4 * (f + I), 0, 0));
                        }
                }
                float h[NT][2][4];
                #pragma unroll
                for (int tt = 0; tt < NT; ++tt) {
                    const int tok = 16 * tt + r;
                    // rows past the pass have zero sums, a zero weight and h = 0
                    const float wl = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rww, (uint32_t)(tok * 4), 0, 0));
                    const float wgt = p.use_w ? wl : (tok < nrows ? 1.0f : 0.0f);
                    // unit u pairs gate features 32 u + [0, 32) (tiles 0, 1)
                    // with the same up features (tiles 2, 3): h of feature
                    // 32 u + 16 a + 4 q + v in this lane
                    float amf = 0.f;
                    #pragma unroll
                    for (int a = 0; a < 2; ++a) {
                        if constexpr (MODE == kPassW1Gen) {
                            float gz[4], uz[4];
                            #pragma unroll
                            for (int v = 0; v < 4; ++v) {
                                gz[v] = acc[tt][a][v] + bg[a][v];
                                uz[v] = acc[tt][a + 2][v] + bu[a][v];
                            }
                            u32x2 pg, pu;
                            pg.x = bf16x2(gz[0], gz[1]); pg.y = bf16x2(gz[2], gz[3]);
                            pu.x = bf16x2(uz[0], uz[1]); pu.y = bf16x2(uz[2], uz[3]);
                            const uint32_t po = (uint32_t)((tok * 2 * I + 32 * u + 16 * a + 4 * q) * 2);
                            __builtin_amdgcn_raw_buffer_store_b64(pg, rpre, po, 0, 0);
                            __builtin_amdgcn_raw_buffer_store_b64(pu, rpre, po + (uint32_t)(2 * I), 0, 0);
                            #pragma unroll
                            for (int v = 0; v < 4; ++v) {
                                float gv = gz[v], uv = uz[v];
                                if (p.limit > 0.f) {
                                    gv = fminf(fmaxf(gv, -p.limit), p.limit);
                                    uv = fminf(fmaxf(uv, -p.limit), p.limit);
                                }
                                h[tt][a][v] = act_value(gv, p.act, p.beta) * uv * wgt;
                                amf = fmaxf(amf, fabsf(h[tt][a][v]));
                            }
                        } else {
                            #pragma unroll
                            for (int v = 0; v < 4; ++v) {
                                h[tt][a][v] = silu_fast(acc[tt][a][v]) * acc[tt][a + 2][v] * wgt;
                                amf = fmaxf(amf, fabsf(h[tt][a][v]));
                            }
                        }
                    }
                    // the token's 32 features of this unit: lanes r, r + 16, r + 32, r + 48
                    const uint32_t am = rows4_umax(__float_as_uint(amf));
                    const uint32_t code = e4m3_scale_code(__uint_as_float(am), p.ceil_rule);
                    const float inv = inv_scale(code);
                    #pragma unroll
                    for (int a = 0; a < 2; ++a)
                        __builtin_amdgcn_raw_buffer_store_b32(
                            e4m3x4(h[tt][a][0] * inv, h[tt][a][1] * inv, h[tt][a][2] * inv, h[tt][a][3] * inv),
                            rhq, (uint32_t)(tok * I + 32 * u + 16 * a + 4 * q), 0, 0);
                    __builtin_amdgcn_raw_buffer_store_b8((unsigned char)code, rhs,
                                                         q == 0 ? (uint32_t)(tok * (I / 32) + u) : kInvalid, 0, 0);
                }
                // transposed copy (passes of 32 or 64 rows: one or two whole
                // 32-token blocks, at columns offsets32[g] + R pass + 32 jp):
                // per feature the amax over a block's 32 tokens (16 lanes x 2
                // tiles), its E8M0 code and the E4M3 codes, one byte each;
                // padding tokens are zeros; blocks that start past the rows
                // belong to the next group's columns and are not written
                if (NT >= 2 && p.transpose) {
                    const rsrc_t rT = make_rsrc(p.hTq, (uint32_t)((size_t)I * p.ldT));
                    const rsrc_t rTs = make_rsrc(p.hTs, (uint32_t)((size_t)I * (p.ldT / 32)));
                    #pragma unroll
                    for (int jp = 0; jp < NT / 2; ++jp) {
                        if (32 * jp >= nrows) break;                    // uniform
                        const int col0 = p.offsets32[g] + pass * R + 32 * jp;
                        #pragma unroll
                        for (int a = 0; a < 2; ++a)
                            #pragma unroll
                            for (int v = 0; v < 4; ++v) {
                                const float m = fmaxf(fabsf(h[2 * jp][a][v]), fabsf(h[(2 * jp + 1) % NT][a][v]));
                                const uint32_t am = row16_umax(__float_as_uint(m));
                                const uint32_t code = e4m3_scale_code(__uint_as_float(am), p.ceil_rule);
                                const float inv = inv_scale(code);
                                const uint32_t f = (uint32_t)(32 * u + 16 * a + 4 * q + v);
                                #pragma unroll
                                for (int jj = 0; jj < 2; ++jj)
                                    __builtin_amdgcn_raw_buffer_store_b8(
                                        (unsigned char)(e4m3x2(h[(2 * jp + jj) % NT][a][v] * inv, 0.f) & 0xFFu), rT,
                                        f * (uint32_t)p.ldT + (uint32_t)(col0 + 16 * jj + r), 0, 0);
                                __builtin_amdgcn_raw_buffer_store_b8(
                                    (unsigned char)code, rTs,
                                    r == 0 ? f * (uint32_t)(p.ldT / 32) + (uint32_t)(col0 >> 5) : kInvalid, 0, 0);
                            }
                    }
                }
            } else {
                const int H = p.N;
                const rsrc_t ry = make_rsrc(p.y + (size_t)rbase * H, (uint32_t)(nrows * H * 2));
                #pragma unroll
                for (int tt = 0; tt < NT; ++tt) {
                    const int tok = 16 * tt + r;
                    #pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        u32x2 o;
                        o.x = bf16x2(acc[tt][t][0], acc[tt][t][1]);
                        o.y = bf16x2(acc[tt][t][2], acc[tt][t][3]);
                        __builtin_amdgcn_raw_buffer_store_b64(o, ry, (uint32_t)((tok * H + 64 * u + 16 * t + 4 * q) * 2),
                                                              0, 0);
                    }
                }
            }
        }
        if (more) cur = nxt;
    }
}

// LDS bytes for chunks of KC K-tiles in nbuf buffers
size_t pass_lds(int KC, int nbuf, int R, int G) {
    return (size_t)nbuf * KC * R * 128 + (size_t)nbuf * ((KC * R + 63) / 64) * 64 * 4 + (size_t)(G + 1) * 4;
}

constexpr size_t kPassLdsCap = 160 * 1024;          // LDS of one compute unit

// The chunk size of a pass-resident launch: the whole K if it fits twice
// (two buffers), else the largest even number of weight batches that fits
// twice; 0 if not even that fits.
int pass_chunk(int K, int G, int NT, int fmt, size_t* lds) {
    const int nkt = K / 128, R = 16 * NT;
    const int KB = (fmt == MOE_FMT_MXFP4 ? 4 : 2) / (NT == 4 ? 2 : 1);
    if (pass_lds(nkt, 2, R, G) <= kPassLdsCap) {
        *lds = pass_lds(nkt, 2, R, G);
        return nkt;
    }
    for (int kc = ((nkt - 1) / (2 * KB)) * 2 * KB; kc >= 2 * KB; kc -= 2 * KB)
        if (pass_lds(kc, 2, R, G) <= kPassLdsCap) {
            *lds = pass_lds(kc, 2, R, G);
            return kc;
        }
    return 0;
}

template <int WFMT, int MODE, int NT>
int launch_pass(KParams p, int R_max, hipStream_t stream) {
    auto kern = pass_gemm_kernel<WFMT, MODE, NT>;
    size_t lds = 0;
    p.pass_kc = pass_chunk(p.K, p.G, NT, WFMT == MFMA_FMT_FP4 ? MOE_FMT_MXFP4 : MOE_FMT_MXFP8, &lds);
    if (p.pass_kc == 0) return (int)hipErrorInvalidValue;
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kPThreads, lds) != hipSuccess || per_cu < 1)
        per_cu = 1;
    const long nub = (p.N / 64 + kPWaves - 1) / kPWaves;
    // passes never exceed R_max / R + G: each group adds at most one partial pass
    const long max_items = nub * ((long)R_max / (16 * NT) + p.G);
    const long grid = std::max<long>(1, std::min<long>(max_items, (long)per_cu * device_cu_count()));
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kPThreads), lds, stream, p);
    return (int)hipGetLastError();
}

}  // namespace

// Whether the pass-resident kernel can stage passes of NT token tiles for
// this K and G (NT = 1, 2 or 4).
bool moe_pass_fits(int K, int G, int NT, int fmt) {
    size_t lds = 0;
    return pass_chunk(K, G, NT, fmt, &lds) > 0;
}

// Runs a grouped GEMM on the pass-resident kernel with NT token tiles per
// pass (1, 2 or 4; 2 or 4 with the transposed copy); the caller has checked
// moe_pass_fits.
int moe_launch_pass(const GemmArgs& a, bool w1, int NT, hipStream_t stream) {
    if (a.G == 0 || a.R_max == 0) return 0;
    const KParams p = make_params(a, w1);
    const bool fp4 = a.fmt == MOE_FMT_MXFP4;
#define MOE_PASS_CASE(MODE)                                                                        \
    if (NT == 4) return fp4 ? launch_pass<MFMA_FMT_FP4, MODE, 4>(p, a.R_max, stream)               \
                            : launch_pass<MFMA_FMT_FP8, MODE, 4>(p, a.R_max, stream);              \
    if (NT == 2) return fp4 ? launch_pass<MFMA_FMT_FP4, MODE, 2>(p, a.R_max, stream)               \
                            : launch_pass<MFMA_FMT_FP8, MODE, 2>(p, a.R_max, stream);              \
    return fp4 ? launch_pass<MFMA_FMT_FP4, MODE, 1>(p, a.R_max, stream)                           \
               : launch_pass<MFMA_FMT_FP8, MODE, 1>(p, a.R_max, stream);
    if (!w1) { MOE_PASS_CASE(kPassW2) }
    if (p.generic) { MOE_PASS_CASE(kPassW1Gen) }
    MOE_PASS_CASE(kPassW1)
#undef MOE_PASS_CASE
}
