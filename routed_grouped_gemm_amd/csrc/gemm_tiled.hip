// S4-S6 for groups with many rows (prefill and training-forward shapes, where
// the grouped GEMMs are bound by the matrix cores, not by HBM; GC-MoE page,
// "Limitations": at large token counts the compute partition is the
// bottleneck).
//
// A workgroup of 8 waves (two per SIMD) computes 256 x 256 output tiles of
// one group: four prepacked 64-row weight units (for W1: 32 gate rows and the
// matching 32 up rows each) against 256 of the group's token rows, over the
// whole K. Wave w owns weight unit w % 4 and token half w / 4: 64 x 128
// outputs = 4 x 8 tiles of the 16x16x128 scaled MFMA, 32 MFMAs per 128-wide
// K-tile.
//
// The tile size is set by L2 traffic: every operand byte is fetched into the
// CU once per workgroup tile (no wave loads what another already loaded), so
// a 128-wide K-tile moves 64 KiB for 16.8 MFLOP.
//
//  - Both operands of a K-tile (the 256 weight rows of the four units, the
//    256 token rows, and their E8M0 words) are staged in LDS by buffer loads
//    that write LDS directly, double-buffered: the next K-tile is in flight
//    while this one is multiplied. The prepacked weight tiles are copied
//    verbatim (1 KiB contiguous per load instruction) and are already in the
//    A operand's lane order. Token rows are copied as whole 128-byte lines
//    (8 rows per instruction), their 16-byte chunks XOR-swizzled by row so
//    that the B operand reads (16 rows, one chunk each) hit 16 distinct bank
//    groups. Rows past the group's end read as zero.
//  - The token rows' E8M0 words are read from scale tiles that a small kernel
//    writes first: per K-tile and 256-row pass, the 256 rows' 4-byte words
//    side by side (zero past the group's end), so one 1 KiB load stages them
//    instead of 256 scattered 4-byte reads.
//  - One barrier per K-tile. The loop runs over the workgroup's whole
//    sequence of (item, K-tile) steps, so the next item's first K-tile is in
//    flight while an item's epilogue runs. Within a K-tile each wave keeps its
//    4 weight tiles in registers and streams its 8 token tiles from LDS
//    through two register buffers: the next token tile's reads are in flight
//    while the current one's 4 MFMAs run.
//  - Memory requests that an item waits for are issued together: the routing
//    weights of the item's rows (W1 epilogue) and the source rows of the next
//    item, one latency each per item.
//  - In a pass of at most 128 rows (a group's last), the four waves of the
//    empty token half only stage their share of the operands and keep the
//    barriers; the other wave of each SIMD then runs alone.
//  - Epilogues run on the accumulators. W1: gate and up of the same feature
//    sit in the same lane (the prepacked units pair them), so
//    h = SiLU(gate) * up * w is formed in place; the 32 features of a unit are
//    one MX block along I (4 lanes x 8 values) and go out as one dword per
//    lane; the transposed copy (32-token blocks along the group's rows) is
//    transposed through an fp32 tile in LDS, so that each lane scales 8
//    tokens of one feature, and leaves as 16-byte row stores. W2: BF16 rows.
//    Conversions use the hardware's round-to-nearest-even converters.
//
// Work items are (group, 256-row pass, 256-row weight tile), weight tile
// fastest; a persistent grid walks them, with item order swizzled so the
// workgroups that run together on one XCD (blockIdx % 8) take consecutive
// items and share operands in that XCD's L2.
#include <algorithm>
#include <type_traits>

#include "gemm_common.h"

namespace {

constexpr int kRows = 256;                  // token rows per workgroup tile
constexpr int kUnits = 4;                   // 64-row weight units per workgroup tile
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBT = 8;                      // 16-row token tiles per wave
constexpr int kAT = 4;                      // 16-row weight tiles per wave (one unit)
constexpr int kTStride = 136;               // bytes per feature row of the transposed staging
constexpr int kTWave = 32 * kTStride;       // per-wave staging of the transposed copy
constexpr int kYStride = 144;               // bytes per token row of the BF16 output staging (conflict-free)
constexpr int kRingPasses = 64;             // token ring: 256-row passes per chunk (one slot)
constexpr int kRingCUs = 16;                // compute units the W1 consumer leaves to the ring's producer

typedef __attribute__((address_space(3))) void lds_void_t;
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// One LDS stage (one K-tile of both operands):
//   B  [256 token rows][8 chunks of 16 B], chunk c of row at slot c ^ bswz(row)   32 KiB
//   A  [16 weight tiles][(half)][lane][16 B]        32 KiB (FP8) / 16 KiB (FP4)
//   BS [256 token rows] E8M0 words                   1 KiB
//   AS [16 weight tiles][lane] E8M0 words            4 KiB (byte kt % 4 is this K-tile's)
template <int WFMT>
struct Stage {
    static constexpr int kBPL = WFMT == MFMA_FMT_FP4 ? 16 : 32;    // bytes per lane per tile
    static constexpr int B = 0;
    static constexpr int A = kRows * 128;
    static constexpr int BS = A + 16 * 64 * kBPL;
    static constexpr int AS = BS + kRows * 4;
    static constexpr int Bytes = AS + 16 * 64 * 4;
};
// the W1 epilogue's scratch (per wave: transposed staging, its scales, a
// 2 KiB fp32 tile) fits in one stage
static_assert(kWaves * (kTWave + 128 + 2048) <= Stage<MFMA_FMT_FP4>::Bytes, "W1 epilogue scratch");

MOE_DEV int bswz(int row) { return (row >> 1) & 7; }

// One work item as seen by this lane.
struct Ctx {
    int g, pass, wt, rbase, nrows;
    const uint8_t* wgrp;                    // prepacked group base
    uint32_t xoff[4];                       // staged token rows 32 w + 8 i + lane / 8: byte offset of the row
    int pidx;                               // pass index over all groups (scale tile column)
};

MOE_DEV Ctx decode(const KParams& p, const int* pass_off, int item, int wtiles, int w, int lane, int r0) {
    Ctx c;
    const int pg = item / wtiles;
    c.wt = item - pg * wtiles;
    int glo = 0, ghi = p.G;                 // largest g with pass_off[g] <= pg
    while (ghi - glo > 1) {
        const int mid = (glo + ghi) >> 1;
        if (pass_off[mid] <= pg) glo = mid; else ghi = mid;
    }
    c.g = __builtin_amdgcn_readfirstlane(glo);
    c.pidx = pg;
    c.pass = pg - __builtin_amdgcn_readfirstlane(pass_off[c.g]);
    const int n_g = p.counts[c.g];
    c.rbase = p.offsets[c.g] + c.pass * kRows;
    c.nrows = min(kRows, n_g - c.pass * kRows);
    const int sel = c.g < p.E_loc ? 0 : 1;
    const int gi = c.g < p.E_loc ? c.g : 0;
    c.wgrp = p.wbase[sel] + gi * p.gstride;
    // source rows of the item's grouped rows (branch-free: rows past the
    // item read as 0 through the bounded resource and are marked invalid)
    // (all four requested before any is used: one memory latency, not four;
    // without row_src the resource is empty and the row itself is the source)
    const rsrc_t rsrcs = make_rsrc(p.row_src + c.rbase, p.row_src ? (uint32_t)(c.nrows * 4) : 0u);
    uint32_t xr[4];
    #pragma unroll
    for (int i = 0; i < 4; ++i)
        xr[i] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(
            rsrcs, (uint32_t)((32 * w + 8 * i + (lane >> 3)) * 4), 0, 0);
    #pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 32 * w + 8 * i + (lane >> 3);
        const uint32_t src = p.row_src ? xr[i] : (uint32_t)(c.rbase + row - r0);
        c.xoff[i] = row < c.nrows ? src * (uint32_t)p.K : kInvalid;
    }
    return c;
}

// Stage K-tile kt of an item into one LDS stage with buffer loads that write
// LDS directly (each lane's bytes land at the wave's LDS base + size * lane).
// Wave w stages token rows [32w, 32w + 32) (lane l of instruction i: row
// 32w + 8i + l/8, LDS slot l%8 holding chunk (l%8) ^ bswz(row)) and the
// weight tiles 2w, 2w+1 of the four units with their E8M0 words (copied
// verbatim); wave 0 also stages the E8M0 words of the 256 token rows (one
// 1 KiB scale tile). With valid == false every load is out of range: zeros
// land and no memory is read.
template <int WFMT>
MOE_DEV void stage_all(const KParams& p, rsrc_t rx, rsrc_t rxs, const Ctx& c, int kt, bool valid,
                       uint8_t* st, int w, int lane) {
    using S = Stage<WFMT>;
    #pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 32 * w + 8 * i + (lane >> 3);
        const int chunk = (lane & 7) ^ bswz(row);
        const uint32_t xo = c.xoff[i];
        const uint32_t o = (xo == kInvalid || !valid) ? kInvalid : xo + (uint32_t)(kt * 128 + 16 * chunk);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void_t*)(st + S::B + (32 * w + 8 * i) * 128), 16, o, 0, 0, 0);
    }
    if (w == 0)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rxs, (lds_void_t*)(st + S::BS), 16,
            valid ? (uint32_t)((kt * p.npass + c.pidx) * (kRows * 4) + lane * 16) : kInvalid, 0, 0, 0);
    #pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int T = 2 * w + i;                // weight tile within the workgroup tile
        const int u = c.wt * kUnits + (T >> 2), t = T & 3;
        // a partial last workgroup tile (N not a multiple of 256: the
        // backward's N = I) stages zeros for the units past the last one
        const bool uok = valid && u < p.N / 64;
        const rsrc_t rw = make_rsrc(c.wgrp + (size_t)u * p.dpu, uok ? (uint32_t)p.dpu : 0u);
        const rsrc_t rs = make_rsrc(c.wgrp + p.dpg + (size_t)u * p.spu, uok ? (uint32_t)p.spu : 0u);
        #pragma unroll
        for (int half = 0; half < S::kBPL / 16; ++half)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rw, (lds_void_t*)(st + S::A + T * 64 * S::kBPL + half * 1024), 16,
                (uint32_t)((kt * 4 + t) * 64 * S::kBPL + half * 1024 + lane * 16), 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (lds_void_t*)(st + S::AS + T * 256), 4,
            (uint32_t)((((kt >> 2) * 4 + t) * 64 + lane) * 4), 0, 0, 0);
    }
}

// Quad transpose of bytes: lane k of each group of 4 lanes receives byte k of
// the dword `x` of every lane of its quad, lane i's byte in byte i. Every
// lane is active and reads a lane of its own quad, so the broadcasts need no
// fallback value (one DPP move each).
MOE_DEV uint32_t quad_byte_transpose(uint32_t x, int lane) {
    const uint32_t q0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x00, 0xF, 0xF, true);  // quad_perm(0,0,0,0)
    const uint32_t q1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x55, 0xF, 0xF, true);  // (1,1,1,1)
    const uint32_t q2 = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xAA, 0xF, 0xF, true);  // (2,2,2,2)
    const uint32_t q3 = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xFF, 0xF, 0xF, true);  // (3,3,3,3)
    const uint32_t k = (uint32_t)(lane & 3);
    // v_perm_b32(a, b, sel): selector byte values 0-3 pick bytes of b, 4-7 bytes of a
    const uint32_t sel01 = (k) | ((k + 4) << 8);                        // byte0 = b[k], byte1 = a[k]
    const uint32_t lo = __builtin_amdgcn_perm(q1, q0, sel01 | (sel01 << 16));
    const uint32_t hi = __builtin_amdgcn_perm(q3, q2, sel01 | (sel01 << 16));
    return __builtin_amdgcn_perm(hi, lo, 0x05040100u);                  // lo bytes 0,1 then hi bytes 0,1
}

// Sum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (the same lane of each
// row of the wave), returned to all four, in a fixed order.
MOE_DEV float rows4_sum(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Transposed copy, staging of one 32-token block jp of a wave (tokens
// tok0 + 32 jp + [0, 32): token tiles 2 jp and 2 jp + 1) for 32 features
// (two 16-feature tiles a, the lane's 4 features 16 a + 4 q + v): per feature
// the amax over its 32 tokens (16 lanes x 2 tiles), the E8M0 code, and the
// E4M3 codes, into the wave's LDS staging as [feature][token] bytes (tw) and
// [block][feature] scale bytes (tsw, written by the lanes with r = 0).
MOE_DEV void transpose_stage(const float (&h)[2][2][4], int jp, uint8_t* tw, uint8_t* tsw, int lane,
                             bool ceil_rule, int stride = kTStride) {
    const int q = lane >> 4, r = lane & 15;
    #pragma unroll
    for (int a = 0; a < 2; ++a) {
        float sc[2][4];
        uint32_t cw = 0;
        #pragma unroll
        for (int v = 0; v < 4; ++v) {
            const uint32_t am = row16_umax(__float_as_uint(fmaxf(fabsf(h[0][a][v]), fabsf(h[1][a][v]))));
            const uint32_t code = e4m3_scale_code(__uint_as_float(am), ceil_rule);
            const float inv = inv_scale(code);
            sc[0][v] = h[0][a][v] * inv;
            sc[1][v] = h[1][a][v] * inv;
            cw |= code << (8 * v);
        }
        if (r == 0) *(uint32_t*)(tsw + jp * 32 + 16 * a + 4 * q) = cw;
        // lane 4m + k: feature 16a + 4q + k, tokens 16 j + 4m .. +3
        #pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const uint32_t pk = e4m3x4(sc[jj][0], sc[jj][1], sc[jj][2], sc[jj][3]);
            const uint32_t tr = quad_byte_transpose(pk, lane);
            const int fl = 16 * a + 4 * q + (lane & 3);
            *(uint32_t*)(tw + fl * stride + 16 * (2 * jp + jj) + 4 * ((lane >> 2) & 3)) = tr;
        }
    }
}

// Transposed copy, staging of one 32-token block jp of a wave through an
// fp32 tile in LDS, one 16-feature half a at a time: the lanes write their
// values (token 16 jj + r, features 16 a + 4 q + [0, 4)) as [token][feature]
// rows, then lane l reads feature l % 16 of tokens 8 (l / 16) + [0, 8), takes
// their amax locally and over the four lanes of its feature, and writes its
// 8 E4M3 codes as one 8-byte piece of the feature's row of tw, and lanes
// 0-15 the E8M0 byte to tsw. Same values and order of operations per code
// as the register-only staging above, with one scale computation per lane
// and half instead of eight.
// xs (2 KiB, 16 B aligned): row t at 64-byte half (t & 1) ^ ((t >> 3) & 1)
// of line t / 2, its 16-byte chunks XOR-swizzled by (t >> 1) & 3: the
// writes of 8 consecutive lanes and the reads of 32 hit distinct banks.
MOE_DEV int xs_word(int t, int f) {
    return (t >> 1) * 32 + (((t & 1) ^ ((t >> 3) & 1)) << 4) + ((((f >> 2) ^ (t >> 1)) & 3) << 2) + (f & 3);
}
MOE_DEV void transpose_stage_f32(const float (&h)[2][2][4], int jp, float* xs, uint8_t* tw, uint8_t* tsw,
                                 int lane, bool ceil_rule) {
    const int q = lane >> 4, r = lane & 15;
    const int f = lane & 15, tg = lane >> 4;
    #pragma unroll
    for (int a = 0; a < 2; ++a) {
        #pragma unroll
        for (int jj = 0; jj < 2; ++jj)
            *(f32x4*)(xs + xs_word(16 * jj + r, 4 * q)) =
                f32x4{h[jj][a][0], h[jj][a][1], h[jj][a][2], h[jj][a][3]};
        float v[8];
        #pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = xs[xs_word(8 * tg + i, f)];
        float amf = 0.f;
        #pragma unroll
        for (int i = 0; i < 8; ++i) amf = fmaxf(amf, fabsf(v[i]));
        const uint32_t code = e4m3_scale_code(__uint_as_float(rows4_umax(__float_as_uint(amf))), ceil_rule);
        const float inv = inv_scale(code);
        u32x2 pk;
        pk.x = e4m3x4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
        pk.y = e4m3x4(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
        *(u32x2*)(tw + (16 * a + f) * kTStride + 32 * jp + 8 * tg) = pk;
        if (tg == 0) tsw[jp * 32 + 16 * a + f] = (uint8_t)code;
    }
}

// The staged 32 features x 128 tokens of a wave -> transposed rows
// [fbase, fbase + 32) of a [rows, ldT] copy at columns col0 + [0, 128), as
// 16-byte row stores, and their scales; only 32-token blocks that start
// inside the item's rows (nrows counted from the wave's first token tok0).
MOE_DEV void transpose_flush(const uint8_t* tw, const uint8_t* tsw, uint8_t* dq, uint8_t* ds, int rows,
                             int ldT, int fbase, int col0, int tok0, int nrows, int lane) {
    const rsrc_t rhT = make_rsrc(dq, (uint32_t)((size_t)rows * ldT));
    const rsrc_t rhTs = make_rsrc(ds, (uint32_t)((size_t)rows * (ldT / 32)));
    #pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int fl = 8 * i + (lane >> 3), c = lane & 7;
        const i32x4 d = *(const i32x4*)(tw + fl * kTStride + 16 * c);
        __builtin_amdgcn_raw_buffer_store_b128(
            d, rhT, tok0 + 32 * (c >> 1) < nrows ? (uint32_t)((fbase + fl) * ldT + col0 + 16 * c) : kInvalid, 0, 0);
    }
    // scales: feature lane (< 32), 4 blocks -> bytes [col0/32, +4) of its scale row
    const uint32_t so = (uint32_t)((fbase + (lane & 31)) * (ldT / 32) + (col0 >> 5));
    #pragma unroll
    for (int b = 0; b < 4; ++b)
        __builtin_amdgcn_raw_buffer_store_b8(tsw[b * 32 + (lane & 31)], rhTs,
                                             (lane < 32 && tok0 + 32 * b < nrows) ? so + b : kInvalid, 0, 0);
}

// One staged 32-token block (32 features x 32 tokens at row stride
// kT32Stride, from transpose_stage with jp = 0) -> rows [fbase, fbase + 32)
// of the transposed copy at columns [col, col + 32), two 16-byte stores per
// feature row, and its scale bytes at column block col / 32.
constexpr int kT32Stride = 48;
MOE_DEV void transpose_flush32(const uint8_t* tw, const uint8_t* tsw, uint8_t* dq, uint8_t* ds, int rows,
                               int ldT, int fbase, int col, int lane) {
    const rsrc_t rhT = make_rsrc(dq, (uint32_t)((size_t)rows * ldT));
    const rsrc_t rhTs = make_rsrc(ds, (uint32_t)((size_t)rows * (ldT / 32)));
    const int fl = lane >> 1, h = lane & 1;
    const i32x4 d = *(const i32x4*)(tw + fl * kT32Stride + 16 * h);
    // non-temporal: these 32-byte pieces of 32 rows are not kept in L2
    // (backward 1319-1352 -> 1263-1292 us; the same hint on the row-major
    // stores of either epilogue was slower)
    __builtin_amdgcn_raw_buffer_store_b128(d, rhT, (uint32_t)((fbase + fl) * ldT + col + 16 * h), 0, 2);
    __builtin_amdgcn_raw_buffer_store_b8(tsw[lane & 31], rhTs,
                                         lane < 32 ? (uint32_t)((fbase + lane) * (ldT / 32) + (col >> 5)) : kInvalid,
                                         0, 0);
}

// Kernel modes: the epilogue that follows the shared K-loop.
enum { kModeW2 = 0, kModeW1 = 1, kModeW1Gen = 2, kModeBwd = 3 };

template <int WFMT, int MODE>
__global__ __launch_bounds__(kThreads, 1)
void tiled_gemm_kernel(KParams p) {
    constexpr bool IS_W1 = MODE == kModeW1 || MODE == kModeW1Gen;
    using S = Stage<WFMT>;
    const int G = p.G, units = p.N / 64;
    const int wtiles = (units + kUnits - 1) / kUnits;   // a multiple of 4 units but for the backward

    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    uint8_t* ring = smem;                                               // [2][S::Bytes]
    int* pass_off = (int*)(smem + 2 * S::Bytes);                        // [G + 1]

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int q = lane >> 4, r = lane & 15;
    const int wi = w & 3, ti = w >> 2;       // weight unit, token half
    if (w == 0) pass_prefix(p.counts, G, kRows, lane, pass_off);
    __syncthreads();
    // the items of this launch: [item_lo, item_hi) of all (pass, weight tile) items
    const int i_lo = p.item_lo, i_hi = min(p.item_hi, pass_off[G] * wtiles);
    const int n_items = max(0, i_hi - i_lo);
    const int grid = gridDim.x;
    const int slot = (grid % 8 == 0) ? (blockIdx.x % 8) * (grid / 8) + blockIdx.x / 8 : blockIdx.x;
    if (slot >= n_items) return;
    // token rows from a ring slot: the slot's first row is the first row of pass ring_pass0
    int r0 = 0;
    if (p.ring_pass0 >= 0) {
        int glo = 0, ghi = G;                   // largest g with pass_off[g] <= ring_pass0
        while (ghi - glo > 1) {
            const int mid = (glo + ghi) >> 1;
            if (pass_off[mid] <= p.ring_pass0) glo = mid; else ghi = mid;
        }
        r0 = p.offsets[glo] + (p.ring_pass0 - pass_off[glo]) * kRows;
    }
    const int n_my = (n_items - slot + grid - 1) / grid;                 // this workgroup's items
    const int nkt = p.kt;
    const int total = n_my * nkt;

    const rsrc_t rx = make_rsrc(p.aq, p.aq_bytes);
    const rsrc_t rxs = make_rsrc(p.bst, p.bst_bytes);

    Ctx cur = decode(p, pass_off, i_lo + slot, wtiles, w, lane, r0);
    Ctx nxt = n_my > 1 ? decode(p, pass_off, i_lo + slot + grid, wtiles, w, lane, r0) : cur;

    stage_all<WFMT>(p, rx, rxs, cur, 0, true, ring, w, lane);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // B operand addresses of this lane's 8 token tiles within a stage: row
    // 16 j + r, chunks q (bytes 0-15) and 4 + q (bytes 16-31), swizzled
    int boff_lo[kBT], boff_hi[kBT];
    #pragma unroll
    for (int j = 0; j < kBT; ++j) {
        const int row = ti * 128 + 16 * j + r;
        boff_lo[j] = S::B + row * 128 + 16 * (q ^ bswz(row));
        boff_hi[j] = S::B + row * 128 + 16 * ((4 + q) ^ bswz(row));
    }

    f32x4 acc[kBT][kAT];
    // one K-tile of the item: step s of the workgroup's sequence
    // (full: false for a wave with no rows in the item, which only stages
    // its share of the operands and keeps the barriers)
    auto kstep = [&](int kt, int s, auto full) {
        // prefetch step s + 1 into the other stage (zeros past the last step)
        {
            const bool same = kt + 1 < nkt;
            stage_all<WFMT>(p, rx, rxs, same ? cur : nxt, same ? kt + 1 : 0, s + 1 < total,
                            ring + ((s + 1) & 1) * S::Bytes, w, lane);
        }
        if constexpr (decltype(full)::value) {
            const uint8_t* st = ring + (s & 1) * S::Bytes;
            // this wave's 4 weight tiles stay in registers for the K-tile; its
            // 8 token tiles stream from LDS, each against all 4, the next token
            // tile's reads in flight while the current one is multiplied
            const int ash = 8 * (kt & 3);
            i32x8 A[kAT];
            int sa[kAT];
            #pragma unroll
            for (int t = 0; t < kAT; ++t) {
                const int T = wi * kAT + t;
                const uint8_t* ap = st + S::A + T * 64 * S::kBPL + lane * 16;
                const i32x4 alo = *(const i32x4*)ap;
                const i32x4 ahi = WFMT == MFMA_FMT_FP8 ? *(const i32x4*)(ap + 1024) : i32x4{0, 0, 0, 0};
                A[t] = __builtin_shufflevector(alo, ahi, 0, 1, 2, 3, 4, 5, 6, 7);
                sa[t] = ((const int*)(st + S::AS))[T * 64 + lane];
            }
            auto load_b = [&](int j, i32x8& B, int& bs) {
                const i32x4 blo = *(const i32x4*)(st + boff_lo[j]);
                const i32x4 bhi = *(const i32x4*)(st + boff_hi[j]);
                B = __builtin_shufflevector(blo, bhi, 0, 1, 2, 3, 4, 5, 6, 7);
                bs = ((const int*)(st + S::BS))[ti * 128 + 16 * j + r];
            };
            i32x8 Bb[2];
            int bsb[2];
            load_b(0, Bb[0], bsb[0]);
            #pragma unroll
            for (int t = 0; t < kAT; ++t) sa[t] >>= ash;
            #pragma unroll
            for (int j = 0; j < kBT; ++j) {
                if (j + 1 < kBT) load_b(j + 1, Bb[(j + 1) & 1], bsb[(j + 1) & 1]);
                const int bs = bsb[j & 1] >> (8 * q);
                #pragma unroll
                for (int t = 0; t < kAT; ++t)
                    acc[j][t] = mfma16x16x128<WFMT, MFMA_FMT_FP8, 0, 0>(A[t], Bb[j & 1], acc[j][t], sa[t], bs);
            }
            // issue order: the weight tiles, their scales and the first two token
            // tiles; then per token tile its 4 MFMAs followed by the reads of the
            // token tile after next (the scheduler would otherwise reuse one
            // register buffer for every token tile and wait for each read)
            constexpr int kAR = WFMT == MFMA_FMT_FP8 ? 3 : 2;      // LDS reads per weight tile
            __builtin_amdgcn_sched_group_barrier(0x100, kAR * kAT + 6, 0);
            #pragma unroll
            for (int j = 0; j < kBT; ++j) {
                __builtin_amdgcn_sched_group_barrier(0x008, kAT, 0);
                if (j + 2 < kBT) __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
            }
        }
        __builtin_amdgcn_s_waitcnt(0);       // the next step's operands have landed
        __syncthreads();
    };
    for (int it = 0; it < n_my; ++it) {
        int s = it * nkt;
        // the waves of the second token half of a half pass (at most 128
        // rows) have no rows: they skip the MFMAs, LDS reads and epilogue
        // (whose stores all stop at the item's rows), and the other wave of
        // their SIMD runs alone (the forward modes; in the backward the
        // second copy of the K-loop made its epilogue spill 70% more)
        const bool idle = MODE != kModeBwd && ti * (kBT * 16) >= __builtin_amdgcn_readfirstlane(cur.nrows);
        if (idle) {
            for (int kt = 0; kt < nkt; ++kt, ++s) kstep(kt, s, std::false_type{});
        } else {
            #pragma unroll
            for (int j = 0; j < kBT; ++j)
                #pragma unroll
                for (int t = 0; t < kAT; ++t) acc[j][t] = f32x4{0.f, 0.f, 0.f, 0.f};
            for (int kt = 0; kt < nkt; ++kt, ++s) kstep(kt, s, std::true_type{});
        }

        // ---------------------------------------------------- epilogue
        const int tok0 = ti * (kBT * 16);
        const int uu = cur.wt * kUnits + wi;                    // this wave's unit
        if constexpr (IS_W1) {
            if (!idle) {
                // the stage just consumed serves as scratch; the next step's
                // prefetch lands in it only after the barrier below
                uint8_t* scratch = ring + ((s - 1) & 1) * S::Bytes;
                uint8_t* tw = scratch + w * kTWave;
                uint8_t* tsw = scratch + kWaves * kTWave + w * 128;
                float* xs = (float*)(scratch + kWaves * (kTWave + 128) + w * 2048);
                const int I = p.N / 2;
                // the item's rows of h, its scales and its routing weights
                const rsrc_t rhq = make_rsrc(p.hq + (size_t)cur.rbase * I, (uint32_t)(cur.nrows * I));
                const rsrc_t rhs = make_rsrc(p.hs + (size_t)cur.rbase * (I / 32), (uint32_t)(cur.nrows * (I / 32)));
                const rsrc_t rw_w = make_rsrc(p.row_w + cur.rbase, p.use_w ? (uint32_t)(cur.nrows * 4) : 0u);
                // the routing weights of this lane's 8 token rows, all requested
                // before the first is used (one memory latency per item, not 8);
                // rows past the item read 0 and have zero sums anyway
                // (without weights the resource is empty: the loads return 0 and
                // are replaced by 1 without a branch)
                float wrow[kBT];
                #pragma unroll
                for (int j = 0; j < kBT; ++j)
                    wrow[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                        rw_w, (uint32_t)((tok0 + 16 * j + r) * 4), 0, 0));
                #pragma unroll
                for (int j = 0; j < kBT; ++j) wrow[j] = p.use_w ? wrow[j] : 1.0f;
                // generic variant: this lane's 8 gate and 8 up biases (features
                // 32 uu + 16 a + 4 q + v), zero without a bias; the BF16
                // pre-activation copy goes to rows of 2I
                float bg[2][4] = {}, bu[2][4] = {};
                const bool spre = MODE == kModeW1Gen && p.save_pre;
                const rsrc_t rpre = make_rsrc(spre ? p.save_pre + (size_t)cur.rbase * 2 * I : (uint16_t*)p.hq,
                                              spre ? (uint32_t)(cur.nrows * 2 * I * 2) : 0u);
                if constexpr (MODE == kModeW1Gen) {
                    const rsrc_t rb = make_rsrc(p.bias + (size_t)cur.g * 2 * I, p.bias ? (uint32_t)(2 * I * 4) : 0u);
                    #pragma unroll
                    for (int a = 0; a < 2; ++a)
                        #pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            const uint32_t f = (uint32_t)(32 * uu + 16 * a + 4 * q + v);
                            bg[a][v] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rb, 4 * f, 0, 0));
                            bu[a][v] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rb, 4 * (f + I), 0, 0));
                        }
                }
                #pragma unroll
                for (int jp = 0; jp < kBT / 2; ++jp) {
                    float h[2][2][4];                               // [j in pair][gate tile][v]
                    #pragma unroll
                    for (int jj = 0; jj < 2; ++jj) {
                        const int j = 2 * jp + jj;
                        const int tok = tok0 + 16 * j + r;
                        // rows past the item have zero token rows, so zero sums and h = 0
                        const float wgt = wrow[j];
                        float amf = 0.f;
                        #pragma unroll
                        for (int a = 0; a < 2; ++a) {
                            if constexpr (MODE == kModeW1Gen) {
                                float gz[4], uz[4];
                                #pragma unroll
                                for (int v = 0; v < 4; ++v) {
                                    gz[v] = acc[j][a][v] + bg[a][v];
                                    uz[v] = acc[j][a + 2][v] + bu[a][v];
                                }
                                // pre-activation rows (dropped past the item's rows)
                                u32x2 pg, pu;
                                pg.x = bf16x2(gz[0], gz[1]); pg.y = bf16x2(gz[2], gz[3]);
                                pu.x = bf16x2(uz[0], uz[1]); pu.y = bf16x2(uz[2], uz[3]);
                                const uint32_t po = (uint32_t)((tok * 2 * I + 32 * uu + 16 * a + 4 * q) * 2);
                                __builtin_amdgcn_raw_buffer_store_b64(pg, rpre, po, 0, 0);
                                __builtin_amdgcn_raw_buffer_store_b64(pu, rpre, po + (uint32_t)(2 * I), 0, 0);
                                #pragma unroll
                                for (int v = 0; v < 4; ++v) {
                                    float g = gz[v], u = uz[v];
                                    if (p.limit > 0.f) {
                                        g = fminf(fmaxf(g, -p.limit), p.limit);
                                        u = fminf(fmaxf(u, -p.limit), p.limit);
                                    }
                                    const float hv = act_value(g, p.act, p.beta) * u * wgt;
                                    h[jj][a][v] = hv;
                                    amf = fmaxf(amf, fabsf(hv));
                                }
                            } else {
                                #pragma unroll
                                for (int v = 0; v < 4; ++v) {
                                    const float hv = silu_fast(acc[j][a][v]) * acc[j][a + 2][v] * wgt;
                                    h[jj][a][v] = hv;
                                    amf = fmaxf(amf, fabsf(hv));
                                }
                            }
                        }
                        // the unit's 32 features of this token: 4 lanes (q) x 8 values
                        const uint32_t am = rows4_umax(__float_as_uint(amf));
                        const uint32_t code = e4m3_scale_code(__uint_as_float(am), p.ceil_rule);
                        const float inv = inv_scale(code);
                        // rows past the item fall outside the resources' range: dropped
                        #pragma unroll
                        for (int a = 0; a < 2; ++a)
                            __builtin_amdgcn_raw_buffer_store_b32(
                                e4m3x4(h[jj][a][0] * inv, h[jj][a][1] * inv, h[jj][a][2] * inv, h[jj][a][3] * inv),
                                rhq, (uint32_t)(tok * I + 32 * uu + 16 * a + 4 * q), 0, 0);
                        __builtin_amdgcn_raw_buffer_store_b8((unsigned char)code, rhs,
                                                             q == 0 ? (uint32_t)(tok * (I / 32) + uu) : kInvalid, 0, 0);
                    }
                    // 32-token block jp of this wave, staged in LDS for the transposed copy
                    // (the generic variant keeps the register-only staging:
                    // its bias and pre-activation leave no registers for this one)
                    if (p.transpose) {
                        if constexpr (MODE == kModeW1) transpose_stage_f32(h, jp, xs, tw, tsw, lane, p.ceil_rule);
                        else transpose_stage(h, jp, tw, tsw, lane, p.ceil_rule);
                    }
                }
                if (p.transpose)
                    transpose_flush(tw, tsw, p.hTq, p.hTs, I, p.ldT, 32 * uu,
                                    p.offsets32[cur.g] + cur.pass * kRows + tok0, tok0, cur.nrows, lane);
            }
            __syncthreads();                 // scratch free before the next prefetch lands in it
        } else if constexpr (MODE == kModeBwd) {
            // dActivation epilogue. acc holds dh for this wave's 64 features
            // (weight tile t: features 64 uu + 16 t + 4 q + v) of 128 token
            // rows. Output rows are [dg | du], L = 2I bytes of E4M3 codes.
            uint8_t* scratch = ring + ((s - 1) & 1) * S::Bytes;
            uint8_t* tw = scratch + w * kTWave;
            uint8_t* tsw = scratch + kWaves * kTWave + w * 128;
            const int I = p.N, L = 2 * I;
            if (uu < units) {                // a partial last tile: waves past the last unit idle
                const rsrc_t rpre = make_rsrc(p.pre + (size_t)cur.rbase * L, (uint32_t)(cur.nrows * L * 2));
                const rsrc_t rdq = make_rsrc(p.hq + (size_t)cur.rbase * L, (uint32_t)(cur.nrows * L));
                const rsrc_t rds = make_rsrc(p.hs + (size_t)cur.rbase * (L / 32), (uint32_t)(cur.nrows * (L / 32)));
                const rsrc_t rw_w = make_rsrc(p.row_w + cur.rbase, p.use_w ? (uint32_t)(cur.nrows * 4) : 0u);
                const rsrc_t rdw = make_rsrc(p.dw_part + (size_t)cur.rbase * units,
                                             p.dw_part ? (uint32_t)(cur.nrows * units * 4) : 0u);
                const float lim = p.limit;
                // The epilogue walks the token tiles in runtime loops (compiled
                // once, not unrolled per tile, chunk and activation): the
                // token tile in hand is always acc[0] (acc[0..1] for a pair),
                // and the accumulators rotate by one tile per step, so every
                // index stays a compile-time one. A token tile's
                // pre-activations (gate and up of the unit's 64 features) and
                // routing weight are requested one step ahead.
                // weight tiles [T0, T0 + NTL): BF16 gate / up of features
                // 64 uu + 16 t + 4 q + [0, 4), and the token's routing weight
                struct PreAll { u32x2 g[kAT], u[kAT]; float w; };
                struct PrePair { u32x2 g[2], u[2]; float w; };
                auto load_pre = [&](int j, int T0, auto& P) {
                    constexpr int NTL = sizeof(P.g) / sizeof(P.g[0]);
                    const int tok = tok0 + 16 * j + r;
                    #pragma unroll
                    for (int i = 0; i < NTL; ++i) {
                        const uint32_t po = (uint32_t)((tok * L + 64 * uu + 16 * (T0 + i) + 4 * q) * 2);
                        P.g[i] = __builtin_amdgcn_raw_buffer_load_b64(rpre, po, 0, 0);
                        P.u[i] = __builtin_amdgcn_raw_buffer_load_b64(rpre, po + (uint32_t)(2 * I), 0, 0);
                    }
                    const float wl = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rw_w, (uint32_t)(tok * 4), 0, 0));
                    P.w = p.use_w ? wl : 1.0f;
                };
                // dg (xg) and du (xu) of one weight tile (entry i of P) for one
                // token tile's dh; returns the tile's part of the
                // routing-weight gradient, dh * act(g) * u over its 4 features
                auto dact_tile = [&](const f32x4& dh, const auto& P, int i, float (&xg)[4], float (&xu)[4]) -> float {
                    const float gv[4] = {bf16_to_f32(P.g[i].x & 0xFFFFu), bf16_to_f32(P.g[i].x >> 16),
                                         bf16_to_f32(P.g[i].y & 0xFFFFu), bf16_to_f32(P.g[i].y >> 16)};
                    const float uv[4] = {bf16_to_f32(P.u[i].x & 0xFFFFu), bf16_to_f32(P.u[i].x >> 16),
                                         bf16_to_f32(P.u[i].y & 0xFFFFu), bf16_to_f32(P.u[i].y >> 16)};
                    float dwp = 0.f;
                    #pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        float g = gv[v], u = uv[v], mg = 1.f, mu = 1.f;
                        if (lim > 0.f) {
                            mg = fabsf(g) <= lim ? 1.f : 0.f;
                            mu = fabsf(u) <= lim ? 1.f : 0.f;
                            g = fminf(fmaxf(g, -lim), lim);
                            u = fminf(fmaxf(u, -lim), lim);
                        }
                        float a, da;
                        act_and_grad(g, p.act, p.beta, a, da);
                        xg[v] = dh[v] * P.w * u * da * mg;
                        xu[v] = dh[v] * P.w * a * mu;
                        dwp += dh[v] * a * u;
                    }
                    return dwp;
                };
                auto rotate = [&](int by) {             // acc[i] <- acc[i + by], cyclically
                    f32x4 keep[2][kAT];
                    #pragma unroll
                    for (int i = 0; i < 2; ++i)
                        #pragma unroll
                        for (int t = 0; t < kAT; ++t) keep[i][t] = acc[i][t];
                    #pragma unroll
                    for (int i = 0; i < kBT - 2; ++i)
                        #pragma unroll
                        for (int t = 0; t < kAT; ++t) acc[i][t] = by == 1 ? acc[i + 1][t] : acc[i + 2][t];
                    #pragma unroll
                    for (int t = 0; t < kAT; ++t) {
                        acc[kBT - 2][t] = by == 1 ? acc[kBT - 1][t] : keep[0][t];
                        acc[kBT - 1][t] = by == 1 ? keep[0][t] : keep[1][t];
                    }
                };
                // Token tiles in pairs (one 32-token block): dg and du of both
                // tiles computed once, then their E4M3 rows with scales
                // (32-feature blocks: tiles 2b, 2b + 1), the dw part, and with
                // the transposed copy the block's four 32-feature chunks (dg
                // or du of tiles 2b, 2b + 1), staged in the wave's LDS area
                // and flushed as 32-byte row pieces.
                uint8_t* tw4 = scratch + w * (4 * (32 * kT32Stride + 32));
                const int col0 = p.transpose ? p.offsets32[cur.g] + cur.pass * kRows + tok0 : 0;
                #pragma nounroll
                for (int jp = 0; jp < kBT / 2; ++jp) {
                    PreAll P[2];
                    load_pre(2 * jp, 0, P[0]);
                    load_pre(2 * jp + 1, 0, P[1]);
                    float x[2][2][kAT][4];              // [token tile of the pair][dg, du][weight tile][v]
                    #pragma unroll
                    for (int jj = 0; jj < 2; ++jj) {
                        const int tok = tok0 + 16 * (2 * jp + jj) + r;
                        float dwp = 0.f;
                        #pragma unroll
                        for (int t = 0; t < kAT; ++t) dwp += dact_tile(acc[jj][t], P[jj], t, x[jj][0][t], x[jj][1][t]);
                        #pragma unroll
                        for (int half = 0; half < 2; ++half)
                            #pragma unroll
                            for (int b = 0; b < 2; ++b) {
                                float amf = 0.f;
                                #pragma unroll
                                for (int tt = 0; tt < 2; ++tt)
                                    #pragma unroll
                                    for (int v = 0; v < 4; ++v) amf = fmaxf(amf, fabsf(x[jj][half][2 * b + tt][v]));
                                const uint32_t am = rows4_umax(__float_as_uint(amf));
                                const uint32_t code = e4m3_scale_code(__uint_as_float(am), p.ceil_rule);
                                const float inv = inv_scale(code);
                                #pragma unroll
                                for (int tt = 0; tt < 2; ++tt) {
                                    const float* xv = x[jj][half][2 * b + tt];
                                    __builtin_amdgcn_raw_buffer_store_b32(
                                        e4m3x4(xv[0] * inv, xv[1] * inv, xv[2] * inv, xv[3] * inv), rdq,
                                        (uint32_t)(tok * L + half * I + 64 * uu + 16 * (2 * b + tt) + 4 * q), 0, 0);
                                }
                                __builtin_amdgcn_raw_buffer_store_b8(
                                    (unsigned char)code, rds,
                                    q == 0 ? (uint32_t)(tok * (L / 32) + half * (I / 32) + 2 * uu + b) : kInvalid, 0, 0);
                            }
                        // the routing weight's gradient: this unit's 64 features of the token
                        const float dws = rows4_sum(dwp);
                        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(dws), rdw,
                                                              q == 0 ? (uint32_t)((tok * units + uu) * 4) : kInvalid, 0, 0);
                    }
                    // a block that starts past the item's rows belongs to the
                    // next group's columns: not written
                    if (p.transpose && tok0 + 32 * jp < cur.nrows) {
                        #pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            const int half = c >> 1, b = c & 1;
                            float h2[2][2][4];
                            #pragma unroll
                            for (int jj = 0; jj < 2; ++jj)
                                #pragma unroll
                                for (int tt = 0; tt < 2; ++tt)
                                    #pragma unroll
                                    for (int v = 0; v < 4; ++v) h2[jj][tt][v] = x[jj][half][2 * b + tt][v];
                            uint8_t* twc = tw4 + c * (32 * kT32Stride + 32);
                            transpose_stage(h2, 0, twc, twc + 32 * kT32Stride, lane, p.ceil_rule, kT32Stride);
                        }
                        #pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            const int half = c >> 1, b = c & 1;
                            const uint8_t* twc = tw4 + c * (32 * kT32Stride + 32);
                            transpose_flush32(twc, twc + 32 * kT32Stride, p.hTq, p.hTs, L, p.ldT,
                                              half * I + 64 * uu + 32 * b, col0 + 32 * jp, lane);
                        }
                    }
                    rotate(2);
                }
            }
            __syncthreads();                 // scratch free before the next prefetch lands in it
        } else {
            // BF16 rows through LDS, 32 tokens at a time, so that each store
            // instruction writes whole 128-byte lines (8 rows x 64 features),
            // streamed out non-temporally: the burst of stores at the end of
            // an item then drains sooner, before the next K-tile's wait
            if (!idle) {
                const int H = p.N;
                uint8_t* ys = ring + ((s - 1) & 1) * S::Bytes + w * (32 * kYStride);
                #pragma unroll
                for (int c = 0; c < kBT / 2; ++c) {
                    #pragma unroll
                    for (int jj = 0; jj < 2; ++jj) {
                        const int j = 2 * c + jj;
                        #pragma unroll
                        for (int t = 0; t < kAT; ++t) {
                            uint2 o;
                            o.x = bf16x2(acc[j][t][0], acc[j][t][1]);
                            o.y = bf16x2(acc[j][t][2], acc[j][t][3]);
                            *(uint2*)(ys + (16 * jj + r) * kYStride + (16 * t + 4 * q) * 2) = o;
                        }
                    }
                    #pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int row = 8 * i + (lane >> 3), k16 = lane & 7;
                        const i32x4 d = *(const i32x4*)(ys + row * kYStride + 16 * k16);
                        const int tok = tok0 + 32 * c + row;
                        if (tok < cur.nrows)
                            __builtin_nontemporal_store(d, (i32x4*)(p.y + (size_t)(cur.rbase + tok) * H + 64 * uu + 8 * k16));
                    }
                }
            }
            __syncthreads();                 // scratch free before the next prefetch lands in it
        }
        cur = nxt;
        if (it + 2 < n_my) nxt = decode(p, pass_off, i_lo + slot + (it + 2) * grid, wtiles, w, lane, r0);
    }
}

// Scale tiles: out[(kt * npass + pass) * 256 + i] = the 4 E8M0 bytes of
// K-tile kt of row i of pass `pass` (passes numbered over all groups, as the
// GEMM numbers them), 0 for rows past the group's end. One workgroup per pass
// and 4 K-tiles; passes past the total are left unwritten (the GEMM never
// reads them).
__global__ __launch_bounds__(kRows)
void scale_tiles_kernel(const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets, int G,
                        const int32_t* __restrict__ row_src, const uint8_t* as, uint32_t as_bytes,
                        int K, int npass, uint32_t* __restrict__ out, int pass_lo = 0) {
    extern __shared__ int pass_off[];                                   // [G + 1]
    const int tid = threadIdx.x;
    if (tid < 64) pass_prefix(counts, G, kRows, tid, pass_off);
    __syncthreads();
    const int b = pass_lo + (int)blockIdx.x;
    if (b >= pass_off[G]) return;
    int glo = 0, ghi = G;                   // largest g with pass_off[g] <= b
    while (ghi - glo > 1) {
        const int mid = (glo + ghi) >> 1;
        if (pass_off[mid] <= b) glo = mid; else ghi = mid;
    }
    const int row = (b - pass_off[glo]) * kRows + tid;
    const bool valid = row < counts[glo];
    const int r = offsets[glo] + row;
    const uint32_t src = valid ? (uint32_t)(row_src ? row_src[r] : r) : 0u;
    const rsrc_t rs = make_rsrc(as, valid ? as_bytes : 0u);
    const int nkt = K / 128, kt0 = 4 * blockIdx.y;
    const uint32_t base = src * (uint32_t)(K / 32);
    uint32_t v[4];
    #pragma unroll
    for (int i = 0; i < 4; ++i)
        v[i] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rs, base + 4u * (kt0 + i), 0, 0);
    #pragma unroll
    for (int i = 0; i < 4; ++i)
        if (kt0 + i < nkt) out[((size_t)(kt0 + i) * npass + b) * kRows + tid] = v[i];
}

// Token ring fill: the grouped token rows of passes [pass0, pass0 + gridDim.x)
// copied one after another into a ring slot (the slot's first row is the
// first row of pass pass0), and their scale tiles written as
// scale_tiles_kernel writes them. Workgroup (x, y) serves rows
// [32y, 32y + 32) of pass pass0 + x: 16-byte pieces with kFillBatch loads in
// flight per thread before their stores; passes past the total are skipped.
constexpr int kFillRows = 32;               // rows per fill workgroup
constexpr int kFillBatch = 8;               // 16-byte loads in flight per thread

__global__ __launch_bounds__(kRows)
void ring_fill_kernel(const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets, int G,
                      const int32_t* __restrict__ row_src, const uint8_t* __restrict__ xq, uint32_t x_bytes,
                      const uint8_t* as, uint32_t as_bytes, int K, int npass, uint32_t* __restrict__ tiles,
                      int pass0, uint8_t* __restrict__ ring, uint32_t ring_bytes) {
    extern __shared__ int pass_off[];                                   // [G + 1], then kFillRows sources
    int* src_row = pass_off + G + 1;
    const int tid = threadIdx.x;
    if (tid < 64) pass_prefix(counts, G, kRows, tid, pass_off);
    __syncthreads();
    const int b = pass0 + (int)blockIdx.x;
    if (b >= pass_off[G] || pass0 >= pass_off[G]) return;
    auto row_of = [&](int pass) {           // group and first grouped row of a pass
        int glo = 0, ghi = G;
        while (ghi - glo > 1) {
            const int mid = (glo + ghi) >> 1;
            if (pass_off[mid] <= pass) glo = mid; else ghi = mid;
        }
        return std::pair<int, int>(glo, offsets[glo] + (pass - pass_off[glo]) * kRows);
    };
    const auto [g, pstart] = row_of(b);
    const int r0 = row_of(pass0).second;
    const int rin0 = kFillRows * (int)blockIdx.y;                       // first row within the pass
    const int rstart = pstart + rin0;
    const int nrows = max(0, min(kFillRows, offsets[g] + counts[g] - rstart));
    if (tid < kFillRows) src_row[tid] = tid < nrows ? row_src[rstart + tid] : -1;
    __syncthreads();

    // scale tiles of these rows (0 past the group's end)
    const rsrc_t rs = make_rsrc(as, as_bytes);
    const int nkt = K / 128;
    for (int t = tid; t < kFillRows * nkt; t += kRows) {
        const int i = t % kFillRows, kt = t / kFillRows;
        const int src = src_row[i];
        const uint32_t v = src >= 0 ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(
                                          rs, (uint32_t)src * (uint32_t)(K / 32) + 4u * kt, 0, 0)
                                    : 0u;
        tiles[((size_t)kt * npass + b) * kRows + rin0 + i] = v;
    }

    // token rows
    const rsrc_t rx = make_rsrc(xq, x_bytes);
    const rsrc_t rr = make_rsrc(ring, ring_bytes);
    const int chunks = K / 16;                                          // 16-byte pieces per row
    const int n = nrows * chunks;
    for (int e0 = 0; e0 < n; e0 += kRows * kFillBatch) {
        i32x4 v[kFillBatch];
        uint32_t dst[kFillBatch];
        #pragma unroll
        for (int j = 0; j < kFillBatch; ++j) {
            const int e = e0 + j * kRows + tid;
            const int i = e / chunks, c = e - i * chunks;
            const bool ok = e < n;
            const uint32_t src = ok ? (uint32_t)src_row[i] : 0u;
            v[j] = ok ? __builtin_amdgcn_raw_buffer_load_b128(rx, src * (uint32_t)K + 16 * c, 0, 0) : i32x4{0, 0, 0, 0};
            dst[j] = ok ? (uint32_t)(rstart + i - r0) * K + 16 * c : 0xFFFFFFFFu;
        }
        #pragma unroll
        for (int j = 0; j < kFillBatch; ++j)
            if (dst[j] != 0xFFFFFFFFu) __builtin_amdgcn_raw_buffer_store_b128(v[j], rr, dst[j], 0, 0);
    }
}

template <int WFMT, int MODE>
int launch_tiled(const KParams& p, int R_max, hipStream_t stream, int max_grid = 0) {
    auto kern = tiled_gemm_kernel<WFMT, MODE>;
    const size_t lds = 2 * (size_t)Stage<WFMT>::Bytes + (size_t)(p.G + 1) * 4;
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kThreads, lds) != hipSuccess || per_cu < 1)
        per_cu = 1;
    const long wtiles = (p.N / 64 + kUnits - 1) / kUnits;
    // passes never exceed R_max / 256 + G: each group adds at most one partial pass
    const long max_items = wtiles * ((long)R_max / kRows + p.G);
    long grid = std::max<long>(1, std::min<long>(max_items, (long)per_cu * device_cu_count()));
    if (max_grid > 0) grid = std::min<long>(grid, max_grid);
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreads), lds, stream, p);
    return (int)hipGetLastError();
}

// dw[r] = sum over the units u of part[r][u], in unit order, for the rows of
// the groups (r < offsets[G]); one thread per row.
__global__ __launch_bounds__(256)
void dw_reduce_kernel(const float* __restrict__ part, int units, const int32_t* __restrict__ offsets,
                      int G, int R_max, float* __restrict__ dw) {
    const int r = blockIdx.x * 256 + threadIdx.x;
    if (r >= R_max || r >= offsets[G]) return;
    float s = 0.f;
    for (int u = 0; u < units; ++u) s += part[(size_t)r * units + u];
    dw[r] = s;
}

// The activation scales as scale tiles in the workspace; fills p.bst.
int launch_scale_tiles(const GemmArgs& a, KParams& p, hipStream_t stream) {
    const int npass = a.R_max / kRows + a.G;
    const size_t need = moe_tiled_scale_bytes(a.R_max, a.G, a.K);
    if (!a.ws || a.ws_bytes < need || need > 0x7FFFFFFFu) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(scale_tiles_kernel, dim3((unsigned)npass, (unsigned)(a.K / 128 + 3) / 4), dim3(kRows),
                       (size_t)(a.G + 1) * 4, stream,
                       a.counts, a.offsets, a.G, a.row_src, a.as, p.as_bytes, a.K, npass, (uint32_t*)a.ws);
    p.bst = (const uint32_t*)a.ws;
    p.bst_bytes = (uint32_t)need;
    p.npass = npass;
    return (int)hipGetLastError();
}

}  // namespace

// bytes of one token-ring slot: kRingPasses passes of 256 rows of K bytes
size_t moe_ring_slot_bytes(int K) { return (size_t)kRingPasses * kRows * K; }

// passes never exceed R_max / 256 + G (each group adds at most one partial
// pass); one 4-byte word per row, pass and K-tile
size_t moe_tiled_scale_bytes(int R_max, int G, int K) {
    return ((size_t)R_max / kRows + G) * kRows * (size_t)(K / 128) * 4;
}

int moe_launch_tiled_w1(const GemmArgs& a, hipStream_t stream) {
    if (a.G == 0 || a.R_max == 0) return 0;
    KParams p = make_params(a, true);
    if (int e = launch_scale_tiles(a, p, stream)) return e;
    const bool fp4 = a.fmt == MOE_FMT_MXFP4;
    if (p.generic)
        return fp4 ? launch_tiled<MFMA_FMT_FP4, kModeW1Gen>(p, a.R_max, stream)
                   : launch_tiled<MFMA_FMT_FP8, kModeW1Gen>(p, a.R_max, stream);
    return fp4 ? launch_tiled<MFMA_FMT_FP4, kModeW1>(p, a.R_max, stream)
               : launch_tiled<MFMA_FMT_FP8, kModeW1>(p, a.R_max, stream);
}

// W1 fed through a token ring (see moe_layer, MOE_LAYER_TOKEN_RING): chunks of
// kRingPasses passes; for chunk c, on `side`: wait until the slot's previous
// chunk is consumed (event), fill the slot with the chunk's rows and write
// their scale tiles (one kernel), record "ready"; on `stream`: wait for "ready", run W1 on the chunk's
// items (grid capped so that kRingCUs compute units stay free for the
// producer), record "consumed". ev: [0] fork, [1 + s] ready of slot s,
// [1 + slots + s] consumed of slot s.
int moe_launch_tiled_w1_ring(const GemmArgs& a, uint8_t* ring, size_t slot_bytes, int slots,
                             hipStream_t stream, hipStream_t side, hipEvent_t* ev) {
    if (a.G == 0 || a.R_max == 0) return 0;
    KParams p = make_params(a, true);
    const int npass = a.R_max / kRows + a.G;                 // every pass the layout allows
    const size_t need = moe_tiled_scale_bytes(a.R_max, a.G, a.K);
    if (!a.ws || a.ws_bytes < need || need > 0x7FFFFFFFu) return (int)hipErrorInvalidValue;
    p.bst = (const uint32_t*)a.ws;
    p.bst_bytes = (uint32_t)need;
    p.npass = npass;
    const int wtiles = (a.N / 64 + kUnits - 1) / kUnits;     // as the kernel counts them
    const int chunks = (npass + kRingPasses - 1) / kRingPasses;
    const int max_grid = std::max(1, device_cu_count() - kRingCUs);
    const bool fp4 = a.fmt == MOE_FMT_MXFP4;
    int e;
    if ((e = (int)hipEventRecord(ev[0], stream))) return e;
    if ((e = (int)hipStreamWaitEvent(side, ev[0], 0))) return e;
    for (int c = 0; c < chunks; ++c) {
        const int sl = c % slots;
        uint8_t* slot = ring + (size_t)sl * slot_bytes;
        if (c >= slots && (e = (int)hipStreamWaitEvent(side, ev[1 + slots + sl], 0))) return e;
        hipLaunchKernelGGL(ring_fill_kernel, dim3(kRingPasses, kRows / kFillRows), dim3(kRows),
                           (size_t)(a.G + 1 + kFillRows) * 4, side, a.counts, a.offsets, a.G, a.row_src, a.aq,
                           p.aq_bytes, a.as, p.as_bytes, a.K, npass, (uint32_t*)a.ws, c * kRingPasses, slot,
                           (uint32_t)slot_bytes);
        if ((e = (int)hipGetLastError())) return e;
        if ((e = (int)hipEventRecord(ev[1 + sl], side))) return e;
        if ((e = (int)hipStreamWaitEvent(stream, ev[1 + sl], 0))) return e;
        KParams q = p;
        q.item_lo = c * kRingPasses * wtiles;
        q.item_hi = (c + 1) * kRingPasses * wtiles;
        q.ring_pass0 = c * kRingPasses;
        q.aq = slot;
        q.aq_bytes = (uint32_t)slot_bytes;
        q.row_src = nullptr;
        e = p.generic ? (fp4 ? launch_tiled<MFMA_FMT_FP4, kModeW1Gen>(q, a.R_max, stream, max_grid)
                             : launch_tiled<MFMA_FMT_FP8, kModeW1Gen>(q, a.R_max, stream, max_grid))
                      : (fp4 ? launch_tiled<MFMA_FMT_FP4, kModeW1>(q, a.R_max, stream, max_grid)
                             : launch_tiled<MFMA_FMT_FP8, kModeW1>(q, a.R_max, stream, max_grid));
        if (e) return e;
        if ((e = (int)hipEventRecord(ev[1 + slots + sl], stream))) return e;
    }
    return 0;
}

int moe_launch_tiled_w2(const GemmArgs& a, hipStream_t stream) {
    if (a.G == 0 || a.R_max == 0) return 0;
    KParams p = make_params(a, false);
    if (int e = launch_scale_tiles(a, p, stream)) return e;
    return a.fmt == MOE_FMT_MXFP4 ? launch_tiled<MFMA_FMT_FP4, kModeW2>(p, a.R_max, stream)
                                  : launch_tiled<MFMA_FMT_FP8, kModeW2>(p, a.R_max, stream);
}

int moe_launch_tiled_backward(const GemmArgs& a, float* dw, hipStream_t stream) {
    if (a.G == 0 || a.R_max == 0) return 0;
    KParams p = make_params(a, false);
    // the backward's own parameters: the forward epilogue variant (act, beta,
    // limit), the transposed copy, the routing weights whenever given
    p.transpose = (a.flags & MOE_W1_WRITE_TRANSPOSE) ? 1 : 0;
    p.use_w = a.row_w ? 1 : 0;
    if (a.epi) { p.act = a.epi->act; p.beta = a.epi->beta; p.limit = a.epi->limit; }
    if (int e = launch_scale_tiles(a, p, stream)) return e;
    const int e = a.fmt == MOE_FMT_MXFP4 ? launch_tiled<MFMA_FMT_FP4, kModeBwd>(p, a.R_max, stream)
                                         : launch_tiled<MFMA_FMT_FP8, kModeBwd>(p, a.R_max, stream);
    if (e || !dw) return e;
    hipLaunchKernelGGL(dw_reduce_kernel, dim3((unsigned)((a.R_max + 255) / 256)), dim3(256), 0, stream,
                       a.dw_part, a.N / 64, a.offsets, a.G, a.R_max, dw);
    return (int)hipGetLastError();
}
