// Pieces shared by the grouped GEMM kernels (decode-shaped and tiled): the
// kernel parameter block, buffer resources, the per-group pass prefix and the
// CU count. Internal to libmoe.
#pragma once
#include "moe_device.h"
#include "moe_internal.h"

namespace {

constexpr uint32_t kInvalid = 0x80000000u;  // offset past every bounded region
constexpr int kNonTemporal = 2;             // cache policy of loads streamed once (weights)

struct KParams {
    const uint8_t* wbase[2];
    size_t gstride, dpg, dpu, spu;   // group stride; data bytes per group; per unit data / scales
    int E_loc, G, K, kt, kt4;
    const int32_t* counts;
    const int32_t* offsets;
    const int32_t* offsets32;
    const float* row_w;
    const uint8_t* aq;
    const uint8_t* as;
    uint32_t aq_bytes, as_bytes;      // sizes of the activation arrays (bounds of the loads)
    const int32_t* row_src;           // null: grouped row r is activation row r
    int N;                            // W1: 2I ; W2: H (y row length)
    int ceil_rule, transpose, use_w;
    uint8_t* hq; uint8_t* hs; uint8_t* hTq; uint8_t* hTs; int ldT;
    uint16_t* y;
    const uint32_t* bst;              // tiled kernels: activation scales per K-tile and pass
    uint32_t bst_bytes;
    int npass;                        // passes the scale tiles are laid out for
    // tiled kernels: the work items [item_lo, item_hi) only; with ring_pass0
    // >= 0 the token rows come from a ring slot (aq) holding the grouped rows
    // from the first row of pass ring_pass0 on, one after another
    int item_lo, item_hi, ring_pass0;
    int pass_kc;                      // pass-resident kernel: K-tiles per staged chunk of token rows
    // W1 epilogue variant (act, beta, clamp limit, per-group bias [G][2I],
    // optional BF16 copy of the pre-activation [R_max, 2I]); generic = 0 is
    // SwiGLU with beta = 1 and none of the options
    int generic, act;
    float beta, limit;
    const float* bias;
    uint16_t* save_pre;
    // backward (dActivation) epilogue: the saved pre-activation [R_max, 2I]
    // (BF16), and the per-unit partial sums of the routing-weight gradient
    // [R_max][N / 64]
    const uint16_t* pre;
    float* dw_part;
    // decode W1 that routes its own tokens (logits non-null): every workgroup
    // routes and groups the T tokens in LDS, workgroup 0 writes the results
    // to the routing outputs and to counts .. row_w above
    const float* logits;
    int T, E_tot, k_top, renorm, e0, R_max;
    int32_t* topk_idx; float* topk_w; int32_t* slot_row;
};

typedef __amdgpu_buffer_rsrc_t rsrc_t;
MOE_DEV rsrc_t make_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}

// Wave 0: pass_off[g] = sum over g' < g of ceil(counts[g'] / rpp), and
// pass_off[G] = the total, in LDS.
MOE_DEV void pass_prefix(const int32_t* __restrict__ counts, int G, int rpp, int lane,
                         int* pass_off) {
    const int per = (G + 63) / 64;
    const int lo = min(G, lane * per), hi = min(G, lo + per);
    int s = 0;
    for (int i = lo; i < hi; ++i) s += (counts[i] + rpp - 1) / rpp;
    const int inc = wave_incl_scan(s);
    int run = inc - s;
    for (int i = lo; i < hi; ++i) {
        pass_off[i] = run;
        run += (counts[i] + rpp - 1) / rpp;
    }
    if (lane == 63) pass_off[G] = inc;
}

inline KParams make_params(const GemmArgs& a, bool w1) {
    KParams p{};
    PackGeom geo = moe_pack_geom(1, a.N, a.K, a.fmt);
    for (int i = 0; i < 2; ++i) p.wbase[i] = a.w_base[i];
    p.gstride = geo.group_stride; p.dpg = geo.data_per_group;
    p.dpu = geo.data_per_unit;    p.spu = geo.scale_per_unit;
    p.E_loc = a.E_loc; p.G = a.G; p.K = a.K; p.kt = geo.kt; p.kt4 = geo.kt4;
    p.counts = a.counts; p.offsets = a.offsets; p.offsets32 = a.offsets32;
    p.row_w = a.row_w; p.aq = a.aq; p.as = a.as; p.row_src = a.row_src; p.N = a.N;
    p.aq_bytes = (uint32_t)((size_t)a.x_rows * a.K);
    p.as_bytes = (uint32_t)((size_t)a.x_rows * (a.K / 32));
    p.ceil_rule = (a.flags & MOE_SCALE_RULE_CEIL) ? 1 : 0;
    p.transpose = (w1 && (a.flags & MOE_W1_WRITE_TRANSPOSE)) ? 1 : 0;
    p.use_w = (w1 && a.row_w && !(a.flags & MOE_WEIGHT_AT_COMBINE)) ? 1 : 0;
    p.hq = a.hq; p.hs = a.hs; p.hTq = a.hTq; p.hTs = a.hTs; p.ldT = a.ldT;
    p.y = a.y;
    if (a.epi && w1) {
        p.act = a.epi->act; p.beta = a.epi->beta; p.limit = a.epi->limit;
        p.bias = a.epi->bias; p.save_pre = a.epi->save_pre;
        p.generic = (p.act != MOE_ACT_SWIGLU || p.beta != 1.0f || p.limit > 0.0f || p.bias ||
                     p.save_pre) ? 1 : 0;
    } else {
        p.act = MOE_ACT_SWIGLU; p.beta = 1.0f;
    }
    p.pre = a.pre; p.dw_part = a.dw_part;
    if (a.route) {
        p.logits = a.route->logits;
        p.T = a.route->T; p.E_tot = a.route->E_tot; p.k_top = a.route->k; p.e0 = a.route->e0;
        p.renorm = (a.route->flags & MOE_ROUTE_RENORM) ? 1 : 0;
        p.topk_idx = a.route->topk_idx; p.topk_w = a.route->topk_w; p.slot_row = a.route->slot_row;
    }
    p.R_max = a.R_max;
    p.item_lo = 0;
    p.item_hi = 0x7FFFFFFF;
    p.ring_pass0 = -1;
    return p;
}

inline int device_cu_count() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cached[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

}  // namespace
