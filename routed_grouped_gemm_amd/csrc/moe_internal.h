// Internal launcher interface between the C-ABI layer and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>
#include "../../include/moe.h"

// Prepacked weight geometry (see prepack.hip): 64-row units, 128-wide K tiles.
struct PackGeom {
    int units;        // N / 64
    int kt;           // K / 128
    int kt4;          // ceil(kt / 4)
    int bpl;          // bytes per lane per 16x128 tile: 16 (FP4) or 32 (FP8)
    size_t data_per_unit;   // kt * 4 tiles * 64 lanes * bpl
    size_t scale_per_unit;  // kt4 * 4 tiles * 64 lanes * 4
    size_t data_per_group, scale_per_group;
    size_t group_stride;    // data_per_group + scale_per_group (scales follow the data)
    size_t total;
};
PackGeom moe_pack_geom(int G, int N, int K, int fmt);

// Launchers return 0 or a hipError_t value.
int moe_launch_route(const float* logits, int T, int E, int k, uint32_t flags,
                     int32_t* topk_idx, float* topk_w, hipStream_t stream);

size_t moe_permute_scratch_bytes(int T, int k, int G);
int moe_launch_permute(const int32_t* topk_idx, const float* topk_w, int T, int k, int e0,
                       int E_loc, int s, const uint8_t* xq, const uint8_t* xs, int H,
                       int32_t* counts, int32_t* offsets, int32_t* offsets32, int32_t* row_src,
                       float* row_w, int32_t* slot_row, uint8_t* xq_perm, uint8_t* xs_perm,
                       void* scratch, hipStream_t stream);

bool moe_route_permute_fusable(int T, int E, int k, int E_loc, int s);
int moe_launch_route_permute(const float* logits, int T, int E, int k, uint32_t flags, int e0,
                             int E_loc, int s, int32_t* topk_idx, float* topk_w, int32_t* counts,
                             int32_t* offsets, int32_t* offsets32, int32_t* row_src, float* row_w,
                             int32_t* slot_row, hipStream_t stream);

// Routing inputs and outputs for a W1 launch that routes its own tokens.
struct RouteArgs {
    const float* logits;
    int T, E_tot, k, e0;
    uint32_t flags;
    int32_t* topk_idx; float* topk_w; int32_t* slot_row;
};

struct GemmArgs {
    const uint8_t* w_base[2];    // prepacked routed groups, shared group
    int E_loc;                   // groups < E_loc use [0], group E_loc uses [1]
    int G, N, K, fmt;
    const int32_t* counts;
    const int32_t* offsets;
    const int32_t* offsets32;
    const float* row_w;          // W1 only; null = weight 1
    const uint8_t* aq;           // activations [R_max, K] E4M3 (or [T, K] with row_src)
    const uint8_t* as;           // [R_max, K/32]               (or [T, K/32])
    const int32_t* row_src;      // null, or: grouped row r reads activation row row_src[r]
    int x_rows;                  // rows of aq / as
    int R_max;
    int rows_hint;               // expected rows per group (0: R_max / G)
    int active_hint;             // expected groups with rows (0: derived from rows_hint)
    uint32_t flags;
    uint8_t* hq; uint8_t* hs;    // W1 outputs
    uint8_t* hTq; uint8_t* hTs; int ldT;
    uint16_t* y;                 // W2 output
    void* ws; size_t ws_bytes;   // workspace (moe_grouped_workspace_size bytes)
    // W1 only, optional: the epilogue variant (null: SwiGLU, beta = 1)
    const moe_epilogue* epi;
    // backward only: the saved pre-activation and the routing-weight
    // gradient's per-unit partials (workspace)
    const uint16_t* pre;
    float* dw_part;
    // W1 only, optional: route and group the tokens inside the W1 launch
    // (counts, offsets, offsets32, row_src and row_w are then written, not
    // read); only when moe_w1_can_route says so
    const RouteArgs* route;
};
int moe_launch_grouped_w1(const GemmArgs& a, hipStream_t stream);
// Whether the W1 launch for these shapes can route its own tokens.
bool moe_w1_can_route(int T, int E_tot, int k, int E_loc, int s, int R_max, int H, int I,
                      int rows_hint, uint32_t flags);
int moe_launch_grouped_w2(const GemmArgs& a, hipStream_t stream);
// Whether the grouped GEMM launch takes the LDS-tiled kernel for these arguments.
bool moe_grouped_uses_tiled(const GemmArgs& a);
// LDS-tiled variants for groups with many rows (256 x 256 workgroup tiles)
int moe_launch_tiled_w1(const GemmArgs& a, hipStream_t stream);
// the pass-resident streaming kernel (gemm_pass.hip): whether passes of NT
// 16-row token tiles fit its staging for this K and G, and the launch
bool moe_pass_fits(int K, int G, int NT, int fmt);
int moe_launch_pass(const GemmArgs& a, bool w1, int NT, hipStream_t stream);
int moe_launch_tiled_w2(const GemmArgs& a, hipStream_t stream);
// The backward of the fused W1 epilogue on the LDS-tiled kernel: the W2^T
// GEMM with the dActivation epilogue (outputs in a.hq/hs/hTq/hTs with rows
// of 2 * a.N bytes, partials of the routing-weight gradient in a.dw_part),
// then the sum of those partials into dw (when dw is non-null).
int moe_launch_tiled_backward(const GemmArgs& a, float* dw, hipStream_t stream);
// W1 on the LDS-tiled kernel fed through a token ring filled on `side`
// (events ev: 1 + 2 * slots), and the bytes of one ring slot for K.
int moe_launch_tiled_w1_ring(const GemmArgs& a, uint8_t* ring, size_t slot_bytes, int slots,
                             hipStream_t stream, hipStream_t side, hipEvent_t* ev);
size_t moe_ring_slot_bytes(int K);
// Workspace of the tiled kernels: the activation scales rearranged per K-tile
// and 256-row pass (see gemm_tiled.hip).
size_t moe_tiled_scale_bytes(int R_max, int G, int K);

// The single-launch decode layer (fused_decode.hip): whether it applies, the
// words of its control block, and the launch (a1/a2 as moe_layer prepares
// them for W1, with its routing arguments, and W2).
bool moe_fused_decode_ok(int T, int E_tot, int k, int E_loc, int s, uint32_t flags);
size_t moe_fused_ctrl_words(int G, int H);
int moe_launch_fused_decode(const GemmArgs& a1, const GemmArgs& a2, uint32_t* ctrl, uint16_t* out,
                            hipStream_t stream);

int moe_launch_combine(const uint16_t* y, const int32_t* slot_row, const float* row_w, int T,
                       int ks, int H, uint16_t* out, hipStream_t stream);
// W2 and the combine in one launch for at most 16 tokens and few active
// groups (w2_combine.hip): whether it applies, and the launch (a: the W2
// arguments; comb_w: the routing weights applied in the combine, or null)
bool moe_w2_combine_ok(int T, int R_max, int G, int H, int I, int active_hint, uint32_t flags);
int moe_launch_w2_combine(const GemmArgs& a, const int32_t* slot_row, const float* comb_w, int T, int ks,
                          uint16_t* out, hipStream_t stream);
int moe_launch_hbm_read_probe(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream);
int moe_launch_quantize(const float* src, int rows, int K, int fmt, uint32_t flags,
                        uint8_t* q, uint8_t* s, hipStream_t stream);
int moe_launch_prepack(const uint8_t* q, const uint8_t* sc, int G, int N, int K, int fmt,
                       int is_w1, uint8_t* dst, hipStream_t stream);
