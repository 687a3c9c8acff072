// C ABI of libmoe: argument validation, workspace carving and the launch
// sequence of the layer. Validation touches no HIP API, so argument errors can
// be checked on a machine without a GPU; nothing here allocates device memory,
// synchronises or reads device data.
#include <hip/hip_runtime.h>
#include <math.h>
#include <string.h>

#include <mutex>

#include "moe_internal.h"

#define MOE_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

inline int32_t hip_status(int e) { return e == 0 ? MOE_OK : MOE_ERR_HIP; }

bool fmt_ok(int fmt) { return fmt == MOE_FMT_MXFP4 || fmt == MOE_FMT_MXFP8; }

int32_t check_weights(const moe_weights* w, int G, int N, int K, int is_w1) {
    if (!w || !w->data) return MOE_ERR_NULL;
    if (!fmt_ok(w->fmt)) return MOE_ERR_UNSUPPORTED;
    if (w->G != G || w->N != N || w->K != K || w->is_w1 != is_w1) return MOE_ERR_SHAPE;
    if (w->bytes < moe_prepacked_size(G, N, K, w->fmt)) return MOE_ERR_WORKSPACE;
    return MOE_OK;
}

// Workspace layout of moe_layer (all regions 256-byte aligned).
constexpr int kRegions = 13;
struct LayerLayout {
    size_t off[kRegions];
    size_t total;
};

constexpr int kRingSlots = 2;

LayerLayout layer_layout(int T, int E_tot, int k, int E_loc, int H, int I, int s, uint32_t flags) {
    (void)E_tot;
    const size_t R = (size_t)T * k + (size_t)s * T;
    const int G = E_loc + s;
    size_t sz[kRegions] = {
        (size_t)T * k * 4,            // topk_idx
        (size_t)T * k * 4,            // topk_w
        (size_t)G * 4,                // counts
        (size_t)(G + 1) * 4,          // offsets
        (size_t)(G + 1) * 4,          // offsets32
        R * 4,                        // row_src
        R * 4,                        // row_w
        (size_t)T * (k + s) * 4,      // slot_row
        R * I,                        // hq
        R * (I / 32),                 // hs
        R * H * 2,                    // y
        0,                            // scratch
        moe_fused_ctrl_words(G, H) * 4,   // control block of the single-launch path
    };
    size_t gws1 = moe_grouped_workspace_size((int)R, G, 2 * I, H);
    size_t gws2 = moe_grouped_workspace_size((int)R, G, H, I);
    size_t pws = moe_permute_workspace_size(T, k, G);
    // with the token ring, the ring's slots follow W1's scale tiles
    if (flags & MOE_LAYER_TOKEN_RING) gws1 = align_up(gws1) + kRingSlots * moe_ring_slot_bytes(H);
    size_t scr = pws > gws1 ? pws : gws1;
    sz[11] = scr > gws2 ? scr : gws2;
    LayerLayout L;
    size_t o = 0;
    for (int i = 0; i < kRegions; ++i) {
        L.off[i] = o;
        o += align_up(sz[i]);
    }
    L.total = o;
    return L;
}

// The token ring's producer stream and its events, one set per device,
// created on first use. The stream has the default priority; it is
// restricted to kRingProducerCUs compute units (every 16th) where the
// runtime can create such a stream, and unrestricted otherwise.
constexpr int kRingProducerCUs = 16;
struct RingResources {
    hipStream_t side = nullptr;
    hipEvent_t ev[1 + 2 * kRingSlots] = {};
    bool cu_masked = false;
};
std::mutex g_ring_lock;
RingResources g_ring[64];

const RingResources* ring_resources() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    std::lock_guard<std::mutex> hold(g_ring_lock);
    RingResources& r = g_ring[dev];
    if (!r.side) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            return nullptr;
        const int words = (cus + 31) / 32;
        uint32_t mask[64] = {};
        const int stride = cus / kRingProducerCUs > 0 ? cus / kRingProducerCUs : 1;
        for (int i = 0; i < kRingProducerCUs && i * stride < cus && words <= 64; ++i)
            mask[(i * stride) / 32] |= 1u << ((i * stride) % 32);
        hipStream_t s = nullptr;
        if (words <= 64 && hipExtStreamCreateWithCUMask(&s, (uint32_t)words, mask) == hipSuccess && s) {
            r.cu_masked = true;
        } else {
            (void)hipGetLastError();           // the failed creation's error must not reach later calls
            s = nullptr;
            if (hipStreamCreateWithFlags(&s, hipStreamNonBlocking) != hipSuccess || !s) {
                (void)hipGetLastError();
                return nullptr;
            }
        }
        for (auto& e : r.ev) {
            if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) {
                (void)hipGetLastError();
                return nullptr;
            }
        }
        r.side = s;
    }
    return &r;
}

}  // namespace

MOE_EXPORT const char* moe_status_string(int32_t status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_ERR_NULL: return "a required pointer is NULL";
        case MOE_ERR_SHAPE: return "a size violates the layer's limits";
        case MOE_ERR_UNSUPPORTED: return "unsupported format or flag combination";
        case MOE_ERR_WORKSPACE: return "workspace or destination buffer too small";
        case MOE_ERR_HIP: return "a HIP kernel launch failed";
        default: return "unknown status";
    }
}

MOE_EXPORT const char* moe_version(void) { return "moe-mi355x 0.1.0 gfx950"; }

// ---------------------------------------------------------------- weights
MOE_EXPORT size_t moe_prepacked_size(int32_t G, int32_t N, int32_t K, int32_t fmt) {
    if (G < 0 || N <= 0 || K <= 0 || N % 64 || K % 128 || !fmt_ok(fmt)) return 0;
    return moe_pack_geom(G, N, K, fmt).total;
}

MOE_EXPORT int32_t moe_prepack_weights(const uint8_t* q, const uint8_t* sc, int32_t G, int32_t N,
                                       int32_t K, int32_t fmt, int32_t is_w1, void* dst,
                                       size_t dst_bytes, hipStream_t stream) {
    if (!fmt_ok(fmt)) return MOE_ERR_UNSUPPORTED;
    if (G < 0 || N <= 0 || K <= 0 || N % 64 || K % 128) return MOE_ERR_SHAPE;
    if (is_w1 && ((N / 2) % 32)) return MOE_ERR_SHAPE;
    if (G == 0) return MOE_OK;
    if (!q || !sc || !dst) return MOE_ERR_NULL;
    if (dst_bytes < moe_prepacked_size(G, N, K, fmt)) return MOE_ERR_WORKSPACE;
    return hip_status(moe_launch_prepack(q, sc, G, N, K, fmt, is_w1, (uint8_t*)dst, stream));
}

MOE_EXPORT int32_t moe_quantize_mx(const float* src, int32_t rows, int32_t K, int32_t fmt,
                                   uint32_t flags, uint8_t* q, uint8_t* s, hipStream_t stream) {
    if (!fmt_ok(fmt)) return MOE_ERR_UNSUPPORTED;
    if (rows < 0 || K <= 0 || K % 32) return MOE_ERR_SHAPE;
    if (rows == 0) return MOE_OK;
    if (!src || !q || !s) return MOE_ERR_NULL;
    return hip_status(moe_launch_quantize(src, rows, K, fmt, flags, q, s, stream));
}

MOE_EXPORT int32_t moe_hbm_read_probe(const void* src, size_t bytes, uint32_t* sink,
                                      hipStream_t stream) {
    if (bytes % 16 || bytes > ((size_t)1 << 31)) return MOE_ERR_SHAPE;
    if (bytes == 0) return MOE_OK;
    if (!src || !sink) return MOE_ERR_NULL;
    return hip_status(moe_launch_hbm_read_probe(src, bytes, sink, stream));
}

// ------------------------------------------------------------------ route
MOE_EXPORT int32_t moe_route(const float* logits, int32_t T, int32_t E_tot, int32_t k,
                             uint32_t flags, int32_t* topk_idx, float* topk_w,
                             hipStream_t stream) {
    if (T < 0 || E_tot < 1 || E_tot > MOE_MAX_EXPERTS || k < 1 || k > E_tot || k > MOE_MAX_SLOTS)
        return MOE_ERR_SHAPE;
    if (T == 0) return MOE_OK;
    if (!logits || !topk_idx || !topk_w) return MOE_ERR_NULL;
    return hip_status(moe_launch_route(logits, T, E_tot, k, flags, topk_idx, topk_w, stream));
}

// ---------------------------------------------------------------- permute
MOE_EXPORT size_t moe_permute_workspace_size(int32_t T, int32_t k, int32_t G) {
    if (T < 0 || k < 1 || G < 1) return 0;
    return moe_permute_scratch_bytes(T, k, G);
}

static int32_t check_permute(int T, int k, int e0, int E_loc, int s, int H) {
    if (T < 0 || k < 1 || E_loc < 1 || e0 < 0 || (s != 0 && s != 1)) return MOE_ERR_SHAPE;
    if (k + s > MOE_MAX_SLOTS || e0 + E_loc > MOE_MAX_EXPERTS) return MOE_ERR_SHAPE;
    if (H <= 0 || H % 256) return MOE_ERR_SHAPE;
    return MOE_OK;
}

MOE_EXPORT int32_t moe_permute(const int32_t* topk_idx, const float* topk_w, int32_t T, int32_t k,
                               int32_t e0, int32_t E_loc, int32_t s, const uint8_t* xq,
                               const uint8_t* xs, int32_t H, int32_t* counts, int32_t* offsets,
                               int32_t* offsets32, int32_t* row_src, float* row_w,
                               int32_t* slot_row, uint8_t* xq_perm, uint8_t* xs_perm, void* ws,
                               size_t ws_bytes, hipStream_t stream) {
    int32_t st = check_permute(T, k, e0, E_loc, s, H);
    if (st) return st;
    if (!counts || !offsets || !row_src || !row_w || !slot_row) return MOE_ERR_NULL;
    if (T > 0 && (!topk_idx || !topk_w)) return MOE_ERR_NULL;
    if (xq_perm && (!xs_perm || !xq || !xs)) return MOE_ERR_NULL;
    const size_t need = moe_permute_workspace_size(T, k, E_loc + s);
    if (ws_bytes < need || (need && !ws)) return MOE_ERR_WORKSPACE;
    return hip_status(moe_launch_permute(topk_idx, topk_w, T, k, e0, E_loc, s, xq, xs, H, counts,
                                         offsets, offsets32, row_src, row_w, slot_row, xq_perm,
                                         xs_perm, ws, stream));
}

// ---------------------------------------------------------------- grouped
MOE_EXPORT int32_t moe_transposed_ld(int32_t R_max, int32_t G) {
    if (R_max < 0 || G < 0) return 0;
    return (R_max + 31 * G + 31) & ~31;
}

MOE_EXPORT size_t moe_grouped_workspace_size(int32_t R_max, int32_t G, int32_t N, int32_t K) {
    (void)N;
    if (R_max < 0 || G < 1 || K <= 0 || K % 128) return 0;
    return moe_tiled_scale_bytes(R_max, G, K);
}

static int32_t fill_gemm_args(GemmArgs& a, const moe_weights* w, const moe_weights* wsh, int G,
                              int N, int K, int is_w1) {
    const int s = (wsh != nullptr) ? 1 : 0;
    const int E_loc = G - s;
    if (E_loc < 1) return MOE_ERR_SHAPE;
    int32_t st = check_weights(w, E_loc, N, K, is_w1);
    if (st) return st;
    if (wsh) {
        st = check_weights(wsh, 1, N, K, is_w1);
        if (st) return st;
        if (wsh->fmt != w->fmt) return MOE_ERR_UNSUPPORTED;
    }
    a.w_base[0] = (const uint8_t*)w->data;
    a.w_base[1] = wsh ? (const uint8_t*)wsh->data : a.w_base[0];
    a.E_loc = E_loc; a.G = G; a.N = N; a.K = K; a.fmt = w->fmt;
    return MOE_OK;
}

static int32_t check_hi(int H, int I) {
    if (H <= 0 || H % 256 || I <= 0 || I % 128 || I > MOE_MAX_I) return MOE_ERR_SHAPE;
    return MOE_OK;
}

constexpr int64_t kI32Lim = 1ll << 31;

// Size limits of the grouped GEMMs that depend on scalars only: every byte
// offset the kernels form is a 32-bit value (buffer resources), so the arrays
// they address must stay below 2 GiB.
static int32_t check_grouped_sizes(int R_max, int G, int x_rows, int H, int I, bool transpose) {
    if (R_max < 0 || G < 1 || G > MOE_MAX_EXPERTS + 1) return MOE_ERR_SHAPE;
    if ((int64_t)x_rows * H >= kI32Lim) return MOE_ERR_SHAPE;               // W1 activations
    if ((int64_t)R_max * I >= kI32Lim) return MOE_ERR_SHAPE;                // h, read by W2
    if (transpose && (int64_t)I * moe_transposed_ld(R_max, G) >= kI32Lim) return MOE_ERR_SHAPE;
    // scale tiles of the LDS-tiled kernels (W1 over K = H, W2 over K = I)
    if (moe_grouped_workspace_size(R_max, G, 2 * I, H) >= (size_t)kI32Lim ||
        moe_grouped_workspace_size(R_max, G, H, I) >= (size_t)kI32Lim) return MOE_ERR_SHAPE;
    return MOE_OK;
}

static int32_t check_gemm_flags(uint32_t flags) {
    const uint32_t fam = flags & (MOE_GEMM_STREAMED | MOE_GEMM_TILED | MOE_GEMM_PASS);
    if (fam & (fam - 1)) return MOE_ERR_UNSUPPORTED;            // more than one family forced
    return MOE_OK;
}

// The epilogue variant: a known activation, a finite positive Swish slope, a
// finite non-negative clamp limit (NULL: SwiGLU with beta = 1).
static int32_t check_epilogue(const moe_epilogue* e) {
    if (!e) return MOE_OK;
    if (e->act != MOE_ACT_SWIGLU && e->act != MOE_ACT_GEGLU && e->act != MOE_ACT_SRELU)
        return MOE_ERR_UNSUPPORTED;
    if (!(e->beta > 0.0f) || !isfinite(e->beta) || !(e->limit >= 0.0f) || !isfinite(e->limit))
        return MOE_ERR_SHAPE;
    return MOE_OK;
}

// Everything moe_grouped_w1 checks before it enqueues; a.* filled on success.
static int32_t prepare_w1(GemmArgs& a, const moe_weights* w1, const moe_weights* w1_shared,
                          const int32_t* counts, const int32_t* offsets, const int32_t* offsets32,
                          const float* row_w, const uint8_t* xq_perm, const uint8_t* xs_perm,
                          const int32_t* row_src, int32_t x_rows, int32_t R_max, int32_t H,
                          int32_t I, int32_t G, const moe_epilogue* epi, uint32_t flags,
                          uint8_t* hq, uint8_t* hs, uint8_t* hTq, uint8_t* hTs, void* ws,
                          size_t ws_bytes) {
    int32_t st = check_hi(H, I);
    if (st) return st;
    if ((st = check_gemm_flags(flags))) return st;
    if ((st = check_epilogue(epi))) return st;
    if (epi && epi->save_pre && (int64_t)R_max * 4 * I >= kI32Lim) return MOE_ERR_SHAPE;
    const bool transpose = (flags & MOE_W1_WRITE_TRANSPOSE) != 0;
    if (x_rows < 1) return MOE_ERR_SHAPE;
    if ((st = check_grouped_sizes(R_max, G, x_rows, H, I, transpose))) return st;
    st = fill_gemm_args(a, w1, w1_shared, G, 2 * I, H, 1);
    if (st) return st;
    if (!row_src && x_rows < R_max) return MOE_ERR_SHAPE;
    if (!counts || !offsets || !xq_perm || !xs_perm || !hq || !hs) return MOE_ERR_NULL;
    if (transpose && (!hTq || !hTs || !offsets32)) return MOE_ERR_NULL;
    if (!(flags & MOE_WEIGHT_AT_COMBINE) && !row_w) return MOE_ERR_NULL;
    const size_t need = moe_grouped_workspace_size(R_max, G, 2 * I, H);
    if (ws_bytes < need || (need && !ws)) return MOE_ERR_WORKSPACE;
    a.counts = counts; a.offsets = offsets; a.offsets32 = offsets32; a.row_w = row_w;
    a.aq = xq_perm; a.as = xs_perm; a.row_src = row_src; a.x_rows = x_rows;
    a.R_max = R_max; a.flags = flags;
    a.hq = hq; a.hs = hs; a.hTq = hTq; a.hTs = hTs; a.ldT = moe_transposed_ld(R_max, G);
    a.ws = ws; a.ws_bytes = ws_bytes;
    a.epi = epi;
    return MOE_OK;
}

MOE_EXPORT int32_t moe_grouped_w1(const moe_weights* w1, const moe_weights* w1_shared,
                                  const int32_t* counts, const int32_t* offsets,
                                  const int32_t* offsets32, const float* row_w,
                                  const uint8_t* xq, const uint8_t* xs, const int32_t* row_src,
                                  int32_t x_rows, int32_t R_max, int32_t H, int32_t I, int32_t G,
                                  const moe_epilogue* epi, uint32_t flags, uint8_t* hq,
                                  uint8_t* hs, uint8_t* hTq, uint8_t* hTs, void* ws,
                                  size_t ws_bytes, hipStream_t stream) {
    GemmArgs a{};
    const int32_t st = prepare_w1(a, w1, w1_shared, counts, offsets, offsets32, row_w, xq, xs,
                                  row_src, x_rows, R_max, H, I, G, epi, flags, hq, hs, hTq, hTs, ws,
                                  ws_bytes);
    if (st) return st;
    return hip_status(moe_launch_grouped_w1(a, stream));
}

// Everything moe_grouped_w2 checks before it enqueues; a.* filled on success.
static int32_t prepare_w2(GemmArgs& a, const moe_weights* w2, const moe_weights* w2_shared,
                          const int32_t* counts, const int32_t* offsets, const uint8_t* hq,
                          const uint8_t* hs, int32_t R_max, int32_t H, int32_t I, int32_t G,
                          uint32_t flags, uint16_t* y, void* ws, size_t ws_bytes) {
    int32_t st = check_hi(H, I);
    if (st) return st;
    if ((st = check_gemm_flags(flags))) return st;
    if (flags & ~(MOE_GEMM_STREAMED | MOE_GEMM_TILED | MOE_GEMM_PASS)) return MOE_ERR_UNSUPPORTED;
    if ((st = check_grouped_sizes(R_max, G, 1, H, I, false))) return st;
    st = fill_gemm_args(a, w2, w2_shared, G, H, I, 0);
    if (st) return st;
    if (!counts || !offsets || !hq || !hs || !y) return MOE_ERR_NULL;
    const size_t need = moe_grouped_workspace_size(R_max, G, H, I);
    if (ws_bytes < need || (need && !ws)) return MOE_ERR_WORKSPACE;
    a.counts = counts; a.offsets = offsets; a.aq = hq; a.as = hs; a.x_rows = R_max; a.R_max = R_max;
    a.flags = flags; a.y = y;
    a.ws = ws; a.ws_bytes = ws_bytes;
    return MOE_OK;
}

MOE_EXPORT int32_t moe_grouped_w2(const moe_weights* w2, const moe_weights* w2_shared,
                                  const int32_t* counts, const int32_t* offsets, const uint8_t* hq,
                                  const uint8_t* hs, int32_t R_max, int32_t H, int32_t I,
                                  int32_t G, uint32_t flags, uint16_t* y, void* ws,
                                  size_t ws_bytes, hipStream_t stream) {
    GemmArgs a{};
    const int32_t st = prepare_w2(a, w2, w2_shared, counts, offsets, hq, hs, R_max, H, I, G, flags,
                                  y, ws, ws_bytes);
    if (st) return st;
    return hip_status(moe_launch_grouped_w2(a, stream));
}

// -------------------------------------------------------------- backward
// Workspace of moe_grouped_w1_backward: the scale tiles of the dy rows (K = H),
// then the routing-weight gradient's partials, one per row and 64-feature unit.
static size_t backward_scale_bytes(int32_t R_max, int32_t G, int32_t H) {
    return align_up(moe_tiled_scale_bytes(R_max, G, H));
}

MOE_EXPORT size_t moe_backward_workspace_size(int32_t R_max, int32_t G, int32_t H, int32_t I) {
    if (R_max < 0 || G < 1 || H <= 0 || H % 128 || I <= 0 || I % 64) return 0;
    return backward_scale_bytes(R_max, G, H) + (size_t)R_max * (I / 64) * 4;
}

MOE_EXPORT int32_t moe_grouped_w1_backward(
        const moe_weights* w2t, const moe_weights* w2t_shared, const int32_t* counts,
        const int32_t* offsets, const int32_t* offsets32, const float* row_w, const uint8_t* dyq,
        const uint8_t* dys, const int32_t* row_src, int32_t x_rows, const uint16_t* pre,
        int32_t R_max, int32_t H, int32_t I, int32_t G, const moe_epilogue* epi, uint32_t flags,
        uint8_t* dq, uint8_t* ds, uint8_t* dTq, uint8_t* dTs, float* dw, void* ws,
        size_t ws_bytes, hipStream_t stream) {
    int32_t st = check_hi(H, I);
    if (st) return st;
    if (flags & ~(MOE_W1_WRITE_TRANSPOSE | MOE_SCALE_RULE_CEIL)) return MOE_ERR_UNSUPPORTED;
    if ((st = check_epilogue(epi))) return st;
    const bool transpose = (flags & MOE_W1_WRITE_TRANSPOSE) != 0;
    if (x_rows < 1) return MOE_ERR_SHAPE;
    if ((st = check_grouped_sizes(R_max, G, x_rows, H, I, false))) return st;
    // outputs of 2I per row: the row copy and, with the transposed copy, 2I rows of ldT
    if ((int64_t)R_max * 4 * I >= kI32Lim) return MOE_ERR_SHAPE;
    if (transpose && (int64_t)2 * I * moe_transposed_ld(R_max, G) >= kI32Lim) return MOE_ERR_SHAPE;
    GemmArgs a{};
    if ((st = fill_gemm_args(a, w2t, w2t_shared, G, I, H, 0))) return st;
    if (!row_src && x_rows < R_max) return MOE_ERR_SHAPE;
    if (!counts || !offsets || !dyq || !dys || !pre || !dq || !ds) return MOE_ERR_NULL;
    if (transpose && (!dTq || !dTs || !offsets32)) return MOE_ERR_NULL;
    if (dw && !row_w) return MOE_ERR_NULL;
    const size_t need = moe_backward_workspace_size(R_max, G, H, I);
    if (ws_bytes < need || (need && !ws)) return MOE_ERR_WORKSPACE;
    a.counts = counts; a.offsets = offsets; a.offsets32 = offsets32; a.row_w = row_w;
    a.aq = dyq; a.as = dys; a.row_src = row_src; a.x_rows = x_rows;
    a.R_max = R_max; a.flags = flags;
    a.hq = dq; a.hs = ds; a.hTq = dTq; a.hTs = dTs; a.ldT = moe_transposed_ld(R_max, G);
    a.ws = ws; a.ws_bytes = ws_bytes;
    a.epi = epi; a.pre = pre;
    a.dw_part = (float*)((char*)ws + backward_scale_bytes(R_max, G, H));
    return hip_status(moe_launch_tiled_backward(a, dw, stream));
}

// The tiling hints moe_layer gives the grouped GEMMs, from uniform routing:
// the expected rows of a routed group, ceil(T * k / E_tot), and the expected
// groups with rows, ceil(E_loc * (1 - (1 - k/E_tot)^T)) + s.
static int32_t layer_active_hint(int32_t T, int32_t E_tot, int32_t k, int32_t E_loc, int32_t s) {
    if (T <= 0 || E_tot <= 0 || k <= 0 || E_loc <= 0) return 0;
    return (int32_t)ceil(E_loc * (1.0 - pow(1.0 - (double)k / E_tot, (double)T))) + (s ? 1 : 0);
}

static int32_t layer_rows_hint(int32_t T, int32_t E_tot, int32_t k) {
    if (T <= 0 || E_tot <= 0 || k <= 0) return 0;
    return (int32_t)(((int64_t)T * k + E_tot - 1) / E_tot);
}

// ---------------------------------------------------------------- combine
MOE_EXPORT int32_t moe_combine(const uint16_t* y, const int32_t* slot_row, const float* row_w,
                               int32_t T, int32_t k_plus_s, int32_t H, uint16_t* out,
                               hipStream_t stream) {
    if (T < 0 || k_plus_s < 1 || k_plus_s > MOE_MAX_SLOTS || H <= 0 || H % 8) return MOE_ERR_SHAPE;
    if (T == 0) return MOE_OK;
    if (!y || !slot_row || !out) return MOE_ERR_NULL;
    return hip_status(moe_launch_combine(y, slot_row, row_w, T, k_plus_s, H, out, stream));
}

// ------------------------------------------------------------------ layer
MOE_EXPORT size_t moe_layer_workspace_size(int32_t T, int32_t E_tot, int32_t k, int32_t E_loc,
                                           int32_t H, int32_t I, int32_t s, uint32_t flags) {
    if (T < 0 || k < 1 || E_loc < 1 || H <= 0 || I <= 0 || (s != 0 && s != 1)) return 0;
    return layer_layout(T, E_tot, k, E_loc, H, I, s, flags).total;
}

MOE_EXPORT int32_t moe_layer_workspace_offsets(int32_t T, int32_t E_tot, int32_t k, int32_t E_loc,
                                               int32_t H, int32_t I, int32_t s, uint32_t flags,
                                               size_t* offsets13) {
    if (!offsets13) return 0;
    LayerLayout L = layer_layout(T, E_tot, k, E_loc, H, I, s, flags);
    memcpy(offsets13, L.off, sizeof(L.off));
    return kRegions;
}

MOE_EXPORT int32_t moe_layer(const moe_layer_args* a, void* ws, size_t ws_bytes,
                             hipStream_t stream) {
    if (!a) return MOE_ERR_NULL;
    const int T = a->T, E_tot = a->E_tot, k = a->k, e0 = a->e0, E_loc = a->E_loc;
    const int H = a->H, I = a->I;
    const int s = a->shared_w1 ? 1 : 0;
    if ((a->shared_w1 == nullptr) != (a->shared_w2 == nullptr)) return MOE_ERR_NULL;
    if (T < 0 || E_tot < 1 || E_tot > MOE_MAX_EXPERTS || k < 1 || k > E_tot) return MOE_ERR_SHAPE;
    if (e0 < 0 || E_loc < 1 || e0 + E_loc > E_tot || k + s > MOE_MAX_SLOTS) return MOE_ERR_SHAPE;
    if ((int64_t)T * (k + s) >= kI32Lim) return MOE_ERR_SHAPE;
    int32_t st = check_hi(H, I);
    if (st) return st;
    if ((st = check_gemm_flags(a->flags))) return st;
    const int G = E_loc + s;
    st = check_weights(a->w1, E_loc, 2 * I, H, 1);
    if (st) return st;
    st = check_weights(a->w2, E_loc, H, I, 0);
    if (st) return st;
    if (s) {
        if ((st = check_weights(a->shared_w1, 1, 2 * I, H, 1))) return st;
        if ((st = check_weights(a->shared_w2, 1, H, I, 0))) return st;
        if (a->shared_w1->fmt != a->w1->fmt || a->shared_w2->fmt != a->w2->fmt)
            return MOE_ERR_UNSUPPORTED;
    }
    const bool transpose = (a->flags & MOE_W1_WRITE_TRANSPOSE) != 0;
    if (transpose && (!a->hTq || !a->hTs)) return MOE_ERR_NULL;
    if (T == 0) return MOE_OK;
    if (!a->logits || !a->xq || !a->xs || !a->out) return MOE_ERR_NULL;
    const int R_max = T * k + s * T;
    if ((st = check_grouped_sizes(R_max, G, T, H, I, transpose))) return st;
    const LayerLayout L = layer_layout(T, E_tot, k, E_loc, H, I, s, a->flags);
    if (!ws || ws_bytes < L.total) return MOE_ERR_WORKSPACE;

    char* base = (char*)ws;
    int32_t* topk_idx = (int32_t*)(base + L.off[0]);
    float* topk_w = (float*)(base + L.off[1]);
    int32_t* counts = (int32_t*)(base + L.off[2]);
    int32_t* offsets = (int32_t*)(base + L.off[3]);
    int32_t* offsets32 = (int32_t*)(base + L.off[4]);
    int32_t* row_src = (int32_t*)(base + L.off[5]);
    float* row_w = (float*)(base + L.off[6]);
    int32_t* slot_row = (int32_t*)(base + L.off[7]);
    uint8_t* hq = (uint8_t*)(base + L.off[8]);
    uint8_t* hs = (uint8_t*)(base + L.off[9]);
    uint16_t* y = (uint16_t*)(base + L.off[10]);
    void* scratch = base + L.off[11];
    const size_t scratch_bytes = L.off[12] - L.off[11];
    uint32_t* ctrl = (uint32_t*)(base + L.off[12]);

    // Both GEMMs are validated before anything is enqueued, so a failing call
    // leaves the stream untouched.
    GemmArgs a1{}, a2{};
    st = prepare_w1(a1, a->w1, a->shared_w1, counts, offsets, offsets32, row_w, a->xq, a->xs,
                    row_src, T, R_max, H, I, G, a->epi, a->flags, hq, hs, a->hTq, a->hTs, scratch,
                    scratch_bytes);
    if (st) return st;
    st = prepare_w2(a2, a->w2, a->shared_w2, counts, offsets, hq, hs, R_max, H, I, G,
                    a->flags & (MOE_GEMM_STREAMED | MOE_GEMM_TILED | MOE_GEMM_PASS), y, scratch, scratch_bytes);
    if (st) return st;

    // expected rows of a routed group under uniform routing; the shared group
    // (T rows) gets more passes from the grid's pass dimension
    const int hint = layer_rows_hint(T, E_tot, k);
    // expected local experts with at least one token: E_loc (1 - (1 - k/E_tot)^T), plus the shared one
    const int active = layer_active_hint(T, E_tot, k, E_loc, s);
    a1.rows_hint = a2.rows_hint = hint;
    a1.active_hint = a2.active_hint = active;
    const RouteArgs ra{a->logits, T, E_tot, k, e0, a->flags, topk_idx, topk_w, slot_row};
    // a decode batch: the whole layer in one persistent launch
    if (moe_fused_decode_ok(T, E_tot, k, E_loc, s, a->flags)) {
        a1.route = &ra;
        a2.y = y;
        return hip_status(moe_launch_fused_decode(a1, a2, ctrl, a->out, stream));
    }
    // few tokens: the W1 launch routes and groups them itself
    const bool self_route = moe_w1_can_route(T, E_tot, k, E_loc, s, R_max, H, I, hint, a->flags);
    if (self_route) a1.route = &ra;

    // the token ring (W1 on the LDS-tiled kernel only)
    const bool ring = (a->flags & MOE_LAYER_TOKEN_RING) && !self_route && moe_grouped_uses_tiled(a1);
    const RingResources* rr = nullptr;
    if (ring && !(rr = ring_resources())) return MOE_ERR_HIP;

    int e;
    if (self_route) {
        // routing and grouping happen inside the W1 launch below
    } else if (moe_route_permute_fusable(T, E_tot, k, E_loc, s)) {
        e = moe_launch_route_permute(a->logits, T, E_tot, k, a->flags, e0, E_loc, s, topk_idx,
                                     topk_w, counts, offsets, offsets32, row_src, row_w, slot_row,
                                     stream);
        if (e) return MOE_ERR_HIP;
    } else {
        e = moe_launch_route(a->logits, T, E_tot, k, a->flags, topk_idx, topk_w, stream);
        if (e) return MOE_ERR_HIP;
        e = moe_launch_permute(topk_idx, topk_w, T, k, e0, E_loc, s, nullptr, nullptr, H, counts,
                               offsets, offsets32, row_src, row_w, slot_row, nullptr, nullptr,
                               scratch, stream);
        if (e) return MOE_ERR_HIP;
    }
    if (ring) {
        // the scale tiles first, then the ring slots, in the scratch region
        uint8_t* slots = (uint8_t*)scratch + align_up(moe_grouped_workspace_size(R_max, G, 2 * I, H));
        e = moe_launch_tiled_w1_ring(a1, slots, moe_ring_slot_bytes(H), kRingSlots, stream, rr->side,
                                     const_cast<hipEvent_t*>(rr->ev));
        if (e) return MOE_ERR_HIP;
    } else if ((e = moe_launch_grouped_w1(a1, stream))) return MOE_ERR_HIP;
    const bool wc = (a->flags & MOE_WEIGHT_AT_COMBINE) != 0;
    // at most 16 tokens on few active groups: W2 and the combine in one
    // launch (column ownership)
    if (moe_w2_combine_ok(T, R_max, G, H, I, active, a->flags))
        return hip_status(moe_launch_w2_combine(a2, slot_row, wc ? row_w : nullptr, T, k + s, a->out, stream));
    if ((e = moe_launch_grouped_w2(a2, stream))) return MOE_ERR_HIP;
    e = moe_launch_combine(y, slot_row, wc ? row_w : nullptr, T, k + s, H, a->out, stream);
    return hip_status(e);
}
