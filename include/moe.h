/*
 * moe.h -- C ABI of libmoe: one GPU's share of a routed Mixture-of-Experts
 * layer on AMD Instinct MI355X (gfx950).
 *
 * The layer (GC-MoE arXiv-wiki summary page, "Approach" and "Key
 * contributions"; fusion-kernel blog, "GLU activation in a fused GEMM
 * epilogue" and "Removing host-device synchronisation"):
 *
 *   route    top-k softmax router over fp32 logits              moe_route
 *   permute  per-expert counts/offsets in device memory, stable
 *            grouping of the local assignments, FP8 row gather   moe_permute
 *   W1       grouped GEMM, FP8 x MXFP4/MXFP8, epilogue fusing
 *            SwiGLU, the routing weight and FP8 requantisation   moe_grouped_w1
 *   W2       grouped GEMM to BF16 rows                           moe_grouped_w2
 *   combine  per-token sum of its rows, BF16                      moe_combine
 *   layer    all of the above in one call                         moe_layer
 *
 * Conventions, for every entry point:
 *  - Tensor pointers are DEVICE pointers owned by the caller. Row-major,
 *    densely packed unless a leading dimension is stated.
 *  - The library never allocates or frees device memory, never synchronises
 *    the host with the device and never reads device data on the host. Each
 *    call validates its scalar arguments, enqueues kernels on `stream` and
 *    returns. Every shape decision that depends on routing is taken on the
 *    device from the counts, so a call sequence can be captured in a graph.
 *  - Validation failures return a nonzero status and enqueue nothing. A
 *    kernel fault surfaces as a HIP error at the caller's next synchronising
 *    call; launch errors are reported as MOE_ERR_HIP.
 *  - Buffers whose size depends on routing are sized for the worst case
 *    R_max = T*k + s*T rows (s = 1 with a shared expert, else 0).
 *  - Calls are reentrant. Two calls in flight at once must not share a
 *    workspace or output buffer (the GC-MoE page's "Limitations": a single
 *    workspace instance serialises the calls that use it).
 *
 * Number formats (OCP Microscaling v1.0): E4M3 and E2M1 element codes, one
 * E8M0 scale byte (2^(c-127)) per 32 consecutive elements along K. FP4 codes
 * are packed two per byte, element 2i in the low nibble.
 *
 * Design limits (GC-MoE page, "Limitations", the paper's Appendix A):
 * I <= 4096, I % 128 == 0, H % 256 == 0, k + s <= 32, E_tot <= 2048.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes -------------------------------------------------- */
#define MOE_OK              0
#define MOE_ERR_NULL        1   /* a required pointer is NULL            */
#define MOE_ERR_SHAPE       2   /* a size violates the design limits     */
#define MOE_ERR_UNSUPPORTED 3   /* format / flag combination not built    */
#define MOE_ERR_WORKSPACE   4   /* workspace or destination too small     */
#define MOE_ERR_HIP         5   /* a kernel launch failed                 */

/* ---- weight formats ------------------------------------------------ */
#define MOE_FMT_MXFP4 0         /* E2M1 elements, E8M0 per 32 along K     */
#define MOE_FMT_MXFP8 1         /* E4M3 elements, E8M0 per 32 along K     */

/* ---- flags ----------------------------------------------------------- */
#define MOE_ROUTE_RENORM       (1u << 0) /* divide the k weights by their sum   */
#define MOE_WEIGHT_AT_COMBINE  (1u << 1) /* apply the routing weight in combine
                                            instead of the W1 epilogue           */
#define MOE_W1_WRITE_TRANSPOSE (1u << 2) /* W1 also writes the transposed MXFP8
                                            copy of h (blocks of 32 tokens)      */
#define MOE_SCALE_RULE_CEIL    (1u << 3) /* requantisation scale 2^ceil(log2(amax/max))
                                            instead of the OCP floor rule        */
/* Kernel family of the grouped GEMMs (moe_grouped_w1 / moe_grouped_w2). By
 * default the library chooses from the expected rows per group, R_max / G:
 * below 16 the weight-streaming kernel (weights read once, K split across
 * waves); from 16 to 95 the pass-resident streaming kernel (a pass of 16 or
 * 32 token rows staged in on-chip memory once, each weight unit streamed over
 * the whole K by one wave), where its staging fits (K * 16 bytes of rows plus
 * scales within the 160 KiB of a compute unit; 32-row passes with the
 * transposed copy), else the K-split kernel; from 96 the LDS-tiled kernel
 * (256 x 256 workgroup tiles). These flags override the choice (a forced
 * pass-resident kernel whose staging does not fit runs the K-split kernel);
 * setting more than one is MOE_ERR_UNSUPPORTED. The families sum the fp32
 * partial products in different orders, so their results may differ in the
 * last bits of the accumulation. */
#define MOE_GEMM_STREAMED      (1u << 8)
#define MOE_GEMM_TILED         (1u << 9)
#define MOE_GEMM_PASS          (1u << 12)
/* moe_layer: run W2 and the combine as separate launches even where one
 * launch does both (at most 16 tokens on few active groups, see moe_layer). */
#define MOE_LAYER_SEPARATE_KERNELS (1u << 10)
/* moe_layer, when W1 runs on the LDS-tiled kernel (many rows per group): the
 * token dispatch as a producer on a second stream. The GC-MoE page's role1
 * fills a token ring in blocks of BM rows and publishes each filled block;
 * role2 runs W1 on filled blocks. Here a producer kernel copies the grouped
 * token rows of 64 256-row blocks at a time into one of two ring slots in the
 * workspace (and writes their scale tiles), on a library stream restricted
 * to 16 compute units where the runtime can create one; W1 runs on each
 * chunk once its "filled" event has fired, on the caller's stream, leaving
 * those 16 units to the producer; the producer refills a slot after the
 * chunk using it has been consumed ("consumed" event). No workgroup waits on
 * another. Results are identical to the unflagged call; the flag is ignored
 * when W1 takes the weight-streaming kernel. Not for calls on the same GPU
 * from several threads at once (the library's stream and events are shared). */
#define MOE_LAYER_TOKEN_RING (1u << 11)

/* ---- epilogue variants of the fused W1 epilogue ------------------------ */
/*
 * The fusion blog's GLU section: SwiGLU(x, W, V, b, c, beta) =
 * Swish_beta(xW + b) (x) (xV + c), with GeGLU and sReLU as the other
 * activations and clamping and bias addition as fused options. Every variant
 * keeps the gate/up structure of W1 (rows [0, I) gate, [I, 2I) up):
 *   g = acc_gate + b, u = acc_up + c          (bias, when given)
 *   g, u clamped to [-limit, limit]           (when limit > 0)
 *   h = a(g) * u * w,  a = Swish_beta (z * sigmoid(beta z)),
 *                          exact GELU (z * Phi(z)), or squared ReLU (max(z,0)^2)
 * save_pre, when non-NULL, receives BF16 [R_max, 2I] of the pre-activation
 * (g | u after the bias, before the clamp): the input of the backward.
 * A NULL moe_epilogue means SwiGLU with beta = 1, no bias, no clamp.
 */
#define MOE_ACT_SWIGLU 0
#define MOE_ACT_GEGLU  1
#define MOE_ACT_SRELU  2
typedef struct moe_epilogue {
    int32_t      act;        /* MOE_ACT_*                                        */
    float        beta;       /* Swish slope (MOE_ACT_SWIGLU only), e.g. 1.0f     */
    float        limit;      /* > 0: clamp both chunks to [-limit, limit]; 0: off */
    int32_t      reserved;
    const float* bias;       /* NULL, or device f32 [G][2I]: b then c per group  */
    uint16_t*    save_pre;   /* NULL, or device bf16 [R_max, 2I] (written)       */
} moe_epilogue;

#define MOE_MAX_EXPERTS 2048
#define MOE_MAX_SLOTS   32      /* k + s */
#define MOE_MAX_I       4096

/* Human-readable text for a status code. Never NULL. */
const char* moe_status_string(int32_t status);

/* Library version string, e.g. "moe-mi355x 0.1.0 gfx950". */
const char* moe_version(void);

/* ---- prepacked expert weights --------------------------------------- */
/*
 * Expert weights are prepacked once, outside the timed path, into the
 * layout the grouped GEMMs stream from (the caller converts weights once and
 * reuses them: GC-MoE page, "Developer view"; the gate/up repack is done at
 * checkpoint load: fusion blog, GLU epilogue section).
 *
 * For W1 (is_w1 = 1, N = 2I) rows [0, I) are the gate projection and rows
 * [I, 2I) the up projection; the prepacked order interleaves them so that one
 * workgroup holds gate row n and up row n. Within a group the layout is
 * opaque; groups are laid out one after another, group g at byte offset
 * g * moe_prepacked_size(1, N, K, fmt), so a buffer can be filled one expert
 * at a time by prepacking with G = 1 into that offset.
 */
typedef struct moe_weights {
    int32_t     fmt;    /* MOE_FMT_MXFP4 or MOE_FMT_MXFP8                    */
    int32_t     G;      /* number of experts in this buffer                   */
    int32_t     N;      /* output rows per expert: 2I for W1, H for W2        */
    int32_t     K;      /* reduction length: H for W1, I for W2               */
    int32_t     is_w1;  /* 1 for W1 (gate/up interleave), 0 for W2           */
    int32_t     reserved;
    const void* data;   /* device pointer to the prepacked buffer             */
    size_t      bytes;  /* its size: moe_prepacked_size(G, N, K, fmt)         */
} moe_weights;

/* Bytes of a prepacked buffer for G experts of N x K weights. 0 on bad args. */
size_t moe_prepacked_size(int32_t G, int32_t N, int32_t K, int32_t fmt);

/*
 * Prepack logical weights.
 *   q   device, uint8 [G, N, K] E4M3 codes (MXFP8) or [G, N, K/2] packed E2M1
 *   sc  device, uint8 [G, N, K/32] E8M0 scales
 *   dst device, >= moe_prepacked_size(...) bytes; written completely.
 * N % 64 == 0, K % 128 == 0. For is_w1, N is even and N/2 % 32 == 0.
 */
int32_t moe_prepack_weights(const uint8_t* q, const uint8_t* sc, int32_t G, int32_t N,
                            int32_t K, int32_t fmt, int32_t is_w1, void* dst,
                            size_t dst_bytes, hipStream_t stream);

/*
 * MX quantisation of fp32 rows (a utility; the layer's inputs arrive
 * quantised). src device f32 [rows, K]; q: E4M3 [rows, K] (MXFP8) or packed
 * E2M1 [rows, K/2] (MXFP4); s: E8M0 [rows, K/32]. Shared exponent
 * floor(log2 amax) - emax (OCP), or the ceil rule with MOE_SCALE_RULE_CEIL;
 * elements rounded to nearest even and saturated. K % 32 == 0.
 */
int32_t moe_quantize_mx(const float* src, int32_t rows, int32_t K, int32_t fmt,
                        uint32_t flags, uint8_t* q, uint8_t* s, hipStream_t stream);

/*
 * HBM read-rate probe (a measurement utility, not a step of the layer): one
 * plain streaming read of `bytes` of device memory at `src`, the practical
 * read rate that the bandwidth-bound kernels are compared with. Every
 * 16-byte chunk is read once; the chunks are folded with XOR into one word
 * per wave, written to sink [MOE_HBM_PROBE_SINK_WORDS] (the XOR of all sink
 * words is the XOR of all 4-byte words of the buffer). bytes % 16 == 0,
 * bytes <= 2^31; 0 bytes enqueues nothing.
 */
#define MOE_HBM_PROBE_SINK_WORDS 8192
int32_t moe_hbm_read_probe(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream);

/* ---- S1: route -------------------------------------------------------- */
/*
 * Top-k softmax router (k appears on the GC-MoE page only in the limit
 * k+1 <= 32; softmax top-k is this library's reading). For each token t:
 * topk_idx[t, j] is the expert with the j-th largest logit (ties to the lower
 * expert id), selected on the fp32 logits; topk_w[t, j] = exp(l - max) / sum
 * over all E_tot experts, in fp32 (renormalised over the k with
 * MOE_ROUTE_RENORM). logits [T, E_tot] f32 (finite); outputs [T, k].
 * 1 <= k <= E_tot <= 2048, T >= 0.
 */
int32_t moe_route(const float* logits, int32_t T, int32_t E_tot, int32_t k, uint32_t flags,
                  int32_t* topk_idx, float* topk_w, hipStream_t stream);

/* ---- S2 + S3: counts, offsets, permutation ---------------------------- */
/*
 * Group the local assignments by expert, stably, on the device (GC-MoE page,
 * "Approach": routing-count aggregation; fusion blog: per-group token counts
 * kept in GPU memory so no host sync is needed).
 *
 * Local experts are [e0, e0 + E_loc); with s = 1 a shared expert forms the
 * last group G-1 = E_loc and takes every token in order with weight 1.
 * Outputs (G = E_loc + s):
 *   counts    [G]        rows per group
 *   offsets   [G + 1]    exclusive prefix sum, offsets[G] = rows used R
 *   offsets32 [G + 1]    exclusive prefix sum of roundup(counts, 32); NULL allowed
 *   row_src   [R_max]    source token of each grouped row (rows >= R untouched)
 *   row_w     [R_max]    routing weight of each row (1 for the shared group)
 *   slot_row  [T, k + s] grouped row of each slot, -1 for a non-local expert
 *   xq_perm   [R_max, H] E4M3 codes of each row's token   (may be NULL: then
 *   xs_perm   [R_max, H/32] its E8M0 scales               xq/xs are unused)
 * Within a group, rows are ordered by the flattened assignment index t*k + j.
 * ws: scratch of moe_permute_workspace_size(T, k, G) bytes.
 * 0 <= e0, e0 + E_loc <= 2048 (the router's E_tot bound), k + s <= 32,
 * H % 256 == 0.
 */
size_t  moe_permute_workspace_size(int32_t T, int32_t k, int32_t G);
int32_t moe_permute(const int32_t* topk_idx, const float* topk_w, int32_t T, int32_t k,
                    int32_t e0, int32_t E_loc, int32_t s,
                    const uint8_t* xq, const uint8_t* xs, int32_t H,
                    int32_t* counts, int32_t* offsets, int32_t* offsets32,
                    int32_t* row_src, float* row_w, int32_t* slot_row,
                    uint8_t* xq_perm, uint8_t* xs_perm,
                    void* ws, size_t ws_bytes, hipStream_t stream);

/* ---- S4 + S5: grouped W1 with the fused epilogue ------------------------ */
/*
 * For every group g and row r in [offsets[g], offsets[g+1]):
 *   acc = dec(x_r) . dec(W1_g)^T  (fp32 accumulation on MFMA)
 *   h   = SiLU(acc[0:I]) * acc[I:2I] * row_w[r]   (row_w ignored, i.e. 1,
 *         with MOE_WEIGHT_AT_COMBINE)
 *   hq[r], hs[r] = MX-E4M3 quantisation of h in blocks of 32 along I
 * (SwiGLU with beta = 1 and no bias: fusion blog, GLU epilogue section; the
 * epilogue fusion: GC-MoE page, "Key contributions".)
 * x_r is row r of xq/xs when row_src is NULL (xq [R_max, H], xs [R_max, H/32],
 * the grouped rows moe_permute gathers), or row row_src[r] of the ungrouped
 * token arrays xq [T, H], xs [T, H/32] when row_src is given (the gather is
 * then done by this kernel's loads). x_rows is the row count of xq/xs
 * (R_max or T); reads are bounded by it. x_rows * H < 2^31.
 * With MOE_W1_WRITE_TRANSPOSE also hTq/hTs: for group g, columns
 * [offsets32[g], offsets32[g+1]) of hTq [I, ldT] hold h_g^T quantised in
 * blocks of 32 tokens counted from the group's first row (hTs [I, ldT/32]);
 * a partial last block takes its amax over valid tokens and its padding
 * columns hold code 0 (fusion blog, MXFP8 section: the transposed copy for
 * backward). ldT = moe_transposed_ld(R_max, G).
 * w1 holds the routed groups [0, E_loc); w1_shared (NULL when G == E_loc)
 * holds group E_loc. hq [R_max, I], hs [R_max, I/32]; rows >= R untouched.
 * The launch configuration is chosen from R_max and G alone (expected rows
 * per group R_max / G, see MOE_GEMM_STREAMED / MOE_GEMM_PASS / MOE_GEMM_TILED), so a caller
 * gets the best configuration by passing the tightest R_max it can
 * guarantee. R_max * I < 2^31; with the transposed copy I * ldT < 2^31.
 * ws: moe_grouped_workspace_size(...) bytes.
 */
int32_t moe_transposed_ld(int32_t R_max, int32_t G);
size_t  moe_grouped_workspace_size(int32_t R_max, int32_t G, int32_t N, int32_t K);
int32_t moe_grouped_w1(const moe_weights* w1, const moe_weights* w1_shared,
                       const int32_t* counts, const int32_t* offsets, const int32_t* offsets32,
                       const float* row_w, const uint8_t* xq, const uint8_t* xs,
                       const int32_t* row_src, int32_t x_rows,
                       int32_t R_max, int32_t H, int32_t I, int32_t G,
                       const moe_epilogue* epi, uint32_t flags,
                       uint8_t* hq, uint8_t* hs, uint8_t* hTq, uint8_t* hTs, void* ws,
                       size_t ws_bytes, hipStream_t stream);

/* ---- backward of the fused W1 epilogue ----------------------------------- */
/*
 * The fusion blog's "GroupGemm + dActivation + Quantize/Transpose" kernel
 * (the backward epilogue reads the GEMM output, forms the activation's
 * derivative and quantises it). For every group g and row r:
 *   dh  = dec(dy_r) . dec(W2T_g)^T           (fp32 on MFMA; W2T_g = W2_g^T,
 *                                              [I, H], MX-quantised along H)
 *   with (g, u) the saved pre-activation row pre[r] (BF16, see moe_epilogue)
 *   and w = row_w[r] (1 when row_w is NULL):
 *   dg  = dh * w * clamp(u) * a'(clamp(g)) * [|g| <= limit]
 *   du  = dh * w * a(clamp(g)) * [|u| <= limit]          ([...] = 1 without clamp)
 *   dw[r] = sum_i dh * a(clamp(g)) * clamp(u)    (the routing weight's gradient)
 *   dq[r], ds[r] = MX-E4M3 quantisation of [dg | du] in blocks of 32 along 2I
 * and, with MOE_W1_WRITE_TRANSPOSE, the transposed copy dTq [2I, ldT],
 * dTs [2I, ldT/32] in 32-row blocks per group, laid out as the forward's hT
 * (ldT = moe_transposed_ld(R_max, G)). dy_r is row row_src[r] of dyq/dys
 * ([x_rows, H] E4M3 + [x_rows, H/32] E8M0: the layer output's gradient, in
 * token order). epi: act, beta and limit as in the forward (bias unused: it
 * is part of pre). flags: MOE_W1_WRITE_TRANSPOSE, MOE_SCALE_RULE_CEIL. dw
 * may be NULL; it needs row_w. Runs on the LDS-tiled GEMM kernel. Limits as
 * moe_grouped_w1, and R_max * 2I < 2^31. ws: moe_backward_workspace_size.
 */
size_t  moe_backward_workspace_size(int32_t R_max, int32_t G, int32_t H, int32_t I);
int32_t moe_grouped_w1_backward(const moe_weights* w2t, const moe_weights* w2t_shared,
                                const int32_t* counts, const int32_t* offsets,
                                const int32_t* offsets32, const float* row_w,
                                const uint8_t* dyq, const uint8_t* dys, const int32_t* row_src,
                                int32_t x_rows, const uint16_t* pre, int32_t R_max, int32_t H,
                                int32_t I, int32_t G, const moe_epilogue* epi, uint32_t flags,
                                uint8_t* dq, uint8_t* ds, uint8_t* dTq, uint8_t* dTs, float* dw,
                                void* ws, size_t ws_bytes, hipStream_t stream);

/* ---- S6: grouped W2 ----------------------------------------------------- */
/*
 * y[r] = BF16_RNE(dec(hq[r]) . dec(W2_g)^T) for every row r of group g
 * (W2 produces BF16 fragments: GC-MoE page, "Approach"). hq [R_max, I],
 * hs [R_max, I/32], y bf16 [R_max, H]; rows >= R untouched. flags: only
 * MOE_GEMM_STREAMED / MOE_GEMM_PASS / MOE_GEMM_TILED; the configuration is chosen as for
 * moe_grouped_w1. R_max * I < 2^31.
 */
int32_t moe_grouped_w2(const moe_weights* w2, const moe_weights* w2_shared,
                       const int32_t* counts, const int32_t* offsets,
                       const uint8_t* hq, const uint8_t* hs,
                       int32_t R_max, int32_t H, int32_t I, int32_t G, uint32_t flags,
                       uint16_t* y, void* ws, size_t ws_bytes, hipStream_t stream);

/* ---- S7: combine ---------------------------------------------------------- */
/*
 * out[t] = BF16_RNE(sum over j < k_plus_s with slot_row[t,j] >= 0 of
 *          y[slot_row[t,j]] (times row_w[slot_row[t,j]] if row_w != NULL)),
 * summed in fp64 in slot order and rounded once (GC-MoE page, "Approach":
 * finalize/combine). A token with no local slot gets +0. y bf16 [R_max, H],
 * slot_row [T, k_plus_s], out bf16 [T, H]. H % 8 == 0.
 */
int32_t moe_combine(const uint16_t* y, const int32_t* slot_row, const float* row_w,
                    int32_t T, int32_t k_plus_s, int32_t H, uint16_t* out, hipStream_t stream);

/* ---- the whole layer ------------------------------------------------------ */
typedef struct moe_layer_args {
    const float*   logits;     /* [T, E_tot] f32                               */
    int32_t        T, E_tot, k;
    int32_t        e0, E_loc;  /* local experts [e0, e0 + E_loc)               */
    const uint8_t* xq;         /* [T, H] E4M3                                  */
    const uint8_t* xs;         /* [T, H/32] E8M0                               */
    int32_t        H, I;
    const moe_weights* w1;     /* E_loc experts, N = 2I, K = H                 */
    const moe_weights* w2;     /* E_loc experts, N = H,  K = I                 */
    const moe_weights* shared_w1;  /* NULL: no shared expert                   */
    const moe_weights* shared_w2;
    uint32_t       flags;
    uint8_t*       hTq;        /* with MOE_W1_WRITE_TRANSPOSE: [I, ldT]        */
    uint8_t*       hTs;        /*                               [I, ldT/32]    */
    uint16_t*      out;        /* [T, H] bf16                                  */
    const moe_epilogue* epi;   /* NULL: SwiGLU, beta = 1 (see moe_epilogue)    */
} moe_layer_args;

/* Workspace of moe_layer: every intermediate sized for R_max, plus scratch. */
size_t  moe_layer_workspace_size(int32_t T, int32_t E_tot, int32_t k, int32_t E_loc,
                                 int32_t H, int32_t I, int32_t s, uint32_t flags);

/*
 * Run route -> permute -> W1 -> W2 -> combine on `stream`. W1 routes and
 * groups the tokens itself when T <= 16 and groups average under 16 rows
 * (every W1 workgroup does it), router and grouping share one workgroup when
 * T <= 64, and W2 and the combine are one launch when T <= 16 and at most
 * 4 groups are expected to be active, or at most 8 whose W2 weights total at
 * most 2^24 elements (each workgroup owns 32 output columns of every token:
 * W2 for every active group, then the fp64 slot sum); so 2
 * launches for a single decode token on a large expert set, up to 5
 * otherwise. The grouped token rows are not materialised:
 * W1 reads them through row_src. Intermediates live in ws at offsets given
 * by moe_layer_workspace_offsets. Region [12] is the control block of a
 * single-launch decode path (every workgroup routes, W2 work on a group
 * waits for that group's W1 work, the last W2 item of a column block
 * combines it), which is built but switched off in this version.
 */
int32_t moe_layer(const moe_layer_args* a, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * moe_layer without a caller workspace, for callers that cannot allocate
 * device memory (code under graph capture, tight serving loops, harnesses
 * that forbid allocation): the same kernels as moe_layer, with the workspace
 * in a fixed array of MOE_NOALLOC_SCRATCH_BYTES inside this library, one per
 * GPU, held from its first use until the process ends. Nothing is allocated
 * or freed. Calls whose moe_layer_workspace_size exceeds the array return
 * MOE_ERR_WORKSPACE with nothing enqueued (64 MiB holds the layer at up to
 * 256 tokens of the 7168 x 2048, 32-expert decode share, or of the 6144 x 1536,
 * 128-expert set). All calls on one GPU share that GPU's array: calls that
 * overlap in time on the same GPU (two streams, two threads) race and must
 * be serialised by the caller. The intermediates of the last call stay in the
 * array; nothing carries over into the next call.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
int32_t moe_layer_noalloc(const moe_layer_args* a, hipStream_t stream);

/* Byte offsets of the intermediates inside the moe_layer workspace, for
 * inspection by tests: [0] topk_idx [1] topk_w [2] counts [3] offsets
 * [4] offsets32 [5] row_src [6] row_w [7] slot_row [8] hq [9] hs [10] y
 * [11] scratch [12] control block. Returns the number written (13). */
int32_t moe_layer_workspace_offsets(int32_t T, int32_t E_tot, int32_t k, int32_t E_loc,
                                    int32_t H, int32_t I, int32_t s, uint32_t flags,
                                    size_t* offsets13);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
