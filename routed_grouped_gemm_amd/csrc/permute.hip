// S2 + S3: per-expert counts and offsets in device memory, and a stable
// grouping of the local assignments (GC-MoE page, "Approach": routing-count
// aggregation before the token blocks are filled; fusion blog, "Removing
// host-device synchronisation": the group sizes stay in GPU memory).
//
// Row order: experts ascending, and within an expert the flattened assignment
// index a = t*k + j ascending; the shared expert (s = 1) is the last group and
// takes tokens 0..T-1. Determinism comes from construction, not from the
// order of atomics: per-wave ranks use a ballot "match any" loop, per-chunk
// wave totals are scanned in LDS, and chunk bases come from a scan over chunks.
//
// Paths: up to 4096 assignments a single workgroup does everything; for a few
// tokens the router runs in that same workgroup (one launch for S1-S3). Larger
// inputs use three kernels: per-chunk histograms, a scan, a scatter.
#include "permute_block.h"

namespace {

constexpr int kChunkThreads = 512;      // chunked path: one chunk = 512 assignments
constexpr int kSmallMax = 4096;         // single-workgroup path up to this many assignments
constexpr int kFusedThreads = 1024;     // route + permute in one workgroup
constexpr int kFusedMaxT = kFusedThreads / 64 * 4;   // four tokens per wave
constexpr int kFusedMaxG = 513;

// ---- single-workgroup path ---------------------------------------------
__global__ __launch_bounds__(kFusedThreads)
void permute_small_kernel(const int32_t* __restrict__ topk_idx, const float* __restrict__ topk_w,
                          int T, int k, int e0, int E_loc, int s,
                          int32_t* counts, int32_t* offsets, int32_t* offsets32,
                          int32_t* row_src, float* row_w, int32_t* slot_row) {
    extern __shared__ int lds[];
    permute_in_block<kFusedThreads / 64>(
        [&](int a) { return topk_idx[a]; }, [&](int a) { return topk_w[a]; },
        T, k, e0, E_loc, s, counts, offsets, offsets32, row_src, row_w, slot_row, lds);
}

// ---- router + single-workgroup permute in one launch (few tokens) -------
// LPT lanes per token: 64 (one token per wave, T <= 16) or 16 (four tokens
// per wave, T <= 64), so all tokens are routed in one pass of the 16 waves.
template <int LPT, int VPL>
__global__ __launch_bounds__(kFusedThreads)
void route_permute_kernel(const float* __restrict__ logits, int T, int E, int k, int renorm,
                          int e0, int E_loc, int s, int32_t* __restrict__ topk_idx,
                          float* __restrict__ topk_w, int32_t* counts, int32_t* offsets,
                          int32_t* offsets32, int32_t* row_src, float* row_w, int32_t* slot_row) {
    extern __shared__ int lds[];
    int* sidx = lds;                        // [T*k]
    float* sw = (float*)(lds + T * k);      // [T*k]
    constexpr int NW = kFusedThreads / 64;
    route_block<NW, LPT, VPL>(logits, T, E, k, renorm != 0, sidx, sw, topk_idx, topk_w);
    __syncthreads();
    permute_in_block<NW>([&](int a) { return sidx[a]; }, [&](int a) { return sw[a]; },
                         T, k, e0, E_loc, s, counts, offsets, offsets32, row_src, row_w, slot_row,
                         lds + 2 * T * k);
}

// ---- chunked path: count, scan, scatter --------------------------------
__global__ __launch_bounds__(kChunkThreads)
void permute_count_kernel(const int32_t* __restrict__ topk_idx, int Tk, int e0, int E_loc,
                          int32_t* __restrict__ chunk_hist) {
    extern __shared__ int lds[];
    const int tid = threadIdx.x, c = blockIdx.x;
    for (int g = tid; g < E_loc; g += kChunkThreads) lds[g] = 0;
    __syncthreads();
    int a = c * kChunkThreads + tid;
    if (a < Tk) {
        int g = topk_idx[a] - e0;
        if (g >= 0 && g < E_loc) atomicAdd(&lds[g], 1);
    }
    __syncthreads();
    for (int g = tid; g < E_loc; g += kChunkThreads) chunk_hist[(size_t)c * E_loc + g] = lds[g];
}

// Scan of the per-chunk histograms: for every expert, the exclusive prefix over
// chunks plus the expert's offset. P threads share an expert, each owning a
// run of ceil(nchunks / P) chunks, so no thread walks all chunks serially;
// within a run, values are loaded in batches before they are stored.
constexpr int kScanThreads = 1024;
constexpr int kScanBatch = 16;

MOE_DEV int run_sum(const int32_t* ch, int E_loc, int g, int c0, int c1) {
    int sum = 0;
    for (int c = c0; c < c1; ++c) sum += ch[(size_t)c * E_loc + g];
    return sum;
}

__global__ __launch_bounds__(kScanThreads)
void permute_scan_kernel(int32_t* __restrict__ chunk_hist, int nchunks, int T, int E_loc, int s,
                         int P, int32_t* counts, int32_t* offsets, int32_t* offsets32) {
    extern __shared__ int lds[];
    const int G = E_loc + s;
    int* cnt = lds;                     // [G]  counts, then offsets
    int* psum = cnt + G;                // [kScanThreads] per-thread run sums
    const int tid = threadIdx.x;
    const int seg = (nchunks + P - 1) / P;
    const int gpp = kScanThreads / P;
    const int p = tid % P;
    const int c0 = min(nchunks, p * seg), c1 = min(nchunks, (p + 1) * seg);

    for (int g0 = 0; g0 < E_loc; g0 += gpp) {          // counts
        const int g = g0 + tid / P;
        psum[tid] = g < E_loc ? run_sum(chunk_hist, E_loc, g, c0, c1) : 0;
        __syncthreads();
        if (g < E_loc && p == 0) {
            int tot = 0;
            for (int q = 0; q < P; ++q) tot += psum[tid + q];
            cnt[g] = tot;
        }
        __syncthreads();
    }
    if (s && tid == 0) cnt[E_loc] = T;
    __syncthreads();
    write_offsets(cnt, G, counts, offsets, offsets32);

    for (int g0 = 0; g0 < E_loc; g0 += gpp) {          // chunk bases
        const int g = g0 + tid / P;
        psum[tid] = g < E_loc ? run_sum(chunk_hist, E_loc, g, c0, c1) : 0;
        __syncthreads();
        if (g < E_loc && p == 0) {
            int run = 0;
            for (int q = 0; q < P; ++q) { int v = psum[tid + q]; psum[tid + q] = run; run += v; }
        }
        __syncthreads();
        if (g < E_loc) {
            int run = cnt[g] + psum[tid];
            for (int cb = c0; cb < c1; cb += kScanBatch) {
                int v[kScanBatch];
                #pragma unroll
                for (int i = 0; i < kScanBatch; ++i)
                    v[i] = (cb + i < c1) ? chunk_hist[(size_t)(cb + i) * E_loc + g] : 0;
                #pragma unroll
                for (int i = 0; i < kScanBatch; ++i) {
                    if (cb + i < c1) chunk_hist[(size_t)(cb + i) * E_loc + g] = run;
                    run += v[i];
                }
            }
        }
        __syncthreads();
    }
}

// The same scan with the whole chunk histogram held in LDS (rows padded to
// E_loc + 1 ints so that a wave reading one group's column hits 64 distinct
// banks): one coalesced pass in, a per-group wave scan (each lane a run of
// chunks), one coalesced pass out.
constexpr int kLdsScanMaxBytes = 120 * 1024;

__global__ __launch_bounds__(kScanThreads)
void permute_scan_lds_kernel(int32_t* __restrict__ chunk_hist, int nchunks, int T, int E_loc, int s,
                             int32_t* counts, int32_t* offsets, int32_t* offsets32) {
    extern __shared__ int lds[];
    constexpr int NW = kScanThreads / 64;
    const int G = E_loc + s, ld = E_loc + 1;
    int* h = lds;                                  // [nchunks][ld]
    int* cnt = h + nchunks * ld;                   // [G]: counts, then offsets
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    // in batches of 16 values per thread, all requested before any is stored
    // (one memory latency per batch, not per value)
    constexpr int kB = 16;
    const int n = nchunks * E_loc;
    for (int i0 = 0; i0 < n; i0 += kB * kScanThreads) {
        int v[kB];
        #pragma unroll
        for (int u = 0; u < kB; ++u) {
            const int i = i0 + u * kScanThreads + tid;
            v[u] = i < n ? chunk_hist[i] : 0;
        }
        #pragma unroll
        for (int u = 0; u < kB; ++u) {
            const int i = i0 + u * kScanThreads + tid;
            if (i < n) {
                const int c = i / E_loc;
                h[c * ld + (i - c * E_loc)] = v[u];
            }
        }
    }
    __syncthreads();
    const int per = (nchunks + 63) / 64;
    const int c0 = min(nchunks, lane * per), c1 = min(nchunks, c0 + per);
    for (int g = w; g < E_loc; g += NW) {
        int sum = 0;
        for (int c = c0; c < c1; ++c) sum += h[c * ld + g];
        int inc = sum;                             // inclusive scan over the lanes' runs
        #pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int a = __shfl_up(inc, d, 64);
            if (lane >= d) inc += a;
        }
        int run = inc - sum;
        for (int c = c0; c < c1; ++c) {
            const int v = h[c * ld + g];
            h[c * ld + g] = run;
            run += v;
        }
        if (lane == 63) cnt[g] = inc;
    }
    if (s && tid == 0) cnt[E_loc] = T;
    write_offsets(cnt, G, counts, offsets, offsets32);
    __syncthreads();
    for (int i = tid; i < nchunks * E_loc; i += kScanThreads) {
        const int c = i / E_loc, g = i - c * E_loc;
        chunk_hist[i] = cnt[g] + h[c * ld + g];
    }
}

__global__ __launch_bounds__(kChunkThreads)
void permute_scatter_kernel(const int32_t* __restrict__ topk_idx, const float* __restrict__ topk_w,
                            int T, int k, int e0, int E_loc, int s,
                            const int32_t* __restrict__ chunk_base, const int32_t* __restrict__ offsets,
                            int32_t* row_src, float* row_w, int32_t* slot_row) {
    constexpr int NW = kChunkThreads / 64;
    extern __shared__ int lds[];
    uint16_t* cnt = (uint16_t*)lds;          // [NW][E_loc]
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, c = blockIdx.x;
    const int Tk = T * k, ks = k + s;
    const int gbits = group_bits(E_loc);
    for (int i = tid; i < NW * E_loc; i += kChunkThreads) cnt[i] = 0;
    __syncthreads();
    int a = c * kChunkThreads + tid;
    int g = -1;
    if (a < Tk) {
        int gg = topk_idx[a] - e0;
        if (gg >= 0 && gg < E_loc) g = gg;
    }
    int rank = wave_match_rank(g, lane, gbits, cnt + w * E_loc);
    __syncthreads();
    scan_waves<NW>(cnt, E_loc, nullptr);
    __syncthreads();
    if (a < Tk) {
        int row = g >= 0 ? chunk_base[(size_t)c * E_loc + g] + cnt[w * E_loc + g] + rank : -1;
        write_row(a, g, row, k, ks, g >= 0 ? topk_w[a] : 0.f, row_src, row_w, slot_row);
    }
    if (s) write_shared_rows(c * kChunkThreads, (c + 1) * kChunkThreads, T, k, ks, offsets[E_loc],
                             row_src, row_w, slot_row);
}

// ---- gather of the FP8 rows and their scales ---------------------------
constexpr int kGatherRows = 8;

__global__ __launch_bounds__(256)
void gather_kernel(const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs, int H,
                   const int32_t* __restrict__ row_src, const int32_t* __restrict__ offsets, int G,
                   uint8_t* __restrict__ xq_perm, uint8_t* __restrict__ xs_perm) {
    const int R = offsets[G];
    const int r0 = blockIdx.x * kGatherRows;
    if (r0 >= R) return;
    const int nvec = H / 16, nsv = H / 256;      // uint4 per row, uint2 of scales per row
    for (int i = 0; i < kGatherRows; ++i) {
        int r = r0 + i;
        if (r >= R) break;
        int t = row_src[r];
        const uint4* src = (const uint4*)(xq + (size_t)t * H);
        uint4* dst = (uint4*)(xq_perm + (size_t)r * H);
        for (int v = threadIdx.x; v < nvec; v += 256) dst[v] = src[v];
        const uint2* ss = (const uint2*)(xs + (size_t)t * (H / 32));
        uint2* sd = (uint2*)(xs_perm + (size_t)r * (H / 32));
        for (int v = threadIdx.x; v < nsv; v += 256) sd[v] = ss[v];
    }
}

int launch_gather(const uint8_t* xq, const uint8_t* xs, int H, const int32_t* row_src,
                  const int32_t* offsets, int G, int R_max, uint8_t* xq_perm, uint8_t* xs_perm,
                  hipStream_t stream) {
    int blocks = (R_max + kGatherRows - 1) / kGatherRows;
    hipLaunchKernelGGL(gather_kernel, dim3(blocks), dim3(256), 0, stream, xq, xs, H, row_src,
                       offsets, G, xq_perm, xs_perm);
    return (int)hipGetLastError();
}

}  // namespace

size_t moe_permute_scratch_bytes(int T, int k, int G) {
    size_t Tk = (size_t)T * k;
    size_t nchunks = (Tk + kChunkThreads - 1) / kChunkThreads;
    return (Tk > (size_t)kSmallMax) ? nchunks * (size_t)G * 4 : 0;
}

int moe_launch_permute(const int32_t* topk_idx, const float* topk_w, int T, int k, int e0,
                       int E_loc, int s, const uint8_t* xq, const uint8_t* xs, int H,
                       int32_t* counts, int32_t* offsets, int32_t* offsets32, int32_t* row_src,
                       float* row_w, int32_t* slot_row, uint8_t* xq_perm, uint8_t* xs_perm,
                       void* scratch, hipStream_t stream) {
    const int G = E_loc + s;
    const int Tk = T * k;
    hipError_t e;
    if (Tk <= kSmallMax) {
        size_t lds = block_lds_ints(kFusedThreads / 64, G, E_loc) * 4;
        hipLaunchKernelGGL(permute_small_kernel, dim3(1), dim3(kFusedThreads), lds, stream,
                           topk_idx, topk_w, T, k, e0, E_loc, s, counts, offsets, offsets32,
                           row_src, row_w, slot_row);
    } else {
        const int nchunks = (Tk + kChunkThreads - 1) / kChunkThreads;
        int32_t* chunk_hist = (int32_t*)scratch;
        hipLaunchKernelGGL(permute_count_kernel, dim3(nchunks), dim3(kChunkThreads),
                           (size_t)E_loc * 4, stream, topk_idx, Tk, e0, E_loc, chunk_hist);
        int P = 1;
        while (P * 2 <= kScanThreads / E_loc && P * 2 <= nchunks) P *= 2;
        const size_t lds_scan = ((size_t)nchunks * (E_loc + 1) + G) * 4;
        if (lds_scan <= (size_t)kLdsScanMaxBytes)
            hipLaunchKernelGGL(permute_scan_lds_kernel, dim3(1), dim3(kScanThreads), lds_scan, stream,
                               chunk_hist, (int)nchunks, T, E_loc, s, counts, offsets, offsets32);
        else
            hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(kScanThreads),
                               (size_t)(G + kScanThreads) * 4, stream, chunk_hist, nchunks, T,
                               E_loc, s, P, counts, offsets, offsets32);
        hipLaunchKernelGGL(permute_scatter_kernel, dim3(nchunks), dim3(kChunkThreads),
                           (size_t)(kChunkThreads / 64) * E_loc * 2 + 4, stream, topk_idx, topk_w,
                           T, k, e0, E_loc, s, chunk_hist, offsets, row_src, row_w, slot_row);
    }
    if ((e = hipGetLastError()) != hipSuccess) return (int)e;
    if (xq_perm && T > 0)
        return launch_gather(xq, xs, H, row_src, offsets, G, Tk + s * T, xq_perm, xs_perm, stream);
    return 0;
}

bool moe_route_permute_fusable(int T, int E, int k, int E_loc, int s) {
    return T <= kFusedMaxT && E <= 256 && k <= 16 && E_loc + s <= kFusedMaxG && T * k <= kSmallMax;
}

int moe_launch_route_permute(const float* logits, int T, int E, int k, uint32_t flags, int e0,
                             int E_loc, int s, int32_t* topk_idx, float* topk_w, int32_t* counts,
                             int32_t* offsets, int32_t* offsets32, int32_t* row_src, float* row_w,
                             int32_t* slot_row, hipStream_t stream) {
    const int G = E_loc + s;
    const int renorm = (flags & MOE_ROUTE_RENORM) ? 1 : 0;
    const size_t lds = ((size_t)2 * T * k + block_lds_ints(kFusedThreads / 64, G, E_loc)) * 4;
#define MOE_RP_CASE(L, N)                                                                      \
    if (vpl <= N) {                                                                            \
        hipLaunchKernelGGL((route_permute_kernel<L, N>), dim3(1), dim3(kFusedThreads), lds,      \
                           stream, logits, T, E, k, renorm, e0, E_loc, s, topk_idx, topk_w,    \
                           counts, offsets, offsets32, row_src, row_w, slot_row);              \
        return (int)hipGetLastError();                                                         \
    }
    if (T <= kFusedThreads / 64) {          // a whole wave per token
        const int vpl = (E + 63) / 64;
        MOE_RP_CASE(64, 1)
        MOE_RP_CASE(64, 2)
        MOE_RP_CASE(64, 4)
    } else {
        const int vpl = (E + 15) / 16;
        MOE_RP_CASE(16, 4)
        MOE_RP_CASE(16, 8)
        MOE_RP_CASE(16, 16)
    }
#undef MOE_RP_CASE
    return -1;
}
