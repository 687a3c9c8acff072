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
#include "moe_device.h"
#include "moe_internal.h"

namespace {

constexpr int kThreads = 512;          // 8 waves; one chunk = 512 assignments
constexpr int kWaves = kThreads / 64;
constexpr int kSmallChunks = 8;        // single-workgroup path up to 4096 assignments

MOE_DEV uint64_t lanemask_lt(int lane) { return (lane == 0) ? 0ull : (~0ull >> (64 - lane)); }

// Block-wide exclusive scan of n values in LDS (in place), n <= 4 * blockDim.
// part: LDS scratch of blockDim ints. Returns the total to every thread.
MOE_DEV int block_exclusive_scan(int* vals, int n, int* part) {
    const int tid = threadIdx.x, nt = blockDim.x;
    const int per = (n + nt - 1) / nt;
    const int lo = tid * per, hi = min(n, lo + per);
    int s = 0;
    for (int i = lo; i < hi; ++i) s += vals[i];
    part[tid] = s;
    __syncthreads();
    for (int off = 1; off < nt; off <<= 1) {
        int add = tid >= off ? part[tid - off] : 0;
        __syncthreads();
        part[tid] += add;
        __syncthreads();
    }
    int run = part[tid] - s;            // exclusive prefix of this thread's segment
    int total = part[nt - 1];
    for (int i = lo; i < hi; ++i) { int v = vals[i]; vals[i] = run; run += v; }
    __syncthreads();
    return total;
}

// counts (LDS, G entries) -> counts/offsets/offsets32 in global memory.
MOE_DEV void write_offsets(int* lds_counts, int* lds_tmp, int G, int* part,
                           int32_t* counts, int32_t* offsets, int32_t* offsets32) {
    const int tid = threadIdx.x, nt = blockDim.x;
    for (int g = tid; g < G; g += nt) {
        counts[g] = lds_counts[g];
        lds_tmp[g] = (lds_counts[g] + 31) & ~31;
    }
    __syncthreads();
    int total = block_exclusive_scan(lds_counts, G, part);   // lds_counts becomes offsets
    int total32 = 0;
    if (offsets32) total32 = block_exclusive_scan(lds_tmp, G, part);
    for (int g = tid; g < G; g += nt) {
        offsets[g] = lds_counts[g];
        if (offsets32) offsets32[g] = lds_tmp[g];
    }
    if (tid == 0) {
        offsets[G] = total;
        if (offsets32) offsets32[G] = total32;
    }
    __syncthreads();
}

// One wave: rank of each lane's group among the lanes below it with the same
// group, and the per-group lane count written by the group's leader lane.
MOE_DEV int wave_match_rank(int g, int lane, uint16_t* wave_cnt /* [E_loc] of this wave */) {
    uint64_t rem = __ballot(g >= 0);
    int rank = 0;
    while (rem) {
        int leader = __ffsll((unsigned long long)rem) - 1;
        int lg = __shfl(g, leader, 64);
        uint64_t m = __ballot(g == lg) & rem;
        if (g == lg) rank = __popcll(m & lanemask_lt(lane));
        if (lane == leader) wave_cnt[lg] = (uint16_t)__popcll(m);
        rem &= ~m;
    }
    return rank;
}

// Chunk: wave ranks -> per-wave exclusive prefix in cnt (in place) and the
// chunk totals in tot (if non-null). Callers zero cnt beforehand.
MOE_DEV void scan_waves(uint16_t* cnt, int E_loc, int* tot) {
    for (int g = threadIdx.x; g < E_loc; g += blockDim.x) {
        int run = 0;
        #pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            int v = cnt[w * E_loc + g];
            cnt[w * E_loc + g] = (uint16_t)run;
            run += v;
        }
        if (tot) tot[g] = run;
    }
}

MOE_DEV void write_row(int a, int g, int row, int k, int ks, const float* topk_w,
                       int32_t* row_src, float* row_w, int32_t* slot_row) {
    int t = a / k, j = a - t * k;
    if (g >= 0) {
        row_src[row] = t;
        row_w[row] = topk_w[a];
        slot_row[(size_t)t * ks + j] = row;
    } else {
        slot_row[(size_t)t * ks + j] = -1;
    }
}

MOE_DEV void write_shared_rows(int t0, int t1, int T, int k, int ks, int base,
                               int32_t* row_src, float* row_w, int32_t* slot_row) {
    for (int t = t0 + (int)threadIdx.x; t < min(T, t1); t += blockDim.x) {
        int r = base + t;
        row_src[r] = t;
        row_w[r] = 1.0f;
        slot_row[(size_t)t * ks + k] = r;
    }
}

// ---- single-workgroup path ---------------------------------------------
__global__ __launch_bounds__(kThreads)
void permute_small_kernel(const int32_t* __restrict__ topk_idx, const float* __restrict__ topk_w,
                          int T, int k, int e0, int E_loc, int s,
                          int32_t* counts, int32_t* offsets, int32_t* offsets32,
                          int32_t* row_src, float* row_w, int32_t* slot_row) {
    extern __shared__ int lds[];
    const int G = E_loc + s;
    int* hist = lds;                       // [G]   counts, then offsets
    int* tmp = hist + G;                   // [G]   roundup counts / chunk totals
    int* base = tmp + G;                   // [G]   running row of each group
    int* part = base + G;                  // [kThreads]
    uint16_t* cnt = (uint16_t*)(part + kThreads);   // [kWaves][E_loc]
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int Tk = T * k, ks = k + s;

    for (int g = tid; g < G; g += kThreads) hist[g] = 0;
    __syncthreads();
    for (int a = tid; a < Tk; a += kThreads) {
        int g = topk_idx[a] - e0;
        if (g >= 0 && g < E_loc) atomicAdd(&hist[g], 1);
    }
    __syncthreads();
    if (s && tid == 0) hist[E_loc] = T;
    __syncthreads();
    write_offsets(hist, tmp, G, part, counts, offsets, offsets32);
    for (int g = tid; g < G; g += kThreads) base[g] = hist[g];
    __syncthreads();

    for (int c0 = 0; c0 < Tk; c0 += kThreads) {
        for (int i = tid; i < kWaves * E_loc; i += kThreads) cnt[i] = 0;
        __syncthreads();
        int a = c0 + tid;
        int g = -1;
        if (a < Tk) {
            int gg = topk_idx[a] - e0;
            if (gg >= 0 && gg < E_loc) g = gg;
        }
        int rank = wave_match_rank(g, lane, cnt + w * E_loc);
        __syncthreads();
        scan_waves(cnt, E_loc, tmp);
        __syncthreads();
        if (a < Tk) {
            int row = g >= 0 ? base[g] + cnt[w * E_loc + g] + rank : -1;
            write_row(a, g, row, k, ks, topk_w, row_src, row_w, slot_row);
        }
        __syncthreads();
        for (int gg = tid; gg < E_loc; gg += kThreads) base[gg] += tmp[gg];
        __syncthreads();
    }
    if (s) write_shared_rows(0, T, T, k, ks, hist[E_loc], row_src, row_w, slot_row);
}

// ---- chunked path: count, scan, scatter --------------------------------
__global__ __launch_bounds__(kThreads)
void permute_count_kernel(const int32_t* __restrict__ topk_idx, int Tk, int e0, int E_loc,
                          int32_t* __restrict__ chunk_hist) {
    extern __shared__ int lds[];
    const int tid = threadIdx.x, c = blockIdx.x;
    for (int g = tid; g < E_loc; g += kThreads) lds[g] = 0;
    __syncthreads();
    int a = c * kThreads + tid;
    if (a < Tk) {
        int g = topk_idx[a] - e0;
        if (g >= 0 && g < E_loc) atomicAdd(&lds[g], 1);
    }
    __syncthreads();
    for (int g = tid; g < E_loc; g += kThreads) chunk_hist[(size_t)c * E_loc + g] = lds[g];
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
    int* tmp = cnt + G;                 // [G]
    int* part = tmp + G;                // [kScanThreads] block-scan scratch
    int* psum = part + kScanThreads;    // [kScanThreads] per-thread run sums
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
    write_offsets(cnt, tmp, G, part, counts, offsets, offsets32);

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

__global__ __launch_bounds__(kThreads)
void permute_scatter_kernel(const int32_t* __restrict__ topk_idx, const float* __restrict__ topk_w,
                            int T, int k, int e0, int E_loc, int s,
                            const int32_t* __restrict__ chunk_base, const int32_t* __restrict__ offsets,
                            int32_t* row_src, float* row_w, int32_t* slot_row) {
    extern __shared__ int lds[];
    uint16_t* cnt = (uint16_t*)lds;          // [kWaves][E_loc]
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, c = blockIdx.x;
    const int Tk = T * k, ks = k + s;
    for (int i = tid; i < kWaves * E_loc; i += kThreads) cnt[i] = 0;
    __syncthreads();
    int a = c * kThreads + tid;
    int g = -1;
    if (a < Tk) {
        int gg = topk_idx[a] - e0;
        if (gg >= 0 && gg < E_loc) g = gg;
    }
    int rank = wave_match_rank(g, lane, cnt + w * E_loc);
    __syncthreads();
    scan_waves(cnt, E_loc, nullptr);
    __syncthreads();
    if (a < Tk) {
        int row = g >= 0 ? chunk_base[(size_t)c * E_loc + g] + cnt[w * E_loc + g] + rank : -1;
        write_row(a, g, row, k, ks, topk_w, row_src, row_w, slot_row);
    }
    if (s) write_shared_rows(c * kThreads, (c + 1) * kThreads, T, k, ks, offsets[E_loc],
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

}  // namespace

size_t moe_permute_scratch_bytes(int T, int k, int G) {
    size_t nchunks = ((size_t)T * k + kThreads - 1) / kThreads;
    return (nchunks > (size_t)kSmallChunks) ? nchunks * (size_t)G * 4 : 0;
}

int moe_launch_permute(const int32_t* topk_idx, const float* topk_w, int T, int k, int e0,
                       int E_loc, int s, const uint8_t* xq, const uint8_t* xs, int H,
                       int32_t* counts, int32_t* offsets, int32_t* offsets32, int32_t* row_src,
                       float* row_w, int32_t* slot_row, uint8_t* xq_perm, uint8_t* xs_perm,
                       void* scratch, hipStream_t stream) {
    const int G = E_loc + s;
    const int Tk = T * k;
    const int nchunks = (Tk + kThreads - 1) / kThreads;
    hipError_t e;
    if (nchunks <= kSmallChunks) {
        size_t lds = (size_t)(3 * G + kThreads) * 4 + (size_t)kWaves * E_loc * 2;
        hipLaunchKernelGGL(permute_small_kernel, dim3(1), dim3(kThreads), lds, stream,
                           topk_idx, topk_w, T, k, e0, E_loc, s, counts, offsets, offsets32,
                           row_src, row_w, slot_row);
    } else {
        int32_t* chunk_hist = (int32_t*)scratch;
        hipLaunchKernelGGL(permute_count_kernel, dim3(nchunks), dim3(kThreads),
                           (size_t)E_loc * 4, stream, topk_idx, Tk, e0, E_loc, chunk_hist);
        int P = 1;
        while (P * 2 <= kScanThreads / E_loc && P * 2 <= nchunks) P *= 2;
        hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(kScanThreads),
                           (size_t)(2 * G + 2 * kScanThreads) * 4, stream, chunk_hist, nchunks, T,
                           E_loc, s, P, counts, offsets, offsets32);
        hipLaunchKernelGGL(permute_scatter_kernel, dim3(nchunks), dim3(kThreads),
                           (size_t)kWaves * E_loc * 2 + 4, stream, topk_idx, topk_w, T, k, e0,
                           E_loc, s, chunk_hist, offsets, row_src, row_w, slot_row);
    }
    if ((e = hipGetLastError()) != hipSuccess) return (int)e;
    if (xq_perm && T > 0) {
        const int R_max = Tk + s * T;
        int blocks = (R_max + kGatherRows - 1) / kGatherRows;
        hipLaunchKernelGGL(gather_kernel, dim3(blocks), dim3(256), 0, stream, xq, xs, H, row_src,
                           offsets, G, xq_perm, xs_perm);
        if ((e = hipGetLastError()) != hipSuccess) return (int)e;
    }
    return 0;
}
