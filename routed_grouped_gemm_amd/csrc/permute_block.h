// Block-level S1-S3 pieces shared by the permute kernels and the decode W1
// kernel that routes its own tokens: routing of a few tokens by the waves of
// one workgroup, and the whole grouping of up to a few thousand assignments
// in one workgroup (GC-MoE page, "Approach": routing-count aggregation before
// the token blocks are filled; fusion blog, "Removing host-device
// synchronisation"). Internal to libmoe.
#pragma once
#include "moe_device.h"
#include "moe_internal.h"

namespace {

MOE_DEV uint64_t lanemask_lt(int lane) { return (lane == 0) ? 0ull : (~0ull >> (64 - lane)); }

// counts (LDS, G entries) -> counts/offsets/offsets32 in global memory; the
// LDS array holds the offsets afterwards. Wave 0 scans: each lane takes a run
// of ceil(G/64) consecutive groups, the lanes' run totals are scanned with
// shuffles, then each lane writes its run.
MOE_DEV void write_offsets(int* lds_counts, int G, int32_t* counts, int32_t* offsets,
                           int32_t* offsets32) {
    __syncthreads();
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        const int per = (G + 63) / 64;
        const int lo = min(G, lane * per), hi = min(G, lo + per);
        int s = 0, s32 = 0;
        for (int i = lo; i < hi; ++i) {
            const int c = lds_counts[i];
            s += c;
            s32 += (c + 31) & ~31;
        }
        const int inc = wave_incl_scan(s), inc32 = wave_incl_scan(s32);   // inclusive scans over lanes
        int run = inc - s, run32 = inc32 - s32;
        for (int i = lo; i < hi; ++i) {
            const int c = lds_counts[i];
            counts[i] = c;
            offsets[i] = run;
            if (offsets32) offsets32[i] = run32;
            lds_counts[i] = run;
            run += c;
            run32 += (c + 31) & ~31;
        }
        if (lane == 63) {
            offsets[G] = inc;
            if (offsets32) offsets32[G] = inc32;
        }
    }
    __syncthreads();
}

// One wave: rank of each lane's group among the lanes below it with the same
// group, and the per-group lane count written by the group's lowest lane.
// The lanes sharing a lane's group are found with one ballot per bit of the
// group index (gbits bits), in constant time however many groups the wave
// holds. Lanes with g < 0 take no part; their rank is meaningless.
MOE_DEV int wave_match_rank(int g, int lane, int gbits, uint16_t* wave_cnt /* [E_loc] of this wave */) {
    uint64_t same = __ballot(g >= 0);
    for (int b = 0; b < gbits; ++b) {
        const bool bit = (g >> b) & 1;
        const uint64_t m = __ballot(bit);
        same &= bit ? m : ~m;
    }
    const int rank = __popcll(same & lanemask_lt(lane));
    if (g >= 0 && rank == 0) wave_cnt[g] = (uint16_t)__popcll(same);
    return rank;
}

// Bits of a group index in [0, E_loc).
__host__ __device__ inline int group_bits(int E_loc) { return E_loc > 1 ? 32 - __builtin_clz((unsigned)(E_loc - 1)) : 0; }

// Per-wave lane counts of one chunk -> per-wave exclusive prefix (in place),
// and the chunk totals in tot (if non-null).
template <int NW>
MOE_DEV void scan_waves(uint16_t* cnt, int E_loc, int* tot) {
    for (int g = threadIdx.x; g < E_loc; g += blockDim.x) {
        int run = 0;
        #pragma unroll
        for (int w = 0; w < NW; ++w) {
            int v = cnt[w * E_loc + g];
            cnt[w * E_loc + g] = (uint16_t)run;
            run += v;
        }
        if (tot) tot[g] = run;
    }
}

MOE_DEV void write_row(int a, int g, int row, int k, int ks, float w,
                       int32_t* row_src, float* row_w, int32_t* slot_row) {
    int t = a / k, j = a - t * k;
    if (g >= 0) {
        row_src[row] = t;
        row_w[row] = w;
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

// LDS ints needed by permute_in_block.
constexpr size_t block_lds_ints(int NW, int G, int E_loc) {
    return (size_t)3 * G + ((size_t)NW * E_loc * 2 + 3) / 4;
}

// The whole S2/S3 computation for at most 64 * APL assignments and 64 groups,
// in one wave with neither LDS nor barriers: slot i of lane l holds
// assignment a = 64 i + l, lane q stands for group q. Each lane compares the
// groups of every lane's slot i with its own target bit by bit, most
// significant first, through one ballot per slot and bit: with target q this
// counts group q's assignments in each slot and those of lower groups (count
// and offset of group q); with target g(a) it finds the lower lanes of the
// same group in a's slot. An assignment's row is then its group's offset,
// plus the group's assignments in earlier slots, plus its rank in its slot:
// stable in a.
template <int APL, class IdxF, class WF>
MOE_DEV void permute_in_wave(IdxF idx_of, WF w_of, int T, int k, int e0, int E_loc, int s,
                             int32_t* counts, int32_t* offsets, int32_t* offsets32,
                             int32_t* row_src, float* row_w, int32_t* slot_row, int lane) {
    const int Tk = T * k, ks = k + s, G = E_loc + s;
    const int gbits = group_bits(E_loc);
    const int q = lane;
    int g[APL];
    uint64_t eq_q[APL], lt_q[APL], eq_a[APL];
    #pragma unroll
    for (int i = 0; i < APL; ++i) {
        const int a = 64 * i + lane;
        g[i] = -1;
        if (a < Tk) {
            const int gg = idx_of(a) - e0;
            if (gg >= 0 && gg < E_loc) g[i] = gg;
        }
        eq_q[i] = eq_a[i] = __ballot(g[i] >= 0);
        lt_q[i] = 0;
    }
    for (int b = gbits - 1; b >= 0; --b) {
        const bool qb = (q >> b) & 1;
        #pragma unroll
        for (int i = 0; i < APL; ++i) {
            const bool gb = g[i] >= 0 && ((g[i] >> b) & 1);
            const uint64_t m = __ballot(gb);
            lt_q[i] = qb ? (lt_q[i] | (eq_q[i] & ~m)) : lt_q[i];
            eq_q[i] = qb ? (eq_q[i] & m) : (eq_q[i] & ~m);
            eq_a[i] = gb ? (eq_a[i] & m) : (eq_a[i] & ~m);
        }
    }
    int routed = 0, cnt = 0, off = 0;
    int before[APL];                        // group q's assignments in slots < i
    #pragma unroll
    for (int i = 0; i < APL; ++i) {
        before[i] = cnt;
        routed += __popcll(__ballot(g[i] >= 0));
        cnt += __popcll(eq_q[i]);
        off += __popcll(lt_q[i]);
    }
    if (q >= E_loc) {                       // the shared group (every token, after the routed rows), or none
        cnt = q < G ? T : 0;
        off = q < G ? routed : 0;
    }
    // offsets32: exclusive scan over the groups of the 32-rounded counts
    const int c32 = (cnt + 31) & ~31;
    const int inc = wave_incl_scan(c32);
    if (q < G) {
        counts[q] = cnt;
        offsets[q] = off;
        if (offsets32) offsets32[q] = inc - c32;
    }
    if (q == G - 1) {
        offsets[G] = off + cnt;
        if (offsets32) offsets32[G] = inc;
    }
    #pragma unroll
    for (int i = 0; i < APL; ++i) {
        const int base = __shfl(off + before[i], g[i] >= 0 ? g[i] : 0, 64);
        const int a = 64 * i + lane;
        if (a < Tk) {
            const int row = g[i] >= 0 ? base + __popcll(eq_a[i] & lanemask_lt(lane)) : -1;
            write_row(a, g[i], row, k, ks, g[i] >= 0 ? w_of(a) : 0.f, row_src, row_w, slot_row);
        }
    }
    if (s)
        for (int t = lane; t < T; t += 64) {
            const int r = routed + t;
            row_src[r] = t;
            row_w[r] = 1.0f;
            slot_row[(size_t)t * ks + k] = r;
        }
}

// The whole S2/S3 computation of up to 4096 assignments in one workgroup of
// NW waves. idx_of(a) / w_of(a) read the routing of flattened assignment a.
// At most 256 assignments and 64 groups: wave 0 alone (permute_in_wave).
template <int NW, class IdxF, class WF>
MOE_DEV void permute_in_block(IdxF idx_of, WF w_of, int T, int k, int e0, int E_loc, int s,
                              int32_t* counts, int32_t* offsets, int32_t* offsets32,
                              int32_t* row_src, float* row_w, int32_t* slot_row, int* lds) {
    constexpr int NT = NW * 64;
    const int G = E_loc + s;
    if (T * k <= 256 && G <= 64) {
        if (threadIdx.x < 64) {
            const int Tk = T * k, l = (int)threadIdx.x;
            if (Tk <= 64)
                permute_in_wave<1>(idx_of, w_of, T, k, e0, E_loc, s, counts, offsets, offsets32,
                                   row_src, row_w, slot_row, l);
            else if (Tk <= 128)
                permute_in_wave<2>(idx_of, w_of, T, k, e0, E_loc, s, counts, offsets, offsets32,
                                   row_src, row_w, slot_row, l);
            else
                permute_in_wave<4>(idx_of, w_of, T, k, e0, E_loc, s, counts, offsets, offsets32,
                                   row_src, row_w, slot_row, l);
        }
        return;
    }
    int* hist = lds;                       // [G]   counts, then offsets
    int* tmp = hist + G;                   // [G]   chunk totals
    int* base = tmp + G;                   // [G]   running row of each group
    uint16_t* cnt = (uint16_t*)(base + G);     // [NW][E_loc]
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int Tk = T * k, ks = k + s;
    const int gbits = group_bits(E_loc);

    for (int g = tid; g < G; g += NT) hist[g] = 0;
    __syncthreads();
    for (int a = tid; a < Tk; a += NT) {
        int g = idx_of(a) - e0;
        if (g >= 0 && g < E_loc) atomicAdd(&hist[g], 1);
    }
    __syncthreads();
    if (s && tid == 0) hist[E_loc] = T;
    __syncthreads();
    write_offsets(hist, G, counts, offsets, offsets32);
    for (int g = tid; g < G; g += NT) base[g] = hist[g];
    __syncthreads();

    for (int c0 = 0; c0 < Tk; c0 += NT) {
        for (int i = tid; i < NW * E_loc; i += NT) cnt[i] = 0;
        __syncthreads();
        const int a = c0 + tid;
        int g = -1;
        if (a < Tk) {
            int gg = idx_of(a) - e0;
            if (gg >= 0 && gg < E_loc) g = gg;
        }
        const int rank = wave_match_rank(g, lane, gbits, cnt + w * E_loc);
        __syncthreads();
        scan_waves<NW>(cnt, E_loc, tmp);
        __syncthreads();
        if (a < Tk) {
            int row = g >= 0 ? base[g] + cnt[w * E_loc + g] + rank : -1;
            write_row(a, g, row, k, ks, g >= 0 ? w_of(a) : 0.f, row_src, row_w, slot_row);
        }
        __syncthreads();
        for (int gg = tid; gg < E_loc; gg += NT) base[gg] += tmp[gg];
        __syncthreads();
    }
    if (s) write_shared_rows(0, T, T, k, ks, hist[E_loc], row_src, row_w, slot_row);
}

// Route tokens [0, T) in the waves of one workgroup (NW waves), LPT lanes per
// token: each round a wave takes 64 / LPT tokens. sidx / sw receive the k
// selected experts and weights of each token (flattened assignment a = t * k
// + j); topk_idx / topk_w, when not null, receive them too.
template <int NW, int LPT, int VPL>
MOE_DEV void route_block(const float* __restrict__ logits, int T, int E, int k, bool renorm,
                         int* sidx, float* sw, int32_t* topk_idx, float* topk_w) {
    constexpr int TPW = 64 / LPT;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    for (int t0 = TPW * w; t0 < T; t0 += TPW * NW) {
        const int t = t0 + lane / LPT;
        float v[VPL];
        if (t < T) load_logits<LPT, VPL>(logits + (size_t)t * E, E, lane, v);
        else {
            #pragma unroll
            for (int i = 0; i < VPL; ++i) v[i] = -INFINITY;
        }
        int e = 0;
        float wt = 0.f;
        route_values<LPT, VPL>(v, t < T ? E : 0, k, renorm, lane, e, wt);
        const int j = lane & (LPT - 1);
        if (t < T && j < k) {
            sidx[t * k + j] = e;
            sw[t * k + j] = wt;
            if (topk_idx) {
                topk_idx[(size_t)t * k + j] = e;
                topk_w[(size_t)t * k + j] = wt;
            }
        }
    }
}

}  // namespace
