// Weight-streaming pieces shared by the decode-shaped grouped GEMM kernel
// and the single-launch decode layer: one wave's batch of K-tiles of a 64-row
// prepacked weight unit (the scaled MFMA's A operand, streamed from HBM into
// registers) against 16-row token tiles (the B operand), and the MFMAs over
// it. Internal to libmoe.
#pragma once
#include "gemm_common.h"

namespace {

// K-tiles per load batch: four FP4 (two FP8) weight K-tiles for one token
// tile, fewer when several token tiles share the batch.
template <int WFMT, int NTT>
constexpr int batch_kt() {
    return ((WFMT == MFMA_FMT_FP4 ? 4 : 2) / NTT) > 0 ? (WFMT == MFMA_FMT_FP4 ? 4 : 2) / NTT : 1;
}

template <int WFMT>
struct ATile {                        // one lane's part of a 16x128 weight tile
    i32x4 lo, hi;                     // hi used for FP8 only
};

template <int WFMT>
MOE_DEV i32x8 a_operand(const ATile<WFMT>& t) {
    i32x8 r;
    r[0] = t.lo[0]; r[1] = t.lo[1]; r[2] = t.lo[2]; r[3] = t.lo[3];
    if (WFMT == MFMA_FMT_FP8) { r[4] = t.hi[0]; r[5] = t.hi[1]; r[6] = t.hi[2]; r[7] = t.hi[3]; }
    else { r[4] = 0; r[5] = 0; r[6] = 0; r[7] = 0; }
    return r;
}

// Operands of one batch of KBT K-tiles for one wave: TPI of the unit's four
// 16-row weight tiles (all four, or a half unit).
template <int WFMT, int NTT, int TPI = 4, int KBT = batch_kt<WFMT, NTT>()>
struct Batch {
    static constexpr int KB = KBT;
    ATile<WFMT> A[KB][TPI];           // [kt][tile]
    int sA[KB][TPI];                  // E8M0 of (tile row, kt) in the low byte after the shift
    i32x4 Blo[NTT][KB], Bhi[NTT][KB];
    int sB[NTT][KB];
};

// CP: cache policy of the weight loads (kNonTemporal when no other pass of
// the group reads the same weights, 0 when other passes do and can find them
// in L2); XCP: cache policy of the activation loads (agent-coherent when
// other workgroups wrote them during the same launch)
template <int WFMT, int NTT, int CP, int TPI = 4, int KBT = batch_kt<WFMT, NTT>(), int XCP = 0>
MOE_DEV void load_batch(Batch<WFMT, NTT, TPI, KBT>& b, int kt_first, int kt_end, int lane,
                        rsrc_t rw, rsrc_t rs, rsrc_t rx, rsrc_t rxs, const uint32_t (&xoff)[NTT],
                        const uint32_t (&xsoff)[NTT], int t0 = 0) {
    constexpr int BPL = WFMT == MFMA_FMT_FP4 ? 16 : 32;
    constexpr int KB = KBT;
    const int grp = lane >> 4;
    // weight scales: batches never straddle a group of four K-tiles, so one
    // dword per tile covers the batch
    int sword[TPI];
    #pragma unroll
    for (int t = 0; t < TPI; ++t) {
        const uint32_t soff = kt_first < kt_end ? (uint32_t)((((kt_first >> 2) * 4 + t0 + t) * 64 + lane) * 4)
                                                : kInvalid;
        sword[t] = (int)__builtin_amdgcn_raw_buffer_load_b32(rs, soff, 0, CP);
    }
    #pragma unroll
    for (int i = 0; i < KB; ++i) {
        const int kt = kt_first + i;
        const bool ok = kt < kt_end;                       // uniform
        #pragma unroll
        for (int t = 0; t < TPI; ++t) {
            // FP4: lane's 16 B at lane*16; FP8: the two 16 B halves at lane*16 and 1024 + lane*16
            const uint32_t off = ok ? (uint32_t)((kt * 4 + t0 + t) * 64 * BPL + lane * 16) : kInvalid;
            b.A[i][t].lo = __builtin_amdgcn_raw_buffer_load_b128(rw, off, 0, CP);
            if (WFMT == MFMA_FMT_FP8)
                b.A[i][t].hi = __builtin_amdgcn_raw_buffer_load_b128(rw, off + (ok ? 1024u : 0u), 0, CP);
            b.sA[i][t] = sword[t] >> (8 * (kt & 3));
        }
        #pragma unroll
        for (int tt = 0; tt < NTT; ++tt) {
            const bool v = ok && xoff[tt] != kInvalid;
            const uint32_t o = v ? xoff[tt] + (uint32_t)(kt * 128 + 16 * grp) : kInvalid;
            b.Blo[tt][i] = __builtin_amdgcn_raw_buffer_load_b128(rx, o, 0, XCP);
            b.Bhi[tt][i] = __builtin_amdgcn_raw_buffer_load_b128(rx, v ? o + 64u : kInvalid, 0, XCP);
            const uint32_t so = v ? xsoff[tt] + (uint32_t)(kt * 4 + grp) : kInvalid;
            b.sB[tt][i] = (int)__builtin_amdgcn_raw_buffer_load_b8(rxs, so, 0, XCP);
        }
    }
}

template <int WFMT, int NTT, int TPI = 4, int KBT = batch_kt<WFMT, NTT>()>
MOE_DEV void mma_batch(const Batch<WFMT, NTT, TPI, KBT>& b, int ntt_active, f32x4 (&acc)[NTT][TPI]) {
    constexpr int KB = KBT;
    #pragma unroll
    for (int i = 0; i < KB; ++i) {
        #pragma unroll
        for (int tt = 0; tt < NTT; ++tt) {
            if (tt < ntt_active) {
                i32x8 B;
                B[0] = b.Blo[tt][i][0]; B[1] = b.Blo[tt][i][1]; B[2] = b.Blo[tt][i][2]; B[3] = b.Blo[tt][i][3];
                B[4] = b.Bhi[tt][i][0]; B[5] = b.Bhi[tt][i][1]; B[6] = b.Bhi[tt][i][2]; B[7] = b.Bhi[tt][i][3];
                #pragma unroll
                for (int t = 0; t < TPI; ++t)
                    acc[tt][t] = mfma16x16x128<WFMT, MFMA_FMT_FP8, 0, 0>(a_operand<WFMT>(b.A[i][t]), B,
                                                                        acc[tt][t], b.sA[i][t], b.sB[tt][i]);
            }
        }
    }
}

}  // namespace
