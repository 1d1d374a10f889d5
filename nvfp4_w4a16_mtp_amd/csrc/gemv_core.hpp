// W4A16 decode GEMV core: y[m][n] = sum_k x[m][k] * e2m1[n][k] * e4m3[n][k/16]
// (times the global scale in the epilogue), for M <= 8 activation rows.
//
// The operation is the `w4a16_decode_gemv` of mtp_head.rs (`MtpHead::gemv`)
// and its batched-M tiers (one pass over the weight serves all rows).  On
// gfx950 it is bound by HBM: every weight byte is read exactly once with
// 16-byte loads, the activations are staged once per workgroup in LDS.
//
// Work mapping (workgroup = 256 threads = 4 wavefronts):
//  * a "slot" is 16 lanes (one DPP row); a slot owns R weight rows and the
//    16 lanes split the row's K/32 chunks (16 bytes of codes + 2 scale bytes
//    = 32 weights per chunk) round-robin;
//  * with KS > 1 the 4 wavefronts split K into KS segments over the same
//    rows (for short-and-wide matrices that would otherwise leave CUs idle);
//  * a workgroup tile is 16 * R / KS rows; workgroups stride over tiles.
// Per chunk a lane converts 32 E2M1 codes to bf16 with the hardware FP4
// converter (exact), takes bf16 dot products with the activation chunk read
// from LDS (fp32 accumulation), and applies the two E4M3 block scales with
// one FMA each.  The 16 lanes of a slot are summed with a fixed DPP
// butterfly, so every row is reduced in the same order wherever it runs.
#pragma once

#include <climits>
#include <math.h>

#include "common.hpp"

namespace nvfp4 {

// LDS image of x: 16-byte units, unit (m, q, c) = x[m][32c + 8q .. 32c + 8q + 8)
// at index (m * 4 + q) * C + c, so that the 16 lanes of a slot reading
// consecutive chunks hit consecutive LDS addresses.
__device__ __forceinline__ void stage_x(uint4 *xs, const uint4 *__restrict__ x, int m, int k) {
    const int C = k >> 5;
    const int units = m * (k >> 3);
    for (int p = threadIdx.x; p < units; p += blockDim.x) {
        int mm = p / (k >> 3), w = p - mm * (k >> 3);
        int c = w >> 2, q = w & 3;
        xs[(mm * 4 + q) * C + c] = x[p];
    }
}

template <int M, int R, int KS>
struct GemvTile {
    static constexpr int kRowsPerTile = 16 * R / KS;
};

// Computes the tile's dot products; calls epi(row, m, value) once per
// (row < n, m < M) with the fp32 sum (before the global scale), from lane
// m of the slot in the K-segment-0 wavefront.  red: LDS scratch of
// 16 * R * M floats (used when KS > 1).
template <int M, int R, int KS, class Epi>
__device__ __forceinline__ void gemv_tile(const uint4 *xs, const uint8_t *__restrict__ codes,
                                          const uint8_t *__restrict__ scales, int n, int k, int row0,
                                          float *red, Epi &&epi) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int slot = lane >> 4, t = lane & 15;
    const int ks = (KS == 1) ? 0 : (wave % KS);
    const int rg = wave / KS;
    const int C = k >> 5;
    const int cs = (C + KS - 1) / KS;
    const int c_lo = ks * cs;
    const int c_hi = min(C, c_lo + cs);
    const int rbase = row0 + (rg * 4 + slot) * R;

    float acc[R][M];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int mm = 0; mm < M; ++mm) acc[r][mm] = 0.0f;

    const size_t row_code_bytes = (size_t)(k >> 1), row_scale_bytes = (size_t)(k >> 4);

    for (int c = c_lo + t; c < c_hi; c += 16) {
        uint4 cw[R];
        uint32_t sw[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int row = rbase + r;
            if (row < n) {
                cw[r] = *reinterpret_cast<const uint4 *>(codes + (size_t)row * row_code_bytes + 16 * (size_t)c);
                sw[r] = *reinterpret_cast<const uint16_t *>(scales + (size_t)row * row_scale_bytes + 2 * (size_t)c);
            } else {
                cw[r] = make_uint4(0, 0, 0, 0);
                sw[r] = 0;
            }
        }
        uint4 xv[M][4];
#pragma unroll
        for (int mm = 0; mm < M; ++mm)
#pragma unroll
            for (int q = 0; q < 4; ++q) xv[mm][q] = xs[(mm * 4 + q) * C + c];

#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float sf0 = e4m3_to_f32(sw[r] & 0xFFu), sf1 = e4m3_to_f32(sw[r] >> 8);
            const uint32_t cwd[4] = {cw[r].x, cw[r].y, cw[r].z, cw[r].w};
            bf16x2 wv[16];
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                wv[4 * d + 0] = e2m1x2_to_bf16<0>(cwd[d]);
                wv[4 * d + 1] = e2m1x2_to_bf16<1>(cwd[d]);
                wv[4 * d + 2] = e2m1x2_to_bf16<2>(cwd[d]);
                wv[4 * d + 3] = e2m1x2_to_bf16<3>(cwd[d]);
            }
#pragma unroll
            for (int mm = 0; mm < M; ++mm) {
                const uint32_t x0[8] = {xv[mm][0].x, xv[mm][0].y, xv[mm][0].z, xv[mm][0].w,
                                        xv[mm][1].x, xv[mm][1].y, xv[mm][1].z, xv[mm][1].w};
                const uint32_t x1[8] = {xv[mm][2].x, xv[mm][2].y, xv[mm][2].z, xv[mm][2].w,
                                        xv[mm][3].x, xv[mm][3].y, xv[mm][3].z, xv[mm][3].w};
                float b0 = 0.0f, b1 = 0.0f;
#pragma unroll
                for (int i = 0; i < 8; ++i) b0 = dot2(wv[i], as_bf16x2(x0[i]), b0);
#pragma unroll
                for (int i = 0; i < 8; ++i) b1 = dot2(wv[8 + i], as_bf16x2(x1[i]), b1);
                acc[r][mm] = __builtin_fmaf(b0, sf0, acc[r][mm]);
                acc[r][mm] = __builtin_fmaf(b1, sf1, acc[r][mm]);
            }
        }
    }

#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int mm = 0; mm < M; ++mm) acc[r][mm] = row16_sum(acc[r][mm]);

    if constexpr (KS == 1) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int row = rbase + r;
#pragma unroll
            for (int mm = 0; mm < M; ++mm)
                if (t == mm && row < n) epi(row, mm, acc[r][mm]);
        }
    } else {
        // red[((rg * 4 + slot) * R + r) * KS + ks][M]
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int mm = 0; mm < M; ++mm)
                if (t == mm) red[((((rg * 4 + slot) * R + r) * KS + ks) * M) + mm] = acc[r][mm];
        __syncthreads();
        if (ks == 0) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int row = rbase + r;
#pragma unroll
                for (int mm = 0; mm < M; ++mm) {
                    if (t == mm && row < n) {
                        const float *p = red + (((rg * 4 + slot) * R + r) * KS) * M + mm;
                        float v = p[0];
#pragma unroll
                        for (int s = 1; s < KS; ++s) v += p[s * M];
                        epi(row, mm, v);
                    }
                }
            }
        }
        __syncthreads();
    }
}

// Host-side choice of the tile shape for an n-row weight: the largest R
// (fewest, fattest tiles) that still gives at least two workgroups per CU,
// else split K across the wavefronts.
struct TileChoice {
    int R, KS;
};
// allow_ksplit is false when the K-split reduction scratch would not fit
// next to the activation image in LDS.
inline TileChoice choose_tile(int n, int cus, bool allow_ksplit) {
    static const TileChoice order[] = {{4, 1}, {2, 1}, {1, 1}, {1, 2}, {1, 4}};
    for (const TileChoice &c : order) {
        if (c.KS > 1 && !allow_ksplit) break;
        int rows = 16 * c.R / c.KS;
        if ((n + rows - 1) / rows >= 2 * cus) return c;
    }
    return allow_ksplit ? TileChoice{1, 4} : TileChoice{1, 1};
}

constexpr int kLdsBytes = 64 * 1024;   // LDS budget of one workgroup

// LDS bytes of a GEMV workgroup: the activation image plus, with a K split,
// 16 * R * M fp32 partial sums.
inline size_t gemv_lds_bytes(int m, int k, TileChoice tc) {
    return (size_t)m * k * 2 + (tc.KS > 1 ? (size_t)16 * tc.R * m * 4 : 0);
}
inline bool ksplit_fits(int m, int k) { return gemv_lds_bytes(m, k, TileChoice{1, 2}) <= (size_t)kLdsBytes; }

}  // namespace nvfp4
