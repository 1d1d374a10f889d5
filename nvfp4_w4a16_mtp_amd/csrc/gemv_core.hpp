// W4A16 decode GEMV core: y[m][n] = sum_k x[m][k] * e2m1[n][k] * e4m3[n][k/16]
// (times the global scale in the epilogue), for M <= 8 activation rows.
//
// The operation is the `w4a16_decode_gemv` of mtp_head.rs (`MtpHead::gemv`)
// and its batched-M tiers (one pass over the weight serves all rows).  On
// gfx950 it is bound by HBM: every weight byte is read exactly once, with
// 16-byte non-temporal loads (the weights stream; keeping them out of the
// caches leaves room for the activations), and the activations are staged
// once per workgroup in LDS.
//
// Work mapping (workgroup = 256 threads = 4 wavefronts):
//  * a "slot" is 16 lanes (one DPP row); a slot owns R weight rows and the
//    16 lanes split the row's K/32 chunks (16 bytes of codes + 2 scale bytes
//    = 32 weights per chunk) round-robin;
//  * with KS > 1 the 4 wavefronts split K into KS segments over the same
//    rows (for short-and-wide matrices that would otherwise leave CUs idle);
//  * a workgroup tile is 16 * R / KS rows;
//  * a wide workgroup (NW = 4 * KS wavefronts) keeps 16 * R rows a tile and
//    splits their K over KS wavefront groups: for activation images so large
//    that one workgroup fills a CU's LDS, it puts 4 * KS wavefronts on the
//    CU instead of 4.
// When every lane owns exactly CPL chunks of each row (K = 512 * KS * CPL),
// all R * CPL chunk loads of a tile are issued before any arithmetic, so a
// wavefront keeps R * CPL * 1 KiB in flight; other shapes take a loop.
// Per chunk a lane converts 32 E2M1 codes to bf16 with the hardware FP4
// converter and its two E4M3 scales with the hardware FP8 converter (both
// exact), takes bf16 dot products with the activation chunk read from LDS
// (fp32 accumulation), and applies the block scales with one FMA each.  The
// 16 lanes of a slot are summed with a fixed DPP butterfly, so every row is
// reduced in the same order wherever it runs (identical rows give identical
// results).
#pragma once

#include <climits>
#include <math.h>

#include "common.hpp"

namespace nvfp4 {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 ld_stream16(const uint8_t *p) {
    u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t ld_stream2(const uint8_t *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const uint16_t *>(p));
}
// A 16-byte load with the default cache policy (its line stays in the L2
// for a later load of the rest of it).
__device__ __forceinline__ uint4 ld_l2_16(const uint8_t *p) { return *reinterpret_cast<const uint4 *>(p); }

// Both E4M3FN scale bytes of a chunk (low byte first) -> fp32, exactly.
__device__ __forceinline__ void e4m3x2_to_f32(uint32_t two, float &s0, float &s1) {
    typedef __attribute__((ext_vector_type(2))) float f32x2;
    f32x2 f = __builtin_amdgcn_cvt_pk_f32_fp8((int)two, false);
    s0 = f.x;
    s1 = f.y;
}

// Copies `units` 16-byte units into LDS: unit p is src(p) (a load, or zero)
// and lands where dst(p, value) puts it.  Each thread issues the loads of a
// batch of kStageBatch units before it stores any of them, so a batch
// costs one round trip to memory (a loop that stores each unit as it
// arrives waits one round trip per unit).
constexpr int kStageBatch = 8;
template <class Src, class Dst>
__device__ __forceinline__ void stage_batched(int units, int tid, int nthreads, Src &&src, Dst &&dst) {
    for (int p0 = tid; p0 < units; p0 += kStageBatch * nthreads) {
        uint4 v[kStageBatch];
#pragma unroll
        for (int j = 0; j < kStageBatch; ++j) {
            const int p = p0 + j * nthreads;
            v[j] = p < units ? src(p) : make_uint4(0, 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < kStageBatch; ++j) {
            const int p = p0 + j * nthreads;
            if (p < units) dst(p, v[j]);
        }
    }
}

// The activation rows of a call.  Row mm, element kk: x[mm][kk] for a plain
// call (kt = 0); with a gathered prefix (the next draft step's fc input, its
// first kt elements the embedding row of the token the LM head chose),
// element kk < kt of table row idx[mm] (a zero row for an id outside
// [0, vocab)) and element kk >= kt of x[mm][kk - kt] (rows of k - kt
// elements).  kt % 32 == 0.
struct XRows {
    const uint16_t *x;
    const int32_t *idx;
    const uint16_t *table;
    int vocab, kt;
};
__host__ __device__ inline XRows xrows_plain(const uint16_t *x) { return XRows{x, nullptr, nullptr, 0, 0}; }

// The table rows of the first (up to 64) activation rows: lane l loads
// idx[min(l, m_rt - 1)].  Issued before the weights, it is the first vector
// load to return, so waiting for it does not wait for them.
__device__ __forceinline__ int xids_issue(const XRows &xr, int m_rt) {
    const int lane = threadIdx.x & 63;
    const int v = xr.idx[lane < m_rt ? lane : m_rt - 1];
    __builtin_amdgcn_sched_barrier(0);
    return v;
}
// One gathered activation row, wavefront-uniform: its table row (row 0 for
// an id outside the table, then read as zeros) and the rest of its elements.
// lid: xids_issue()'s value; m < 64.
struct XRow {
    const uint16_t *t;   // table row
    const uint16_t *r;   // elements kt .. k-1
    bool z;              // the prefix reads as zeros
};
__device__ __forceinline__ XRow xrow(const XRows &xr, int m, int k, int lid) {
    const int id = __builtin_amdgcn_readlane(lid, m);
    XRow g;
    g.z = (unsigned int)id >= (unsigned int)xr.vocab;
    g.t = xr.table + (size_t)(g.z ? 0 : id) * xr.kt;
    g.r = xr.x + (size_t)m * (k - xr.kt);
    return g;
}
// Address of elements [kk, ...) of a gathered row, within one 32-element
// chunk (kt % 32 == 0, so a chunk lies wholly in the prefix or wholly after
// it), and whether that chunk reads as zeros.
__device__ __forceinline__ const uint16_t *xrow_addr(const XRow &g, int kk, int kt) {
    return kk < kt ? g.t + kk : g.r + (kk - kt);
}
__device__ __forceinline__ bool xrow_zero(const XRow &g, int kk, int kt) { return kk < kt && g.z; }
// The loads are unconditional (their addresses are always valid) and a zero
// chunk is masked where the value is first used, after the batch of loads
// has been issued: masking at the load made every load wait for the one
// before it.
__device__ __forceinline__ uint4 xmask(uint4 v, bool zero) {
    const uint32_t keep = zero ? 0u : ~0u;
    return make_uint4(v.x & keep, v.y & keep, v.z & keep, v.w & keep);
}
// Addresses of row mm (per lane) among the first MT gathered rows (a select
// chain; the zero flag is not picked).
template <int MT>
__device__ __forceinline__ XRow xrow_pick(const XRow (&g)[MT], int mm) {
    XRow o = g[0];
#pragma unroll
    for (int m = 1; m < MT; ++m) {
        o.t = mm == m ? g[m].t : o.t;
        o.r = mm == m ? g[m].r : o.r;
    }
    return o;
}

// LDS image of x: 16-byte units, unit (m, q, c) = x[m][32c + 8q .. 32c + 8q + 8)
// at index (m * 4 + q) * C + c, so that the 16 lanes of a slot reading
// consecutive chunks hit consecutive LDS addresses.  Rows m_rt .. MT-1 are
// zero-filled (the kernel is instantiated for MT >= m_rt rows).
template <int MT, bool XG>
__device__ __forceinline__ void stage_x(uint4 *xs, const XRows &xr, int m_rt, int k, int lid = 0) {
    static_assert(MT <= 8, "up to 8 activation rows");
    const int C = k >> 5, upr = k >> 3;
    auto put = [&](int p, uint4 v) {
        const int mm = p / upr, w = p - mm * upr;
        xs[(mm * 4 + (w & 3)) * C + (w >> 2)] = v;
    };
    if constexpr (!XG) {
        const uint4 *x = reinterpret_cast<const uint4 *>(xr.x);
        stage_batched(
            MT * upr, threadIdx.x, blockDim.x, [&](int p) { return p / upr < m_rt ? x[p] : make_uint4(0, 0, 0, 0); },
            put);
    } else {
        // rows from m_rt on load row m_rt - 1 and are masked
        XRow g[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) g[m] = xrow(xr, m < m_rt ? m : m_rt - 1, k, lid);
        uint32_t zrows = 0;   // rows whose prefix reads as zeros, and rows from m_rt on
#pragma unroll
        for (int m = 0; m < MT; ++m) zrows |= (m >= m_rt || g[m].z) ? 1u << m : 0u;
        stage_batched(
            MT * upr, threadIdx.x, blockDim.x,
            [&](int p) {
                const int mm = p / upr;
                return *reinterpret_cast<const uint4 *>(xrow_addr(xrow_pick<MT>(g, mm), 8 * (p - mm * upr), xr.kt));
            },
            [&](int p, uint4 v) {
                const int mm = p / upr;
                const int kk = 8 * (p - mm * upr);
                put(p, xmask(v, mm >= m_rt || (kk < xr.kt && ((zrows >> mm) & 1u))));
            });
    }
}

template <int R, int KS, int NW = 4>
struct GemvTile {
    static constexpr int kRowsPerTile = 4 * (NW / KS) * R;
};

// One chunk of one row: dot products with the MT activation rows, scaled.
template <int MT>
__device__ __forceinline__ void chunk_fma(const uint4 cw, uint32_t sw, const uint4 *xs, int C, int c, float (&acc)[MT]) {
    float sf0, sf1;
    e4m3x2_to_f32(sw, sf0, sf1);
    const uint32_t cwd[4] = {cw.x, cw.y, cw.z, cw.w};
    bf16x2 wv[16];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        wv[4 * d + 0] = e2m1x2_to_bf16<0>(cwd[d]);
        wv[4 * d + 1] = e2m1x2_to_bf16<1>(cwd[d]);
        wv[4 * d + 2] = e2m1x2_to_bf16<2>(cwd[d]);
        wv[4 * d + 3] = e2m1x2_to_bf16<3>(cwd[d]);
    }
#pragma unroll
    for (int mm = 0; mm < MT; ++mm) {
        const uint4 x0 = xs[(mm * 4 + 0) * C + c], x1 = xs[(mm * 4 + 1) * C + c];
        const uint4 x2 = xs[(mm * 4 + 2) * C + c], x3 = xs[(mm * 4 + 3) * C + c];
        const uint32_t xa[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
        const uint32_t xb[8] = {x2.x, x2.y, x2.z, x2.w, x3.x, x3.y, x3.z, x3.w};
        float b0 = 0.0f, b1 = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) b0 = dot2(wv[i], as_bf16x2(xa[i]), b0);
#pragma unroll
        for (int i = 0; i < 8; ++i) b1 = dot2(wv[8 + i], as_bf16x2(xb[i]), b1);
        acc[mm] = __builtin_fmaf(b0, sf0, acc[mm]);
        acc[mm] = __builtin_fmaf(b1, sf1, acc[mm]);
    }
}

// Tiles: a workgroup tile is 16 * R / KS rows (four wavefronts of four
// 16-lane slots, R rows per slot, K split over KS wavefronts).  With WT (a
// wavefront tile, KS = 1) the tile is the calling wavefront's own 4 * R rows
// starting at row0, so wavefronts can take tiles independently.
// The tile functions compute the dot products and call epi(row, m, value)
// once per (row < n, m < MT) with the fp32 sum (before the global scale),
// from lane m of the slot in the K-segment-0 wavefront.  red: LDS scratch
// of 16 * R * MT floats (used when KS > 1).
template <int MT, int R, int KS, int CPL>
struct TileRegs {
    uint4 c[R][CPL > 0 ? CPL : 1];
    uint32_t s[R][CPL > 0 ? CPL : 1];
};

template <int MT, int R, int KS, int CPL, bool WT = false>
__device__ __forceinline__ void gemv_tile_load(TileRegs<MT, R, KS, CPL> &t, const uint8_t *__restrict__ codes,
                                               const uint8_t *__restrict__ scales, int n, int k, int row0) {
    static_assert(CPL > 0, "preloading needs a fixed chunk count");
    static_assert(!WT || KS == 1, "a wavefront tile has no K split");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int slot = lane >> 4, tl = lane & 15;
    const int ks = (KS == 1) ? 0 : (wave % KS);
    const int rg = WT ? 0 : wave / KS;
    const int rbase = row0 + (rg * 4 + slot) * R;
    const int c_lo = ks * 16 * CPL;
    // rows past n load row n - 1 instead (no branch around the loads); their
    // sums are never passed to the epilogue
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int row = min(rbase + r, n - 1);
        const uint8_t *cp = codes + (size_t)row * (size_t)(k >> 1);
        const uint8_t *sp = scales + (size_t)row * (size_t)(k >> 4);
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int c = c_lo + tl + 16 * j;
            t.c[r][j] = ld_stream16(cp + 16 * (size_t)c);
            t.s[r][j] = ld_stream2(sp + 2 * (size_t)c);
        }
    }
    // keep every load of the tile ahead of the arithmetic that follows (the
    // scheduler would otherwise sink some of them next to their first use
    // and serialise their latency)
    __builtin_amdgcn_sched_barrier(0);
}

template <int MT, int R, int KS, int CPL, bool WT = false, class Epi>
__device__ __forceinline__ void gemv_tile_finish(float (&acc)[R][MT], int n, int row0, float *red, Epi &&epi) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int slot = lane >> 4, t = lane & 15;
    const int ks = (KS == 1) ? 0 : (wave % KS);
    const int rg = WT ? 0 : wave / KS;
    const int rbase = row0 + (rg * 4 + slot) * R;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int mm = 0; mm < MT; ++mm) acc[r][mm] = row16_sum(acc[r][mm]);

    if constexpr (KS == 1) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int row = rbase + r;
#pragma unroll
            for (int mm = 0; mm < MT; ++mm)
                if (t == mm && row < n) epi(row, mm, acc[r][mm]);
        }
    } else {
        // red[((rg * 4 + slot) * R + r) * KS + ks][MT]
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int mm = 0; mm < MT; ++mm)
                if (t == mm) red[((((rg * 4 + slot) * R + r) * KS + ks) * MT) + mm] = acc[r][mm];
        __syncthreads();
        if (ks == 0) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int row = rbase + r;
#pragma unroll
                for (int mm = 0; mm < MT; ++mm) {
                    if (t == mm && row < n) {
                        const float *p = red + (((rg * 4 + slot) * R + r) * KS) * MT + mm;
                        float v = p[0];
#pragma unroll
                        for (int s = 1; s < KS; ++s) v += p[s * MT];
                        epi(row, mm, v);
                    }
                }
            }
        }
        __syncthreads();
    }
}

// Full tile with fixed chunk count: loads already issued into `t`.
template <int MT, int R, int KS, int CPL, bool WT = false, class Epi>
__device__ __forceinline__ void gemv_tile_compute(const TileRegs<MT, R, KS, CPL> &t, const uint4 *xs, int n, int k,
                                                  int row0, float *red, Epi &&epi) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int tl = lane & 15;
    const int ks = (KS == 1) ? 0 : (wave % KS);
    const int C = k >> 5;
    const int c_lo = ks * 16 * CPL;
    float acc[R][MT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int mm = 0; mm < MT; ++mm) acc[r][mm] = 0.0f;
#pragma unroll
    for (int j = 0; j < CPL; ++j)
#pragma unroll
        for (int r = 0; r < R; ++r) chunk_fma<MT>(t.c[r][j], t.s[r][j], xs, C, c_lo + tl + 16 * j, acc[r]);
    gemv_tile_finish<MT, R, KS, CPL, WT>(acc, n, row0, red, epi);
}

// Single activation row with a fixed chunk count: a lane always works on the
// same CPL chunks of K, so its 32 * CPL activations live in registers for
// the whole kernel (no LDS image, no LDS reads in the inner loop).
template <int CPL>
struct XRegs {
    uint32_t w[CPL][16];
};

template <int KS, int CPL, bool XG>
__device__ __forceinline__ void load_xregs(XRegs<CPL> &xr, const XRows &x, int k, int lid = 0) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int tl = lane & 15;
    const int ks = (KS == 1) ? 0 : (wave % KS);
    const int c_lo = ks * 16 * CPL;
    XRow g{};
    if constexpr (XG) g = xrow(x, 0, k, lid);
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int kk = 32 * (c_lo + tl + 16 * j);
        const uint4 *p = reinterpret_cast<const uint4 *>(XG ? xrow_addr(g, kk, x.kt) : x.x + kk);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint4 u = p[q];
            xr.w[j][4 * q + 0] = u.x;
            xr.w[j][4 * q + 1] = u.y;
            xr.w[j][4 * q + 2] = u.z;
            xr.w[j][4 * q + 3] = u.w;
        }
    }
    if constexpr (XG) {
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const uint32_t keep = xrow_zero(g, 32 * (c_lo + tl + 16 * j), x.kt) ? 0u : ~0u;
#pragma unroll
            for (int i = 0; i < 16; ++i) xr.w[j][i] &= keep;
        }
    }
}

// One chunk of one row against register-held activations.
__device__ __forceinline__ float chunk_dot_xreg(const uint4 cw, uint32_t sw, const uint32_t (&xr)[16], float acc) {
    float sf0, sf1;
    e4m3x2_to_f32(sw, sf0, sf1);
    const uint32_t cwd[4] = {cw.x, cw.y, cw.z, cw.w};
    float b0 = 0.0f, b1 = 0.0f;
#pragma unroll
    for (int d = 0; d < 2; ++d) {
        b0 = dot2(e2m1x2_to_bf16<0>(cwd[d]), as_bf16x2(xr[4 * d + 0]), b0);
        b0 = dot2(e2m1x2_to_bf16<1>(cwd[d]), as_bf16x2(xr[4 * d + 1]), b0);
        b0 = dot2(e2m1x2_to_bf16<2>(cwd[d]), as_bf16x2(xr[4 * d + 2]), b0);
        b0 = dot2(e2m1x2_to_bf16<3>(cwd[d]), as_bf16x2(xr[4 * d + 3]), b0);
    }
#pragma unroll
    for (int d = 2; d < 4; ++d) {
        b1 = dot2(e2m1x2_to_bf16<0>(cwd[d]), as_bf16x2(xr[4 * d + 0]), b1);
        b1 = dot2(e2m1x2_to_bf16<1>(cwd[d]), as_bf16x2(xr[4 * d + 1]), b1);
        b1 = dot2(e2m1x2_to_bf16<2>(cwd[d]), as_bf16x2(xr[4 * d + 2]), b1);
        b1 = dot2(e2m1x2_to_bf16<3>(cwd[d]), as_bf16x2(xr[4 * d + 3]), b1);
    }
    acc = __builtin_fmaf(b0, sf0, acc);
    return __builtin_fmaf(b1, sf1, acc);
}

template <int R, int KS, int CPL, bool WT = false, class Epi>
__device__ __forceinline__ void gemv_tile_compute_x1(const TileRegs<1, R, KS, CPL> &t, const XRegs<CPL> &xr, int n,
                                                     int row0, float *red, Epi &&epi) {
    float acc[R][1];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r][0] = 0.0f;
#pragma unroll
    for (int j = 0; j < CPL; ++j)
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r][0] = chunk_dot_xreg(t.c[r][j], t.s[r][j], xr.w[j], acc[r][0]);
    gemv_tile_finish<1, R, KS, CPL, WT>(acc, n, row0, red, epi);
}

// One stage of the pipelined loop: chunks c0, c0 + 16, ... of the slot's R
// rows, the first `left` of them (uniform where every lane of the wavefront
// owns the same chunk count).
template <int U, int R>
__device__ __forceinline__ void stage_load(uint4 (&cw)[U][R], uint32_t (&sw)[U][R], const uint8_t *const (&cp)[R],
                                           const uint8_t *const (&sp)[R], int c0, int left) {
#pragma unroll
    for (int q = 0; q < U; ++q) {
        if (q < left) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                cw[q][r] = ld_stream16(cp[r] + 16 * (size_t)(c0 + 16 * q));
                sw[q][r] = ld_stream2(sp[r] + 2 * (size_t)(c0 + 16 * q));
            }
        }
    }
}

template <int MT, int U, int R>
__device__ __forceinline__ void stage_fma(const uint4 (&cw)[U][R], const uint32_t (&sw)[U][R], const uint4 *xs, int C,
                                          int c0, int left, float (&acc)[R][MT]) {
#pragma unroll
    for (int q = 0; q < U; ++q) {
        if (q < left) {
#pragma unroll
            for (int r = 0; r < R; ++r) chunk_fma<MT>(cw[q][r], sw[q][r], xs, C, c0 + 16 * q, acc[r]);
        }
    }
}

// R rows (code and scale row pointers cp, sp) against the activation image
// (C chunks a row), for a lane that owns the nc chunks tl, tl + 16, ...:
// stages of U chunks, the loads of stage s + 1 in flight while stage s is
// computed.
template <int MT, int R, int U>
__device__ __forceinline__ void pipe_rows(const uint4 *xs, const uint8_t *const (&cp)[R], const uint8_t *const (&sp)[R],
                                          int C, int tl, int nc, float (&acc)[R][MT]) {
    const int ns = (nc + U - 1) / U;
    uint4 ca[U][R], cb[U][R];
    uint32_t sa[U][R], sb[U][R];
    stage_load<U, R>(ca, sa, cp, sp, tl, nc);
    for (int st = 0; st < ns; st += 2) {
        if (st + 1 < ns) stage_load<U, R>(cb, sb, cp, sp, tl + 16 * U * (st + 1), nc - U * (st + 1));
        __builtin_amdgcn_sched_barrier(0);
        stage_fma<MT, U, R>(ca, sa, xs, C, tl + 16 * U * st, nc - U * st, acc);
        if (st + 1 >= ns) break;
        if (st + 2 < ns) stage_load<U, R>(ca, sa, cp, sp, tl + 16 * U * (st + 2), nc - U * (st + 2));
        __builtin_amdgcn_sched_barrier(0);
        stage_fma<MT, U, R>(cb, sb, xs, C, tl + 16 * U * (st + 1), nc - U * (st + 1), acc);
    }
}

// Generic shape (any K % 32 == 0): loop over the lane's chunks.  U > 0:
// pipelined stages of U chunks where every lane owns the same number of
// chunks, or (UNEVEN) in any K split; otherwise one chunk at a time (the
// fewest registers).
template <int MT, int R, int KS, int U = (R >= 4 ? 1 : 4 / R), bool WT = false, bool UNEVEN = false, class Epi>
__device__ __forceinline__ void gemv_tile_loop(const uint4 *xs, const uint8_t *__restrict__ codes,
                                               const uint8_t *__restrict__ scales, int n, int k, int row0, float *red,
                                               Epi &&epi) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int slot = lane >> 4, tl = lane & 15;
    const int ks = (KS == 1) ? 0 : (wave % KS);
    const int rg = WT ? 0 : wave / KS;
    const int C = k >> 5;
    const int cs = (C + KS - 1) / KS;
    const int c_lo = ks * cs;
    const int c_hi = min(C, c_lo + cs);
    const int rbase = row0 + (rg * 4 + slot) * R;
    float acc[R][MT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int mm = 0; mm < MT; ++mm) acc[r][mm] = 0.0f;
    const uint8_t *cp[R], *sp[R];
    auto row_ptrs = [&]() {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int row = min(rbase + r, n - 1);   // rows past n: never passed to the epilogue
            cp[r] = codes + (size_t)row * (size_t)(k >> 1);
            sp[r] = scales + (size_t)row * (size_t)(k >> 4);
        }
    };
    constexpr int UP = U > 0 ? U : 1;
    if (U > 0 && (cs & 15) == 0 && c_hi - c_lo == cs) {
        // the same count in every lane, from the kernel arguments alone: a
        // scalar loop
        row_ptrs();
        pipe_rows<MT, R, UP>(xs, cp, sp, C, c_lo + tl, cs >> 4, acc);
    } else if constexpr (U > 0 && KS > 1 && UNEVEN) {
        // K slices whose counts differ by one between the lanes: still
        // pipelined (elsewhere the single-chunk loop below keeps the register
        // count of the common kernels down)
        const int c0 = c_lo + tl;
        row_ptrs();
        pipe_rows<MT, R, UP>(xs, cp, sp, C, c0, c0 < c_hi ? (c_hi - c0 + 15) >> 4 : 0, acc);
    } else {
        for (int c = c_lo + tl; c < c_hi; c += 16) {
            uint4 cw[R];
            uint32_t sw[R];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int row = min(rbase + r, n - 1);   // rows past n: never passed to the epilogue
                cw[r] = ld_stream16(codes + (size_t)row * (size_t)(k >> 1) + 16 * (size_t)c);
                sw[r] = ld_stream2(scales + (size_t)row * (size_t)(k >> 4) + 2 * (size_t)c);
            }
#pragma unroll
            for (int r = 0; r < R; ++r) chunk_fma<MT>(cw[r], sw[r], xs, C, c, acc[r]);
        }
    }
    gemv_tile_finish<MT, R, KS, 0, WT>(acc, n, row0, red, epi);
}

// ------------------------------------------------------------ MFMA path ----
// For M >= 2 activation rows a unit of 16 weight rows is one wavefront's
// v_mfma_f32_16x16x32_bf16 tile: B = the 16 rows dequantized exactly to bf16,
// A = the activation rows, padded to 16 with zeros.  Lane (n = l % 16,
// q = l / 16) covers, in 128-k step s, the k = 128 s + 32 q .. + 31 of row n:
// one 16-byte code chunk and its two scale bytes.  Inside a step the MFMA k
// order is chosen so that block b takes k = 128 s + 32 q + 8 b .. + 7 from
// every lane group q; each block still sums 32 products of the row, and the
// activations are read from LDS in the same order.  The result C[m][n]
// leaves lane (n, q) as rows m = 4 q + r, r = 0..3.

// Activation image of the MFMA path: row m is K / 8 chunks of 16 bytes,
// chunk c stored at c ^ (m % 8), so that the rows a lane group reads at one
// chunk hit different bank groups.  K % 128 == 0.
__device__ __forceinline__ void stage_x_mf(uint4 *xs, const uint4 *__restrict__ x, int m_rt, int mt, int k) {
    const int cpr = k >> 3;
    stage_batched(
        mt * cpr, threadIdx.x, blockDim.x,
        [&](int p) { return p / cpr < m_rt ? x[p] : make_uint4(0, 0, 0, 0); },
        [&](int p, uint4 v) {
            const int m = p / cpr, c = p - m * cpr;
            xs[m * cpr + (c ^ (m & 7))] = v;
        });
}
// stage_x_mf in two steps, so that loads issued in between (the first
// weights) are in flight with the activations and the image's stores wait
// for the activations only: the first kStageBatch units of each thread into
// registers, then their stores and the rest of the image.
__device__ __forceinline__ void stage_x_mf_first(uint4 (&v)[kStageBatch], const uint4 *__restrict__ x, int m_rt,
                                                 int mt, int k) {
    const int cpr = k >> 3, units = mt * cpr;
#pragma unroll
    for (int j = 0; j < kStageBatch; ++j) {
        const int p = threadIdx.x + j * blockDim.x;
        v[j] = p < units && p / cpr < m_rt ? x[p] : make_uint4(0, 0, 0, 0);
    }
}
__device__ __forceinline__ void stage_x_mf_rest(uint4 *xs, const uint4 (&v)[kStageBatch], const uint4 *__restrict__ x,
                                                int m_rt, int mt, int k) {
    const int cpr = k >> 3, units = mt * cpr, done = kStageBatch * blockDim.x;
    auto put = [&](int p, uint4 val) {
        const int m = p / cpr, c = p - m * cpr;
        xs[m * cpr + (c ^ (m & 7))] = val;
    };
#pragma unroll
    for (int j = 0; j < kStageBatch; ++j) {
        const int p = threadIdx.x + j * blockDim.x;
        if (p < units) put(p, v[j]);
    }
    if (units > done)
        stage_batched(
            units - done, threadIdx.x, blockDim.x,
            [&](int q) { return (q + done) / cpr < m_rt ? x[q + done] : make_uint4(0, 0, 0, 0); },
            [&](int q, uint4 val) { put(q + done, val); });
}

// Two E2M1 codes (byte SEL of word) times sf as two bf16 (exact: e2m1 times
// an E4M3 scale has at most 6 significant bits).
template <int SEL>
__device__ __forceinline__ uint32_t mf_dq2(uint32_t word, float sf) {
    typedef __attribute__((ext_vector_type(2))) float f32x2;
    f32x2 f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, SEL);
    const uint32_t lo = __float_as_uint(f.x * sf), hi = __float_as_uint(f.y * sf);
    return __builtin_amdgcn_perm(hi, lo, 0x07060302u);
}

// One 128-k step in two halves.  mf_dequant: the lane's code chunk and
// scale bytes as the four bf16x8 B blocks; mf_mma: the activation rows
// against them (lanes n >= MT read row n % MT and zero it), four MFMAs into
// two accumulators (blocks 0, 2 and 1, 3).  Split so that the registers of
// the chunk can be reloaded between the halves.
__device__ __forceinline__ void mf_dequant(uint4 cw, uint32_t sw, uint4 (&bw)[4]) {
    float sf0, sf1;
    e4m3x2_to_f32(sw, sf0, sf1);
    const uint32_t w[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const float sf = b < 2 ? sf0 : sf1;
        bw[b] = make_uint4(mf_dq2<0>(w[b], sf), mf_dq2<1>(w[b], sf), mf_dq2<2>(w[b], sf), mf_dq2<3>(w[b], sf));
    }
}

// xa[b]: block b of this lane's activation row in LDS (mf_xrow); lanes
// n >= MT read row n % MT, whose products land in output rows >= MT that are
// never read.  Read apart from the MFMAs so that the four LDS reads are in
// flight together.
__device__ __forceinline__ void mf_xload(const uint4 *const (&xa)[4], int s, uint4 (&a)[4]) {
#pragma unroll
    for (int b = 0; b < 4; ++b) a[b] = xa[b][16 * s];
}

__device__ __forceinline__ void mf_mma(const uint4 (&a)[4], const uint4 (&bw)[4], f32x4 &acc0, f32x4 &acc1) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        f32x4 &acc = (b & 1) ? acc1 : acc0;
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[b]), __builtin_bit_cast(bf16x8, bw[b]),
                                                    acc, 0, 0, 0);
    }
}

// Chunk 16 s + 4 q + b of lane (n, q)'s activation row sits at
// mf_xrow(..., b)[16 s]: the swizzle c ^ (m % 8) only touches the low three
// bits of c, so it is folded into one base per block.
__device__ __forceinline__ const uint4 *mf_xrow(const uint4 *xs, int cpr, int mt, int li, int q, int b) {
    const int xr = li & (mt - 1);
    return xs + xr * cpr + ((4 * q + b) ^ (xr & 7));
}

// Loads of a 16-row unit that fill whole 128-byte lines (one instruction
// touching 16 rows x 64 bytes, the MFMA layout, costs about twice the time
// of one touching 8 rows x 128 bytes).  Codes: step pair p (256 k) of rows
// 0-7 is one instruction (lane l: row l / 8, bytes 128 p + 16 (l % 8)), of
// rows 8-15 the next; scales: 8 steps (1024 k, 64 bytes a row) of all 16
// rows are one instruction (lane l: row l / 4, bytes 16 (l % 4)).  Rows past
// n read row n - 1, never passed on.
struct MfLines {
    const uint8_t *ca, *cb, *sp;
};
__device__ __forceinline__ MfLines mf_lines(const uint8_t *__restrict__ codes, const uint8_t *__restrict__ scales,
                                            int n, int k, int row0, int lane) {
    const int ra = min(row0 + (lane >> 3), n - 1), rb = min(row0 + 8 + (lane >> 3), n - 1);
    const int rs = min(row0 + (lane >> 2), n - 1);
    return MfLines{codes + (size_t)ra * (size_t)(k >> 1) + 16 * (lane & 7),
                   codes + (size_t)rb * (size_t)(k >> 1) + 16 * (lane & 7),
                   scales + (size_t)rs * (size_t)(k >> 4) + 16 * (lane & 3)};
}

// The lines go through a per-wavefront LDS area to the MFMA layout: code
// slot (8 r + (i ^ (r % 8))) holds 16-byte segment i of row r of the pair
// (the swizzle keeps the 16 rows one layout read touches on different
// banks); the scale area holds row r's 64 bytes at 64 r.
__device__ __forceinline__ int mf_code_wslot(int lane, int half) {   // lane's store, rows 8 half + lane / 8
    const int r = 8 * half + (lane >> 3), i = lane & 7;
    return 8 * r + (i ^ (r & 7));
}
__device__ __forceinline__ int mf_code_rslot(int li, int q, int h) {   // step h of the pair, lane (n = li, q)
    const int i = 4 * h + q;
    return 8 * li + (i ^ (li & 7));
}

// ---------------------------------------------------------------- host ----
struct TileChoice {
    int R, KS, CPL;   // CPL 0: generic loop
    int NW = 4;       // wavefronts a workgroup
};

constexpr int kLdsBytes = 64 * 1024;   // LDS budget of one workgroup when choosing a K split
constexpr size_t kMaxLds = 160 * 1024 - 8192;   // largest activation image (LDS per workgroup, static LDS aside)

// LDS bytes of a GEMV workgroup: the activation image plus, with a K split,
// 4 * NW * R * MT fp32 partial sums (one a slot, row and activation row).
inline size_t gemv_lds_bytes(int mt, int k, TileChoice tc) {
    return (size_t)mt * k * 2 + (tc.KS > 1 ? (size_t)4 * tc.NW * tc.R * mt * 4 : 0);
}

// Tile shape for an n x k weight and MT activation rows: the largest R
// (fewest, fattest tiles) that still gives at least `min_tiles` workgroups,
// else a K split across the wavefronts (if its scratch fits in LDS next to
// the activations, `extra_lds` bytes of static LDS included).  CPL is the
// fixed per-lane chunk count when K splits evenly into 16-lane rows.
inline TileChoice choose_tile(int n, int k, int mt, int min_tiles, size_t extra_lds) {
    static const int order[][2] = {{4, 1}, {2, 1}, {1, 1}, {1, 2}, {1, 4}};
    TileChoice pick{1, 1, 0};
    bool found = false;
    for (const auto &o : order) {
        TileChoice c{o[0], o[1], 0};
        if (c.KS > 1 && gemv_lds_bytes(mt, k, c) + extra_lds > (size_t)kLdsBytes) break;
        // a K split only where every lane gets the same chunk count (the
        // fixed counts 1, 2, 4, or the pipelined generic loop).  With one
        // activation row the generic loop splits only a grid under a third
        // of min_tiles: there a lane's loads already cover the latency, and
        // the split's partial-sum exchange costs more than the extra tiles
        // gain (measured at 17408 x 5120 and 18432 x 7168).
        if (c.KS > 1 && k % (512 * c.KS) != 0) continue;
        if (c.KS > 1 && mt == 1) {
            const int cpl = k / (512 * c.KS);
            if (cpl != 1 && cpl != 2 && cpl != 4 && (n + 15) / 16 >= min_tiles / 3) continue;
        }
        pick = c;
        const int rows = 16 * c.R / c.KS;
        if ((n + rows - 1) / rows >= min_tiles) {
            found = true;
            break;
        }
    }
    (void)found;
    const int per = 512 * pick.KS;
    if (k % per == 0) {
        const int cpl = k / per;
        if (cpl == 1 || cpl == 2 || cpl == 4) pick.CPL = cpl;
    }
    return pick;
}

__host__ __device__ inline int round_up_mt(int m) { return m <= 1 ? 1 : m <= 2 ? 2 : m <= 4 ? 4 : 8; }

}  // namespace nvfp4
