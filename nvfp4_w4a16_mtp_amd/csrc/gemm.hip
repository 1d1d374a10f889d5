// W4A16 GEMM for prompt-sized row counts (drafter prefill): the
// `w4a16_gemm_m128_dispatch` of prefill_weights.rs in its lossless variant --
// NVFP4 weights dequantized exactly to bf16, bf16 matrix products, fp32
// accumulation, activations never quantized.  y[m][n] = sum_k x[m][k] W^[n][k].
//
// gfx950 design: a 128- or 256-row by 128-column output tile per workgroup
// (4 or 8 wavefronts, each 64 x 64 = 4 x 4 blocks of
// v_mfma_f32_16x16x32_bf16), K in steps of 64.  Per step the workgroup
// stages the activation tile and the 128 x 64 weight tile in LDS; the
// weight tile is dequantized on the way in (hardware E2M1 -> fp32 convert,
// times the E4M3 block scale, packed to bf16 -- exact, since e2m1 * e4m3 has
// at most 6 significant bits).  The next step's global loads are issued
// before the current step's MFMAs.  LDS chunks are XOR-swizzled (lds_off)
// to spread the rows of an operand load and of a staging store over the
// banks.  The global scale is applied in the epilogue.
//
// The tiles of a call fill the chip in rounds of resident workgroups, and a
// last round that is only partly filled costs a full one.  With a workspace
// the tiles of that last round (all tiles, for prompt chunks too short to
// fill one round) split K over up to 16 workgroups each, in the same launch
// as the whole tiles; the slices write fp32 tile-shaped partial planes and a
// second kernel sums them in slice order and applies the global scale.
//
// The dequantization runs on the same SIMDs as the MFMAs and the two hardly
// overlap (timed: 4 MFMAs and 32 fp32 multiplies per wavefront cost close to
// the sum of either alone), so its share is what the tile height sets.
#include "common.hpp"

namespace nvfp4 {

constexpr int kBN = 128, kBK = 64;
constexpr int kLdsRow = kBK * 2;   // bytes per LDS row (64 bf16 of one K step)

// Byte offset of 16-byte chunk c (8 bf16) of tile row r in LDS.  The chunk is
// stored at position c ^ (r % 8): each 8 consecutive rows of one operand
// read at a fixed chunk, and the 4 rows of one staging store, hit 8
// different 16-byte bank groups of a 128-byte bank row.
__device__ __forceinline__ int lds_off(int r, int c) { return r * kLdsRow + 16 * (c ^ (r & 7)); }

// Two E2M1 codes (byte SEL of word) times sf, packed as two bf16 (exact).
template <int SEL>
__device__ __forceinline__ uint32_t dq2(uint32_t word, float sf) {
    typedef __attribute__((ext_vector_type(2))) float f32x2;
    f32x2 f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, SEL);
    const uint32_t lo = __float_as_uint(f.x * sf), hi = __float_as_uint(f.y * sf);
    return __builtin_amdgcn_perm(hi, lo, 0x07060302u);   // upper halves: exact bf16
}

// BM x 128 output tile per workgroup: BM / 64 x 2 wavefronts of 64 x 64.
// The weight tile is dequantized once per workgroup, so a taller tile
// spends fewer dequantization instructions per MFMA (a BM = 256 tile half as
// many as BM = 128); each of the 2 BM threads stages one half row of the
// activation tile and 8192 / (2 BM) weights.  Tall tiles raise the wave
// priority over their MFMA phase, so that the CU's other workgroup stages
// in the gaps (measured +1-5% at 8192 rows; it slowed the 128-row tile).
// Work items (blockIdx.x): tiles [0, full) in row-major tile order (column
// tiles fastest) over the whole K, written to y; then `nz` slices of each
// later tile.  Slice z takes the K steps [z S / nz, (z + 1) S / nz) of the
// S = ceil(K / 64) and writes its fp32 sums without the global scale to
// partial plane (tile - full) nz + z of `part`, a BM x 128 row-major plane
// per (tile, slice), for k_gemm_reduce.
struct GemmWork {
    int cols;      // column tiles
    int full;      // tiles computed whole
    int nz;        // K slices of each later tile
    float *part;   // partial planes of the split tiles
};

template <int BM, bool BF16OUT>
__global__ __launch_bounds__(2 * BM) __attribute__((amdgpu_waves_per_eu(BM == 256 ? 4 : 3))) void k_gemm(
    const uint16_t *__restrict__ x, const uint8_t *__restrict__ codes, const uint8_t *__restrict__ scales,
    const nvfp4_global *__restrict__ g, int M, int N, int K, void *__restrict__ y, GemmWork wk) {
    constexpr int NT = 2 * BM;          // threads
    constexpr int BPR = NT / kBN;       // weight staging parts per tile row: 2 or 4
    constexpr int CPT = 64 / BPR / 8;   // code dwords (8 codes each) per thread: 4 or 2
    static_assert(BPR == 2 || BPR == 4, "BM is 128 or 256");
    __shared__ __attribute__((aligned(16))) uint8_t lds_a[BM * kLdsRow];
    __shared__ __attribute__((aligned(16))) uint8_t lds_b[kBN * kLdsRow];

    const int th = threadIdx.x, lane = th & 63, wave = th >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int id = blockIdx.x;
    const bool split = id >= wk.full;
    const int tile = split ? wk.full + (id - wk.full) / wk.nz : id;
    const int z = split ? (id - wk.full) % wk.nz : 0, nz = split ? wk.nz : 1;
    const int m0 = tile / wk.cols * BM, n0 = tile % wk.cols * kBN;

    // staging roles: activation rows th / 8 + (NT / 8) q, q = 0..3, chunk th % 8
    // (8 bf16) of the K step -- each load instruction of a wavefront covers
    // 8 rows x 128 bytes, whole lines; weight row th / BPR, part th % BPR
    // (64 / BPR k)
    const int xrow0 = th >> 3, xch = th & 7;
    const int brow = th / BPR, bpart = th % BPR;
    const int wnr = n0 + brow;
    const bool wval = wnr < N;
    const uint8_t *crow = codes + (size_t)(wval ? wnr : 0) * (K >> 1);
    const uint8_t *srow_p = scales + (size_t)(wval ? wnr : 0) * (K >> 4);

    // rows m0 + xrow0 + (NT / 8) q exist for q < xq
    const int xleft = M - m0 - xrow0;
    const int xq = xleft <= 0 ? 0 : (xleft + NT / 8 - 1) / (NT / 8);
    const uint16_t *xb = x + (size_t)(m0 + (xq > 0 ? xrow0 : 0)) * K + 8 * xch;
    const size_t xstep = (size_t)(NT / 8) * K;
    uint4 xr[4];
    uint32_t cr[CPT];
    uint32_t sr;
    auto load_step = [&](int k0) {
        const bool kin = k0 + 8 * xch < K;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            xr[q] = (q < xq && kin) ? *reinterpret_cast<const uint4 *>(xb + q * xstep + k0) : make_uint4(0, 0, 0, 0);
        const int kb = k0 + (64 / BPR) * bpart;
        if (wval && kb < K) {
            if constexpr (CPT == 4) {
                const uint4 c = *reinterpret_cast<const uint4 *>(crow + (kb >> 1));
                cr[0] = c.x;
                cr[1] = c.y;
                cr[2] = c.z;
                cr[3] = c.w;
                sr = *reinterpret_cast<const uint16_t *>(srow_p + (kb >> 4));
            } else {
                const uint2 c = *reinterpret_cast<const uint2 *>(crow + (kb >> 1));
                cr[0] = c.x;
                cr[1] = c.y;
                sr = srow_p[kb >> 4];
            }
        } else {
#pragma unroll
            for (int d = 0; d < CPT; ++d) cr[d] = 0;
            sr = 0;
        }
    };

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    const int steps = (K + kBK - 1) / kBK;
    const int kb0 = (int)((long)z * steps / nz) * kBK, kb1 = min(K, (int)((long)(z + 1) * steps / nz) * kBK);
    if (kb0 < kb1) load_step(kb0);
    for (int k0 = kb0; k0 < kb1; k0 += kBK) {
        // stage: activations as they are, weights dequantized
        {
#pragma unroll
            for (int q = 0; q < 4; ++q) *reinterpret_cast<uint4 *>(lds_a + lds_off(xrow0 + (NT / 8) * q, xch)) = xr[q];
            typedef __attribute__((ext_vector_type(2))) float f32x2;
            const f32x2 sfv = __builtin_amdgcn_cvt_pk_f32_fp8((int)sr, false);   // E4M3 block scales, exact
#pragma unroll
            for (int d = 0; d < CPT; ++d) {
                const float sf = (CPT == 4 && d >= 2) ? sfv.y : sfv.x;   // 16 codes per scale
                *reinterpret_cast<uint4 *>(lds_b + lds_off(brow, CPT * bpart + d)) =
                    make_uint4(dq2<0>(cr[d], sf), dq2<1>(cr[d], sf), dq2<2>(cr[d], sf), dq2<3>(cr[d], sf));
            }
        }
        __syncthreads();
        if (k0 + kBK < kb1) load_step(k0 + kBK);
        if constexpr (BM == 256) __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            bf16x8 af[4], bfr[4];
            const int kc = 4 * ks + (lane >> 4);   // 16-byte chunk of the K step
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                af[i] = *reinterpret_cast<const bf16x8 *>(lds_a + lds_off(64 * wm + 16 * i + (lane & 15), kc));
                bfr[i] = *reinterpret_cast<const bf16x8 *>(lds_b + lds_off(64 * wn + 16 * i + (lane & 15), kc));
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
        if constexpr (BM == 256) __builtin_amdgcn_s_setprio(0);
        __syncthreads();
    }

    if (split) {
        // the whole plane, rows and columns past the matrix included (the
        // reduction reads them and drops them)
        float *pz = wk.part + ((size_t)(tile - wk.full) * nz + z) * (BM * kBN);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int c = 64 * wn + 16 * j + (lane & 15);
#pragma unroll
                for (int r = 0; r < 4; ++r) pz[(64 * wm + 16 * i + 4 * (lane >> 4) + r) * kBN + c] = acc[i][j][r];
            }
        return;
    }
    const float dec = g->dec;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + 64 * wn + 16 * j + (lane & 15);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + 64 * wm + 16 * i + 4 * (lane >> 4) + r;
                if (m < M && n < N) {
                    const float o = acc[i][j][r] * dec;
                    if constexpr (BF16OUT)
                        reinterpret_cast<uint16_t *>(y)[(size_t)m * N + n] = (uint16_t)f32_to_bf16_bits(o);
                    else
                        reinterpret_cast<float *>(y)[(size_t)m * N + n] = o;
                }
            }
        }
}

// Sum of the K-slice partials of each output of the split tiles in slice
// order (the same order on every call), times the global scale, as fp32 or
// bf16.  Thread items are 4 consecutive columns of one tile row.
template <int BM, bool BF16OUT>
__global__ __launch_bounds__(256) void k_gemm_reduce(const float *__restrict__ part, int tiles, int nz, int first,
                                                     int cols, int M, int N, const nvfp4_global *__restrict__ g,
                                                     void *__restrict__ y) {
    constexpr int kPlane = BM * kBN;
    const float dec = g->dec;
    const size_t count = (size_t)tiles * kPlane, stride = (size_t)gridDim.x * 256 * 4;
    for (size_t e = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4; e < count; e += stride) {
        const int t = (int)(e / kPlane), local = (int)(e % kPlane);
        const float *src = part + (size_t)t * nz * kPlane + local;
        float4 a = *reinterpret_cast<const float4 *>(src);
        for (int s = 1; s < nz; ++s) {
            const float4 b = *reinterpret_cast<const float4 *>(src + (size_t)s * kPlane);
            a.x += b.x;
            a.y += b.y;
            a.z += b.z;
            a.w += b.w;
        }
        const int tile = first + t;
        const int m = tile / cols * BM + local / kBN, n = tile % cols * kBN + local % kBN;
        if (m >= M) continue;
        const float v[4] = {a.x * dec, a.y * dec, a.z * dec, a.w * dec};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            if (n + c >= N) break;
            if constexpr (BF16OUT)
                reinterpret_cast<uint16_t *>(y)[(size_t)m * N + n + c] = (uint16_t)f32_to_bf16_bits(v[c]);
            else
                reinterpret_cast<float *>(y)[(size_t)m * N + n + c] = v[c];
        }
    }
}

// Tile choice by rounds of resident workgroups: a 256-row round (2 per CU)
// takes about kTallRound times a 128-row round (3 per CU) -- measured at
// 8192 x 17408 x 5120, where both fill the chip: 919 against 815 TFLOP/s,
// 2 x 256 / 919 over 3 x 128 / 815.  Without a split a partly filled last
// round costs a full one (1024 x 17408: 544 tall tiles on 512 slots take two
// rounds).  With a workspace the last round's tiles are split over K: S
// slices each, S = min(kMaxSplit, slots / tiles of that round, steps /
// kMinSliceSteps), so the slices take about 1 / S of a round, plus the
// reduction's traffic.
constexpr double kTallRound = 1.18;
constexpr int kMaxSplit = 16;             // K slices at most
// 64-k steps per slice at least: at 128 x 2048 x 4096 slices of 8 steps
// (8 slices) took 18.8-19.6 us against 21.4-22.3 for 16 slices of 4; the
// other 128- and 1024-row shapes were within noise; at most 4 or 8 slices
// instead of 16 made 128 x 5120 x 17408 slower (79, 60 against 52 us).
// 256-row tiles that all split (less than one round of them) need longer
// slices: 4 and 8 ways in slices of 8 steps, 8192 x 512 x 2048 and 1024 x
// 2048 x 4096 took 43.6 and 40.9 us against 35.9 and 37.0 us as 128-row
// tiles; the tiles of a last round split in slices of 8 steps (1024 x 17408
// x 5120: 32 tiles in 10 slices, 204 us against 238-252 us unsplit).
constexpr int kMinSliceSteps = 8, kMinSliceSteps256 = 24;
constexpr long kMaxSplitRounds = 3;   // split the last round of at most this many
// Rates of whole rounds (bf16 TFLOP/s, 128- and 256-row tiles) and of the
// reduction (bytes/us), for the cost of a split in rounds.
constexpr double kRate128 = 815e6, kRate256 = 919e6, kReduceRate = 5e6, kReduceLaunchUs = 4.0;

struct GemmPlan {
    int bm;       // 128 or 256
    int cols;     // column tiles
    int full;     // tiles computed whole
    int split;    // tiles split over K (the last ones)
    int nz;       // K slices of a split tile
    size_t ws;    // workspace bytes for the partial planes
};

static GemmPlan gemm_plan_bm(int bm, long slots, int m, int n, int k, bool can_split, double &cost) {
    const long cols = (n + kBN - 1) / kBN, tiles = cols * ((m + bm - 1) / bm);
    const long steps = (k + kBK - 1) / kBK;
    const double c = bm == 256 ? kTallRound : 1.0;
    const long rounds = (tiles + slots - 1) / slots;
    GemmPlan p{bm, (int)cols, (int)tiles, 0, 1, 0};
    cost = rounds * c;
    // after several rounds the workgroups no longer start in step, and a
    // last partial round costs less than a whole one: 8192 x 17408 x 5120
    // (8.5 rounds of tall tiles) took 1445 us with its last 256 tiles split
    // against 1302-1310 us unsplit, while 8192 x 5120 x 17408 (2.5 rounds)
    // gained 1459 -> 1375 us
    if (!can_split || rounds > kMaxSplitRounds) return p;
    const long tail = tiles - (rounds - 1) * slots;   // tiles of the last round
    long nz = slots / tail;
    nz = nz < kMaxSplit ? nz : kMaxSplit;
    const long min_steps = bm == 256 && rounds == 1 ? kMinSliceSteps256 : kMinSliceSteps;
    nz = nz < steps / min_steps ? nz : steps / min_steps;
    if (nz < 2) return p;
    const double round_us = 2.0 * bm * kBN * (double)k * slots / (bm == 256 ? kRate256 : kRate128);
    const double red_us = (double)tail * nz * bm * kBN * 4 / kReduceRate + kReduceLaunchUs;
    const double split_cost = (rounds - 1) * c + c / nz + red_us / round_us;
    if (split_cost >= cost) return p;
    cost = split_cost;
    p.full = (int)(tiles - tail);
    p.split = (int)tail;
    p.nz = (int)nz;
    p.ws = (size_t)tail * nz * bm * kBN * sizeof(float);
    return p;
}

static GemmPlan gemm_plan(int m, int n, int k, bool can_split) {
    const long slots_s = (long)num_cus() * blocks_per_cu(reinterpret_cast<const void *>(k_gemm<128, false>), 256, 0);
    const long slots_t = (long)num_cus() * blocks_per_cu(reinterpret_cast<const void *>(k_gemm<256, false>), 512, 0);
    double cs, ct;
    const GemmPlan ps = gemm_plan_bm(128, slots_s, m, n, k, can_split, cs);
    const GemmPlan pt = gemm_plan_bm(256, slots_t, m, n, k, can_split, ct);
    return ct < cs ? pt : ps;
}

template <int BM>
static void launch_gemm(const uint16_t *x, int m, const nvfp4_weight *w, void *y, bool bf16, const GemmPlan &p,
                        float *part, hipStream_t s) {
    const GemmWork wk{p.cols, p.full, p.nz, part};
    const dim3 grid(p.full + p.split * p.nz);
    if (bf16)
        hipLaunchKernelGGL((k_gemm<BM, true>), grid, dim3(2 * BM), 0, s, x, w->codes, w->scales, w->global, m, w->n,
                           w->k, y, wk);
    else
        hipLaunchKernelGGL((k_gemm<BM, false>), grid, dim3(2 * BM), 0, s, x, w->codes, w->scales, w->global, m, w->n,
                           w->k, y, wk);
    if (p.split == 0) return;
    const size_t groups = (size_t)p.split * BM * kBN / 4;
    const size_t want = (groups + 255) / 256, cap = (size_t)num_cus() * 8;
    const unsigned blocks = (unsigned)(want < cap ? want : cap);
    if (bf16)
        hipLaunchKernelGGL((k_gemm_reduce<BM, true>), dim3(blocks), dim3(256), 0, s, part, p.split, p.nz, p.full,
                           p.cols, m, w->n, w->global, y);
    else
        hipLaunchKernelGGL((k_gemm_reduce<BM, false>), dim3(blocks), dim3(256), 0, s, part, p.split, p.nz, p.full,
                           p.cols, m, w->n, w->global, y);
}

}  // namespace nvfp4

using namespace nvfp4;

extern "C" size_t w4a16_gemm_m128_workspace_bytes(int32_t m, int32_t n, int32_t k) {
    if (m < 1 || n < 1 || k < 32) return 0;
    return gemm_plan(m, n, k, true).ws;
}

extern "C" int w4a16_gemm_m128(const uint16_t *x_bf16, int32_t m, const nvfp4_weight *w, void *y, int32_t y_dtype,
                               void *workspace, size_t ws_bytes, void *stream) {
    int rc = validate_weight(w, "w4a16_gemm_m128");
    if (rc) return rc;
    if (w->n == 0 && m >= 1) return ok();   // empty output: nothing to read or write
    if (!x_bf16 || !y) return fail(NVFP4_ERR_ARG, "w4a16_gemm_m128: NULL x or y");
    if (m < 1) return fail(NVFP4_ERR_SHAPE, "w4a16_gemm_m128: m=%d < 1", m);
    if (y_dtype != NVFP4_OUT_F32 && y_dtype != NVFP4_OUT_BF16)
        return fail(NVFP4_ERR_ARG, "w4a16_gemm_m128: unknown y_dtype %d", y_dtype);
    if (!aligned(x_bf16, 16)) return fail(NVFP4_ERR_ALIGN, "w4a16_gemm_m128: x not 16-byte aligned");
    if (!aligned(y, 4)) return fail(NVFP4_ERR_ALIGN, "w4a16_gemm_m128: y not 4-byte aligned");
    const long items = (long)((w->n + kBN - 1) / kBN) * ((m + 127) / 128) * kMaxSplit;
    if (items > 2147483647L) return fail(NVFP4_ERR_UNSUPPORTED, "w4a16_gemm_m128: grid too large");
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const bool bf16 = y_dtype == NVFP4_OUT_BF16;
    const GemmPlan p = gemm_plan(m, w->n, w->k, workspace != nullptr);   // no workspace: one pass over K
    if (p.split > 0) {
        if (ws_bytes < p.ws)
            return fail(NVFP4_ERR_WORKSPACE, "w4a16_gemm_m128: workspace of %zu bytes, %zu needed", ws_bytes, p.ws);
        if (!aligned(workspace, 16)) return fail(NVFP4_ERR_ALIGN, "w4a16_gemm_m128: workspace not 16-byte aligned");
    }
    float *part = reinterpret_cast<float *>(workspace);
    if (p.bm == 256)
        launch_gemm<256>(x_bf16, m, w, y, bf16, p, part, s);
    else
        launch_gemm<128>(x_bf16, m, w, y, bf16, p, part, s);
    return check_launch("w4a16_gemm_m128");
}
