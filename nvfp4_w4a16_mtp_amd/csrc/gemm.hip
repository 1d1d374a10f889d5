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
// Prompt chunks too short to fill the chip with output tiles (a few hundred
// rows) split K over up to 16 workgroups per tile, which write fp32 partial
// planes to the caller's workspace; a second kernel sums them in slice order
// and applies the global scale.
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
// K split: slice z = blockIdx.z of gridDim.z takes the K steps
// [z S / Z, (z + 1) S / Z) of the S = ceil(K / 64) and, with PART, writes
// its fp32 sums without the global scale to plane z of `part` (row-major
// [M][N] planes, `plane` floats apart) for k_gemm_reduce.
template <int BM, bool BF16OUT, bool PART>
__global__ __launch_bounds__(2 * BM) __attribute__((amdgpu_waves_per_eu(BM == 256 ? 4 : 3))) void k_gemm(
    const uint16_t *__restrict__ x, const uint8_t *__restrict__ codes, const uint8_t *__restrict__ scales,
    const nvfp4_global *__restrict__ g, int M, int N, int K, void *__restrict__ y, float *__restrict__ part,
    size_t plane) {
    constexpr int NT = 2 * BM;          // threads
    constexpr int BPR = NT / kBN;       // weight staging parts per tile row: 2 or 4
    constexpr int CPT = 64 / BPR / 8;   // code dwords (8 codes each) per thread: 4 or 2
    static_assert(BPR == 2 || BPR == 4, "BM is 128 or 256");
    __shared__ __attribute__((aligned(16))) uint8_t lds_a[BM * kLdsRow];
    __shared__ __attribute__((aligned(16))) uint8_t lds_b[kBN * kLdsRow];

    const int th = threadIdx.x, lane = th & 63, wave = th >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int m0 = blockIdx.y * BM, n0 = blockIdx.x * kBN;

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

    const int steps = (K + kBK - 1) / kBK, nz = gridDim.z, z = blockIdx.z;
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

    const float dec = PART ? 1.0f : g->dec;
    float *pz = PART ? part + (size_t)z * plane : nullptr;
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
                    if constexpr (PART)
                        pz[(size_t)m * N + n] = o;
                    else if constexpr (BF16OUT)
                        reinterpret_cast<uint16_t *>(y)[(size_t)m * N + n] = (uint16_t)f32_to_bf16_bits(o);
                    else
                        reinterpret_cast<float *>(y)[(size_t)m * N + n] = o;
                }
            }
        }
}

// Sum of the K-slice partials of each output in slice order (the same
// order on every call), times the global scale, as fp32 or bf16.  Planes are
// padded to a multiple of 4 floats, so the float4 reads of a last group stay
// inside the plane.
template <bool BF16OUT>
__global__ __launch_bounds__(256) void k_gemm_reduce(const float *__restrict__ part, size_t plane, int nz,
                                                     size_t count, const nvfp4_global *__restrict__ g,
                                                     void *__restrict__ y) {
    const float dec = g->dec;
    const size_t stride = (size_t)gridDim.x * 256 * 4;
    for (size_t e = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4; e < count; e += stride) {
        float4 a = *reinterpret_cast<const float4 *>(part + e);
        for (int z = 1; z < nz; ++z) {
            const float4 b = *reinterpret_cast<const float4 *>(part + (size_t)z * plane + e);
            a.x += b.x;
            a.y += b.y;
            a.z += b.z;
            a.w += b.w;
        }
        const float v[4] = {a.x * dec, a.y * dec, a.z * dec, a.w * dec};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            if (e + c >= count) break;
            if constexpr (BF16OUT)
                reinterpret_cast<uint16_t *>(y)[e + c] = (uint16_t)f32_to_bf16_bits(v[c]);
            else
                reinterpret_cast<float *>(y)[e + c] = v[c];
        }
    }
}

// Tile choice by rounds of resident workgroups: a 256-row round (2 per CU)
// takes about kTallRound times a 128-row round (3 per CU) -- measured at
// 8192 x 17408 x 5120, where both fill the chip: 919 against 815 TFLOP/s,
// 2 x 256 / 919 over 3 x 128 / 815.  A partly filled last round costs a
// full one, so e.g. 1024 x 17408 (544 tall tiles, 2 rounds) keeps the
// 128-row tile (1088 tiles, 2 rounds).
constexpr double kTallRound = 1.18;
constexpr int kMaxSplit = 16;             // K slices at most
// 64-k steps per slice at least: at 128 x 2048 x 4096 slices of 8 steps
// (8 slices) took 18.8-19.6 us against 21.4-22.3 for 16 slices of 4; the
// other 128- and 1024-row shapes were within noise; at most 4 or 8 slices
// instead of 16 made 128 x 5120 x 17408 slower (79, 60 against 52 us).
constexpr int kMinSliceSteps = 8;

struct GemmPlan {
    int bm;       // 128 or 256
    int split;    // K slices (128-row tiles only)
    size_t plane; // floats per partial plane (split > 1)
};

// 256-row tiles where they take fewer rounds; else 128-row tiles, with K cut
// into slices when the tiles fill less than one round of resident
// workgroups (prompt chunks of a few hundred rows): then up to kMaxSplit
// slices bring the grid to about one round.
static GemmPlan gemm_plan(int m, int n, int k) {
    const long cols = (n + kBN - 1) / kBN;
    const long slots_s = (long)num_cus() * blocks_per_cu(reinterpret_cast<const void *>(k_gemm<128, false, false>), 256, 0);
    const long slots_t = (long)num_cus() * blocks_per_cu(reinterpret_cast<const void *>(k_gemm<256, false, false>), 512, 0);
    const long tiles_s = cols * ((m + 127) / 128), tiles_t = cols * ((m + 255) / 256);
    const long rounds_s = (tiles_s + slots_s - 1) / slots_s, rounds_t = (tiles_t + slots_t - 1) / slots_t;
    GemmPlan p{128, 1, 0};
    if (kTallRound * rounds_t < rounds_s) {
        p.bm = 256;
        return p;
    }
    const long steps = (k + kBK - 1) / kBK;
    long split = slots_s / (tiles_s > 0 ? tiles_s : 1);
    split = split < kMaxSplit ? split : kMaxSplit;
    split = split < steps / kMinSliceSteps ? split : steps / kMinSliceSteps;
    if (split >= 2) {
        p.split = (int)split;
        p.plane = ((size_t)m * n + 3) & ~(size_t)3;
    }
    return p;
}

template <int BM, bool PART>
static void launch_gemm(const uint16_t *x, int m, const nvfp4_weight *w, void *y, bool bf16, float *part, size_t plane,
                        int split, hipStream_t s) {
    dim3 grid((w->n + kBN - 1) / kBN, (m + BM - 1) / BM, split);
    if (bf16)
        hipLaunchKernelGGL((k_gemm<BM, true, PART>), grid, dim3(2 * BM), 0, s, x, w->codes, w->scales, w->global, m,
                           w->n, w->k, y, part, plane);
    else
        hipLaunchKernelGGL((k_gemm<BM, false, PART>), grid, dim3(2 * BM), 0, s, x, w->codes, w->scales, w->global,
                           m, w->n, w->k, y, part, plane);
}

}  // namespace nvfp4

using namespace nvfp4;

extern "C" size_t w4a16_gemm_m128_workspace_bytes(int32_t m, int32_t n, int32_t k) {
    if (m < 1 || n < 1 || k < 32) return 0;
    const GemmPlan p = gemm_plan(m, n, k);
    return p.split > 1 ? (size_t)p.split * p.plane * sizeof(float) : 0;
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
    if ((w->n + kBN - 1) / kBN > 2147483647 || (m + 127) / 128 > 65535)
        return fail(NVFP4_ERR_UNSUPPORTED, "w4a16_gemm_m128: grid too large");
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const bool bf16 = y_dtype == NVFP4_OUT_BF16;
    GemmPlan p = gemm_plan(m, w->n, w->k);
    if (p.split > 1 && workspace == nullptr) p.split = 1;   // no workspace: one pass over K
    if (p.split > 1) {
        const size_t need = (size_t)p.split * p.plane * sizeof(float);
        if (ws_bytes < need)
            return fail(NVFP4_ERR_WORKSPACE, "w4a16_gemm_m128: workspace of %zu bytes, %zu needed", ws_bytes, need);
        if (!aligned(workspace, 16)) return fail(NVFP4_ERR_ALIGN, "w4a16_gemm_m128: workspace not 16-byte aligned");
        float *part = reinterpret_cast<float *>(workspace);
        launch_gemm<128, true>(x_bf16, m, w, y, bf16, part, p.plane, p.split, s);
        rc = check_launch("w4a16_gemm_m128");
        if (rc) return rc;
        const size_t count = (size_t)m * w->n;
        const size_t groups = (count + 3) / 4;
        const size_t want = (groups + 255) / 256, cap = (size_t)num_cus() * 8;
        const unsigned blocks = (unsigned)(want < cap ? want : cap);
        if (bf16)
            hipLaunchKernelGGL(k_gemm_reduce<true>, dim3(blocks), dim3(256), 0, s, part, p.plane, p.split, count,
                               w->global, y);
        else
            hipLaunchKernelGGL(k_gemm_reduce<false>, dim3(blocks), dim3(256), 0, s, part, p.plane, p.split, count,
                               w->global, y);
        return check_launch("w4a16_gemm_m128");
    }
    if (p.bm == 256)
        launch_gemm<256, false>(x_bf16, m, w, y, bf16, nullptr, 0, 1, s);
    else
        launch_gemm<128, false>(x_bf16, m, w, y, bf16, nullptr, 0, 1, s);
    return check_launch("w4a16_gemm_m128");
}
