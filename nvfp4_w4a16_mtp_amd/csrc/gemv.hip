// W4A16 decode GEMV and the LM-head GEMV fused with argmax.
//
// w4a16_gemv: the projection GEMV of mtp_head.rs (`MtpHead::gemv` ->
// `w4a16_decode_gemv`) for M = 1..8 rows, used for the head's fc, q/k/v/o
// projections (new.rs, `MtpHead::new` quantizes exactly these).
//
// lmhead_gemv_argmax: the NVFP4 LM head over the first V vocabulary rows and
// the argmax that turns it into the draft token (new.rs resolves the NVFP4
// LM head and `argmax_bf16`; deepseek_v4_mtp.rs `forward_one` runs LM head
// then argmax, with the reduced vocabulary).  Pass 1 computes logits tile by
// tile and keeps, per workgroup and row m, the best (key, index); no logits
// tensor is written.  Pass 2 (one workgroup) combines the partials.  The
// combine keeps the larger key and, on equal keys, the lower index, which is
// exactly the ascending strict-greater scan of `argmax_grammar_masked`.
#include <float.h>

#include "gemv_core.hpp"

namespace nvfp4 {

constexpr int kMaxPartials = 4096;        // LM-head pass-1 workgroups at most
constexpr int kLmStaticLds = 16 * 8 * 16; // per-slot argmax candidates of pass 1

template <int M, int R, int KS, bool BF16OUT>
__global__ __launch_bounds__(256) void k_gemv(const uint16_t *__restrict__ x, const uint8_t *__restrict__ codes,
                                             const uint8_t *__restrict__ scales, const nvfp4_global *__restrict__ g,
                                             int n, int k, void *__restrict__ y) {
    extern __shared__ uint4 smem[];
    uint4 *xs = smem;
    float *red = reinterpret_cast<float *>(smem + (M * k) / 8);
    stage_x(xs, reinterpret_cast<const uint4 *>(x), M, k);
    __syncthreads();
    const float dec = g->dec;
    constexpr int rows = GemvTile<M, R, KS>::kRowsPerTile;
    const int ntiles = (n + rows - 1) / rows;
    for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        gemv_tile<M, R, KS>(xs, codes, scales, n, k, tile * rows, red, [&](int row, int mm, float v) {
            const float o = v * dec;
            if constexpr (BF16OUT)
                reinterpret_cast<uint16_t *>(y)[(size_t)mm * n + row] = (uint16_t)f32_to_bf16_bits(o);
            else
                reinterpret_cast<float *>(y)[(size_t)mm * n + row] = o;
        });
    }
}

struct ArgPart {
    float key;    // compared value (fp32 logit or its bf16 rounding)
    float val;    // fp32 logit of that row
    int idx;
    int pad;
};

template <int M, int R, int KS, bool BF16KEY>
__global__ __launch_bounds__(256) void k_lmhead_pass1(const uint16_t *__restrict__ x, const uint8_t *__restrict__ codes,
                                                     const uint8_t *__restrict__ scales,
                                                     const nvfp4_global *__restrict__ g, int v, int k,
                                                     ArgPart *__restrict__ parts, float *__restrict__ row0) {
    extern __shared__ uint4 smem[];
    uint4 *xs = smem;
    float *red = reinterpret_cast<float *>(smem + (M * k) / 8);
    stage_x(xs, reinterpret_cast<const uint4 *>(x), M, k);
    __syncthreads();
    const float dec = g->dec;
    constexpr int rows = GemvTile<M, R, KS>::kRowsPerTile;
    const int ntiles = (v + rows - 1) / rows;
    // lane m of every slot keeps the best of the rows it was handed for m
    float bkey = -INFINITY, bval = -INFINITY;
    int bidx = INT_MAX;
    for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        gemv_tile<M, R, KS>(xs, codes, scales, v, k, tile * rows, red, [&](int row, int mm, float s) {
            const float logit = s * dec;
            const float key = BF16KEY ? bf16_bits_to_f32(f32_to_bf16_bits(logit)) : logit;
            if (row == 0) row0[mm] = logit;
            if (beats(key, row, bkey, bidx)) {
                bkey = key;
                bval = logit;
                bidx = row;
            }
        });
    }
    // workgroup combine: 16 slots x M candidates -> M partials
    __shared__ ArgPart cand[16][8];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int slot = lane >> 4, t = lane & 15;
    const int gslot = wave * 4 + slot;
    if (t < M) cand[gslot][t] = ArgPart{bkey, bval, bidx, 0};
    __syncthreads();
    if (threadIdx.x < M) {
        const int mm = threadIdx.x;
        ArgPart best{-INFINITY, -INFINITY, INT_MAX, 0};
        for (int s = 0; s < 16; ++s) {
            // wavefronts of K segments other than 0 never produced candidates
            ArgPart c = cand[s][mm];
            if (KS > 1 && ((s >> 2) % KS) != 0) continue;
            if (beats(c.key, c.idx, best.key, best.idx)) best = c;
        }
        parts[(size_t)blockIdx.x * M + mm] = best;
    }
}

__global__ __launch_bounds__(256) void k_lmhead_pass2(const ArgPart *__restrict__ parts, int nparts, int m,
                                                     const float *__restrict__ row0, int32_t *__restrict__ out_idx,
                                                     float *__restrict__ out_max) {
    __shared__ ArgPart red[256];
    for (int mm = 0; mm < m; ++mm) {
        ArgPart best{-INFINITY, -INFINITY, INT_MAX, 0};
        for (int p = threadIdx.x; p < nparts; p += blockDim.x) {
            ArgPart c = parts[(size_t)p * m + mm];
            if (beats(c.key, c.idx, best.key, best.idx)) best = c;
        }
        red[threadIdx.x] = best;
        __syncthreads();
        for (int s = 128; s > 0; s >>= 1) {
            if (threadIdx.x < s) {
                ArgPart c = red[threadIdx.x + s];
                if (beats(c.key, c.idx, red[threadIdx.x].key, red[threadIdx.x].idx)) red[threadIdx.x] = c;
            }
            __syncthreads();
        }
        if (threadIdx.x == 0) {
            ArgPart b = red[0];
            // nothing above -inf: the scan keeps its initial index 0
            if (!(b.key > -INFINITY)) {
                out_idx[mm] = 0;
                out_max[mm] = row0[mm];
            } else {
                out_idx[mm] = b.idx;
                out_max[mm] = b.val;
            }
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------ dispatch ----
template <int M>
static int launch_gemv_m(const uint16_t *x, const nvfp4_weight *w, void *y, bool bf16, hipStream_t s) {
    const TileChoice tc = choose_tile(w->n, num_cus(), ksplit_fits(M, w->k));
    const int rows = 16 * tc.R / tc.KS;
    const int ntiles = (w->n + rows - 1) / rows;
    const int grid = ntiles;
    const size_t lds = gemv_lds_bytes(M, w->k, tc);
#define NVFP4_GEMV_CASE(RR, KK)                                                                           \
    if (tc.R == RR && tc.KS == KK) {                                                                      \
        if (bf16)                                                                                         \
            hipLaunchKernelGGL((k_gemv<M, RR, KK, true>), dim3(grid), dim3(256), lds, s, x, w->codes,     \
                               w->scales, w->global, w->n, w->k, y);                                      \
        else                                                                                              \
            hipLaunchKernelGGL((k_gemv<M, RR, KK, false>), dim3(grid), dim3(256), lds, s, x, w->codes,    \
                               w->scales, w->global, w->n, w->k, y);                                      \
        return check_launch("w4a16_gemv");                                                                \
    }
    NVFP4_GEMV_CASE(4, 1)
    NVFP4_GEMV_CASE(2, 1)
    NVFP4_GEMV_CASE(1, 1)
    NVFP4_GEMV_CASE(1, 2)
    NVFP4_GEMV_CASE(1, 4)
#undef NVFP4_GEMV_CASE
    return fail(NVFP4_ERR_UNSUPPORTED, "w4a16_gemv: no tile shape");
}

template <int M>
static int launch_lmhead_m(const uint16_t *h, const nvfp4_weight *w, int v, ArgPart *parts, float *row0,
                           int32_t *out_idx, float *out_max, bool bf16key, hipStream_t s) {
    const bool ks_ok = gemv_lds_bytes(M, w->k, TileChoice{1, 2}) + kLmStaticLds <= (size_t)kLdsBytes;
    const TileChoice tc = choose_tile(v, num_cus(), ks_ok);
    const int rows = 16 * tc.R / tc.KS;
    const int ntiles = (v + rows - 1) / rows;
    int grid = num_cus() * 4;
    if (grid > ntiles) grid = ntiles;
    if (grid > kMaxPartials) grid = kMaxPartials;
    const size_t lds = gemv_lds_bytes(M, w->k, tc);
#define NVFP4_LM_CASE(RR, KK)                                                                             \
    if (tc.R == RR && tc.KS == KK) {                                                                      \
        if (bf16key)                                                                                      \
            hipLaunchKernelGGL((k_lmhead_pass1<M, RR, KK, true>), dim3(grid), dim3(256), lds, s, h,       \
                               w->codes, w->scales, w->global, v, w->k, parts, row0);                     \
        else                                                                                              \
            hipLaunchKernelGGL((k_lmhead_pass1<M, RR, KK, false>), dim3(grid), dim3(256), lds, s, h,      \
                               w->codes, w->scales, w->global, v, w->k, parts, row0);                     \
        int rc = check_launch("lmhead_gemv_argmax(pass 1)");                                              \
        if (rc) return rc;                                                                                \
        hipLaunchKernelGGL(k_lmhead_pass2, dim3(1), dim3(256), 0, s, parts, grid, M, row0, out_idx,       \
                           out_max);                                                                      \
        return check_launch("lmhead_gemv_argmax(pass 2)");                                                \
    }
    NVFP4_LM_CASE(4, 1)
    NVFP4_LM_CASE(2, 1)
    NVFP4_LM_CASE(1, 1)
    NVFP4_LM_CASE(1, 2)
    NVFP4_LM_CASE(1, 4)
#undef NVFP4_LM_CASE
    return fail(NVFP4_ERR_UNSUPPORTED, "lmhead_gemv_argmax: no tile shape");
}

}  // namespace nvfp4

using namespace nvfp4;

extern "C" int w4a16_gemv(const uint16_t *x_bf16, int32_t m, const nvfp4_weight *w, void *y, int32_t y_dtype,
                          void *stream) {
    int rc = validate_weight(w, "w4a16_gemv");
    if (rc) return rc;
    if (w->n == 0 && m >= 1) return ok();   // empty output: nothing to read or write
    if (!x_bf16 || !y) return fail(NVFP4_ERR_ARG, "w4a16_gemv: NULL x or y");
    if (m < 1 || m > 8) return fail(NVFP4_ERR_SHAPE, "w4a16_gemv: m=%d outside 1..8", m);
    if (y_dtype != NVFP4_OUT_F32 && y_dtype != NVFP4_OUT_BF16)
        return fail(NVFP4_ERR_ARG, "w4a16_gemv: unknown y_dtype %d", y_dtype);
    if (!aligned(x_bf16, 16)) return fail(NVFP4_ERR_ALIGN, "w4a16_gemv: x not 16-byte aligned");
    if (!aligned(y, 4)) return fail(NVFP4_ERR_ALIGN, "w4a16_gemv: y not 4-byte aligned");
    if ((size_t)m * w->k * 2 > (size_t)kLdsBytes)
        return fail(NVFP4_ERR_UNSUPPORTED, "w4a16_gemv: m * k = %lld exceeds %d activations", (long long)m * w->k,
                    kLdsBytes / 2);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const bool bf16 = y_dtype == NVFP4_OUT_BF16;
    switch (m) {
        case 1: return launch_gemv_m<1>(x_bf16, w, y, bf16, s);
        case 2: return launch_gemv_m<2>(x_bf16, w, y, bf16, s);
        case 3: return launch_gemv_m<3>(x_bf16, w, y, bf16, s);
        case 4: return launch_gemv_m<4>(x_bf16, w, y, bf16, s);
        case 5: return launch_gemv_m<5>(x_bf16, w, y, bf16, s);
        case 6: return launch_gemv_m<6>(x_bf16, w, y, bf16, s);
        case 7: return launch_gemv_m<7>(x_bf16, w, y, bf16, s);
        default: return launch_gemv_m<8>(x_bf16, w, y, bf16, s);
    }
}

extern "C" size_t lmhead_gemv_argmax_workspace_bytes(int32_t m, int32_t vocab_rows) {
    (void)vocab_rows;
    if (m < 1) m = 1;
    if (m > 8) m = 8;
    return (size_t)kMaxPartials * m * sizeof(ArgPart) + 256;
}

extern "C" int lmhead_gemv_argmax(const uint16_t *h_bf16, int32_t m, const nvfp4_weight *w, int32_t vocab_rows,
                                  int32_t *out_idx, float *out_max, void *workspace, size_t ws_bytes,
                                  uint32_t flags, void *stream) {
    int rc = validate_weight(w, "lmhead_gemv_argmax");
    if (rc) return rc;
    if (!h_bf16 || !out_idx || !out_max) return fail(NVFP4_ERR_ARG, "lmhead_gemv_argmax: NULL h/out_idx/out_max");
    if (m < 1 || m > 8) return fail(NVFP4_ERR_SHAPE, "lmhead_gemv_argmax: m=%d outside 1..8", m);
    if (vocab_rows < 0) return fail(NVFP4_ERR_ARG, "lmhead_gemv_argmax: vocab_rows=%d < 0", vocab_rows);
    if (flags & ~NVFP4_ARGMAX_BF16_KEYS) return fail(NVFP4_ERR_ARG, "lmhead_gemv_argmax: unknown flags 0x%x", flags);
    const int v = (vocab_rows == 0 || vocab_rows > w->n) ? w->n : vocab_rows;
    if (v < 1) return fail(NVFP4_ERR_SHAPE, "lmhead_gemv_argmax: empty vocabulary");
    if (!aligned(h_bf16, 16) || !aligned(out_idx, 4) || !aligned(out_max, 4))
        return fail(NVFP4_ERR_ALIGN, "lmhead_gemv_argmax: h needs 16-byte, outputs 4-byte alignment");
    if ((size_t)m * w->k * 2 + kLmStaticLds > (size_t)kLdsBytes)
        return fail(NVFP4_ERR_UNSUPPORTED, "lmhead_gemv_argmax: m * k exceeds %d activations",
                    (kLdsBytes - kLmStaticLds) / 2);
    if (!workspace || ws_bytes < lmhead_gemv_argmax_workspace_bytes(m, vocab_rows))
        return fail(NVFP4_ERR_WORKSPACE, "lmhead_gemv_argmax: workspace needs %zu bytes",
                    lmhead_gemv_argmax_workspace_bytes(m, vocab_rows));
    if (!aligned(workspace, 256)) return fail(NVFP4_ERR_ALIGN, "lmhead_gemv_argmax: workspace not 256-byte aligned");
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    float *row0 = reinterpret_cast<float *>(workspace);
    ArgPart *parts = reinterpret_cast<ArgPart *>(reinterpret_cast<char *>(workspace) + 256);
    const bool bk = (flags & NVFP4_ARGMAX_BF16_KEYS) != 0;
    switch (m) {
        case 1: return launch_lmhead_m<1>(h_bf16, w, v, parts, row0, out_idx, out_max, bk, s);
        case 2: return launch_lmhead_m<2>(h_bf16, w, v, parts, row0, out_idx, out_max, bk, s);
        case 3: return launch_lmhead_m<3>(h_bf16, w, v, parts, row0, out_idx, out_max, bk, s);
        case 4: return launch_lmhead_m<4>(h_bf16, w, v, parts, row0, out_idx, out_max, bk, s);
        case 5: return launch_lmhead_m<5>(h_bf16, w, v, parts, row0, out_idx, out_max, bk, s);
        case 6: return launch_lmhead_m<6>(h_bf16, w, v, parts, row0, out_idx, out_max, bk, s);
        case 7: return launch_lmhead_m<7>(h_bf16, w, v, parts, row0, out_idx, out_max, bk, s);
        default: return launch_lmhead_m<8>(h_bf16, w, v, parts, row0, out_idx, out_max, bk, s);
    }
}
