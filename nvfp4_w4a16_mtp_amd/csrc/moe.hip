// Routed-expert MoE FFN for decode rows on NVFP4 experts: the
// `moe_topk_softmax` -> `moe_silu_mul` -> weighted-sum chain that new.rs
// (`MtpHead::new`) names for the head's MoE, with the NVFP4 expert
// gate/up [inter][hidden] and down [hidden][inter] matrices it quantizes.
//
// Four launches, all sized for the worst case and reading the routing from
// device memory (no host round trip):
//  1. route    (1 workgroup): top-k by logit (lower id first on ties),
//              softmax over the selected logits, and the list of distinct
//              experts in ascending id with the mask of tokens that chose
//              each one;
//  2. gate_up  (experts x row tiles): for each distinct expert, the gate and
//              up GEMVs over exactly the tokens that chose it -- the expert's
//              weights are streamed once however many tokens use it -- then
//              a = bf16(silu(g) * u) per (token, slot) pair;
//  3. down     (experts x row tiles): d = down(a) for the same pairs, fp32;
//  4. combine  y[t] = sum_j w[t][j] * d[t][j] in slot order (deterministic;
//              no floating-point atomics).
#include "gemv_core.hpp"

namespace nvfp4 {

constexpr int kMoeMaxTopK = 16;
constexpr int kMoeMaxExperts = 1024;
constexpr int kMoeHeader = 4096;   // route header bytes at the start of the workspace

struct MoeRoute {
    int n_distinct;
    int pad[3];
    int expert[128];      // distinct experts, ascending id
    int mask[128];        // bit t set: token t chose expert[u]
};
static_assert(sizeof(MoeRoute) <= kMoeHeader, "route header");

__global__ __launch_bounds__(256) void k_moe_route(const float *__restrict__ logits, int m, int E, int topk,
                                                  int32_t *__restrict__ ids, float *__restrict__ wts,
                                                  MoeRoute *__restrict__ route) {
    __shared__ float sv[256];
    __shared__ int si[256];
    __shared__ unsigned char taken[kMoeMaxExperts];
    __shared__ unsigned char tokmask[kMoeMaxExperts];
    __shared__ int sel[kMoeMaxTopK];
    __shared__ int counts[256];
    for (int e = threadIdx.x; e < E; e += blockDim.x) tokmask[e] = 0;
    __syncthreads();
    for (int t = 0; t < m; ++t) {
        const float *lg = logits + (size_t)t * E;
        for (int e = threadIdx.x; e < E; e += blockDim.x) taken[e] = 0;
        __syncthreads();
        for (int j = 0; j < topk; ++j) {
            float bv = -INFINITY;
            int bi = INT_MAX;
            for (int e = threadIdx.x; e < E; e += blockDim.x)
                if (!taken[e] && (bi == INT_MAX || beats(lg[e], e, bv, bi))) {
                    bv = lg[e];
                    bi = e;
                }
            sv[threadIdx.x] = bv;
            si[threadIdx.x] = bi;
            __syncthreads();
            for (int s = 128; s > 0; s >>= 1) {
                if (threadIdx.x < s) {
                    const int o = threadIdx.x + s;
                    if (si[o] != INT_MAX && (si[threadIdx.x] == INT_MAX || beats(sv[o], si[o], sv[threadIdx.x], si[threadIdx.x]))) {
                        sv[threadIdx.x] = sv[o];
                        si[threadIdx.x] = si[o];
                    }
                }
                __syncthreads();
            }
            if (threadIdx.x == 0) {
                sel[j] = si[0];
                taken[si[0]] = 1;
                tokmask[si[0]] |= (unsigned char)(1u << t);
            }
            __syncthreads();
        }
        if (threadIdx.x == 0) {
            // softmax over the selected logits (the largest is the first)
            const float lmax = lg[sel[0]];
            float ex[kMoeMaxTopK];
            float den = 0.0f;
            for (int j = 0; j < topk; ++j) {
                ex[j] = expf(lg[sel[j]] - lmax);
                den += ex[j];
            }
            for (int j = 0; j < topk; ++j) {
                ids[t * topk + j] = sel[j];
                wts[t * topk + j] = ex[j] / den;
            }
        }
        __syncthreads();
    }
    // compact the experts with a nonzero token mask, ascending id
    const int per = (E + blockDim.x - 1) / blockDim.x;
    const int e0 = threadIdx.x * per;
    int c = 0;
    for (int e = e0; e < min(E, e0 + per); ++e) c += tokmask[e] != 0;
    counts[threadIdx.x] = c;
    __syncthreads();
    if (threadIdx.x == 0) {
        int run = 0;
        for (int i = 0; i < (int)blockDim.x; ++i) {
            int v = counts[i];
            counts[i] = run;
            run += v;
        }
        route->n_distinct = run;
    }
    __syncthreads();
    int pos = counts[threadIdx.x];
    for (int e = e0; e < min(E, e0 + per); ++e)
        if (tokmask[e]) {
            route->expert[pos] = e;
            route->mask[pos] = tokmask[e];
            ++pos;
        }
}

// Index of the (token, slot) pair of token t that chose expert e.
__device__ __forceinline__ int pair_of(const int32_t *ids, int topk, int t, int e) {
    for (int j = 0; j < topk; ++j)
        if (ids[t * topk + j] == e) return t * topk + j;
    return -1;
}

// Runs the GEMV core for a runtime token count 1..8.
template <int R, class Epi>
__device__ __forceinline__ void gemv_tile_rt(int cnt, const uint4 *xs, const uint8_t *codes, const uint8_t *scales,
                                             int n, int k, int row0, Epi &&epi) {
    switch (cnt) {
        case 1: gemv_tile<1, R, 1>(xs, codes, scales, n, k, row0, nullptr, epi); break;
        case 2: gemv_tile<2, R, 1>(xs, codes, scales, n, k, row0, nullptr, epi); break;
        case 3: gemv_tile<3, R, 1>(xs, codes, scales, n, k, row0, nullptr, epi); break;
        case 4: gemv_tile<4, R, 1>(xs, codes, scales, n, k, row0, nullptr, epi); break;
        case 5: gemv_tile<5, R, 1>(xs, codes, scales, n, k, row0, nullptr, epi); break;
        case 6: gemv_tile<6, R, 1>(xs, codes, scales, n, k, row0, nullptr, epi); break;
        case 7: gemv_tile<7, R, 1>(xs, codes, scales, n, k, row0, nullptr, epi); break;
        default: gemv_tile<8, R, 1>(xs, codes, scales, n, k, row0, nullptr, epi); break;
    }
}

// Stages the rows listed in rows[0..cnt) of a [*, k] bf16 matrix into the
// swizzled LDS image of gemv_core.
__device__ __forceinline__ void stage_rows(uint4 *xs, const uint16_t *__restrict__ src, const int *rows, int cnt, int k) {
    const int C = k >> 5, upr = k >> 3;
    for (int p = threadIdx.x; p < cnt * upr; p += blockDim.x) {
        int mm = p / upr, w = p - mm * upr;
        int c = w >> 2, q = w & 3;
        xs[(mm * 4 + q) * C + c] = reinterpret_cast<const uint4 *>(src + (size_t)rows[mm] * k)[w];
    }
}

constexpr int kMoeR = 1;                     // rows per slot in the expert GEMVs
constexpr int kMoeRows = 16 * kMoeR;         // rows per workgroup tile

__global__ __launch_bounds__(256) void k_moe_gate_up(const uint16_t *__restrict__ x, nvfp4_moe_weights e, int topk,
                                                    const int32_t *__restrict__ ids, const MoeRoute *__restrict__ route,
                                                    uint16_t *__restrict__ act) {
    const int u = blockIdx.y;
    if (u >= route->n_distinct) return;
    const int ex = route->expert[u];
    const int mask = route->mask[u];
    const int H = e.hidden, I = e.inter;
    extern __shared__ uint4 smem[];
    uint4 *xs = smem;
    __shared__ int tok[8];
    __shared__ int prs[8];
    __shared__ float gbuf[kMoeRows][8];
    if (threadIdx.x == 0) {
        int c = 0;
        for (int t = 0; t < 8; ++t)
            if (mask & (1 << t)) {
                tok[c] = t;
                prs[c] = pair_of(ids, topk, t, ex);
                ++c;
            }
    }
    __syncthreads();
    const int cnt = __popc(mask);
    stage_rows(xs, x, tok, cnt, H);
    __syncthreads();
    const size_t wsz = (size_t)I * H;
    const uint8_t *gc = e.gate_codes + (size_t)ex * (wsz / 2), *gs = e.gate_scales + (size_t)ex * (wsz / 16);
    const uint8_t *uc = e.up_codes + (size_t)ex * (wsz / 2), *us = e.up_scales + (size_t)ex * (wsz / 16);
    const float gdec = e.gate_global[ex].dec, udec = e.up_global[ex].dec;
    const int row0 = blockIdx.x * kMoeRows;
    gemv_tile_rt<kMoeR>(cnt, xs, gc, gs, I, H, row0, [&](int row, int mm, float v) { gbuf[row - row0][mm] = v * gdec; });
    __syncthreads();
    gemv_tile_rt<kMoeR>(cnt, xs, uc, us, I, H, row0, [&](int row, int mm, float v) {
        const float g = gbuf[row - row0][mm];
        const float up = v * udec;
        const float a = g / (1.0f + expf(-g)) * up;
        act[(size_t)prs[mm] * I + row] = (uint16_t)f32_to_bf16_bits(a);
    });
}

__global__ __launch_bounds__(256) void k_moe_down(nvfp4_moe_weights e, int topk, const int32_t *__restrict__ ids,
                                                 const MoeRoute *__restrict__ route, const uint16_t *__restrict__ act,
                                                 float *__restrict__ dbuf) {
    const int u = blockIdx.y;
    if (u >= route->n_distinct) return;
    const int ex = route->expert[u];
    const int mask = route->mask[u];
    const int H = e.hidden, I = e.inter;
    extern __shared__ uint4 smem[];
    uint4 *xs = smem;
    __shared__ int prs[8];
    if (threadIdx.x == 0) {
        int c = 0;
        for (int t = 0; t < 8; ++t)
            if (mask & (1 << t)) prs[c++] = pair_of(ids, topk, t, ex);
    }
    __syncthreads();
    const int cnt = __popc(mask);
    stage_rows(xs, act, prs, cnt, I);
    __syncthreads();
    const size_t wsz = (size_t)H * I;
    const uint8_t *dc = e.down_codes + (size_t)ex * (wsz / 2), *ds = e.down_scales + (size_t)ex * (wsz / 16);
    const float ddec = e.down_global[ex].dec;
    gemv_tile_rt<kMoeR>(cnt, xs, dc, ds, H, I, blockIdx.x * kMoeRows,
                        [&](int row, int mm, float v) { dbuf[(size_t)prs[mm] * H + row] = v * ddec; });
}

__global__ __launch_bounds__(256) void k_moe_combine(const float *__restrict__ dbuf, const float *__restrict__ wts,
                                                    int m, int topk, int H, float *__restrict__ y) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= m * H) return;
    const int t = i / H, h = i - t * H;
    float acc = 0.0f;
    for (int j = 0; j < topk; ++j) acc = __builtin_fmaf(wts[t * topk + j], dbuf[(size_t)(t * topk + j) * H + h], acc);
    y[i] = acc;
}

static size_t moe_ws_bytes(int m, int topk, int H, int I) {
    const size_t pairs = (size_t)m * topk;
    size_t act = (pairs * I * 2 + 255) & ~(size_t)255;
    size_t d = pairs * H * 4;
    return kMoeHeader + act + d;
}

}  // namespace nvfp4

using namespace nvfp4;

extern "C" size_t moe_w4a16_gemv_workspace_bytes(int32_t m, int32_t top_k, const nvfp4_moe_weights *e) {
    if (!e || m < 1 || top_k < 1) return 0;
    return moe_ws_bytes(m, top_k, e->hidden, e->inter);
}

extern "C" int moe_w4a16_gemv(const uint16_t *x_bf16, int32_t m, const float *router_logits, int32_t top_k,
                              const nvfp4_moe_weights *e, float *y, int32_t *topk_ids, float *topk_w, void *workspace,
                              size_t ws_bytes, void *stream) {
    if (!e) return fail(NVFP4_ERR_ARG, "moe_w4a16_gemv: NULL expert descriptor");
    if (!x_bf16 || !router_logits || !y || !topk_ids || !topk_w)
        return fail(NVFP4_ERR_ARG, "moe_w4a16_gemv: NULL x/router_logits/y/topk_ids/topk_w");
    if (!e->gate_codes || !e->gate_scales || !e->gate_global || !e->up_codes || !e->up_scales || !e->up_global ||
        !e->down_codes || !e->down_scales || !e->down_global)
        return fail(NVFP4_ERR_ARG, "moe_w4a16_gemv: NULL expert weight pointer");
    if (m < 1 || m > 8) return fail(NVFP4_ERR_SHAPE, "moe_w4a16_gemv: m=%d outside 1..8", m);
    const int E = e->num_experts, H = e->hidden, I = e->inter;
    if (E < 1 || E > kMoeMaxExperts) return fail(NVFP4_ERR_SHAPE, "moe_w4a16_gemv: num_experts=%d outside 1..%d", E, kMoeMaxExperts);
    if (top_k < 1 || top_k > kMoeMaxTopK || top_k > E)
        return fail(NVFP4_ERR_SHAPE, "moe_w4a16_gemv: top_k=%d outside 1..min(E, %d)", top_k, kMoeMaxTopK);
    if (H < 32 || I < 32 || H % 32 || I % 32) return fail(NVFP4_ERR_SHAPE, "moe_w4a16_gemv: hidden/inter must be multiples of 32");
    if ((size_t)8 * H * 2 > (size_t)kLdsBytes - 2048 || (size_t)8 * I * 2 > (size_t)kLdsBytes - 2048)
        return fail(NVFP4_ERR_UNSUPPORTED, "moe_w4a16_gemv: hidden/inter above %d", (kLdsBytes - 2048) / 16);
    if (!aligned(x_bf16, 16) || !aligned(e->gate_codes, 16) || !aligned(e->up_codes, 16) || !aligned(e->down_codes, 16))
        return fail(NVFP4_ERR_ALIGN, "moe_w4a16_gemv: x and codes need 16-byte alignment");
    if (!aligned(e->gate_scales, 2) || !aligned(e->up_scales, 2) || !aligned(e->down_scales, 2) ||
        !aligned(router_logits, 4) || !aligned(y, 4) || !aligned(topk_ids, 4) || !aligned(topk_w, 4))
        return fail(NVFP4_ERR_ALIGN, "moe_w4a16_gemv: scales 2-byte, logits/outputs 4-byte alignment");
    const size_t need = moe_ws_bytes(m, top_k, H, I);
    if (!workspace || ws_bytes < need) return fail(NVFP4_ERR_WORKSPACE, "moe_w4a16_gemv: workspace needs %zu bytes", need);
    if (!aligned(workspace, 256)) return fail(NVFP4_ERR_ALIGN, "moe_w4a16_gemv: workspace not 256-byte aligned");
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    char *ws = reinterpret_cast<char *>(workspace);
    MoeRoute *route = reinterpret_cast<MoeRoute *>(ws);
    uint16_t *act = reinterpret_cast<uint16_t *>(ws + kMoeHeader);
    float *dbuf = reinterpret_cast<float *>(ws + kMoeHeader + (((size_t)m * top_k * I * 2 + 255) & ~(size_t)255));
    const int maxd = min(E, m * top_k);
    hipLaunchKernelGGL(k_moe_route, dim3(1), dim3(256), 0, s, router_logits, m, E, top_k, topk_ids, topk_w, route);
    int rc = check_launch("moe_w4a16_gemv(route)");
    if (rc) return rc;
    hipLaunchKernelGGL(k_moe_gate_up, dim3((I + kMoeRows - 1) / kMoeRows, maxd), dim3(256), (size_t)8 * H * 2, s, x_bf16,
                       *e, top_k, topk_ids, route, act);
    rc = check_launch("moe_w4a16_gemv(gate_up)");
    if (rc) return rc;
    hipLaunchKernelGGL(k_moe_down, dim3((H + kMoeRows - 1) / kMoeRows, maxd), dim3(256), (size_t)8 * I * 2, s, *e, top_k,
                       topk_ids, route, act, dbuf);
    rc = check_launch("moe_w4a16_gemv(down)");
    if (rc) return rc;
    hipLaunchKernelGGL(k_moe_combine, dim3((m * H + 255) / 256), dim3(256), 0, s, dbuf, topk_w, m, top_k, H, y);
    return check_launch("moe_w4a16_gemv(combine)");
}
