// Routed-expert MoE FFN for decode rows on NVFP4 experts: the
// `moe_topk_softmax` -> `moe_silu_mul` -> weighted-sum chain that new.rs
// (`MtpHead::new`) names for the head's MoE, with the NVFP4 expert
// gate/up [inter][hidden] and down [hidden][inter] matrices it quantizes.
//
// Three launches, sized for the worst case and reading the routing from
// device memory (no host round trip):
//  1. route   (one workgroup, one wavefront per token): top-k by logit with
//             the lower id first on ties (shuffle argmax over register-held
//             logits), softmax over the selected logits, and for each
//             distinct expert (ascending id) the tokens that chose it and
//             their (token, slot) pair indices;
//  2. gate_up (row tiles x distinct experts): the gate and up GEMVs over
//             exactly the tokens that chose the expert -- its weights are
//             streamed once however many tokens use it -- then
//             a = bf16(silu(g) * u) for each (token, slot) pair;
//  3. down    (row tiles x distinct experts): d = down(a) for the same
//             pairs; the last expert to finish a 16-row tile (a ticket per
//             tile, returned to zero afterwards) writes y[t] = sum_j w[t][j] *
//             d[t][j] in slot order for those rows -- deterministic, no
//             floating-point atomics.
#include "gemv_core.hpp"

namespace nvfp4 {

constexpr int kMoeMaxTopK = 16;
constexpr int kMoeMaxExperts = 1024;
constexpr int kMoeHeader = 12288;   // route header bytes at the start of the workspace
constexpr int kMoeRows = 16;        // rows per workgroup tile (R = 1, KS = 1)

// One distinct expert of a call: the tokens that chose it (ascending) and,
// for each, the index t * top_k + j of its (token, slot) pair.
struct MoeExpert {
    int expert;
    int cnt;
    int tok[8];
    int pair[8];
    int pad[2];
};
struct MoeRoute {
    int n_distinct;
    int pad[3];
    MoeExpert ex[128];   // ascending expert id
};
static_assert(sizeof(MoeRoute) <= kMoeHeader, "route header");

__global__ __launch_bounds__(256) void k_moe_route(const float *__restrict__ logits, int m, int E, int topk,
                                                  int32_t *__restrict__ ids, float *__restrict__ wts,
                                                  MoeRoute *__restrict__ route) {
    __shared__ int tokmask[kMoeMaxExperts];
    __shared__ unsigned char jof[kMoeMaxExperts][8];   // slot at which token t chose expert e
    __shared__ int wsum[4];
    for (int e = threadIdx.x; e < E; e += blockDim.x) tokmask[e] = 0;
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int per = (E + 63) / 64;   // logits per lane, <= 16
    for (int t = wave; t < m; t += 4) {
        const float *lg = logits + (size_t)t * E;
        float v[16];
        uint32_t taken = 0;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int e = lane + 64 * j;
            const bool in = j < per && e < E;
            v[j] = in ? lg[e] : 0.0f;
            if (!in) taken |= 1u << j;
        }
        float my_v = -INFINITY;   // lane s keeps the s-th selection
        int my_i = 0;
        for (int s = 0; s < topk; ++s) {
            float bv = -INFINITY;
            int bi = INT_MAX;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int e = lane + 64 * j;
                if (!(taken & (1u << j)) && (bi == INT_MAX || beats(v[j], e, bv, bi))) {
                    bv = v[j];
                    bi = e;
                }
            }
            for (int off = 32; off > 0; off >>= 1) {
                const float ov = __shfl_xor(bv, off, 64);
                const int oi = __shfl_xor(bi, off, 64);
                if (oi != INT_MAX && (bi == INT_MAX || beats(ov, oi, bv, bi))) {
                    bv = ov;
                    bi = oi;
                }
            }
            if (lane == s) {
                my_v = bv;
                my_i = bi;
            }
            if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
        }
        // softmax over the selected logits (selection 0 is the largest)
        const float vmax = __shfl(my_v, 0, 64);
        const float ex = lane < topk ? expf(my_v - vmax) : 0.0f;
        float den = ex;
        for (int off = 32; off > 0; off >>= 1) den += __shfl_xor(den, off, 64);
        if (lane < topk) {
            ids[t * topk + lane] = my_i;
            wts[t * topk + lane] = ex / den;
            atomicOr(&tokmask[my_i], 1 << t);
            jof[my_i][t] = (unsigned char)lane;
        }
    }
    __syncthreads();
    // compact the experts with a nonzero token mask, ascending id
    const int epp = (E + 255) / 256;     // experts per thread, <= 4
    const int e0 = threadIdx.x * epp;
    int c = 0;
    for (int e = e0; e < min(E, e0 + epp); ++e) c += tokmask[e] != 0;
    int incl = c;   // inclusive scan over the workgroup
    for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off, 64);
        if (lane >= off) incl += o;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wave; ++w) base += wsum[w];
    int pos = base + incl - c;
    for (int e = e0; e < min(E, e0 + epp); ++e) {
        const int mask = tokmask[e];
        if (!mask) continue;
        MoeExpert me;
        me.expert = e;
        me.cnt = 0;
        for (int t = 0; t < 8; ++t) {
            me.tok[t] = 0;
            me.pair[t] = 0;
        }
        for (int t = 0; t < 8; ++t)
            if (mask & (1 << t)) {
                me.tok[me.cnt] = t;
                me.pair[me.cnt] = t * topk + jof[e][t];
                ++me.cnt;
            }
        me.pad[0] = me.pad[1] = 0;
        route->ex[pos++] = me;
    }
    if (threadIdx.x == 255) route->n_distinct = base + incl;
}

// Stages rows rows[0..cnt) of a [*, k] bf16 matrix into the swizzled LDS
// image of gemv_core, zero-filling rows cnt..mt-1.
__device__ __forceinline__ void stage_rows(uint4 *xs, const uint16_t *__restrict__ src, const int *rows, int cnt, int mt,
                                           int k) {
    const int C = k >> 5, upr = k >> 3;
    for (int p = threadIdx.x; p < mt * upr; p += blockDim.x) {
        int mm = p / upr, w = p - mm * upr;
        int c = w >> 2, q = w & 3;
        xs[(mm * 4 + q) * C + c] =
            mm < cnt ? reinterpret_cast<const uint4 *>(src + (size_t)rows[mm] * k)[w] : make_uint4(0, 0, 0, 0);
    }
}

// gate/up body for MT >= cnt token rows.
template <int MT, int CPL>
__device__ __forceinline__ void gate_up_body(uint4 *xs, const uint16_t *x, const int *tok, const int *prs, int cnt,
                                             const uint8_t *gc, const uint8_t *gs, float gdec, const uint8_t *uc,
                                             const uint8_t *us, float udec, int I, int H, int row0,
                                             uint16_t *__restrict__ act) {
    float gl = 0.0f;   // gate value of this lane's (row, token)
    auto epi_g = [&](int row, int mm, float v) { gl = v * gdec; };
    auto epi_u = [&](int row, int mm, float v) {
        if (mm >= cnt) return;
        const float up = v * udec;
        const float a = gl / (1.0f + expf(-gl)) * up;
        act[(size_t)prs[mm] * I + row] = (uint16_t)f32_to_bf16_bits(a);
    };
    if constexpr (CPL > 0) {
        TileRegs<MT, 1, 1, CPL> tg, tu;
        gemv_tile_load(tg, gc, gs, I, H, row0);
        gemv_tile_load(tu, uc, us, I, H, row0);
        stage_rows(xs, x, tok, cnt, MT, H);
        __syncthreads();
        gemv_tile_compute(tg, xs, I, H, row0, nullptr, epi_g);
        gemv_tile_compute(tu, xs, I, H, row0, nullptr, epi_u);
    } else {
        stage_rows(xs, x, tok, cnt, MT, H);
        __syncthreads();
        gemv_tile_loop<MT, 1, 1>(xs, gc, gs, I, H, row0, nullptr, epi_g);
        gemv_tile_loop<MT, 1, 1>(xs, uc, us, I, H, row0, nullptr, epi_u);
    }
}

template <int CPL>
__global__ __launch_bounds__(256) void k_moe_gate_up(const uint16_t *__restrict__ x, nvfp4_moe_weights e,
                                                    const MoeRoute *__restrict__ route, uint16_t *__restrict__ act) {
    const int u = blockIdx.y;
    if (u >= route->n_distinct) return;
    const MoeExpert *me = &route->ex[u];
    const int ex = me->expert;
    const int cnt = me->cnt;
    const int H = e.hidden, I = e.inter;
    extern __shared__ uint4 smem[];
    const size_t wsz = (size_t)I * H;
    const uint8_t *gc = e.gate_codes + (size_t)ex * (wsz / 2), *gs = e.gate_scales + (size_t)ex * (wsz / 16);
    const uint8_t *uc = e.up_codes + (size_t)ex * (wsz / 2), *us = e.up_scales + (size_t)ex * (wsz / 16);
    const float gdec = e.gate_global[ex].dec, udec = e.up_global[ex].dec;
    const int row0 = blockIdx.x * kMoeRows;
    const int mt = round_up_mt(cnt);
    if (mt == 1) gate_up_body<1, CPL>(smem, x, me->tok, me->pair, cnt, gc, gs, gdec, uc, us, udec, I, H, row0, act);
    else if (mt == 2) gate_up_body<2, CPL>(smem, x, me->tok, me->pair, cnt, gc, gs, gdec, uc, us, udec, I, H, row0, act);
    else if (mt == 4) gate_up_body<4, CPL>(smem, x, me->tok, me->pair, cnt, gc, gs, gdec, uc, us, udec, I, H, row0, act);
    else gate_up_body<8, CPL>(smem, x, me->tok, me->pair, cnt, gc, gs, gdec, uc, us, udec, I, H, row0, act);
}

template <int MT, int CPL>
__device__ __forceinline__ void down_body(uint4 *xs, const uint16_t *act, const int *prs, int cnt, const uint8_t *dc,
                                          const uint8_t *ds, float ddec, int H, int I, int row0, float *__restrict__ dbuf) {
    auto epi = [&](int row, int mm, float v) {
        if (mm < cnt) st_dev(&dbuf[(size_t)prs[mm] * H + row], v * ddec);
    };
    if constexpr (CPL > 0) {
        TileRegs<MT, 1, 1, CPL> t;
        gemv_tile_load(t, dc, ds, H, I, row0);
        stage_rows(xs, act, prs, cnt, MT, I);
        __syncthreads();
        gemv_tile_compute(t, xs, H, I, row0, nullptr, epi);
    } else {
        stage_rows(xs, act, prs, cnt, MT, I);
        __syncthreads();
        gemv_tile_loop<MT, 1, 1>(xs, dc, ds, H, I, row0, nullptr, epi);
    }
}

template <int CPL>
__global__ __launch_bounds__(256) void k_moe_down(nvfp4_moe_weights e, int m, int topk, const float *__restrict__ wts,
                                                 const MoeRoute *__restrict__ route, const uint16_t *__restrict__ act,
                                                 float *__restrict__ dbuf, unsigned int *__restrict__ tickets,
                                                 float *__restrict__ y) {
    const int u = blockIdx.y;
    const int nd = route->n_distinct;
    if (u >= nd) return;
    const MoeExpert *me = &route->ex[u];
    const int ex = me->expert;
    const int cnt = me->cnt;
    const int H = e.hidden, I = e.inter;
    extern __shared__ uint4 smem[];
    __shared__ int s_last;
    const size_t wsz = (size_t)H * I;
    const uint8_t *dc = e.down_codes + (size_t)ex * (wsz / 2), *ds = e.down_scales + (size_t)ex * (wsz / 16);
    const float ddec = e.down_global[ex].dec;
    const int row0 = blockIdx.x * kMoeRows;
    const int mt = round_up_mt(cnt);
    if (mt == 1) down_body<1, CPL>(smem, act, me->pair, cnt, dc, ds, ddec, H, I, row0, dbuf);
    else if (mt == 2) down_body<2, CPL>(smem, act, me->pair, cnt, dc, ds, ddec, H, I, row0, dbuf);
    else if (mt == 4) down_body<4, CPL>(smem, act, me->pair, cnt, dc, ds, ddec, H, I, row0, dbuf);
    else down_body<8, CPL>(smem, act, me->pair, cnt, dc, ds, ddec, H, I, row0, dbuf);

    // the last expert to finish this row tile writes y for its rows
    wait_mem();   // this workgroup's d values have reached device scope
    __syncthreads();
    if (threadIdx.x == 0) s_last = atomicAdd(&tickets[blockIdx.x], 1u) == (unsigned)(nd - 1);
    __syncthreads();
    if (!s_last) return;
    const int i = threadIdx.x;
    if (i < m * kMoeRows) {
        const int t = i / kMoeRows, row = row0 + (i - t * kMoeRows);
        if (row < H) {
            float acc = 0.0f;
            for (int j = 0; j < topk; ++j)
                acc = __builtin_fmaf(wts[t * topk + j], ld_dev(&dbuf[(size_t)(t * topk + j) * H + row]), acc);
            y[(size_t)t * H + row] = acc;
        }
    }
    if (threadIdx.x == 0) st_dev(&tickets[blockIdx.x], 0u);   // ready for the next call
}

struct MoeLayout {
    size_t tickets, act, dbuf, total;
};
static MoeLayout moe_layout(int m, int topk, int H, int I) {
    MoeLayout L;
    const size_t pairs = (size_t)m * topk;
    L.tickets = kMoeHeader;
    L.act = L.tickets + (((size_t)(H + kMoeRows - 1) / kMoeRows * 4 + 255) & ~(size_t)255);
    L.dbuf = L.act + ((pairs * I * 2 + 255) & ~(size_t)255);
    L.total = L.dbuf + pairs * H * 4;
    return L;
}

template <int CPL>
static void launch_gate_up(dim3 g, size_t lds, hipStream_t s, const uint16_t *x, const nvfp4_moe_weights &e,
                           const MoeRoute *route, uint16_t *act) {
    hipLaunchKernelGGL(k_moe_gate_up<CPL>, g, dim3(256), lds, s, x, e, route, act);
}
template <int CPL>
static void launch_down(dim3 g, size_t lds, hipStream_t s, const nvfp4_moe_weights &e, int m, int topk, const float *wts,
                        const MoeRoute *route, const uint16_t *act, float *dbuf, unsigned int *tickets, float *y) {
    hipLaunchKernelGGL(k_moe_down<CPL>, g, dim3(256), lds, s, e, m, topk, wts, route, act, dbuf, tickets, y);
}

static int cpl_for(int k) {
    if (k % 512) return 0;
    const int c = k / 512;
    return (c == 1 || c == 2 || c == 4) ? c : 0;
}

}  // namespace nvfp4

using namespace nvfp4;

extern "C" size_t moe_w4a16_gemv_workspace_bytes(int32_t m, int32_t top_k, const nvfp4_moe_weights *e) {
    if (!e || m < 1 || top_k < 1 || e->hidden < 1 || e->inter < 1) return 0;
    return moe_layout(m, top_k, e->hidden, e->inter).total;
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
    if (E < 1 || E > kMoeMaxExperts)
        return fail(NVFP4_ERR_SHAPE, "moe_w4a16_gemv: num_experts=%d outside 1..%d", E, kMoeMaxExperts);
    if (top_k < 1 || top_k > kMoeMaxTopK || top_k > E)
        return fail(NVFP4_ERR_SHAPE, "moe_w4a16_gemv: top_k=%d outside 1..min(E, %d)", top_k, kMoeMaxTopK);
    if (H < 32 || I < 32 || H % 32 || I % 32)
        return fail(NVFP4_ERR_SHAPE, "moe_w4a16_gemv: hidden/inter must be multiples of 32");
    if ((size_t)8 * H * 2 > (size_t)kLdsBytes - 1024 || (size_t)8 * I * 2 > (size_t)kLdsBytes - 1024)
        return fail(NVFP4_ERR_UNSUPPORTED, "moe_w4a16_gemv: hidden/inter above %d", (kLdsBytes - 1024) / 16);
    if (!aligned(x_bf16, 16) || !aligned(e->gate_codes, 16) || !aligned(e->up_codes, 16) || !aligned(e->down_codes, 16))
        return fail(NVFP4_ERR_ALIGN, "moe_w4a16_gemv: x and codes need 16-byte alignment");
    if (!aligned(e->gate_scales, 2) || !aligned(e->up_scales, 2) || !aligned(e->down_scales, 2) ||
        !aligned(router_logits, 4) || !aligned(y, 4) || !aligned(topk_ids, 4) || !aligned(topk_w, 4))
        return fail(NVFP4_ERR_ALIGN, "moe_w4a16_gemv: scales 2-byte, logits/outputs 4-byte alignment");
    const MoeLayout L = moe_layout(m, top_k, H, I);
    if (!workspace || ws_bytes < L.total)
        return fail(NVFP4_ERR_WORKSPACE, "moe_w4a16_gemv: workspace needs %zu bytes", L.total);
    if (!aligned(workspace, 256)) return fail(NVFP4_ERR_ALIGN, "moe_w4a16_gemv: workspace not 256-byte aligned");
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    char *ws = reinterpret_cast<char *>(workspace);
    MoeRoute *route = reinterpret_cast<MoeRoute *>(ws);
    unsigned int *tickets = reinterpret_cast<unsigned int *>(ws + L.tickets);
    uint16_t *act = reinterpret_cast<uint16_t *>(ws + L.act);
    float *dbuf = reinterpret_cast<float *>(ws + L.dbuf);
    const int maxd = min(E, m * top_k);
    hipLaunchKernelGGL(k_moe_route, dim3(1), dim3(256), 0, s, router_logits, m, E, top_k, topk_ids, topk_w, route);
    int rc = check_launch("moe_w4a16_gemv(route)");
    if (rc) return rc;
    const nvfp4_moe_weights ev = *e;
    const dim3 g1((I + kMoeRows - 1) / kMoeRows, maxd), g2((H + kMoeRows - 1) / kMoeRows, maxd);
    const size_t lds1 = (size_t)8 * H * 2, lds2 = (size_t)8 * I * 2;
    switch (cpl_for(H)) {
        case 1: launch_gate_up<1>(g1, lds1, s, x_bf16, ev, route, act); break;
        case 2: launch_gate_up<2>(g1, lds1, s, x_bf16, ev, route, act); break;
        case 4: launch_gate_up<4>(g1, lds1, s, x_bf16, ev, route, act); break;
        default: launch_gate_up<0>(g1, lds1, s, x_bf16, ev, route, act); break;
    }
    rc = check_launch("moe_w4a16_gemv(gate_up)");
    if (rc) return rc;
    switch (cpl_for(I)) {
        case 1: launch_down<1>(g2, lds2, s, ev, m, top_k, topk_w, route, act, dbuf, tickets, y); break;
        case 2: launch_down<2>(g2, lds2, s, ev, m, top_k, topk_w, route, act, dbuf, tickets, y); break;
        case 4: launch_down<4>(g2, lds2, s, ev, m, top_k, topk_w, route, act, dbuf, tickets, y); break;
        default: launch_down<0>(g2, lds2, s, ev, m, top_k, topk_w, route, act, dbuf, tickets, y); break;
    }
    return check_launch("moe_w4a16_gemv(down)");
}
