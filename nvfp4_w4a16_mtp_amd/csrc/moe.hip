// Routed-expert MoE FFN for decode rows on NVFP4 experts: the
// `moe_topk_softmax` -> `moe_silu_mul` -> weighted-sum chain that new.rs
// (`MtpHead::new`) names for the head's MoE, with the NVFP4 expert
// gate/up [inter][hidden] and down [hidden][inter] matrices it quantizes.
// The routing is decided on the device (no host round trip): top-k by
// logit with the lower id first on ties, softmax over the selected logits,
// the distinct experts in ascending id with their tokens and (token, slot)
// pairs.  The gate/up pass takes one column of workgroups per (token, slot)
// pair -- a workgroup needs only its own token's selections up to its slot,
// and an expert two tokens chose is streamed once per pair -- and the down
// pass streams each distinct expert's weights once.
//
// Launch structure:
//  * one token, when the whole grid is resident: one launch (k_moe_fused).
//    The gate/up workgroups of column j select the token's j-th expert, run
//    16 rows of its gate and up and store a = bf16(silu(g) * u); the down
//    workgroups, after them in dispatch order, route for themselves,
//    prefetch their weights and wait for a release per column before
//    reading the activations;
//  * otherwise: gate/up (workgroup (0, 0) also routes every token and
//    publishes the ids, the weights and the down pass's plan), then the down
//    pass: the row-owner pass (k_moe_down_rows: a workgroup owns 8 output
//    rows of every routed expert, all pairs' activations in LDS, y summed
//    per token in ascending expert order) when the activations fit in LDS,
//    else the ticket pass (k_moe_down: 64-row tiles per expert, d per pair
//    to the workspace, the last expert of a tile sums y in slot order).
// No floating-point atomics: y is deterministic for given inputs.
#include <algorithm>

#include "gemv_core.hpp"

namespace nvfp4 {

constexpr int kMoeMaxTopK = 16;
constexpr int kMoeMaxExperts = 1024;
constexpr int kMoeHeader = 16384;   // route header bytes at the start of the workspace
constexpr int kPairU = 1;   // chunks per pipeline stage of the gate|up row pair
constexpr int kMoeRows = 16;        // rows per workgroup tile (R = 1, KS = 1)
constexpr int kSpinLimit = 1 << 22;    // polls of the fused down pass's wait (seconds)
// Hand-off words of the fused launch, each counter on its own 128-byte line:
// per expert column u a count of its finished gate/up workgroups (word
// 32 u, zero between calls); then per down workgroup i, kGoStride words
// apart, its go word (+0) and its count (+1).  The workgroup that completes
// a column adds kGoTag to every down workgroup's go word, so a call releases
// each of them once per column; the count holds kGoTag times the number of
// releases the down workgroup expected up to and including its last call.
// At the start of a call with r columns the go word lies between the count
// c and c + r kGoTag (the releases of this call that have landed); the call
// waits for c + r kGoTag and stores that as the new count.  Releases left
// over from an earlier call whose wait gave up have landed before the next
// launch starts (launches on one workspace are serialized), so they never
// count towards a later call; any other value (an overwritten workspace) is
// reported instead of trusted.
constexpr int kColStride = 32, kSyncWords = 32 * 128, kGoStride = 16;
constexpr unsigned int kGoTag = 0x9E3779B1u;      // odd, so multiplying by it is one-to-one mod 2^32
constexpr unsigned int kGoTagInv = 0x0E8B2F51u;   // its inverse mod 2^32
// Sticky status of a MoE workspace (bit 0: a down pass gave up its wait;
// bit 1: it found its go word overwritten), at a fixed offset at the end of
// the route header; the host reads and clears it with moe_workspace_status.
constexpr int kMoeStatusOffset = 16384 - 64;
constexpr unsigned int kMoeStatusTimeout = 1u, kMoeStatusCorrupt = 2u;
constexpr size_t kMoeMaxLds = 160 * 1024 - 4096;   // dynamic LDS of one workgroup, static LDS aside

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
    int n_pairs;
    int pad[2];
    MoeExpert ex[128];   // ascending expert id
    // flat plan for the down pass, read in one round: per distinct expert its
    // first pair position and down-projection scale, per pair position (in
    // (expert, token) order) the token, the pair index and its weight
    int ex_id[128];
    int pb[129];
    float ddec[128];
    int pos_tok[128];
    int pos_pair[128];
    float pos_w[128];
};
static_assert(sizeof(MoeRoute) <= kMoeStatusOffset, "route header");

// The shared expert of the complete MoE layer (all pointers device memory;
// on == 0 for the routed-only entry point).  Its gate and up outputs come
// from the grouped GEMV that also produces the router logits.
struct MoeShared {
    const float *sg, *su;           // gate / up outputs, fp32 [m][I]
    uint16_t *sact;                 // its activations, bf16 [m][I]
    const uint16_t *gate_w;         // shared_expert_gate, bf16 [H], or nullptr (ungated)
    float *sgate;                   // sigmoid(gate_w . x_t), fp32 [m] (1 when ungated)
    const uint8_t *dcodes, *dscales;
    const nvfp4_global *dglob;      // its down projection [H][I]
    int on;
    // phase timestamps of the one-launch form, or nullptr: event ev of
    // workgroup b at trace[ev * grid + b] (moe_w4a16_gemv_trace)
    unsigned long long *trace;
};

// Events of trace_mark.  Gate/up workgroups: start, routing done,
// activations stored, counted in the column (and, for the last one of a
// column, its release issued).  Down workgroups: start, weight loads issued,
// go word seen, activations staged, sums done, output written.
// Only the traced instantiation records them: a run-time test of the
// pointer alone, in the plain kernel, slowed the one-token launch by 1.6 us.
constexpr int kTraceEvents = 6;
template <bool TRACE>
__device__ __forceinline__ void trace_mark(unsigned long long *trace, int ev) {
    if constexpr (TRACE)
        if (threadIdx.x == 0) trace[(size_t)ev * gridDim.x + blockIdx.x] = __builtin_amdgcn_s_memrealtime();
}

// Sum over the wavefront in a fixed order; every lane gets the result.
__device__ __forceinline__ float wave_sum(float v) {
    v = row16_sum(v);
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return (r0 + r1) + (r2 + r3);
}

// Routing of all m tokens, computed by one workgroup in LDS.
struct RouteLds {
    int tokmask[kMoeMaxExperts];                 // bit t: token t chose expert e
    unsigned char jof[kMoeMaxExperts][8];        // slot at which token t chose e
    int sel_i[8][kMoeMaxTopK];
    float sel_w[8][kMoeMaxTopK];
    int wsum[16];
    int n_distinct;
    MoeExpert ex[128];
};

// Top-k by logit (lower id first on ties), softmax over the selected logits,
// then the distinct experts in ascending id with their tokens and pairs.
// One wavefront per token.  Lane l holds the logits of experts
// [l * PER, (l + 1) * PER), sorted once (larger logit first, lower id first
// on ties), so its head is its best untaken expert.  A selection is a DPP max
// of the heads, a ballot of the lanes whose head equals it and the lowest
// such lane -- its experts all have lower ids than those of higher lanes, so
// it holds the lowest-id maximum -- which then pops its head.  The dependent
// chain of a selection is a few dozen instructions.
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false)));
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// Top-k of one token's logits; lane s < topk receives the s-th selection.
// nsel < topk: only the first nsel selections (the same ones).
template <int PER>
__device__ __forceinline__ void route_token(const float *__restrict__ lg, int E, int topk, int lane, float &my_v,
                                            int &my_i, int nsel = -1) {
    float v[PER];
    int id[PER];
    int rem = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int e = lane * PER + j;
        const bool in = e < E;
        v[j] = in ? lg[e] : -INFINITY;
        id[j] = in ? e : INT_MAX;
        rem += in;
    }
    // odd-even transposition sort: larger logit first, lower id on ties
    // (entries past E carry id INT_MAX and sort last)
#pragma unroll
    for (int r = 0; r < PER; ++r)
#pragma unroll
        for (int j = r & 1; j + 1 < PER; j += 2) {
            const bool sw = v[j + 1] > v[j] || (v[j + 1] == v[j] && id[j + 1] < id[j]);
            const float tv = v[j];
            const int ti = id[j];
            v[j] = sw ? v[j + 1] : v[j];
            id[j] = sw ? id[j + 1] : id[j];
            v[j + 1] = sw ? tv : v[j + 1];
            id[j + 1] = sw ? ti : id[j + 1];
        }
    my_v = -INFINITY;
    my_i = 0;
    const int ns = nsel < 0 ? topk : nsel;
    for (int s = 0; s < ns; ++s) {
        const float mx = wave_max(rem > 0 ? v[0] : -INFINITY);
        uint64_t ball = __ballot(rem > 0 && v[0] == mx);
        if (!ball) ball = __ballot(rem > 0);   // only with NaN logits: any untaken expert, never out of range
        const int wl = (int)__builtin_ctzll(ball);
        const int wid = __builtin_amdgcn_readlane(id[0], wl);
        if (lane == s) {
            my_v = mx;
            my_i = wid;
        }
        const bool pop = lane == wl;
#pragma unroll
        for (int j = 0; j + 1 < PER; ++j) {
            v[j] = pop ? v[j + 1] : v[j];
            id[j] = pop ? id[j + 1] : id[j];
        }
        rem -= pop;
    }
}

template <int PER>
__device__ __forceinline__ void moe_route_per(const float *__restrict__ logits, int m, int E, int topk, RouteLds &L) {
    if (m == 1) {
        // one token: its top_k experts are the distinct ones; wavefront 0
        // selects them and ranks them by id (no masks, atomics or
        // compaction rounds), in the same order as the general path below
        if (threadIdx.x < 64) {
            const int lane = threadIdx.x;
            float my_v;
            int my_i;
            route_token<PER>(logits, E, topk, lane, my_v, my_i);
            const float vmax = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_v), 0));
            const float ex = lane < topk ? expf(my_v - vmax) : 0.0f;
            const float den = wave_sum(ex);
            int rank = 0;
            for (int j = 0; j < topk; ++j) rank += __builtin_amdgcn_readlane(my_i, j) < my_i;
            if (lane < topk) {
                L.sel_i[0][lane] = my_i;
                L.sel_w[0][lane] = ex / den;
                MoeExpert &me = L.ex[rank];
                me.expert = my_i;
                me.cnt = 1;
                me.tok[0] = 0;
                me.pair[0] = lane;
            }
            if (lane == 0) L.n_distinct = topk;
        }
        __syncthreads();
        return;
    }
    for (int e = threadIdx.x; e < E; e += blockDim.x) L.tokmask[e] = 0;
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    for (int t = wave; t < m; t += nw) {
        float my_v;
        int my_i;
        route_token<PER>(logits + (size_t)t * E, E, topk, lane, my_v, my_i);
        const float vmax = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_v), 0));
        const float ex = lane < topk ? expf(my_v - vmax) : 0.0f;
        const float den = wave_sum(ex);
        if (lane < topk) {
            L.sel_i[t][lane] = my_i;
            L.sel_w[t][lane] = ex / den;
            atomicOr(&L.tokmask[my_i], 1 << t);
            L.jof[my_i][t] = (unsigned char)lane;
        }
    }
    __syncthreads();
    // compact the experts with a nonzero token mask, ascending id: thread q
    // looks at experts q, q + blockDim.x, ...; a ballot and the lane's count
    // of lower set lanes place each one
    int base = 0;
    for (int e0 = 0; e0 < E; e0 += blockDim.x) {
        const int e = e0 + (int)threadIdx.x;
        const int mask = e < E ? L.tokmask[e] : 0;
        const uint64_t ball = __ballot(mask != 0);
        const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(ball >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)ball, 0));
        if (lane == 0) L.wsum[wave] = __popcll(ball);
        __syncthreads();
        int pos = base, total = 0;
        for (int w = 0; w < nw; ++w) {
            pos += w < wave ? L.wsum[w] : 0;
            total += L.wsum[w];
        }
        pos += below;
        if (mask) {
            MoeExpert &me = L.ex[pos];
            me.expert = e;
            int cnt = 0;
            for (int t = 0; t < m; ++t)
                if (mask & (1 << t)) {
                    me.tok[cnt] = t;
                    me.pair[cnt] = t * topk + L.jof[e][t];
                    ++cnt;
                }
            me.cnt = cnt;
        }
        base += total;
        __syncthreads();   // wsum is rewritten by the next round
    }
    if (threadIdx.x == 0) L.n_distinct = base;
    __syncthreads();
}

// The expert of the u-th selection of a single token (u < topk), from
// wavefront 0 after u + 1 selections; valid in every lane of wavefront 0.
__device__ __forceinline__ int moe_route_nth(const float *__restrict__ logits, int E, int topk, int u) {
    const int lane = threadIdx.x & 63, per = (E + 63) / 64;
    float v;
    int i;
    if (per <= 1) route_token<1>(logits, E, topk, lane, v, i, u + 1);
    else if (per <= 2) route_token<2>(logits, E, topk, lane, v, i, u + 1);
    else if (per <= 4) route_token<4>(logits, E, topk, lane, v, i, u + 1);
    else if (per <= 8) route_token<8>(logits, E, topk, lane, v, i, u + 1);
    else route_token<16>(logits, E, topk, lane, v, i, u + 1);
    return __builtin_amdgcn_readlane(i, u);
}

__device__ __forceinline__ void moe_route_lds(const float *__restrict__ logits, int m, int E, int topk, RouteLds &L) {
    const int per = (E + 63) / 64;
    if (per <= 1) moe_route_per<1>(logits, m, E, topk, L);
    else if (per <= 2) moe_route_per<2>(logits, m, E, topk, L);
    else if (per <= 4) moe_route_per<4>(logits, m, E, topk, L);
    else if (per <= 8) moe_route_per<8>(logits, m, E, topk, L);
    else moe_route_per<16>(logits, m, E, topk, L);
}

// Stages rows rows[0..cnt) of a [*, k] bf16 matrix into the swizzled LDS
// image of gemv_core, zero-filling rows cnt..mt-1.
__device__ __forceinline__ void stage_rows(uint4 *xs, const uint16_t *__restrict__ src, const int *rows, int cnt, int mt,
                                           int k) {
    const int C = k >> 5, upr = k >> 3;
    stage_batched(
        mt * upr, threadIdx.x, blockDim.x,
        [&](int p) {
            const int mm = p / upr;
            return mm < cnt ? reinterpret_cast<const uint4 *>(src + (size_t)rows[mm] * k)[p - mm * upr]
                            : make_uint4(0, 0, 0, 0);
        },
        [&](int p, uint4 v) {
            const int mm = p / upr, w = p - mm * upr;
            xs[(mm * 4 + (w & 3)) * C + (w >> 2)] = v;
        });
}

// stage_rows for rows another workgroup of the same launch wrote: 16-byte
// buffer loads with the device-coherent cache policy (sc1), over a source of
// src_rows rows.
constexpr int kBufWord3 = 0x00020000;   // buffer resource word 3 for raw byte buffers (gfx9 family)
constexpr int kCoherent = 16;           // sc1: device-scope coherent load
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
__device__ __forceinline__ void stage_rows_dev(uint4 *xs, const uint16_t *__restrict__ src, size_t src_rows,
                                               const int *rows, int cnt, int mt, int k) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void *)src, 0, (int)(src_rows * k * 2), kBufWord3);
    const int C = k >> 5, upr = k >> 3;
    stage_batched(
        mt * upr, threadIdx.x, blockDim.x,
        [&](int p) {
            const int mm = p / upr;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (mm < cnt) {
                const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(r, (rows[mm] * k + 8 * (p - mm * upr)) * 2, 0,
                                                                       kCoherent);
                v = make_uint4(t.x, t.y, t.z, t.w);
            }
            return v;
        },
        [&](int p, uint4 v) {
            const int mm = p / upr, w = p - mm * upr;
            xs[(mm * 4 + (w & 3)) * C + (w >> 2)] = v;
        });
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
        st_dev(&act[(size_t)prs[mm] * I + row], (uint16_t)f32_to_bf16_bits(a));   // read across workgroups
    };
    // Preloading both tiles is kept to MT <= 2 (the common case: most experts
    // serve one or two tokens), so that the 8-token branch does not set the
    // register budget of the whole kernel.
    if constexpr (CPL > 0 && MT <= 2) {
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
        bool pair = false;
        if constexpr (MT <= 2) pair = ((H >> 5) & 15) == 0;
        if (pair) {
            // the gate row and the up row of a lane's slot stream as one
            // two-row pipeline (a 16-row tile: one row per slot; kept to
            // MT <= 2 for the register budget, as above)
            const int lane = threadIdx.x & 63, slot = lane >> 4, tl = lane & 15;
            const int row = row0 + (threadIdx.x >> 6) * 4 + slot;
            const int rc = min(row, I - 1);   // rows past I: never passed to the epilogue
            const uint8_t *const cp[2] = {gc + (size_t)rc * (size_t)(H >> 1), uc + (size_t)rc * (size_t)(H >> 1)};
            const uint8_t *const sp[2] = {gs + (size_t)rc * (size_t)(H >> 4), us + (size_t)rc * (size_t)(H >> 4)};
            float acc[2][MT];
#pragma unroll
            for (int r = 0; r < 2; ++r)
#pragma unroll
                for (int mm = 0; mm < MT; ++mm) acc[r][mm] = 0.0f;
            pipe_rows<MT, 2, kPairU>(xs, cp, sp, H >> 5, tl, H >> 9, acc);
#pragma unroll
            for (int mm = 0; mm < MT; ++mm) {
                const float g = row16_sum(acc[0][mm]), u = row16_sum(acc[1][mm]);
                if (tl == mm && row < I) {
                    epi_g(row, mm, g);
                    epi_u(row, mm, u);
                }
            }
        } else {
            gemv_tile_loop<MT, 1, 1, 0>(xs, gc, gs, I, H, row0, nullptr, epi_g);
            gemv_tile_loop<MT, 1, 1, 0>(xs, uc, us, I, H, row0, nullptr, epi_u);
        }
    }
}

// Routing + gate/up: every workgroup computes the routing in LDS (cheap,
// and it saves a launch), takes the distinct expert u and the row tile bx
// (of gx), and workgroup (0, 0) publishes ids and weights -- and, for a
// separate down launch, the route.  Activations, and the shared expert's
// activations and gate, are stored device-scope: in the fused launch the
// down workgroups read them in the same launch, once the workgroup has
// counted itself in the hand-off words `done` (FUSED).
// gate/up of one token's pair over the row tiles bx0, bx0 + bs, ... (< gx):
// the workgroup routes once and stages the activation row once for all of
// them; each tile's weights are loaded and computed in turn (the other
// workgroups of the CU cover the loads' latency).
template <int CPL>
__device__ __forceinline__ void gate_up_tiles(uint4 *xs, const uint16_t *x, const int *tok, const int *prs,
                                              const uint8_t *gc, const uint8_t *gs, float gdec, const uint8_t *uc,
                                              const uint8_t *us, float udec, int I, int H, int bx0, int bs, int gx,
                                              uint16_t *__restrict__ act) {
    static_assert(CPL > 0, "preloaded tiles need a fixed chunk count");
    TileRegs<1, 1, 1, CPL> tg, tu;
    gemv_tile_load(tg, gc, gs, I, H, bx0 * kMoeRows);
    gemv_tile_load(tu, uc, us, I, H, bx0 * kMoeRows);
    stage_rows(xs, x, tok, 1, 1, H);
    __syncthreads();
    const size_t arow = (size_t)prs[0] * I;
    for (int bx = bx0; bx < gx; bx += bs) {
        if (bx != bx0) {
            gemv_tile_load(tg, gc, gs, I, H, bx * kMoeRows);
            gemv_tile_load(tu, uc, us, I, H, bx * kMoeRows);
        }
        float gl = 0.0f;   // gate value of this lane's row
        auto epi_g = [&](int row, int mm, float v) { gl = v * gdec; };
        auto epi_u = [&](int row, int mm, float v) {
            const float up = v * udec;
            act[arow + row] = (uint16_t)f32_to_bf16_bits(gl / (1.0f + expf(-gl)) * up);
        };
        gemv_tile_compute(tg, xs, I, H, bx * kMoeRows, nullptr, epi_g);
        gemv_tile_compute(tu, xs, I, H, bx * kMoeRows, nullptr, epi_u);
    }
}

// The routing's outputs: ids and weights, and (route != nullptr) the plan of
// the two-launch path -- distinct experts, and per pair position (in
// (expert, token) order) its token, pair and weight.  One workgroup.
__device__ __forceinline__ void write_route(RouteLds &L, const nvfp4_moe_weights &e, int m, int topk,
                                            int32_t *__restrict__ ids, float *__restrict__ wts,
                                            MoeRoute *__restrict__ route, const float *dec_lds = nullptr) {
    for (int p = threadIdx.x; p < m * topk; p += blockDim.x) {
        ids[p] = L.sel_i[p / topk][p % topk];
        wts[p] = L.sel_w[p / topk][p % topk];
    }
    if (route == nullptr) return;
    // thread q writes distinct expert q and its pairs; its first pair
    // position is the exclusive prefix sum of the pair counts (nd <= 128):
    // a scan inside each of the first two wavefronts, the second adding the
    // first's total (a serial sum per thread cost a dependent LDS read per
    // expert before it: about 2 us at 8 tokens)
    const int nd = L.n_distinct;
    const int q = threadIdx.x, lane = q & 63;
    const int c = q < nd ? L.ex[q].cnt : 0;
    int incl = c;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int v = __shfl_up(incl, d, 64);
        if (lane >= d) incl += v;
    }
    if (lane == 63 && q < 128) L.wsum[q >> 6] = incl;
    __syncthreads();
    if (q > nd) return;
    const int pb = q < 64 ? incl - c : q < 128 ? incl - c + L.wsum[0] : L.wsum[0] + L.wsum[1];
    route->pb[q] = pb;
    if (q == nd) {
        route->n_distinct = nd;
        route->n_pairs = pb;
        return;
    }
    const MoeExpert &me = L.ex[q];
    route->ex[q] = me;
    route->ex_id[q] = me.expert;
    route->ddec[q] = dec_lds != nullptr ? dec_lds[me.expert] : e.down_global[me.expert].dec;
    for (int k = 0; k < me.cnt; ++k) {
        route->pos_tok[pb + k] = me.tok[k];
        route->pos_pair[pb + k] = me.pair[k];
        route->pos_w[pb + k] = L.sel_w[me.tok[k]][me.pair[k] - me.tok[k] * topk];
    }
}

template <int CPL, bool FUSED, bool TRACE = false, bool MULTI = false>
__device__ __forceinline__ void gate_up_role(uint4 *smem, int bx, int u, int gx, const uint16_t *__restrict__ x,
                                             const float *__restrict__ logits, int m, int E, int topk,
                                             const nvfp4_moe_weights &e, int32_t *__restrict__ ids,
                                             float *__restrict__ wts, MoeRoute *__restrict__ route,
                                             uint16_t *__restrict__ act, const MoeShared &sh, unsigned int *done,
                                             int n_down, int gx_tiles = 0) {
    RouteLds &L = *reinterpret_cast<RouteLds *>(smem);   // reused for the activations afterwards
    __shared__ int tok[8], prs[8];
    __shared__ int s_ex, s_cnt, s_nd;
    if (FUSED) trace_mark<TRACE>(sh.trace, 0);
    // shared expert: the workgroups of the first expert column form 16 of its
    // activations per token each (loads issued before the routing, stored after)
    const int I = e.inter, H = e.hidden;
    const int si = bx * kMoeRows + (threadIdx.x & 15), st = threadIdx.x >> 4;
    const bool s_act = sh.on && u == 0 && st < m && si < I;
    float sgv = 0.0f, suv = 0.0f;
    if (s_act) {
        sgv = sh.sg[(size_t)st * I + si];
        suv = sh.su[(size_t)st * I + si];
    }
    // shared_expert_gate: the last workgroup of the first column, one wavefront per token
    if (sh.on && u == 0 && bx == gx - 1) {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        for (int t = wave; t < m; t += 4) {
            float z = 0.0f;
            if (sh.gate_w != nullptr)
                for (int h = lane; h < H; h += 64)
                    z = __builtin_fmaf(bf16_bits_to_f32(sh.gate_w[h]), bf16_bits_to_f32(x[(size_t)t * H + h]), z);
            z = wave_sum(z);
            if (lane == 0) st_dev(&sh.sgate[t], sh.gate_w != nullptr ? 1.0f / (1.0f + expf(-z)) : 1.0f);
        }
    }
    if (FUSED || bx != 0 || u != 0) {
        // column u is pair u = t top_k + j: token t's j-th selected expert,
        // known after j + 1 selections of that token alone, so the early
        // columns' weights stream while the later ones still select (an
        // expert two tokens chose is streamed once per pair).  The whole
        // routing is published by workgroup (0, 0), or in the one-token
        // launch by a down workgroup.
        if (threadIdx.x < 64) {
            const int t = u / topk, j = u - t * topk;
            const int id = u < m * topk ? moe_route_nth(logits + (size_t)t * E, E, topk, j) : 0;
            if (threadIdx.x == 0) {
                s_nd = m * topk;
                s_ex = id;
                s_cnt = 1;
                tok[0] = t;
                prs[0] = u;
            }
        }
    } else {
        // workgroup (0, 0) of the two-launch form: the whole routing, the ids
        // and weights and the down pass's plan, then its own pair 0
        moe_route_lds(logits, m, E, topk, L);
        write_route(L, e, m, topk, ids, wts, route);
        if (threadIdx.x == 0) {
            s_nd = m * topk;
            s_ex = L.sel_i[0][0];
            s_cnt = 1;
            tok[0] = 0;
            prs[0] = 0;
        }
    }
    if (s_act) st_dev(&sh.sact[(size_t)st * I + si], (uint16_t)f32_to_bf16_bits(sgv / (1.0f + expf(-sgv)) * suv));
    __syncthreads();   // the routing scratch is free from here on
    if (FUSED) trace_mark<TRACE>(sh.trace, 1);
    if (u >= s_nd) return;
    const int ex = s_ex, cnt = s_cnt;
    const size_t wsz = (size_t)I * H;
    const uint8_t *gc = e.gate_codes + (size_t)ex * (wsz / 2), *gs = e.gate_scales + (size_t)ex * (wsz / 16);
    const uint8_t *uc = e.up_codes + (size_t)ex * (wsz / 2), *us = e.up_scales + (size_t)ex * (wsz / 16);
    const float gdec = e.gate_global[ex].dec, udec = e.up_global[ex].dec;
    const int row0 = bx * kMoeRows;
    if constexpr (MULTI) {
        // tiles bx, bx + gx, ... of gx_tiles (gx: workgroups per pair); no shared expert
        gate_up_tiles<CPL>(smem, x, tok, prs, gc, gs, gdec, uc, us, udec, I, H, bx, gx, gx_tiles, act);
        return;
    }
    gate_up_body<1, CPL>(smem, x, tok, prs, cnt, gc, gs, gdec, uc, us, udec, I, H, row0, act);
    if constexpr (FUSED) {
        // count this workgroup in its column; the one that completes the
        // column releases it to every down workgroup through its go word
        __shared__ int s_release;
        wait_mem();   // this workgroup's activations have reached device scope
        trace_mark<TRACE>(sh.trace, 2);
        __syncthreads();
        if (threadIdx.x == 0) {
            int rel = 0;
            if (atomicAdd(&done[kColStride * u], 1u) == (unsigned int)(gx - 1)) {
                st_dev(&done[kColStride * u], 0u);
                rel = 1;
            }
            s_release = rel;
        }
        __syncthreads();
        if (s_release)
            for (int i = threadIdx.x; i < n_down; i += blockDim.x)
                __hip_atomic_fetch_add(&done[kSyncWords + kGoStride * i], kGoTag, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
        trace_mark<TRACE>(sh.trace, 3);
    }
}

// The two-launch form's gate/up pass (one workgroup per 16-row tile and
// (token, slot) pair), held to four workgroups a CU.  MULTI: a workgroup
// over several tiles of its pair (gate_up_tiles).
template <int CPL, bool MULTI>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void k_moe_gate_up(const uint16_t *__restrict__ x, const float *__restrict__ logits,
                                                    int m, int E, int topk, nvfp4_moe_weights e,
                                                    int32_t *__restrict__ ids, float *__restrict__ wts,
                                                    MoeRoute *__restrict__ route, uint16_t *__restrict__ act,
                                                    MoeShared sh, int gx_tiles) {
    extern __shared__ uint4 smem[];
    gate_up_role<CPL, false, false, MULTI>(smem, blockIdx.x, blockIdx.y, gridDim.x, x, logits, m, E, topk, e, ids,
                                           wts, route, act, sh, nullptr, 0, gx_tiles);
}

// Rows per slot of the ticket down pass: 4 (a 64-row tile, about 37 KB of
// weights per workgroup at inter = 1024; 16-row tiles were launch-bound).
constexpr int kDownR = 4;
constexpr int kDownTile = 16 * kDownR;

template <int MT, int CPL>
__device__ __forceinline__ void down_body(uint4 *xs, const uint16_t *act, const int *prs, int cnt, const uint8_t *dc,
                                          const uint8_t *ds, float ddec, int H, int I, int row0, float *__restrict__ dbuf) {
    auto epi = [&](int row, int mm, float v) {
        if (mm < cnt) st_dev(&dbuf[(size_t)prs[mm] * H + row], v * ddec);
    };
    // preloading is kept to MT <= 2, as in gate/up, so that the rarer wide
    // experts do not set the register budget of the kernel
    if constexpr (CPL > 0 && MT <= 2) {
        TileRegs<MT, kDownR, 1, CPL> t;
        gemv_tile_load(t, dc, ds, H, I, row0);
        stage_rows(xs, act, prs, cnt, MT, I);
        __syncthreads();
        gemv_tile_compute(t, xs, H, I, row0, nullptr, epi);
    } else {
        stage_rows(xs, act, prs, cnt, MT, I);
        __syncthreads();
#pragma unroll 1
        for (int i = 0; i < kDownR; ++i) gemv_tile_loop<MT, 1, 1, 0>(xs, dc, ds, H, I, row0 + 16 * i, nullptr, epi);
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
    const int row0 = blockIdx.x * kDownTile;
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
    for (int i = threadIdx.x; i < m * kDownTile; i += blockDim.x) {
        const int t = i / kDownTile, row = row0 + (i - t * kDownTile);
        if (row < H) {
            float acc = 0.0f;
            for (int j = 0; j < topk; ++j)
                acc = __builtin_fmaf(wts[t * topk + j], ld_dev(&dbuf[(size_t)(t * topk + j) * H + row]), acc);
            y[(size_t)t * H + row] = acc;
        }
    }
    if (threadIdx.x == 0) st_dev(&tickets[blockIdx.x], 0u);   // ready for the next call
}

// Down pass when every (token, slot) activation row fits in LDS (the usual
// decode case: m * top_k <= 31 at inter = 1024).  Workgroup w owns output rows
// [w * kDownRows, (w + 1) * kDownRows) of every routed expert: its 16 slots
// take (expert, row) items in turn, all of a batch's weight loads in flight at
// once, and write d into LDS; the workgroup then forms y = sum of w * d per
// token in ascending expert order.  No scratch buffer, no ticket, one pass.
constexpr int kDownRows = 8;
constexpr int kDownBatch = 2;   // items per slot in a batch; two batches in flight
constexpr int kDownMaxExperts = 129;   // routed (<= 128) + the shared one
constexpr int kDownMaxPos = 136;       // pairs (<= 128) + one per token for the shared expert

// The row-owner down pass of workgroup bx.  Separate launch: the plan comes
// from the route the gate/up launch published.  FUSED (one launch with the
// gate/up workgroups, which come first in dispatch order): the workgroup
// computes the routing itself, builds the plan in LDS, issues its weight
// loads, then waits until its go word holds one release of this call per
// expert column (every gate/up workgroup of the column has stored its
// activations) and reads the activations with device-coherent loads.  The
// wait is bounded: past kSpinLimit polls the workgroup writes NaN rows and
// sets the workspace's status instead of waiting for ever.
// The items of the row-owner down pass: item it is row r0 + it % kDownRows
// of distinct expert it / kDownRows (the shared expert where s_ex is -1).
// Slot sl takes items b0 + sl + kSlots n of a batch; items past the end load
// a valid row (the last one) and are never computed.
struct DownItems {
    const uint8_t *codes, *scales;     // the routed experts' down matrices
    const uint8_t *scodes, *sscales;   // the shared expert's
    const int *s_ex;
    int nitems, r0, H, I, sl, tl;
};

template <int CPL>
__device__ __forceinline__ void down_rows_load(const DownItems &d, int b0, int kSlots, uint4 (&cw)[kDownBatch][CPL],
                                               uint32_t (&sw)[kDownBatch][CPL]) {
    const size_t wsz = (size_t)d.H * d.I;
#pragma unroll
    for (int n = 0; n < kDownBatch; ++n) {
        const int it = min(b0 + d.sl + kSlots * n, d.nitems - 1);
        const int u = it / kDownRows, row = min(d.r0 + it % kDownRows, d.H - 1);
        // selects, not branches: a branch here made the compiler wait for
        // loads already in flight
        const int ex = d.s_ex[u];
        const size_t eo = (size_t)(ex < 0 ? 0 : ex) * wsz;
        const uint8_t *dc = (ex < 0 ? d.scodes : d.codes) + eo / 2 + (size_t)row * (d.I / 2);
        const uint8_t *ds = (ex < 0 ? d.sscales : d.scales) + eo / 16 + (size_t)row * (d.I / 16);
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int c = d.tl + 16 * j;
            cw[n][j] = ld_stream16(dc + 16 * c);
            sw[n][j] = ld_stream2(ds + 2 * c);
        }
    }
}

template <int CPL>
__device__ __forceinline__ void down_rows_fma(const DownItems &d, int b0, int kSlots,
                                              const uint4 (&cw)[kDownBatch][CPL],
                                              const uint32_t (&sw)[kDownBatch][CPL], const int *s_pb,
                                              const float *s_dec, const uint4 *smem, int C,
                                              float (*contrib)[kDownRows], const int *img = nullptr) {
#pragma unroll
    for (int n = 0; n < kDownBatch; ++n) {
        const int it = b0 + d.sl + kSlots * n;
        if (it >= d.nitems) continue;   // uniform over the slot
        const int u = it / kDownRows, r = it % kDownRows;
        for (int pos = s_pb[u]; pos < s_pb[u + 1]; ++pos) {
            float acc[1] = {0.0f};
            const int ir = img ? img[pos] : pos;   // the position's row of the activation image
#pragma unroll
            for (int j = 0; j < CPL; ++j) chunk_fma<1>(cw[n][j], sw[n][j], smem + (size_t)ir * 4 * C, C, d.tl + 16 * j, acc);
            const float v = row16_sum(acc[0]);
            if (d.tl == 0) contrib[pos][r] = v * s_dec[u];
        }
    }
}

// down_rows_fma for one register batch when each expert has a single
// activation row (position u of expert u): the batch's items are computed
// together in one straight-line block, so that their dot products overlap (a
// wavefront per SIMD has no other work to hide their latency behind).
template <int CPL>
__device__ __forceinline__ void down_rows_fma_one(const DownItems &d, int b0, int kSlots,
                                                  const uint4 (&cw)[kDownBatch][CPL],
                                                  const uint32_t (&sw)[kDownBatch][CPL], const float *s_dec,
                                                  const uint4 *smem, int C, float (*contrib)[kDownRows]) {
    int itn[kDownBatch];
    float acc[kDownBatch][1];
#pragma unroll
    for (int n = 0; n < kDownBatch; ++n) {
        itn[n] = b0 + d.sl + kSlots * n;
        // an item past the end is computed on the last item's rows, not stored
        const int u = min(itn[n], d.nitems - 1) / kDownRows;
        acc[n][0] = 0.0f;
#pragma unroll
        for (int j = 0; j < CPL; ++j)
            chunk_fma<1>(cw[n][j], sw[n][j], smem + (size_t)u * 4 * C, C, d.tl + 16 * j, acc[n]);
    }
    float v[kDownBatch];
#pragma unroll
    for (int n = 0; n < kDownBatch; ++n) v[n] = row16_sum(acc[n][0]);
#pragma unroll
    for (int n = 0; n < kDownBatch; ++n)
        if (itn[n] < d.nitems && d.tl == 0) {
            const int u = itn[n] / kDownRows;
            contrib[u][itn[n] % kDownRows] = v[n] * s_dec[u];
        }
}

// stage_rows in two steps, so that loads issued in between do not delay the
// image: the first kStageBatch units of each thread into registers, then
// their stores and the rest of the image.  rows == nullptr: rows 0, 1, ...
__device__ __forceinline__ void stage_rows_first(uint4 (&v)[kStageBatch], const uint16_t *__restrict__ src,
                                                 const int *rows, int cnt, int k) {
    const int upr = k >> 3, units = cnt * upr;
#pragma unroll
    for (int j = 0; j < kStageBatch; ++j) {
        const int p = threadIdx.x + j * blockDim.x, mm = p / upr;
        v[j] = p < units ? reinterpret_cast<const uint4 *>(src + (size_t)(rows ? rows[mm] : mm) * k)[p - mm * upr]
                         : make_uint4(0, 0, 0, 0);
    }
}
__device__ __forceinline__ void stage_rows_rest(uint4 *xs, const uint4 (&v)[kStageBatch],
                                                const uint16_t *__restrict__ src, const int *rows, int cnt, int k) {
    const int C = k >> 5, upr = k >> 3, units = cnt * upr, done = kStageBatch * blockDim.x;
    auto put = [&](int p, uint4 val) {
        const int mm = p / upr, w = p - mm * upr;
        xs[(mm * 4 + (w & 3)) * C + (w >> 2)] = val;
    };
#pragma unroll
    for (int j = 0; j < kStageBatch; ++j) {
        const int p = threadIdx.x + j * blockDim.x;
        if (p < units) put(p, v[j]);
    }
    if (units > done)
        stage_batched(
            units - done, threadIdx.x, blockDim.x,
            [&](int q) {
                const int p = q + done, mm = p / upr;
                return reinterpret_cast<const uint4 *>(src + (size_t)(rows ? rows[mm] : mm) * k)[p - mm * upr];
            },
            [&](int q, uint4 val) { put(q + done, val); });
}

template <int CPL, bool FUSED, int NW = 4, bool TRACE = false>
__device__ __forceinline__ void down_rows_role(uint4 *smem, int bx, const nvfp4_moe_weights &e, int m, int topk,
                                               const MoeRoute *__restrict__ route, const float *__restrict__ logits,
                                               int E, int gx, const uint16_t *__restrict__ act, float *__restrict__ y,
                                               const MoeShared &sh, unsigned int *done, unsigned int *status,
                                               int32_t *__restrict__ ids = nullptr, float *__restrict__ wts = nullptr) {
    __shared__ int s_ex[kDownMaxExperts], s_pb[kDownMaxExperts + 1];
    __shared__ float s_dec[kDownMaxExperts], s_w[kDownMaxPos];
    __shared__ int s_tok[kDownMaxPos], s_pair[kDownMaxPos];
    __shared__ int s_img[kDownMaxPos];   // separate launch: the activation image's row of each position
    uint4 av[kStageBatch];               // separate launch: the first activation loads, issued with the plan's
    __shared__ float contrib[kDownMaxPos][kDownRows];
    __shared__ int s_nr, s_p0, s_late;
    if (FUSED) trace_mark<TRACE>(sh.trace, 0);
    const int H = e.hidden, I = e.inter, C = I >> 5;
    float s_decv = 0.0f;   // one-launch form: the down scale of distinct expert threadIdx.x
    // the plan in LDS; with a shared expert it follows the routed ones as
    // expert nd (id -1), its m positions after the pairs, weighted by the
    // shared gate, activation rows from sh.sact
    if constexpr (FUSED) {
        RouteLds &L = *reinterpret_cast<RouteLds *>(smem);   // the activation image overwrites it later
        moe_route_lds(logits, m, E, topk, L);
        if (bx == 0 && ids != nullptr) write_route(L, e, m, topk, ids, wts, nullptr);
        const int nr = L.n_distinct;
        // the experts' down scales go to LDS after the weight loads are
        // issued (a dependent load: waiting for it here delayed them)
        for (int q = threadIdx.x; q < nr; q += blockDim.x) s_ex[q] = L.ex[q].expert;
        if (threadIdx.x < nr) s_decv = e.down_global[L.ex[threadIdx.x].expert].dec;
        if (m == 1) {
            // one token: expert q is position q, its pair the slot that chose it
            if (threadIdx.x < nr) {
                const int pr = L.ex[threadIdx.x].pair[0];
                s_pb[threadIdx.x] = threadIdx.x;
                s_tok[threadIdx.x] = 0;
                s_pair[threadIdx.x] = pr;
                s_w[threadIdx.x] = L.sel_w[0][pr];
            }
            if (threadIdx.x == 0) {
                s_pb[nr] = nr;
                s_nr = nr;
                s_p0 = nr;
            }
        } else if (threadIdx.x == 0) {
            int pb = 0;
            for (int q = 0; q < nr; ++q) {
                const MoeExpert &me = L.ex[q];
                s_pb[q] = pb;
                for (int c = 0; c < me.cnt; ++c, ++pb) {
                    s_tok[pb] = me.tok[c];
                    s_pair[pb] = me.pair[c];
                    s_w[pb] = L.sel_w[me.tok[c]][me.pair[c] - me.tok[c] * topk];
                }
            }
            s_pb[nr] = pb;
            s_nr = nr;
            s_p0 = pb;
        }
        __syncthreads();
    } else {
        // the plan in one round of loads: every entry up to the m top_k pairs
        // (the distinct count only bounds which are used), then the
        // activation rows, which need no plan (image row u is pair u; the
        // sums look up each position's row): both round trips overlap
        const int P0 = m * topk;   // every (token, slot) pair is a position
        const int i = threadIdx.x;
        int pb = 0, ex = 0, tk = 0, pr = 0, nr = 0;
        float dec = 0.0f, w = 0.0f;
        if (i <= P0) pb = route->pb[i];
        if (i < P0) {
            ex = route->ex_id[i];
            dec = route->ddec[i];
            tk = route->pos_tok[i];
            pr = route->pos_pair[i];
            w = route->pos_w[i];
        }
        if (i == 0) nr = route->n_distinct;
        stage_rows_first(av, act, nullptr, P0, I);
        __builtin_amdgcn_sched_barrier(0);
        if (i <= P0) s_pb[i] = pb;
        if (i < P0) {
            s_ex[i] = ex;
            s_dec[i] = dec;
            s_tok[i] = tk;
            s_pair[i] = pr;
            s_w[i] = w;
            s_img[i] = pr;
        }
        if (i == 0) {
            s_nr = nr;
            s_p0 = P0;
        }
        __syncthreads();
    }
    const int nr = s_nr, P0 = s_p0;
    const int nd = nr + (sh.on ? 1 : 0), P = P0 + (sh.on ? m : 0);
    if (sh.on) {
        if (threadIdx.x == 0) {
            s_ex[nr] = -1;
            s_dec[nr] = sh.dglob->dec;
            s_pb[nr + 1] = P;
        }
        if (threadIdx.x < m) {
            if (!FUSED) s_img[P0 + threadIdx.x] = P0 + threadIdx.x;   // the shared expert's rows follow the pairs'
            s_tok[P0 + threadIdx.x] = threadIdx.x;
            s_pair[P0 + threadIdx.x] = threadIdx.x;   // row of sh.sact
            if (!FUSED) s_w[P0 + threadIdx.x] = sh.sgate[threadIdx.x];   // FUSED: read after the wait
        }
    }
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, tl = lane & 15;
    const int sl = wave * 4 + (lane >> 4);
    const int r0 = bx * kDownRows;
    const int nitems = nd * kDownRows;
    constexpr int kSlots = 4 * NW, kStep = kSlots * kDownBatch;
    const DownItems it{e.down_codes, e.down_scales, sh.dcodes, sh.dscales, s_ex, nitems, r0, H, I, sl, tl};
    // two register batches of weights, both issued before the activation
    // image is complete; from then on the loads of one batch are in flight
    // while the other is computed
    uint4 ca[kDownBatch][CPL], cb[kDownBatch][CPL];
    uint32_t sa[kDownBatch][CPL], sb[kDownBatch][CPL];
    if constexpr (FUSED) {
        // the weights first: they stream while gate/up still runs
        down_rows_load<CPL>(it, 0, kSlots, ca, sa);
        down_rows_load<CPL>(it, kStep, kSlots, cb, sb);   // always (past the end: valid rows, unused)
        __builtin_amdgcn_sched_barrier(0);
        if (threadIdx.x < nr) s_dec[threadIdx.x] = s_decv;   // read at the sums, after the staging barrier
        trace_mark<TRACE>(sh.trace, 1);
        if (threadIdx.x == 0) {
            // one release per routed expert column; the count is advanced
            // whether or not the wait succeeds, so a late release of this
            // call cannot satisfy the next one
            unsigned int *go = done + kSyncWords + kGoStride * bx;
            const unsigned int c = ld_dev(go + 1);
            const unsigned int want = c + (unsigned int)nr * kGoTag;
            st_dev(go + 1, want);
            unsigned int g = ld_dev(go);
            int bad = 0;
            if ((g - c) * kGoTagInv > (unsigned int)nr) {   // not c plus up to nr releases
                bad = (int)kMoeStatusCorrupt;
            } else {
                int n = 0;
                while (g != want && n < kSpinLimit) {
                    __builtin_amdgcn_s_sleep(2);
                    g = ld_dev(go);
                    ++n;
                }
                if (g != want) bad = (int)kMoeStatusTimeout;
            }
            if (bad)
                __hip_atomic_fetch_or(status, (unsigned int)bad, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            s_late = bad;
        }
        __syncthreads();
        trace_mark<TRACE>(sh.trace, 2);
        if (s_late) {
            for (int i = threadIdx.x; i < m * kDownRows; i += blockDim.x) {
                const int row = r0 + i % kDownRows;
                if (row < H) y[(size_t)(i / kDownRows) * H + row] = __builtin_nanf("");
            }
            return;
        }
        if (sh.on && threadIdx.x < m) s_w[P0 + threadIdx.x] = ld_dev(&sh.sgate[threadIdx.x]);
        stage_rows_dev(smem, act, (size_t)m * topk, s_pair, P0, P0, I);
        if (sh.on) stage_rows_dev(smem + (size_t)P0 * 4 * C, sh.sact, (size_t)m, s_pair + P0, m, m, I);
    } else {
        // the activation loads went out with the plan's, before the weights,
        // so that waiting for them does not wait for the weights
        down_rows_load<CPL>(it, 0, kSlots, ca, sa);
        down_rows_load<CPL>(it, kStep, kSlots, cb, sb);   // always (past the end: valid rows, unused)
        __builtin_amdgcn_sched_barrier(0);
        stage_rows_rest(smem, av, act, nullptr, P0, I);   // image row u = pair u
        if (sh.on) stage_rows(smem + (size_t)P0 * 4 * C, sh.sact, s_pair + P0, m, m, I);
    }
    __syncthreads();
    if (FUSED) trace_mark<TRACE>(sh.trace, 3);
    if (FUSED && CPL <= 2 && P == nd && nitems <= 2 * kStep) {
        // one position per expert (position u is expert u's); the separate
        // pass has four times the wavefronts to overlap its items instead,
        // and neither it nor wider rows have the registers
        down_rows_fma_one<CPL>(it, 0, kSlots, ca, sa, s_dec, smem, C, contrib);
        if (kStep < nitems) down_rows_fma_one<CPL>(it, kStep, kSlots, cb, sb, s_dec, smem, C, contrib);
    } else {
        for (int b0 = 0; b0 < nitems; b0 += 2 * kStep) {
            down_rows_fma<CPL>(it, b0, kSlots, ca, sa, s_pb, s_dec, smem, C, contrib, FUSED ? nullptr : s_img);
            if (b0 + 2 * kStep < nitems) down_rows_load<CPL>(it, b0 + 2 * kStep, kSlots, ca, sa);
            __builtin_amdgcn_sched_barrier(0);
            if (b0 + kStep >= nitems) break;
            down_rows_fma<CPL>(it, b0 + kStep, kSlots, cb, sb, s_pb, s_dec, smem, C, contrib, FUSED ? nullptr : s_img);
            if (b0 + 3 * kStep < nitems) down_rows_load<CPL>(it, b0 + 3 * kStep, kSlots, cb, sb);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    if (FUSED) trace_mark<TRACE>(sh.trace, 4);
    __syncthreads();
    // y[t][row] = sum over token t's pairs, in ascending expert order, of
    // w * d: one thread per (token, row); the positions are read four at a
    // time so the LDS reads overlap
    const int i = threadIdx.x;
    if (i < m * kDownRows) {
        const int t = i / kDownRows, r = i % kDownRows, row = r0 + r;
        float acc = 0.0f;
        int pos = 0;
        for (; pos + 4 <= P; pos += 4) {
            int tk[4];
            float wv[4], cv[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                tk[q] = s_tok[pos + q];
                wv[q] = s_w[pos + q];
                cv[q] = contrib[pos + q][r];
            }
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (tk[q] == t) acc = __builtin_fmaf(wv[q], cv[q], acc);
        }
        for (; pos < P; ++pos)
            if (s_tok[pos] == t) acc = __builtin_fmaf(s_w[pos], contrib[pos][r], acc);
        if (row < H) y[(size_t)t * H + row] = acc;
    }
    if (FUSED) trace_mark<TRACE>(sh.trace, 5);
}

// The separate row-owner down pass: 16 wavefronts (64 slots) per
// workgroup, so that a CU keeps 64 items (expert, row) of weights in flight
// (8 wavefronts for four chunks a lane, whose registers would not fit 16).
template <int CPL>
constexpr int down_rows_waves() { return CPL >= 4 ? 8 : 16; }
template <int CPL>
__global__ __launch_bounds__(64 * down_rows_waves<CPL>()) void k_moe_down_rows(nvfp4_moe_weights e, int m, int topk,
                                                                      const float *__restrict__ wts,
                                                                      const MoeRoute *__restrict__ route,
                                                                      const uint16_t *__restrict__ act,
                                                                      float *__restrict__ y, MoeShared sh) {
    extern __shared__ uint4 smem[];
    down_rows_role<CPL, false, down_rows_waves<CPL>()>(smem, blockIdx.x, e, m, topk, route, nullptr, 0, 0, act, y, sh,
                                                       nullptr, nullptr);
}

// Gate/up and the row-owner down pass in one launch: workgroups [0, g1) are
// the gate/up tiles (gx per expert column), the rest own kDownRows output
// rows each.  The down workgroups come after every gate/up workgroup in
// dispatch order, so the ones they wait for are already running.
template <int CPLG, int CPLD, bool TRACE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(CPLD <= 2 ? 3 : 1))) void k_moe_fused(const uint16_t *__restrict__ x, const float *__restrict__ logits,
                                                  int m, int E, int topk, nvfp4_moe_weights e,
                                                  int32_t *__restrict__ ids, float *__restrict__ wts,
                                                  uint16_t *__restrict__ act, float *__restrict__ y, MoeShared sh,
                                                  unsigned int *__restrict__ counters, unsigned int *status, int gx,
                                                  int g1) {
    extern __shared__ uint4 smem[];
    const int b = blockIdx.x;
    if (b < g1)
        gate_up_role<CPLG, true, TRACE>(smem, b % gx, b / gx, gx, x, logits, m, E, topk, e, ids, wts, nullptr, act,
                                        sh, counters, (int)gridDim.x - g1);
    else
        down_rows_role<CPLD, true, 4, TRACE>(smem, b - g1, e, m, topk, nullptr, logits, E, gx, act, y, sh, counters,
                                             status, ids, wts);
}

template <int CPL>
static int launch_down_rows(dim3 g, size_t lds, hipStream_t s, const nvfp4_moe_weights &e, int m, int topk,
                            const float *wts, const MoeRoute *route, const uint16_t *act, float *y,
                            const MoeShared &sh) {
    const int rc = allow_lds(reinterpret_cast<const void *>(k_moe_down_rows<CPL>), lds, "moe_w4a16_gemv");
    if (rc) return rc;
    hipLaunchKernelGGL(k_moe_down_rows<CPL>, g, dim3(64 * down_rows_waves<CPL>()), lds, s, e, m, topk, wts, route, act,
                       y, sh);
    return check_launch("moe_w4a16_gemv(down)");
}

struct MoeLayout {
    size_t tickets, sync, act, dbuf, total;
};
static MoeLayout moe_layout(int m, int topk, int H, int I) {
    MoeLayout L;
    const size_t pairs = (size_t)m * topk;
    L.tickets = kMoeHeader;
    L.sync = L.tickets + (((size_t)(H + kMoeRows - 1) / kMoeRows * 4 + 255) & ~(size_t)255);
    L.act = L.sync + (((size_t)kSyncWords * 4 + (size_t)(H + kDownRows - 1) / kDownRows * kGoStride * 4 + 255) & ~(size_t)255);
    L.dbuf = L.act + ((pairs * I * 2 + 255) & ~(size_t)255);
    L.total = L.dbuf + pairs * H * 4;
    return L;
}


template <int CPL>
static int launch_gate_up(dim3 g, size_t lds, hipStream_t s, const uint16_t *x, const float *logits, int m, int E,
                          int topk, const nvfp4_moe_weights &e, int32_t *ids, float *wts, MoeRoute *route,
                          uint16_t *act, const MoeShared &sh) {
    const int gx = (int)g.x;   // row tiles of a pair
    if constexpr (CPL > 0) {
        // more workgroups than one round holds: fewer, each over several
        // tiles of its pair, as evenly as the round allows (one routing and
        // one activation staging for all of them).  256 experts of 2048 x
        // 1024, top-8: 4 and 8 tokens 33.1 / 55.6 -> 29.2 / 46.3 us; an even
        // share of tiles at 3 tokens 26.2 -> 24.6 us.
        const void *km = reinterpret_cast<const void *>(k_moe_gate_up<CPL, true>);
        const long most = (long)num_cus() * blocks_per_cu(km, 256, lds) / (long)g.y;   // one round
        const long t = most >= 1 ? (gx + most - 1) / most : 0;                        // tiles a workgroup
        const long per_pair = t >= 1 ? (gx + t - 1) / t : 0;   // so that each takes t or t - 1 tiles
        if (!sh.on && t > 1) {
            const int rc = allow_lds(km, lds, "moe_w4a16_gemv");
            if (rc) return rc;
            hipLaunchKernelGGL((k_moe_gate_up<CPL, true>), dim3((unsigned)per_pair, g.y), dim3(256), lds, s, x, logits,
                               m, E, topk, e, ids, wts, route, act, sh, gx);
            return check_launch("moe_w4a16_gemv(gate_up)");
        }
    }
    const int rc = allow_lds(reinterpret_cast<const void *>(k_moe_gate_up<CPL, false>), lds, "moe_w4a16_gemv");
    if (rc) return rc;
    hipLaunchKernelGGL((k_moe_gate_up<CPL, false>), g, dim3(256), lds, s, x, logits, m, E, topk, e, ids, wts, route, act,
                       sh, gx);
    return check_launch("moe_w4a16_gemv(gate_up)");
}
template <int CPL>
static int launch_down(dim3 g, size_t lds, hipStream_t s, const nvfp4_moe_weights &e, int m, int topk, const float *wts,
                       const MoeRoute *route, const uint16_t *act, float *dbuf, unsigned int *tickets, float *y) {
    const int rc = allow_lds(reinterpret_cast<const void *>(k_moe_down<CPL>), lds, "moe_w4a16_gemv");
    if (rc) return rc;
    hipLaunchKernelGGL(k_moe_down<CPL>, g, dim3(256), lds, s, e, m, topk, wts, route, act, dbuf, tickets, y);
    return check_launch("moe_w4a16_gemv(down)");
}

constexpr int kNotResident = 1;   // launch_fused: the grid does not fit at once (nothing launched)

template <int CPLG, int CPLD, bool TRACE>
static int launch_fused_t(int grid, size_t lds, hipStream_t s, const uint16_t *x, const float *logits, int m, int E,
                          int topk, const nvfp4_moe_weights &e, int32_t *ids, float *wts, uint16_t *act, float *y,
                          const MoeShared &sh, unsigned int *counters, unsigned int *status, int gx, int g1) {
    const void *kern = reinterpret_cast<const void *>(k_moe_fused<CPLG, CPLD, TRACE>);
    const int rc = allow_lds(kern, lds, "moe_w4a16_gemv");
    if (rc) return rc;
    // the down workgroups only overlap the gate/up pass when every workgroup
    // of the launch is resident at once
    if (grid > num_cus() * blocks_per_cu(kern, 256, lds)) return kNotResident;
    hipLaunchKernelGGL((k_moe_fused<CPLG, CPLD, TRACE>), dim3(grid), dim3(256), lds, s, x, logits, m, E, topk, e, ids, wts, act,
                       y, sh, counters, status, gx, g1);
    return check_launch("moe_w4a16_gemv");
}
template <int CPLG, bool TRACE>
static int launch_fused_g(int cpld, int grid, size_t lds, hipStream_t s, const uint16_t *x, const float *logits, int m,
                          int E, int topk, const nvfp4_moe_weights &e, int32_t *ids, float *wts, uint16_t *act,
                          float *y, const MoeShared &sh, unsigned int *counters, unsigned int *status, int gx,
                          int g1) {
    switch (cpld) {
        case 1: return launch_fused_t<CPLG, 1, TRACE>(grid, lds, s, x, logits, m, E, topk, e, ids, wts, act, y, sh, counters, status, gx, g1);
        case 2: return launch_fused_t<CPLG, 2, TRACE>(grid, lds, s, x, logits, m, E, topk, e, ids, wts, act, y, sh, counters, status, gx, g1);
        default: return launch_fused_t<CPLG, 4, TRACE>(grid, lds, s, x, logits, m, E, topk, e, ids, wts, act, y, sh, counters, status, gx, g1);
    }
}
template <bool TRACE>
static int launch_fused_c(int cplg, int cpld, int grid, size_t lds, hipStream_t s, const uint16_t *x,
                          const float *logits, int m, int E, int topk, const nvfp4_moe_weights &e, int32_t *ids,
                          float *wts, uint16_t *act, float *y, const MoeShared &sh, unsigned int *counters,
                          unsigned int *status, int gx, int g1) {
    switch (cplg) {
        case 1: return launch_fused_g<1, TRACE>(cpld, grid, lds, s, x, logits, m, E, topk, e, ids, wts, act, y, sh, counters, status, gx, g1);
        case 2: return launch_fused_g<2, TRACE>(cpld, grid, lds, s, x, logits, m, E, topk, e, ids, wts, act, y, sh, counters, status, gx, g1);
        case 4: return launch_fused_g<4, TRACE>(cpld, grid, lds, s, x, logits, m, E, topk, e, ids, wts, act, y, sh, counters, status, gx, g1);
        default: return launch_fused_g<0, TRACE>(cpld, grid, lds, s, x, logits, m, E, topk, e, ids, wts, act, y, sh, counters, status, gx, g1);
    }
}
// The traced instantiation when sh.trace is set (moe_w4a16_gemv_trace).
static int launch_fused(int cplg, int cpld, int grid, size_t lds, hipStream_t s, const uint16_t *x, const float *logits,
                        int m, int E, int topk, const nvfp4_moe_weights &e, int32_t *ids, float *wts, uint16_t *act,
                        float *y, const MoeShared &sh, unsigned int *counters, unsigned int *status, int gx,
                        int g1) {
    if (sh.trace != nullptr)
        return launch_fused_c<true>(cplg, cpld, grid, lds, s, x, logits, m, E, topk, e, ids, wts, act, y, sh, counters,
                                    status, gx, g1);
    return launch_fused_c<false>(cplg, cpld, grid, lds, s, x, logits, m, E, topk, e, ids, wts, act, y, sh, counters,
                                 status, gx, g1);
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

// Checks shared by the routed MoE and the complete layer.
static int moe_validate(const uint16_t *x_bf16, int32_t m, int32_t top_k, const nvfp4_moe_weights *e, const float *y,
                        const int32_t *topk_ids, const float *topk_w, const char *who) {
    if (!e) return fail(NVFP4_ERR_ARG, "%s: NULL expert descriptor", who);
    if (!x_bf16 || !y || !topk_ids || !topk_w) return fail(NVFP4_ERR_ARG, "%s: NULL x/y/topk_ids/topk_w", who);
    if (!e->gate_codes || !e->gate_scales || !e->gate_global || !e->up_codes || !e->up_scales || !e->up_global ||
        !e->down_codes || !e->down_scales || !e->down_global)
        return fail(NVFP4_ERR_ARG, "%s: NULL expert weight pointer", who);
    if (m < 1 || m > 8) return fail(NVFP4_ERR_SHAPE, "%s: m=%d outside 1..8", who, m);
    const int E = e->num_experts, H = e->hidden, I = e->inter;
    if (E < 1 || E > kMoeMaxExperts) return fail(NVFP4_ERR_SHAPE, "%s: num_experts=%d outside 1..%d", who, E, kMoeMaxExperts);
    if (top_k < 1 || top_k > kMoeMaxTopK || top_k > E)
        return fail(NVFP4_ERR_SHAPE, "%s: top_k=%d outside 1..min(E, %d)", who, top_k, kMoeMaxTopK);
    if (H < 32 || I < 32 || H % 32 || I % 32) return fail(NVFP4_ERR_SHAPE, "%s: hidden/inter must be multiples of 32", who);
    // an expert serves at most m tokens: its activation rows are staged for
    // round_up(m) of them (up to 160 KiB of LDS per workgroup)
    const int mt = round_up_mt(m);
    if ((size_t)mt * H * 2 > kMoeMaxLds || (size_t)mt * I * 2 > kMoeMaxLds)
        return fail(NVFP4_ERR_UNSUPPORTED, "%s: %d rows x hidden %d / inter %d exceed the LDS", who, mt, H, I);
    if (!aligned(x_bf16, 16) || !aligned(e->gate_codes, 16) || !aligned(e->up_codes, 16) || !aligned(e->down_codes, 16))
        return fail(NVFP4_ERR_ALIGN, "%s: x and codes need 16-byte alignment", who);
    if (!aligned(e->gate_scales, 2) || !aligned(e->up_scales, 2) || !aligned(e->down_scales, 2) || !aligned(y, 4) ||
        !aligned(topk_ids, 4) || !aligned(topk_w, 4))
        return fail(NVFP4_ERR_ALIGN, "%s: scales 2-byte, outputs 4-byte alignment", who);
    return NVFP4_OK;
}

// Routing + gate/up, then the down pass (row-owner when the activation rows
// fit in LDS -- always with a shared expert -- else the ticket pass).
static int moe_launch(const uint16_t *x_bf16, int32_t m, const float *router_logits, int32_t top_k,
                      const nvfp4_moe_weights *e, float *y, int32_t *topk_ids, float *topk_w, char *ws,
                      const MoeLayout &L, const MoeShared &sh, hipStream_t s) {
    MoeRoute *route = reinterpret_cast<MoeRoute *>(ws);
    unsigned int *tickets = reinterpret_cast<unsigned int *>(ws + L.tickets);
    uint16_t *act = reinterpret_cast<uint16_t *>(ws + L.act);
    float *dbuf = reinterpret_cast<float *>(ws + L.dbuf);
    const int E = e->num_experts, H = e->hidden, I = e->inter, mt = round_up_mt(m);
    const int maxd = min(E, m * top_k);
    const nvfp4_moe_weights ev = *e;
    // gate/up: one column per (token, slot) pair; down (ticket pass): one per distinct expert
    const dim3 g1((I + kMoeRows - 1) / kMoeRows, m * top_k), g2((H + kDownTile - 1) / kDownTile, maxd);
    // gate/up: one token's activation row (or the routing scratch of
    // workgroup (0, 0)); the ticket down pass: an expert's rows of up to m tokens
    const size_t lds1 = std::max((size_t)H * 2, sizeof(RouteLds)), lds2 = (size_t)mt * I * 2;
    const size_t pos = (size_t)m * top_k + (sh.on ? m : 0);
    // the row-owner pass keeps about 8 KiB of static LDS next to the
    // activation rows of every pair; with 16 wavefronts a workgroup it beats
    // the ticket pass at every token count (at 8 tokens 20.8 against 24.4 us)
    const size_t lds_limit = (size_t)160 * 1024 - 10240;
    const bool row_owner = pos <= (size_t)kDownMaxPos && pos * I * 2 <= lds_limit && cpl_for(I) != 0;
    if (row_owner && m == 1) {
        // one launch: gate/up workgroups, then the row-owner down workgroups
        const int gx = (int)g1.x, ng1 = gx * (int)g1.y, ng3 = (H + kDownRows - 1) / kDownRows;
        const size_t lds = std::max(lds1, pos * I * 2);
        const int frc = launch_fused(cpl_for(H), cpl_for(I), ng1 + ng3, lds, s, x_bf16, router_logits, m, E, top_k,
                                     ev, topk_ids, topk_w, act, y, sh, reinterpret_cast<unsigned int *>(ws + L.sync),
                                     reinterpret_cast<unsigned int *>(ws + kMoeStatusOffset), gx, ng1);
        if (frc != kNotResident) return frc;
    }
    if (sh.trace != nullptr)
        return fail(NVFP4_ERR_UNSUPPORTED, "moe_w4a16_gemv_trace: the call does not take the one-launch form (one "
                    "token, every activation row in LDS, the whole grid resident)");
    int rc;
    switch (cpl_for(H)) {
        case 1: rc = launch_gate_up<1>(g1, lds1, s, x_bf16, router_logits, m, E, top_k, ev, topk_ids, topk_w, route, act, sh); break;
        case 2: rc = launch_gate_up<2>(g1, lds1, s, x_bf16, router_logits, m, E, top_k, ev, topk_ids, topk_w, route, act, sh); break;
        case 4: rc = launch_gate_up<4>(g1, lds1, s, x_bf16, router_logits, m, E, top_k, ev, topk_ids, topk_w, route, act, sh); break;
        default: rc = launch_gate_up<0>(g1, lds1, s, x_bf16, router_logits, m, E, top_k, ev, topk_ids, topk_w, route, act, sh); break;
    }
    if (rc) return rc;
    if (row_owner) {
        const dim3 g3((H + kDownRows - 1) / kDownRows);
        const size_t lds3 = pos * I * 2;
        switch (cpl_for(I)) {
            case 1: return launch_down_rows<1>(g3, lds3, s, ev, m, top_k, topk_w, route, act, y, sh);
            case 2: return launch_down_rows<2>(g3, lds3, s, ev, m, top_k, topk_w, route, act, y, sh);
            default: return launch_down_rows<4>(g3, lds3, s, ev, m, top_k, topk_w, route, act, y, sh);
        }
    }
    if (sh.on) return fail(NVFP4_ERR_UNSUPPORTED, "moe_layer_w4a16: %zu activation rows of inter %d exceed the LDS", pos, I);
    switch (cpl_for(I)) {
        case 1: return launch_down<1>(g2, lds2, s, ev, m, top_k, topk_w, route, act, dbuf, tickets, y);
        case 2: return launch_down<2>(g2, lds2, s, ev, m, top_k, topk_w, route, act, dbuf, tickets, y);
        case 4: return launch_down<4>(g2, lds2, s, ev, m, top_k, topk_w, route, act, dbuf, tickets, y);
        default: return launch_down<0>(g2, lds2, s, ev, m, top_k, topk_w, route, act, dbuf, tickets, y);
    }
}

extern "C" int moe_w4a16_gemv(const uint16_t *x_bf16, int32_t m, const float *router_logits, int32_t top_k,
                              const nvfp4_moe_weights *e, float *y, int32_t *topk_ids, float *topk_w, void *workspace,
                              size_t ws_bytes, void *stream) {
    int rc = moe_validate(x_bf16, m, top_k, e, y, topk_ids, topk_w, "moe_w4a16_gemv");
    if (rc) return rc;
    if (!router_logits) return fail(NVFP4_ERR_ARG, "moe_w4a16_gemv: NULL router_logits");
    if (!aligned(router_logits, 4)) return fail(NVFP4_ERR_ALIGN, "moe_w4a16_gemv: router_logits not 4-byte aligned");
    const MoeLayout L = moe_layout(m, top_k, e->hidden, e->inter);
    if (!workspace || ws_bytes < L.total)
        return fail(NVFP4_ERR_WORKSPACE, "moe_w4a16_gemv: workspace needs %zu bytes", L.total);
    if (!aligned(workspace, 256)) return fail(NVFP4_ERR_ALIGN, "moe_w4a16_gemv: workspace not 256-byte aligned");
    return moe_launch(x_bf16, m, router_logits, top_k, e, y, topk_ids, topk_w, reinterpret_cast<char *>(workspace), L,
                      MoeShared{}, reinterpret_cast<hipStream_t>(stream));
}

// The one-launch form's grid: gate/up tiles per pair, then the down workgroups.
static size_t moe_trace_grid(int m, int top_k, const nvfp4_moe_weights *e) {
    return (size_t)(e->inter + kMoeRows - 1) / kMoeRows * m * top_k + (e->hidden + kDownRows - 1) / kDownRows;
}

extern "C" size_t moe_w4a16_gemv_trace_words(int32_t m, int32_t top_k, const nvfp4_moe_weights *e) {
    if (!e || m != 1 || top_k < 1 || e->hidden < 1 || e->inter < 1) return 0;
    return (size_t)kTraceEvents * moe_trace_grid(m, top_k, e);
}

extern "C" int moe_w4a16_gemv_trace(const uint16_t *x_bf16, int32_t m, const float *router_logits, int32_t top_k,
                                    const nvfp4_moe_weights *e, float *y, int32_t *topk_ids, float *topk_w,
                                    void *workspace, size_t ws_bytes, uint64_t *trace, size_t trace_words,
                                    void *stream) {
    const char *who = "moe_w4a16_gemv_trace";
    int rc = moe_validate(x_bf16, m, top_k, e, y, topk_ids, topk_w, who);
    if (rc) return rc;
    if (m != 1) return fail(NVFP4_ERR_UNSUPPORTED, "%s: m=%d; the one-launch form serves one token", who, m);
    if (!router_logits || !aligned(router_logits, 4))
        return fail(NVFP4_ERR_ARG, "%s: router_logits must be a 4-byte aligned device buffer", who);
    if (!trace || !aligned(trace, 8)) return fail(NVFP4_ERR_ARG, "%s: trace must be an 8-byte aligned device buffer", who);
    if (trace_words < moe_w4a16_gemv_trace_words(m, top_k, e))
        return fail(NVFP4_ERR_WORKSPACE, "%s: trace needs %zu words", who, moe_w4a16_gemv_trace_words(m, top_k, e));
    const MoeLayout L = moe_layout(m, top_k, e->hidden, e->inter);
    if (!workspace || ws_bytes < L.total) return fail(NVFP4_ERR_WORKSPACE, "%s: workspace needs %zu bytes", who, L.total);
    if (!aligned(workspace, 256)) return fail(NVFP4_ERR_ALIGN, "%s: workspace not 256-byte aligned", who);
    MoeShared sh{};
    sh.trace = reinterpret_cast<unsigned long long *>(trace);
    return moe_launch(x_bf16, m, router_logits, top_k, e, y, topk_ids, topk_w, reinterpret_cast<char *>(workspace), L,
                      sh, reinterpret_cast<hipStream_t>(stream));
}

extern "C" int moe_workspace_status(void *workspace, size_t ws_bytes, uint32_t *status, void *stream) {
    const char *who = "moe_workspace_status";
    if (!workspace || !status) return fail(NVFP4_ERR_ARG, "%s: NULL workspace or status", who);
    if (ws_bytes < (size_t)kMoeHeader) return fail(NVFP4_ERR_WORKSPACE, "%s: not a MoE workspace (%zu bytes)", who, ws_bytes);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) == hipSuccess && cs != hipStreamCaptureStatusNone)
        return fail(NVFP4_ERR_UNSUPPORTED, "%s: synchronizes the stream; not allowed during graph capture", who);
    char *word = reinterpret_cast<char *>(workspace) + kMoeStatusOffset;
    uint32_t v = 0, zero = 0;
    hipError_t err = hipMemcpyAsync(&v, word, 4, hipMemcpyDeviceToHost, s);
    if (err == hipSuccess) err = hipStreamSynchronize(s);
    if (err == hipSuccess && v != 0) {
        err = hipMemcpyAsync(word, &zero, 4, hipMemcpyHostToDevice, s);
        if (err == hipSuccess) err = hipStreamSynchronize(s);
    }
    if (err != hipSuccess) return fail(NVFP4_ERR_HIP, "%s: %s", who, hipGetErrorString(err));
    *status = v;
    if (v & kMoeStatusCorrupt)
        return fail(NVFP4_ERR_DEVICE, "%s: a down pass found its hand-off word overwritten (status 0x%x); zero the "
                    "workspace before the next call", who, v);
    if (v) return fail(NVFP4_ERR_DEVICE, "%s: a down pass gave up waiting for its gate/up pass (status 0x%x)", who, v);
    return ok();
}

// Workspace of the complete layer: the routed MoE's, then the shared
// expert's gate and up outputs (fp32), its activations (bf16) and the gate
// values (fp32), each 256-byte aligned.
struct LayerLayout {
    MoeLayout moe;
    size_t sg, su, sact, sgate, total;
};
static LayerLayout layer_layout(int m, int topk, int H, int I) {
    LayerLayout L;
    L.moe = moe_layout(m, topk, H, I);
    auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
    L.sg = up(L.moe.total);
    L.su = L.sg + up((size_t)m * I * 4);
    L.sact = L.su + up((size_t)m * I * 4);
    L.sgate = L.sact + up((size_t)m * I * 2);
    L.total = L.sgate + 256;
    return L;
}

extern "C" size_t moe_layer_w4a16_workspace_bytes(int32_t m, int32_t top_k, const nvfp4_moe_weights *e) {
    if (!e || m < 1 || top_k < 1 || e->hidden < 1 || e->inter < 1) return 0;
    return layer_layout(m, top_k, e->hidden, e->inter).total;
}

extern "C" int moe_layer_w4a16(const uint16_t *x_bf16, int32_t m, const nvfp4_weight *router, int32_t top_k,
                               const nvfp4_moe_weights *e, const nvfp4_weight *shared_gate,
                               const nvfp4_weight *shared_up, const nvfp4_weight *shared_down,
                               const uint16_t *shared_gate_w_bf16, float *y, int32_t *topk_ids, float *topk_w,
                               float *router_logits, void *workspace, size_t ws_bytes, void *stream) {
    const char *who = "moe_layer_w4a16";
    int rc = moe_validate(x_bf16, m, top_k, e, y, topk_ids, topk_w, who);
    if (rc) return rc;
    const int E = e->num_experts, H = e->hidden, I = e->inter;
    for (const nvfp4_weight *w : {router, shared_gate, shared_up, shared_down}) {
        rc = validate_weight(w, who);
        if (rc) return rc;
    }
    if (router->n != E || router->k != H)
        return fail(NVFP4_ERR_SHAPE, "%s: router is %dx%d, need %dx%d", who, router->n, router->k, E, H);
    if (shared_gate->n != I || shared_gate->k != H || shared_up->n != I || shared_up->k != H || shared_down->n != H ||
        shared_down->k != I)
        return fail(NVFP4_ERR_SHAPE, "%s: the shared expert must be gate/up %dx%d and down %dx%d", who, I, H, H, I);
    if (!router_logits || !aligned(router_logits, 4))
        return fail(NVFP4_ERR_ARG, "%s: router_logits must be a 4-byte aligned device buffer", who);
    const LayerLayout L = layer_layout(m, top_k, H, I);
    if (!workspace || ws_bytes < L.total) return fail(NVFP4_ERR_WORKSPACE, "%s: workspace needs %zu bytes", who, L.total);
    if (!aligned(workspace, 256)) return fail(NVFP4_ERR_ALIGN, "%s: workspace not 256-byte aligned", who);
    char *ws = reinterpret_cast<char *>(workspace);
    float *sg = reinterpret_cast<float *>(ws + L.sg), *su = reinterpret_cast<float *>(ws + L.su);
    // 1. router logits and the shared expert's gate and up: one grouped GEMV
    const nvfp4_weight *ws3[3] = {router, shared_gate, shared_up};
    void *ys3[3] = {router_logits, sg, su};
    rc = w4a16_gemv_grouped(x_bf16, m, ws3, ys3, 3, NVFP4_OUT_F32, stream);
    if (rc) return rc;
    // 2-3. routed experts with the shared expert folded into the down pass
    MoeShared sh{};
    sh.sg = sg;
    sh.su = su;
    sh.sact = reinterpret_cast<uint16_t *>(ws + L.sact);
    sh.gate_w = shared_gate_w_bf16;
    sh.sgate = reinterpret_cast<float *>(ws + L.sgate);
    sh.dcodes = shared_down->codes;
    sh.dscales = shared_down->scales;
    sh.dglob = shared_down->global;
    sh.on = 1;
    return moe_launch(x_bf16, m, router_logits, top_k, e, y, topk_ids, topk_w, ws, L.moe, sh,
                      reinterpret_cast<hipStream_t>(stream));
}
