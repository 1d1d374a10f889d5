// W4A16 decode GEMV and the LM-head GEMV fused with argmax.
//
// w4a16_gemv: the projection GEMV of mtp_head.rs (`MtpHead::gemv` ->
// `w4a16_decode_gemv`) for M = 1..8 rows, used for the head's fc and q/k/v/o
// projections (new.rs, `MtpHead::new` quantizes exactly these).
//
// lmhead_gemv_argmax: the NVFP4 LM head over the first V vocabulary rows and
// the argmax that turns it into the draft token (new.rs resolves the NVFP4
// LM head and `argmax_bf16`; deepseek_v4_mtp.rs `forward_one` runs LM head
// then argmax, with the reduced vocabulary).  One launch: each workgroup
// scores one tile of rows and writes, per activation row, the best (key,
// index) of its tile; the last workgroup to finish (a ticket counter in the
// workspace, returned to zero afterwards) combines the partials.  No logits
// tensor is written.  The combine keeps the larger key and, on equal keys,
// the lower index -- exactly the ascending strict-greater scan of
// `argmax_grammar_masked`, independent of the order workgroups finish in.
#include <float.h>

#include <mutex>

#include "gemv_core.hpp"

namespace nvfp4 {

// Up to kMaxGroups weights that share K and the activations, scored in one
// launch: the grid is the concatenation of every group's row tiles (tile0
// holds the prefix sums) and each workgroup picks its group by comparing its
// tile index with tile0.  One group is the plain GEMV.
constexpr int kMaxGroups = 8;
struct GemvGroups {
    const uint8_t *codes[kMaxGroups];
    const uint8_t *scales[kMaxGroups];
    const nvfp4_global *g[kMaxGroups];
    void *y[kMaxGroups];
    int n[kMaxGroups];
    int tile0[kMaxGroups + 1];
    int count;
};

// Chunks per lane per pipelined stage of the generic loop (R rows share it).
constexpr int kGemvPipe = 4;
template <int R>
constexpr int gemv_pipe() { return R >= kGemvPipe ? 1 : kGemvPipe / R; }

template <int MT, int R, int KS, int CPL, int NW = 4, bool XG = false>
__global__ __launch_bounds__(64 * NW) void k_gemv(const XRows x, int m_rt, const GemvGroups grp, int k,
                                             int bf16out) {
    extern __shared__ uint4 smem[];
    uint4 *xs = smem;
    float *red = reinterpret_cast<float *>(smem + (MT * k) / 8);
    constexpr int rows = GemvTile<R, KS, NW>::kRowsPerTile;
    // group of this workgroup: selects with constant indices keep the table
    // in scalar registers (a dynamic index would copy it to private memory)
    const int tile = blockIdx.x;
    const uint8_t *codes = grp.codes[0];
    const uint8_t *scales = grp.scales[0];
    const nvfp4_global *g = grp.g[0];
    void *y = grp.y[0];
    int n = grp.n[0], t0 = 0;
#pragma unroll
    for (int i = 1; i < kMaxGroups; ++i) {
        if (i < grp.count && tile >= grp.tile0[i]) {
            codes = grp.codes[i];
            scales = grp.scales[i];
            g = grp.g[i];
            y = grp.y[i];
            n = grp.n[i];
            t0 = grp.tile0[i];
        }
    }
    const int row0 = (tile - t0) * rows;
    const float dec = g->dec;
    auto epi = [&](int row, int mm, float v) {
        if (mm >= m_rt) return;
        const float o = v * dec;
        if (bf16out)
            reinterpret_cast<uint16_t *>(y)[(size_t)mm * n + row] = (uint16_t)f32_to_bf16_bits(o);
        else
            reinterpret_cast<float *>(y)[(size_t)mm * n + row] = o;
    };
    // gathered rows: their table rows first (the row addresses wait for them)
    int lid = 0;
    if constexpr (XG) lid = xids_issue(x, m_rt);
    if constexpr (MT == 1 && CPL > 0) {
        TileRegs<MT, R, KS, CPL> t;
        gemv_tile_load(t, codes, scales, n, k, row0);
        XRegs<CPL> xr;
        load_xregs<KS, CPL, XG>(xr, x, k, lid);
        gemv_tile_compute_x1(t, xr, n, row0, red, epi);
    } else if constexpr (CPL > 0) {
        TileRegs<MT, R, KS, CPL> t;
        gemv_tile_load(t, codes, scales, n, k, row0);   // weight loads in flight while x is staged
        stage_x<MT, XG>(xs, x, m_rt, k, lid);
        __syncthreads();
        gemv_tile_compute(t, xs, n, k, row0, red, epi);
    } else {
        stage_x<MT, XG>(xs, x, m_rt, k, lid);
        __syncthreads();
        gemv_tile_loop<MT, R, KS, gemv_pipe<R>(), false, (NW > 4)>(xs, codes, scales, n, k, row0, red, epi);
    }
}

struct ArgPart {
    float key;    // compared value (fp32 logit or its bf16 rounding)
    float val;    // fp32 logit of that row
    int idx;
    float lm;     // log-sum-exp state of the keys seen: their largest finite
    float ls;     // or +inf key lm, and ls = sum of exp(key - lm) (NaN-sticky)
    int pad[3];
};

// Merges two log-sum-exp states (lm, ls).  -inf keys never enter a state, so
// a state with lm = -inf has ls = 0.
__device__ __forceinline__ void lse_merge(float &lm, float &ls, float om, float os) {
    const float mn = fmaxf(lm, om);
    if (mn == -INFINITY) {
        ls += os;
    } else {
        ls = ls * __expf(lm - mn) + os * __expf(om - mn);
        lm = mn;
    }
}

template <bool LP>
__device__ __forceinline__ void argpart_combine(ArgPart &b, const ArgPart &o) {
    if constexpr (LP) lse_merge(b.lm, b.ls, o.lm, o.ls);
    if (beats(o.key, o.idx, b.key, b.idx)) {
        b.key = o.key;
        b.val = o.val;
        b.idx = o.idx;
    }
}

template <bool LP>
__device__ __forceinline__ void argpart_shfl_combine(ArgPart &b, int off) {
    ArgPart o;
    o.key = __shfl_xor(b.key, off, 64);
    o.val = __shfl_xor(b.val, off, 64);
    o.idx = __shfl_xor(b.idx, off, 64);
    if constexpr (LP) {
        o.lm = __shfl_xor(b.lm, off, 64);
        o.ls = __shfl_xor(b.ls, off, 64);
    }
    argpart_combine<LP>(b, o);
}

// The same combine with the state of the lane OFF places along a 16-lane row
// (DPP row rotate, a VALU operation: a cross-lane shuffle goes through the
// LDS unit and its latency chains through every step).  Rotating by 8, 4, 2
// and 1 leaves every lane of a row with the row's combination; by 8, 4, ...,
// MT the combination of the row's lanes of one class mod MT.
template <bool LP, int OFF>
__device__ __forceinline__ void argpart_row_combine(ArgPart &b) {
    static_assert(OFF >= 1 && OFF < 16, "a rotation inside a 16-lane row");
    constexpr int ctrl = 0x120 + OFF;   // row_ror:OFF
    ArgPart o;
    o.key = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(b.key), ctrl, 0xF, 0xF, false));
    o.val = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(b.val), ctrl, 0xF, 0xF, false));
    o.idx = __builtin_amdgcn_update_dpp(0, b.idx, ctrl, 0xF, 0xF, false);
    if constexpr (LP) {
        o.lm = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(b.lm), ctrl, 0xF, 0xF, false));
        o.ls = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(b.ls), ctrl, 0xF, 0xF, false));
    }
    argpart_combine<LP>(b, o);
}

// Argmax as one unsigned 64-bit word whose order is that of beats(): the
// key's bits made monotone in the upper half (-0 taken as +0, so equal keys
// compare equal), the complemented index in the lower half (a lower index
// wins a tie).  Keys here are never NaN (NaN never beats the initial -inf).
__device__ __forceinline__ unsigned long long pack_best(float key, int idx) {
    const unsigned int kb = __float_as_uint(key == 0.0f ? 0.0f : key);
    const unsigned int ok = (kb & 0x80000000u) ? ~kb : (kb | 0x80000000u);
    return ((unsigned long long)ok << 32) | (unsigned long long)(~(unsigned int)idx);
}
__device__ __forceinline__ float unpack_best_key(unsigned long long p) {
    const unsigned int ok = (unsigned int)(p >> 32);
    return __uint_as_float((ok & 0x80000000u) ? (ok & 0x7FFFFFFFu) : ~ok);
}
__device__ __forceinline__ int unpack_best_idx(unsigned long long p) { return (int)~(unsigned int)p; }

// Workspace layout of lmhead_gemv_argmax.
constexpr int kLmTicket = 0;      // uint32 ticket counter (zero between calls)
constexpr int kLmRow0 = 64;       // fp32[8]: logits of row 0
constexpr int kLmBest = 128;      // uint64[8]: packed best (key, index) per row (zero between calls)
constexpr int kLmFcSpinLimit = 1 << 22;   // polls of the fused fc's wait for the draft id (seconds)
constexpr int kLmFcRows = 2;              // fc rows per wavefront: (NW - 1) G kLmFcRows >= n
constexpr int kLmFcNoFit = 1;             // launch_lm_fc: too many fc rows for the grid (nothing launched)
// uint64: call count (high) and draft id (low) of the fused next fc, on a
// 128-byte line of its own: every waiting workgroup polls it, and on the
// line of the maxima its polls slowed the end chain
constexpr int kLmFcWord = 384;
constexpr int kLmParts = 512;     // ArgPart[grid][MT]

// Optional gather of the selected tokens' embedding rows by the last
// workgroup (the next draft step's input, device-resident): table [vocab][units
// x 16 B], row i written at out + i * stride_units, id_log[i] = index.
// The next draft step's fc, run by the LM head's workgroups once the draft
// id is known (lmhead_gemv_argmax_fc): y[r] = sum_k W[r][k] a[k] with a =
// [table row of the id (kt elements) | rest (k - kt elements)], one
// activation row.  codes == nullptr: none.
struct FcNext {
    const uint8_t *codes, *scales;
    const nvfp4_global *g;
    int n, k;
    const uint16_t *table;   // [vocab][kt] bf16
    int vocab, kt;
    const uint16_t *rest;    // [k - kt] bf16
    void *y;                 // [n] fp32, or bf16 when y_bf16
    int y_bf16;
};

struct EmbedOut {
    const uint4 *table;   // nullptr: no gather
    uint4 *out;
    int32_t *id_log;
    int64_t stride_units;
    int vocab, units;
};
constexpr int kEmbBatch = 16;   // 16-byte loads in flight per lane in the gather

// Wavefronts per LM-head workgroup: one workgroup per CU holding as many
// wavefronts as the kernel's registers leave resident (3 per SIMD up to 170
// VGPRs, 4 up to 128 for the one-row generic loop, 2 up to 256, 1 beyond).
template <int MT, int CPL>
constexpr int lm_waves() {
    return MT == 1 && CPL == 0 ? 16 : MT == 1 ? 8 : MT <= 2 ? 12 : MT == 4 ? 8 : 4;
}

// Rows per slot of an LM-head unit: one activation row takes 4-row units
// (short units keep the wavefronts' end times close together); more rows
// take 8-row units, whose activation reads from LDS serve two rows.
template <int MT>
constexpr int lm_rows_per_slot() {
    return MT == 1 ? 1 : 2;
}

// Wavefronts per workgroup of the MFMA units (M >= 2, K % 128 == 0), and
// whether those units are used.
constexpr int kLmMfWaves = 8;
constexpr int kLmMfDepth = 8;   // 128-k steps of code loads in flight per lane
constexpr int kMfStageBytes = 3072;   // per wavefront: one code pair (2 KiB) and one scale round (1 KiB)

// Fewest activation rows served by the MFMA units.  Their cost per unit does
// not depend on M (16 rows of which M are used, and an fp32 multiply per
// dequantized weight that the dot2 units fold into one per 16), while the
// dot2 units' grows with M: at K = 2048 the LM head with MFMA units measures
// 45-47 us at M = 4..8, with dot2 units 37.5, 55 and 103 us at M = 2, 4, 8.
constexpr int kLmMfMinRows = 4;

// The MFMA units serve MT >= kLmMfMinRows rows when K is a whole number of
// load rounds and the activation image plus the staging areas fit the LDS
// (MT = 8: K <= 8192; larger K takes the dot2 units).
inline bool lm_mf_fits(int mt, int k) {
    return mt >= kLmMfMinRows && k % (128 * kLmMfDepth) == 0 &&
           (size_t)mt * k * 2 + (size_t)kLmMfWaves * kMfStageBytes <= kMaxLds;
}

// Next position in a workgroup's unit sequence: wavefronts draw from an LDS
// counter (positions 0 .. NW-1 are the wavefronts' first units).
template <int NW>
__device__ __forceinline__ int lm_draw(int *q, int lane) {
    int g = 0;
    if (lane == 0) g = atomicAdd(q, 1);
    return NW + __builtin_amdgcn_readfirstlane(g);
}

// Combines per-wavefront candidates wb[0..NW)[m] inside one wavefront: lane
// l takes the entries (w, m = l % MT) for w = l / MT, l / MT + 64 / MT, ...,
// xor shuffles fold the wavefront bits, and lane m < MT ends with the
// combination for activation row m.
template <int MT, int NW, bool LP>
__device__ __forceinline__ ArgPart combine_waves(const ArgPart (&wb)[NW][MT], int lane) {
    static_assert((MT & (MT - 1)) == 0 && MT <= 64, "MT divides the wavefront");
    constexpr int LW = 64 / MT;                              // wavefronts one pass of the lanes covers
    constexpr int NWP = NW <= 1 ? 1 : NW <= 2 ? 2 : NW <= 4 ? 4 : NW <= 8 ? 8 : NW <= 16 ? 16 : 32;
    constexpr int SPAN = NWP < LW ? NWP : LW;                // lane groups holding entries
    const int w0 = lane / MT, mm = lane % MT;
    ArgPart c{-INFINITY, -INFINITY, INT_MAX, -INFINITY, 0.0f, {0, 0, 0}};
    for (int w = w0; w < NW; w += LW) argpart_combine<LP>(c, wb[w][mm]);
#pragma unroll
    for (int off = SPAN * MT / 2; off >= 16; off >>= 1) argpart_shfl_combine<LP>(c, off);   // across rows
    // inside the row: every rotation from 8 down to MT (a rotation covers a
    // window of lanes, not an aligned block, so none may be skipped even when
    // the entries fill only part of the row; the other lanes hold -inf)
    argpart_row_combine<LP, 8>(c);
    if constexpr (MT <= 4) argpart_row_combine<LP, 4>(c);
    if constexpr (MT <= 2) argpart_row_combine<LP, 2>(c);
    if constexpr (MT <= 1) argpart_row_combine<LP, 1>(c);
    return c;
}

// Persistent LM-head pass.  The vocabulary is cut into units of 4 * R rows,
// one wavefront's tile.  Workgroup b (one per CU) owns units b, b + G,
// b + 2G, ... (G = gridDim.x), so that at any moment the chip sweeps one
// contiguous band of the matrix; inside the workgroup the units go to
// whichever wavefront is free next (an LDS counter), so wavefronts that the
// CU's arbitration serves less take fewer units and all of them end
// together.  The activations are loaded once per workgroup.
//
// GOUT: the same streaming loop as a plain GEMV -- every unit's sums, times
// the global scale, go to gy[m][row] (fp32, or bf16 with gy_bf16) and there
// is no argmax, mask or workspace.  Large decode GEMVs use it for the
// persistent grid, the LDS unit queue and the next unit's loads in flight.
//
// FCPL > 0 (one activation row, argmax only; lmhead_gemv_argmax_fc): the
// workgroups then run the next step's fc, a wavefront per row and FCPL
// 32-element chunks a lane (k = 2048 FCPL).  Wavefronts 1.. load their fc
// rows and the rest part of the activations as soon as their LM-head loop
// ends, so the loads stream during the end chain (wavefront 0 carries the
// chain's stores, and its completion wait would wait for them too); the last
// workgroup publishes the draft id with this call's count in the fc word,
// the others compute the rest part's products while they wait for the count
// to change (bounded); then each lane loads its chunks of the id's
// embedding row and the rows are finished.
template <int MT, int R, int CPL, bool BF16KEY, bool LP, int NW, bool MF = false, bool MASKED = true, bool GOUT = false,
          int FCPL = 0>
__global__ __launch_bounds__(64 * NW) void k_lmhead(const uint16_t *__restrict__ x, int m_rt, const uint8_t *__restrict__ codes,
                                                   const uint8_t *__restrict__ scales, const nvfp4_global *__restrict__ g,
                                                   int v, int k, char *__restrict__ ws, int32_t *__restrict__ out_idx,
                                                   float *__restrict__ out_max, float *__restrict__ out_lp,
                                                   const uint32_t *__restrict__ mask, int mask_words, EmbedOut emb,
                                                   void *__restrict__ gy, int gy_bf16, FcNext fc) {
    static_assert(FCPL == 0 || (MT == 1 && !LP && !MASKED && !MF && !GOUT), "the fused fc follows a plain one-row argmax");
    extern __shared__ uint4 smem[];
    uint4 *xs = smem;
    __shared__ ArgPart wbest[NW][MT];
    __shared__ int s_last, s_q;
    unsigned int *ticket = reinterpret_cast<unsigned int *>(ws + kLmTicket);
    float *row0 = reinterpret_cast<float *>(ws + kLmRow0);
    ArgPart *parts = reinterpret_cast<ArgPart *>(ws + kLmParts);
    unsigned long long *best = reinterpret_cast<unsigned long long *>(ws + kLmBest);
    unsigned long long *fcword = reinterpret_cast<unsigned long long *>(ws + kLmFcWord);
    __shared__ unsigned int s_fce;   // FCPL: the fc word's count when the call started
    __shared__ int32_t s_fcidx;      // FCPL: the draft id the fc gathers (-1: the wait gave up)
    unsigned int fce = 0;            // thread 0; the last workgroup advances the word only after every ticket
    if constexpr (FCPL > 0)
        if (threadIdx.x == 0) fce = (unsigned int)(ld_dev(fcword) >> 32);

    constexpr int rows = MF ? 16 : 4 * R;
    static_assert(32 % rows == 0, "a unit lies inside one 32-row mask word");
    static_assert(!MF || MT >= 2, "the MFMA units serve two or more activation rows");
    const int nunits = (v + rows - 1) / rows;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const float dec = g->dec;
    // lane m of every slot keeps the best of its rows for activation row m
    // (scalars rather than an ArgPart: a struct captured by the lambda below
    // is kept in scratch memory by the compiler)
    float b_key = -INFINITY, b_val = -INFINITY, b_lm = -INFINITY, b_ls = 0.0f;
    int b_idx = INT_MAX;
    // Grammar mask word (32 rows) of a unit for the activation row this lane
    // serves in the epilogue; all ones without a mask.  Loaded with the
    // unit's weights, so it adds no latency to the epilogue.
    const int mrow = min(min(lane & 15, MT - 1), m_rt - 1);
    auto load_mask = [&](int unit) -> uint32_t {
        if (!MASKED) return ~0u;   // no mask: no load (an optional load would make the compiler drain every load)
        const int word = (unit * rows) >> 5;
        return word < mask_words ? mask[(size_t)mrow * mask_words + word] : 0u;
    };
    uint32_t mword = ~0u;
    auto gout = [&](int row, int mm, float s) {
        if (mm >= m_rt) return;
        const float o = s * dec;
        if (gy_bf16)
            reinterpret_cast<uint16_t *>(gy)[(size_t)mm * v + row] = (uint16_t)f32_to_bf16_bits(o);
        else
            reinterpret_cast<float *>(gy)[(size_t)mm * v + row] = o;
    };
    auto epi = [&](int row, int mm, float s) {
        if constexpr (GOUT) {
            gout(row, mm, s);
            return;
        }
        const float logit = s * dec;
        float key = BF16KEY ? bf16_bits_to_f32(f32_to_bf16_bits(logit)) : logit;
        if (row == 0) st_dev(&row0[mm], logit);
        // grammar mask: a disallowed row is scored as -inf (mword holds this
        // lane's mask word of the current unit)
        if (!((mword >> (row & 31)) & 1u)) key = -INFINITY;
        if constexpr (LP) {
            if (key != -INFINITY) lse_merge(b_lm, b_ls, key, 1.0f);   // exp(-inf) adds nothing
        }
        if (beats(key, row, b_key, b_idx)) {
            b_key = key;
            b_val = logit;
            b_idx = row;
        }
    };
    const int G = gridDim.x, b0 = blockIdx.x;
    if (threadIdx.x == 0) s_q = 0;
    // MFMA units: lane (n, q) keeps the best of its rows for activation rows
    // 4 q + r, r = 0..3 (the scalars above serve the other paths)
    float mk[4], mv[4], mlm[4], mls[4];
    int mi[4];
    uint32_t mw[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        mk[r] = -INFINITY;
        mv[r] = -INFINITY;
        mlm[r] = -INFINITY;
        mls[r] = 0.0f;
        mi[r] = INT_MAX;
        mw[r] = ~0u;
    }
    if constexpr (MF) {
        const int q = lane >> 4;
        auto epi_mf = [&](int row, int r, float s) {
            const int mm = 4 * q + r;
            if constexpr (GOUT) {
                gout(row, mm, s);
                return;
            }
            const float logit = s * dec;
            float key = BF16KEY ? bf16_bits_to_f32(f32_to_bf16_bits(logit)) : logit;
            if (row == 0) st_dev(&row0[mm], logit);
            if (!((mw[r] >> (row & 31)) & 1u)) key = -INFINITY;
            if constexpr (LP) {
                if (key != -INFINITY) lse_merge(mlm[r], mls[r], key, 1.0f);
            }
            if (beats(key, row, mk[r], mi[r])) {
                mk[r] = key;
                mv[r] = logit;
                mi[r] = row;
            }
        };
        // the code loads run kLmMfDepth steps ahead (and the scale loads one
        // round of kLmMfDepth steps) as one stream across the wavefront's
        // units (the launch keeps the step count a multiple of the depth);
        // past its last unit the stream reads unit 0, unused
        constexpr int D = kLmMfDepth;
        static_assert(D == 8, "a round of 8 steps is one scale line");
        const int li = lane & 15, cpr = k >> 3, S = k >> 7;
        uint4 *cst = smem + (size_t)MT * cpr + (size_t)wave * (kMfStageBytes / 16);   // code pair, 2 KiB
        const uint16_t *sst = reinterpret_cast<const uint16_t *>(cst + 128);            // scale round, 1 KiB
        int u = b0 + G * wave;
        MfLines cur = mf_lines(codes, scales, v, k, (u < nunits ? u : 0) * rows, lane);
        // the activations, then the first unit's weights, all in flight
        // before the image is stored (its stores wait for the activations
        // only).  Issue order as in the loop (scales, then the code pairs),
        // so that each wait there only covers what it needs.  A scale load
        // covers half of each row's 128-byte line (8 steps) and the other
        // half is read a round later: the scales go through the L2 with the
        // normal policy, so that the line is still there (streamed like the
        // codes, the line was fetched twice: 7% more bytes at K = 2048)
        uint4 xv[kStageBatch];
        stage_x_mf_first(xv, reinterpret_cast<const uint4 *>(x), m_rt, MT, k);
        __builtin_amdgcn_sched_barrier(0);
        uint4 sv = ld_l2_16(cur.sp);
        __builtin_amdgcn_sched_barrier(0);
        uint4 cw[D];
#pragma unroll
        for (int d = 0; d < D; ++d) {
            cw[d] = ld_stream16((d & 1 ? cur.cb : cur.ca) + 128 * (d >> 1));
            __builtin_amdgcn_sched_barrier(0);
        }
        stage_x_mf_rest(xs, xv, reinterpret_cast<const uint4 *>(x), m_rt, MT, k);
        __syncthreads();
        int un = b0 + G * lm_draw<NW>(&s_q, lane);
        MfLines nxt = mf_lines(codes, scales, v, k, (un < nunits ? un : 0) * rows, lane);
        const uint4 *xa[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) xa[b] = mf_xrow(xs, cpr, MT, li, q, b);
        const int ws0 = mf_code_wslot(lane, 0), ws1 = mf_code_wslot(lane, 1);
        const int rs0 = mf_code_rslot(li, q, 0), rs1 = mf_code_rslot(li, q, 1);
        while (u < nunits) {
            if constexpr (MASKED) {
                const int word = (u * rows) >> 5;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int mm = min(min(4 * q + r, MT - 1), m_rt - 1);
                    mw[r] = word < mask_words ? mask[(size_t)mm * mask_words + word] : 0u;
                }
            }
            f32x4 acc0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = {0.0f, 0.0f, 0.0f, 0.0f};
            for (int s0 = 0; s0 < S; s0 += D) {
                // this round reloads steps s0 + D .. s0 + 2 D - 1 and the next
                // round's scales: of this unit, or in the last round steps
                // 0 .. D - 1 of the next
                const bool last = s0 + D >= S;
                const uint8_t *la = last ? nxt.ca : cur.ca + 64 * (size_t)(s0 + D);
                const uint8_t *lb = last ? nxt.cb : cur.cb + 64 * (size_t)(s0 + D);
                const uint8_t *ls = last ? nxt.sp : cur.sp + 8 * (size_t)(s0 + D);
                cst[128 + lane] = sv;   // the round's scales to LDS (row r at byte 64 r)
                sv = ld_l2_16(ls);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int d = 0; d < D; d += 2) {
                    cst[ws0] = cw[d];         // the pair's lines to LDS
                    cst[ws1] = cw[d + 1];
                    cw[d] = ld_stream16(la + 128 * (d >> 1));
                    cw[d + 1] = ld_stream16(lb + 128 * (d >> 1));
                    __builtin_amdgcn_sched_barrier(0);   // reloads issued here, D steps ahead
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        uint4 a[4], bw[4];
                        mf_xload(xa, s0 + d + h, a);
                        const uint4 c = cst[h ? rs1 : rs0];
                        const uint32_t sw = sst[32 * li + 4 * (d + h) + q];
                        mf_dequant(c, sw, bw);
                        mf_mma(a, bw, acc0, acc1);
                    }
                }
            }
            const int rowu = u * rows + li;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (4 * q + r < MT && rowu < v) epi_mf(rowu, r, acc0[r] + acc1[r]);
            u = un;
            cur = nxt;
            un = b0 + G * lm_draw<NW>(&s_q, lane);
            nxt = mf_lines(codes, scales, v, k, (un < nunits ? un : 0) * rows, lane);
        }
    } else if constexpr (MT == 1 && CPL > 0) {
        // one activation row: it lives in registers; the next unit's loads
        // are in flight while this one is computed
        int q = wave, u = b0 + G * q;
        TileRegs<MT, R, 1, CPL> cur;
        uint32_t mcur = ~0u;
        if (u < nunits) {
            gemv_tile_load<MT, R, 1, CPL, true>(cur, codes, scales, v, k, u * rows);
            mcur = load_mask(u);
        }
        XRegs<CPL> xr;
        load_xregs<1, CPL, false>(xr, xrows_plain(x), k);
        __syncthreads();
        int qn = lm_draw<NW>(&s_q, lane);
        while (u < nunits) {
            const int un = b0 + G * qn;
            TileRegs<MT, R, 1, CPL> nxt;
            uint32_t mnxt = mcur;
            if (un < nunits) {
                gemv_tile_load<MT, R, 1, CPL, true>(nxt, codes, scales, v, k, un * rows);
                mnxt = load_mask(un);
            } else {
                nxt = cur;
            }
            qn = lm_draw<NW>(&s_q, lane);
            mword = mcur;
            gemv_tile_compute_x1<R, 1, CPL, true>(cur, xr, v, u * rows, nullptr, epi);
            cur = nxt;
            mcur = mnxt;
            u = un;
        }
    } else if constexpr (CPL > 0) {
        // the next unit's loads are in flight while this one is computed
        int q = wave, u = b0 + G * q;
        TileRegs<MT, R, 1, CPL> cur;
        uint32_t mcur = ~0u;
        if (u < nunits) {
            gemv_tile_load<MT, R, 1, CPL, true>(cur, codes, scales, v, k, u * rows);
            mcur = load_mask(u);
        }
        stage_x<MT, false>(xs, xrows_plain(x), m_rt, k);
        __syncthreads();
        int qn = lm_draw<NW>(&s_q, lane);
        while (u < nunits) {
            const int un = b0 + G * qn;
            TileRegs<MT, R, 1, CPL> nxt;
            uint32_t mnxt = mcur;
            if (un < nunits) {
                gemv_tile_load<MT, R, 1, CPL, true>(nxt, codes, scales, v, k, un * rows);
                mnxt = load_mask(un);
            } else {
                nxt = cur;
            }
            qn = lm_draw<NW>(&s_q, lane);
            mword = mcur;
            gemv_tile_compute<MT, R, 1, CPL, true>(cur, xs, v, k, u * rows, nullptr, epi);
            cur = nxt;
            mcur = mnxt;
            u = un;
        }
    } else {
        stage_x<MT, false>(xs, xrows_plain(x), m_rt, k);
        __syncthreads();
        int q = wave, qn = lm_draw<NW>(&s_q, lane);
        for (int u = b0 + G * q; u < nunits; u = b0 + G * q) {
            mword = load_mask(u);
            q = qn;
            qn = lm_draw<NW>(&s_q, lane);
            gemv_tile_loop<MT, R, 1, (R >= 4 ? 1 : 4 / R), true>(xs, codes, scales, v, k, u * rows, nullptr, epi);
        }
    }

    if constexpr (GOUT) return;   // plain GEMV: every output is written

    // FCPL: the fc rows of this wavefront (wavefronts 1..NW-1; row b + G ((w - 1)
    // + (NW - 1) j)), lane l taking 32-element chunks l + 64 i, i < FCPL; the
    // weights and the rest part of the activations now, so that the rest
    // part's products are done while the draft id is awaited
    constexpr int FCP = FCPL > 0 ? FCPL : 1;
    uint4 fcw[kLmFcRows][FCP];
    uint32_t fcs[kLmFcRows][FCP];
    uint32_t fxr[FCP][16];   // the lane's rest-part activations (its emb-part chunks: loaded after the id)
    if constexpr (FCPL > 0) {
        if (wave >= 1) {
#pragma unroll
            for (int j = 0; j < kLmFcRows; ++j) {
                const int row = min((int)blockIdx.x + (int)gridDim.x * (wave - 1 + (NW - 1) * j), fc.n - 1);
                const uint8_t *cp = fc.codes + (size_t)row * (size_t)(fc.k >> 1);
                const uint8_t *sp = fc.scales + (size_t)row * (size_t)(fc.k >> 4);
#pragma unroll
                for (int i = 0; i < FCP; ++i) {
                    fcw[j][i] = ld_stream16(cp + 16 * (size_t)(lane + 64 * i));
                    fcs[j][i] = ld_stream2(sp + 2 * (size_t)(lane + 64 * i));
                }
            }
#pragma unroll
            for (int i = 0; i < FCP; ++i) {
                const int kk = 32 * (lane + 64 * i);
                if (kk >= fc.kt) {
                    const uint4 *p = reinterpret_cast<const uint4 *>(fc.rest + (kk - fc.kt));
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const uint4 u = p[q];
                        fxr[i][4 * q] = u.x;
                        fxr[i][4 * q + 1] = u.y;
                        fxr[i][4 * q + 2] = u.z;
                        fxr[i][4 * q + 3] = u.w;
                    }
                }
            }
        }
        if (threadIdx.x == 0) s_fce = fce;
    }

    // workgroup combine: the four slots of a wavefront by shuffles, then the
    // NW wavefronts in LDS -> MT candidates
    if constexpr (MF) {
        // rows 4 q + r: fold the 16 lanes of group q
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            ArgPart c{mk[r], mv[r], mi[r], mlm[r], mls[r], {0, 0, 0}};
            argpart_row_combine<LP, 8>(c);
            argpart_row_combine<LP, 4>(c);
            argpart_row_combine<LP, 2>(c);
            argpart_row_combine<LP, 1>(c);
            const int mm = 4 * (lane >> 4) + r;
            if ((lane & 15) == 0 && mm < MT) wbest[wave][mm] = c;
        }
    } else {
        ArgPart c{b_key, b_val, b_idx, b_lm, b_ls, {0, 0, 0}};
        argpart_shfl_combine<LP>(c, 16);
        argpart_shfl_combine<LP>(c, 32);
        if (lane < MT) wbest[wave][lane] = c;
    }
    __syncthreads();
    if (wave == 0) {
        const ArgPart b = combine_waves<MT, NW, LP>(wbest, lane);
        if (lane < MT) {
            // the argmax as one 64-bit atomic max per activation row (the
            // fp32 logit of a bf16 key, or the sign of a zero one, is looked
            // up afterwards in the partial of the workgroup that owns the
            // winning row); the log-sum-exp state as a partial
            ArgPart *dst = parts + (size_t)blockIdx.x * MT + lane;
            st_dev(&dst->val, b.val);
            if constexpr (LP) {
                st_dev(&dst->lm, b.lm);
                st_dev(&dst->ls, b.ls);
            }
            __hip_atomic_fetch_max(&best[lane], pack_best(b.key, b.idx), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    // partials, maxima and row-0 logits (wavefront 0's stores) have reached
    // device scope
    if (FCPL == 0 || wave == 0) wait_mem();
    __syncthreads();
    if (threadIdx.x == 0) s_last = atomicAdd(ticket, 1u) == gridDim.x - 1;
    __syncthreads();
    if constexpr (FCPL > 0) {
        float fpart[kLmFcRows];   // the rest part's sum of each fc row (lanes' shares)
        if (s_last) {
            if (wave == 0) {
                // the argmax of the one row (as below), its outputs, and the
                // id published with this call's count
                const unsigned long long pk = ld_dev(&best[0]);
                float key = unpack_best_key(pk), val = key;
                int idx = unpack_best_idx(pk);
                if (key > -INFINITY && (BF16KEY || key == 0.0f))
                    val = ld_dev(&parts[(size_t)((idx / rows) % (int)gridDim.x) * MT].val);
                if (!(key > -INFINITY)) {   // nothing above -inf: index 0
                    idx = 0;
                    val = ld_dev(&row0[0]);
                }
                if (lane == 0) {
                    st_dev(&best[0], 0ull);   // ready for the next call
                    st_dev(ticket, 0u);
                    out_idx[0] = idx;
                    out_max[0] = val;
                    s_fcidx = idx;
                    st_dev(fcword, ((unsigned long long)(s_fce + 1u) << 32) | (unsigned int)idx);
                }
            }
        } else if (threadIdx.x == 0) {
            unsigned long long w = ld_dev(fcword);
            int n = 0;
            while ((unsigned int)(w >> 32) == s_fce && n < kLmFcSpinLimit) {
                __builtin_amdgcn_s_sleep(2);
                w = ld_dev(fcword);
                ++n;
            }
            s_fcidx = (unsigned int)(w >> 32) == s_fce ? -1 : (int32_t)(unsigned int)w;
        }
        if (wave >= 1) {
            // the rest part's products (their loads were issued after the loop)
#pragma unroll
            for (int j = 0; j < kLmFcRows; ++j) {
                float acc = 0.0f;
#pragma unroll
                for (int i = 0; i < FCP; ++i)
                    if (32 * (lane + 64 * i) >= fc.kt) acc = chunk_dot_xreg(fcw[j][i], fcs[j][i], fxr[i], acc);
                fpart[j] = acc;
            }
        }
        __syncthreads();
        const int32_t fid = s_fcidx;
        if (wave >= 1) {
            // the emb part: each lane's chunks of the id's table row (a zero
            // row for an id outside the table, or when the wait gave up)
            const bool in = fid >= 0 && fid < fc.vocab;
            const uint16_t *trow = fc.table + (size_t)(in ? fid : 0) * (size_t)fc.kt;
#pragma unroll
            for (int i = 0; i < FCP; ++i) {
                const int kk = 32 * (lane + 64 * i);
                if (kk < fc.kt) {
                    const uint4 *p = reinterpret_cast<const uint4 *>(trow + kk);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const uint4 u = in ? p[q] : make_uint4(0, 0, 0, 0);
                        fxr[i][4 * q] = u.x;
                        fxr[i][4 * q + 1] = u.y;
                        fxr[i][4 * q + 2] = u.z;
                        fxr[i][4 * q + 3] = u.w;
                    }
                }
            }
            const float fdec = fc.g->dec;
#pragma unroll
            for (int j = 0; j < kLmFcRows; ++j) {
                float acc = fpart[j];
#pragma unroll
                for (int i = 0; i < FCP; ++i)
                    if (32 * (lane + 64 * i) < fc.kt) acc = chunk_dot_xreg(fcw[j][i], fcs[j][i], fxr[i], acc);
                // the row's sum over the 64 lanes, in a fixed order
                const float r16 = row16_sum(acc);
                const float sum = (__shfl(r16, 0, 64) + __shfl(r16, 16, 64)) + (__shfl(r16, 32, 64) + __shfl(r16, 48, 64));
                const int row = (int)blockIdx.x + (int)gridDim.x * (wave - 1 + (NW - 1) * j);
                if (lane == 0 && row < fc.n) {
                    const float o = fid < 0 ? __builtin_nanf("") : sum * fdec;   // a wait that gave up: NaN rows
                    if (fc.y_bf16)
                        reinterpret_cast<uint16_t *>(fc.y)[row] = (uint16_t)f32_to_bf16_bits(o);
                    else
                        reinterpret_cast<float *>(fc.y)[row] = o;
                }
            }
        }
        return;
    }
    if (!s_last) return;

    // last workgroup: its first wavefront reads the maxima and merges the
    // log-sum-exp partials
    if (wave != 0) return;
    ArgPart f{-INFINITY, -INFINITY, INT_MAX, -INFINITY, 0.0f, {0, 0, 0}};
    if constexpr (LP) {
        float lm[MT], ls[MT];
#pragma unroll
        for (int mm = 0; mm < MT; ++mm) {
            lm[mm] = -INFINITY;
            ls[mm] = 0.0f;
        }
        // UB partials per lane per round, all loads issued before any merge
        constexpr int UB = MT <= 2 ? 4 : MT == 4 ? 2 : 1;
        for (int p0 = lane; p0 < (int)gridDim.x; p0 += 64 * UB) {
            float plm[UB][MT], pls[UB][MT];
#pragma unroll
            for (int j = 0; j < UB; ++j) {
                const int p = p0 + 64 * j;
#pragma unroll
                for (int mm = 0; mm < MT; ++mm) {
                    const ArgPart *src = parts + (size_t)(p < (int)gridDim.x ? p : 0) * MT + mm;
                    plm[j][mm] = ld_dev(&src->lm);
                    pls[j][mm] = ld_dev(&src->ls);
                    if (p >= (int)gridDim.x) {
                        plm[j][mm] = -INFINITY;
                        pls[j][mm] = 0.0f;
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < UB; ++j)
#pragma unroll
                for (int mm = 0; mm < MT; ++mm) lse_merge(lm[mm], ls[mm], plm[j][mm], pls[j][mm]);
        }
#pragma unroll
        for (int mm = 0; mm < MT; ++mm) {
#pragma unroll
            for (int off = 32; off > 0; off >>= 1)
                lse_merge(lm[mm], ls[mm], __shfl_xor(lm[mm], off, 64), __shfl_xor(ls[mm], off, 64));
            if (mm == lane) {
                f.lm = lm[mm];
                f.ls = ls[mm];
            }
        }
    }
    if (lane < MT) {
        const unsigned long long pk = ld_dev(&best[lane]);
        st_dev(&best[lane], 0ull);   // ready for the next call
        f.key = unpack_best_key(pk);
        f.idx = unpack_best_idx(pk);
        f.val = f.key;
        if (f.key > -INFINITY && (BF16KEY || f.key == 0.0f)) {
            const int owner = (f.idx / rows) % (int)gridDim.x;
            f.val = ld_dev(&parts[(size_t)owner * MT + lane].val);
        }
    }
    if (lane < m_rt) {
        const int mm = lane;
        // nothing above -inf: the scan keeps its initial index 0
        float wkey = f.key;
        if (!(f.key > -INFINITY)) {
            const float l0 = ld_dev(&row0[mm]);
            out_idx[mm] = 0;
            out_max[mm] = l0;
            wkey = BF16KEY ? bf16_bits_to_f32(f32_to_bf16_bits(l0)) : l0;
        } else {
            out_idx[mm] = f.idx;
            out_max[mm] = f.val;
        }
        // no mass (nothing allowed, or only -inf keys): not measured
        if constexpr (LP) out_lp[mm] = f.ls > 0.0f ? wkey - (f.lm + __logf(f.ls)) : __builtin_nanf("");
    }
    if (emb.table != nullptr) {
        // the selected token of row mm is lane mm's.  Lane l copies units
        // l, l + 64, ... of every row: item t of a lane is unit
        // lane + 64 (t mod per) of row t / per.  A batch's loads are all
        // issued before its stores (a load-store pair per unit waited one
        // memory round trip per unit: 32 of them at eight rows).
        const int sel = lane < m_rt && f.key > -INFINITY ? f.idx : 0;
        if (lane < m_rt && emb.id_log != nullptr) emb.id_log[lane] = sel;
        const int per = (emb.units + 63) / 64, total = m_rt * per;
        for (int t0 = 0; t0 < total; t0 += kEmbBatch) {
            uint4 v[kEmbBatch];
            int row[kEmbBatch], unit[kEmbBatch];   // unit -1: nothing to store
#pragma unroll
            for (int j = 0; j < kEmbBatch; ++j) {
                const int t = t0 + j < total ? t0 + j : total - 1;
                const int mm = t / per, u = lane + 64 * (t - mm * per);
                const int id = __shfl(sel, mm, 64);
                const bool in = id >= 0 && id < emb.vocab, live = t0 + j < total && u < emb.units;
                v[j] = emb.table[(size_t)(in ? id : 0) * emb.units + (live ? u : 0)];
                if (!in) v[j] = make_uint4(0, 0, 0, 0);
                row[j] = mm;
                unit[j] = live ? u : -1;
            }
#pragma unroll
            for (int j = 0; j < kEmbBatch; ++j)
                if (unit[j] >= 0) emb.out[(size_t)row[j] * emb.stride_units + unit[j]] = v[j];
        }
    }
    if (lane == 0) st_dev(ticket, 0u);   // ready for the next call
}

// --------------------------------------------------- MFMA units, K split ----
// Decode GEMV for 4 to 8 activation rows on the MFMA units, for weights too
// small for the persistent grid: one workgroup per 16-row unit, its K split
// into slices of 1024 (8 steps of 128, one scale line), one wavefront per
// slice.  A wavefront issues every load of its slice at once (8 code-line
// pairs and one scale line, 9 KiB), stages them through its LDS area into
// the MFMA layout as the LM head's units do, and runs 16
// v_mfma_f32_16x16x32_bf16; the slices' sums are added in slice order
// through LDS.  With the dot2 units the cost of a weight grows with the row
// count; here it does not, and every load of the launch is in flight at once.
constexpr int kMfSliceSteps = 8;                        // 128-k steps a wavefront
constexpr int kMfSliceK = 128 * kMfSliceSteps;          // 1024
constexpr int kMfMaxSlices = 8;                         // K <= 8192
constexpr long kMfSplitMaxUnits = 1024;                 // 16-row units (4096 at four rows)

template <int MT, bool XG = false>
__global__ __launch_bounds__(64 * kMfMaxSlices) void k_gemv_mf(const XRows x, int m_rt,
                                                               const GemvGroups grp, int k, int bf16out) {
    extern __shared__ uint4 smem[];
    const int tile = blockIdx.x;
    const uint8_t *codes = grp.codes[0];
    const uint8_t *scales = grp.scales[0];
    const nvfp4_global *g = grp.g[0];
    void *y = grp.y[0];
    int n = grp.n[0], t0 = 0;
#pragma unroll
    for (int i = 1; i < kMaxGroups; ++i) {
        if (i < grp.count && tile >= grp.tile0[i]) {
            codes = grp.codes[i];
            scales = grp.scales[i];
            g = grp.g[i];
            y = grp.y[i];
            n = grp.n[i];
            t0 = grp.tile0[i];
        }
    }
    const int row0 = (tile - t0) * 16;
    const int lane = threadIdx.x & 63, ks = threadIdx.x >> 6, nks = blockDim.x >> 6;
    const int li = lane & 15, q = lane >> 4;
    const int s0 = ks * kMfSliceSteps;
    // this wavefront's LDS: its slice of the activation image (MT rows of
    // 128 chunks, chunk c of row m at c ^ (m % 8)), then its stage area
    constexpr int kSliceChunks = kMfSliceK / 8;
    uint4 *xs = smem + (size_t)ks * (MT * kSliceChunks + kMfStageBytes / 16);
    uint4 *cst = xs + MT * kSliceChunks;                                           // code pair, 2 KiB
    const uint16_t *sst = reinterpret_cast<const uint16_t *>(cst + 128);            // scale line, 1 KiB
    // the slice's activations (2 MT chunks a lane), then the weights, all in
    // flight together; the activation stores wait for the activations only
    // (a lane's unit j lies in activation row j / 2: 128 chunks a row)
    constexpr int XU = 2 * MT;
    static_assert(kSliceChunks == 128, "two units a row per lane");
    uint4 xv[XU];
    if constexpr (!XG) {
        const uint4 *xg = reinterpret_cast<const uint4 *>(x.x);
        const int cpr = k >> 3;
#pragma unroll
        for (int j = 0; j < XU; ++j) {
            const int p = lane + 64 * j, m = p / kSliceChunks, c = p % kSliceChunks;
            xv[j] = m < m_rt ? xg[(size_t)m * cpr + kSliceChunks * ks + c] : make_uint4(0, 0, 0, 0);
        }
    }
    int lid = 0;
    if constexpr (XG) lid = xids_issue(x, m_rt);   // before the weights: see below
    const MfLines ln = mf_lines(codes, scales, n, k, row0, lane);
    const uint4 sv = ld_l2_16(ln.sp + 8 * (size_t)s0);   // the slices of a line share it
    uint4 cw[kMfSliceSteps];
#pragma unroll
    for (int d = 0; d < kMfSliceSteps; ++d)
        cw[d] = ld_stream16((d & 1 ? ln.cb : ln.ca) + 64 * (size_t)s0 + 128 * (d >> 1));
    if constexpr (XG) {
        __builtin_amdgcn_sched_barrier(0);
        // gathered rows: their addresses wait for the table rows, so the
        // weights go first (rows from m_rt on load row m_rt - 1 and are masked)
        XRow g[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) g[m] = xrow(x, m < m_rt ? m : m_rt - 1, k, lid);
#pragma unroll
        for (int j = 0; j < XU; ++j) {
            const int c = (lane + 64 * j) % kSliceChunks;
            xv[j] = *reinterpret_cast<const uint4 *>(xrow_addr(g[j / 2], 8 * (kSliceChunks * ks + c), x.kt));
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < XU; ++j) {
            const int m = j / 2, c = (lane + 64 * j) % kSliceChunks;
            xv[j] = xmask(xv[j], m >= m_rt || xrow_zero(g[m], 8 * (kSliceChunks * ks + c), x.kt));
        }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < XU; ++j) {
        const int p = lane + 64 * j, m = p / kSliceChunks, c = p % kSliceChunks;
        xs[m * kSliceChunks + (c ^ (m & 7))] = xv[j];
    }
    const uint4 *xa[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) xa[b] = mf_xrow(xs, kSliceChunks, MT, li, q, b);
    const int ws0 = mf_code_wslot(lane, 0), ws1 = mf_code_wslot(lane, 1);
    const int rs0 = mf_code_rslot(li, q, 0), rs1 = mf_code_rslot(li, q, 1);
    cst[128 + lane] = sv;
    f32x4 acc0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int d = 0; d < kMfSliceSteps; d += 2) {
        cst[ws0] = cw[d];
        cst[ws1] = cw[d + 1];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            uint4 a[4], bw[4];
            mf_xload(xa, d + h, a);
            const uint4 c = cst[h ? rs1 : rs0];
            const uint32_t sw = sst[32 * li + 4 * (d + h) + q];
            mf_dequant(c, sw, bw);
            mf_mma(a, bw, acc0, acc1);
        }
    }
    // the slices' sums in slice order (wavefront 0 adds them)
    float *part = reinterpret_cast<float *>(cst);   // this wavefront's stage area, reused
#pragma unroll
    for (int r = 0; r < 4; ++r) part[4 * lane + r] = acc0[r] + acc1[r];
    __syncthreads();
    if (ks != 0) return;
    const int row = row0 + li;
    const float dec = g->dec;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        float v = part[4 * lane + r];
        for (int j = 1; j < nks; ++j)
            v += reinterpret_cast<const float *>(smem + (size_t)j * (MT * kSliceChunks + kMfStageBytes / 16) +
                                                 MT * kSliceChunks)[4 * lane + r];
        const int mm = 4 * q + r;
        if (mm < m_rt && row < n) {
            const float o = v * dec;
            if (bf16out)
                reinterpret_cast<uint16_t *>(y)[(size_t)mm * n + row] = (uint16_t)f32_to_bf16_bits(o);
            else
                reinterpret_cast<float *>(y)[(size_t)mm * n + row] = o;
        }
    }
}

// The K-split MFMA GEMV serves 4 to 8 rows when K is 1024 to 8192 in whole
// slices and the activation image and the stage areas fit the LDS.
inline size_t gemv_mf_lds(int mt, int k) { return (size_t)(k / kMfSliceK) * ((size_t)mt * kMfSliceK * 2 + kMfStageBytes); }
inline bool gemv_mf_fits(int mt, int k) {
    return mt >= 4 && k % kMfSliceK == 0 && k / kMfSliceK <= kMfMaxSlices && gemv_mf_lds(mt, k) <= kMaxLds;
}

// ------------------------------------------------------------ dispatch ----
// Instantiated tile shapes (R rows per slot, KS K-segments, CPL fixed chunks
// per lane or 0 for the generic loop).
#define NVFP4_TILE_SWITCH(FN, MT, tc, ...)                                               \
    do {                                                                                 \
        if (tc.NW == 16 && tc.KS == 4) FN<MT, 1, 4, 0, 16>(__VA_ARGS__);                 \
        else if (tc.NW == 8 && tc.KS == 2) FN<MT, 1, 2, 0, 8>(__VA_ARGS__);              \
        else if (tc.R == 4 && tc.KS == 1 && tc.CPL == 4) FN<MT, 4, 1, 4>(__VA_ARGS__);   \
        else if (tc.R == 4 && tc.KS == 1 && tc.CPL == 2) FN<MT, 4, 1, 2>(__VA_ARGS__);   \
        else if (tc.R == 4 && tc.KS == 1) FN<MT, 4, 1, 0>(__VA_ARGS__);                  \
        else if (tc.R == 2 && tc.KS == 1 && tc.CPL == 4) FN<MT, 2, 1, 4>(__VA_ARGS__);   \
        else if (tc.R == 2 && tc.KS == 1) FN<MT, 2, 1, 0>(__VA_ARGS__);                  \
        else if (tc.R == 1 && tc.KS == 1 && tc.CPL == 4) FN<MT, 1, 1, 4>(__VA_ARGS__);   \
        else if (tc.R == 1 && tc.KS == 1 && tc.CPL == 2) FN<MT, 1, 1, 2>(__VA_ARGS__);   \
        else if (tc.R == 1 && tc.KS == 1) FN<MT, 1, 1, 0>(__VA_ARGS__);                  \
        else if (tc.KS == 2 && tc.CPL == 2) FN<MT, 1, 2, 2>(__VA_ARGS__);                \
        else if (tc.KS == 2 && tc.CPL == 4) FN<MT, 1, 2, 4>(__VA_ARGS__);                \
        else if (tc.KS == 2) FN<MT, 1, 2, 0>(__VA_ARGS__);                               \
        else if (tc.KS == 4 && tc.CPL == 1) FN<MT, 1, 4, 1>(__VA_ARGS__);                \
        else if (tc.KS == 4 && tc.CPL == 2) FN<MT, 1, 4, 2>(__VA_ARGS__);                \
        else FN<MT, 1, 4, 0>(__VA_ARGS__);                                               \
    } while (0)

// Reduces a tile choice to the instantiated set above.
static TileChoice canonical(TileChoice tc) {
    if (tc.NW != 4) return TileChoice{1, tc.NW == 16 ? 4 : 2, 0, tc.NW == 16 ? 16 : 8};
    if (tc.KS == 1 && tc.R == 4 && tc.CPL != 4 && tc.CPL != 2) tc.CPL = 0;
    if (tc.KS == 1 && tc.R == 2 && tc.CPL != 4) tc.CPL = 0;
    if (tc.KS == 1 && tc.R == 1 && tc.CPL != 4 && tc.CPL != 2) tc.CPL = 0;
    if (tc.KS == 2 && tc.CPL != 2 && tc.CPL != 4) tc.CPL = 0;
    if (tc.KS == 4 && tc.CPL != 1 && tc.CPL != 2) tc.CPL = 0;
    return tc;
}

template <int MT, int R, int KS, int CPL, int NW = 4>
static void launch_gemv_cfg(dim3 grid, size_t lds, hipStream_t s, const XRows &x, int m, const GemvGroups &grp,
                            int k, int bf16) {
    if (x.kt > 0) {   // the activation rows begin with gathered embedding rows
        if (allow_lds(reinterpret_cast<const void *>(k_gemv<MT, R, KS, CPL, NW, true>), lds, "w4a16_gemv")) return;
        hipLaunchKernelGGL((k_gemv<MT, R, KS, CPL, NW, true>), grid, dim3(64 * NW), lds, s, x, m, grp, k, bf16);
        return;
    }
    if (allow_lds(reinterpret_cast<const void *>(k_gemv<MT, R, KS, CPL, NW>), lds, "w4a16_gemv")) return;
    hipLaunchKernelGGL((k_gemv<MT, R, KS, CPL, NW>), grid, dim3(64 * NW), lds, s, x, m, grp, k, bf16);
}

// Tile target of a GEMV launch: at least this many workgroups per CU (a
// sweep of 2, 4, 6, 8 and 12 put the q|k|v grouped GEMV at 5.8, 5.3, 4.9,
// 4.9 and 4.9 us: one tile per workgroup, so more of them keep more loads
// in flight while the launch ramps up).
constexpr int kGemvTilesPerCu = 6;
// From four activation rows on, 2 per CU: each tile then has more rows and
// its lanes more arithmetic between loads (q|k|v grouped at M = 4 in 6.9 us
// against 8.3 at 6 per CU; the single q, fc and 4096 x 2048 GEMVs equal or
// faster).
constexpr int kGemvTilesPerCuM4 = 2;
// One launch over `count` weights with a common K (their tiles concatenated);
// the tile shape is chosen for the total row count.
template <int MT>
static bool launch_gemv_persist(hipStream_t s, const XRows &x, int m, const nvfp4_weight *w, void *y, int bf16);

// An activation image that leaves LDS for at most three workgroups a CU (a
// quarter of it or more) caps the per-tile grid at 4 to 12 wavefronts a CU,
// too few to keep the weight loads in flight: then wide workgroups of
// 16 rows whose K is split over 2 (two workgroups fit) or 4 (one fits)
// wavefront groups.
static TileChoice wide_tile(TileChoice tc, int mt, int k) {
    if (tc.KS != 1 || tc.CPL != 0) return tc;
    const size_t image = (size_t)mt * k * 2, cu_lds = 160 * 1024;
    if (4 * image < cu_lds) return tc;
    const TileChoice w4{1, 4, 0, 16}, w2{1, 2, 0, 8};
    if (2 * gemv_lds_bytes(mt, k, w2) > cu_lds && gemv_lds_bytes(mt, k, w4) <= kMaxLds) return w4;
    return gemv_lds_bytes(mt, k, w2) <= kMaxLds ? w2 : tc;
}

template <int MT>
static int launch_gemv_mf(const XRows &x, int m, const nvfp4_weight *const *w, void *const *y, int count, int bf16,
                          hipStream_t s) {
    const int k = w[0]->k;
    GemvGroups grp{};
    grp.count = count;
    int tiles = 0;
    for (int i = 0; i < count; ++i) {
        grp.codes[i] = w[i]->codes;
        grp.scales[i] = w[i]->scales;
        grp.g[i] = w[i]->global;
        grp.y[i] = y[i];
        grp.n[i] = w[i]->n;
        grp.tile0[i] = tiles;
        tiles += (w[i]->n + 15) / 16;
    }
    for (int i = count; i <= kMaxGroups; ++i) grp.tile0[i] = tiles;
    if (tiles == 0) return ok();
    const int nks = k / kMfSliceK;
    const size_t lds = gemv_mf_lds(MT, k);
    const void *kern = x.kt > 0 ? reinterpret_cast<const void *>(k_gemv_mf<MT, true>)
                                : reinterpret_cast<const void *>(k_gemv_mf<MT, false>);
    const int rc = allow_lds(kern, lds, "w4a16_gemv");
    if (rc) return rc;
    if (x.kt > 0)
        hipLaunchKernelGGL((k_gemv_mf<MT, true>), dim3(tiles), dim3(64 * nks), lds, s, x, m, grp, k, bf16);
    else
        hipLaunchKernelGGL((k_gemv_mf<MT, false>), dim3(tiles), dim3(64 * nks), lds, s, x, m, grp, k, bf16);
    return check_launch("w4a16_gemv");
}

template <int MT>
static int launch_gemv_m(const XRows &x, int m, const nvfp4_weight *const *w, void *const *y, int count, int bf16,
                         hipStream_t s) {
    const int k = w[0]->k;
    if constexpr (MT >= 4) {
        // the K split keeps an activation slice per wavefront in LDS, which at
        // eight rows leaves room for one workgroup a CU: large weights stream
        // faster on the persistent grid (17408 x 5120 at eight rows: 29.6
        // against 20.4 us; at four rows 18.5 against 19.1, and 2048 x 4096,
        // 8192 x 2048 and q|k|v at eight rows 5.6, 6.8, 7.4 against 9.1, 8.0,
        // 12.0 us on the dot2 or persistent paths)
        long units = 0;
        for (int i = 0; i < count; ++i) units += (w[i]->n + 15) / 16;
        const bool small = units <= kMfSplitMaxUnits || (MT == 4 && units <= 4 * kMfSplitMaxUnits);
        if (small && gemv_mf_fits(MT, k)) return launch_gemv_mf<MT>(x, m, w, y, count, bf16, s);
    }
    if (count == 1) {
        ok();   // clears the message that a refused LDS request would leave
        if (launch_gemv_persist<MT>(s, x, m, w[0], y[0], bf16)) return check_launch("w4a16_gemv");
        if (nvfp4_mtp_last_error()[0]) return NVFP4_ERR_UNSUPPORTED;   // allow_lds refused
    }
    int total_n = 0;
    for (int i = 0; i < count; ++i) total_n += w[i]->n;
    const int tpc = MT >= 4 ? kGemvTilesPerCuM4 : kGemvTilesPerCu;
    const TileChoice tc = canonical(wide_tile(choose_tile(total_n, k, MT, tpc * num_cus(), 0), MT, k));
    const int rows = 4 * (tc.NW / tc.KS) * tc.R;
    GemvGroups grp{};
    grp.count = count;
    int tiles = 0;
    for (int i = 0; i < count; ++i) {
        grp.codes[i] = w[i]->codes;
        grp.scales[i] = w[i]->scales;
        grp.g[i] = w[i]->global;
        grp.y[i] = y[i];
        grp.n[i] = w[i]->n;
        grp.tile0[i] = tiles;
        tiles += (w[i]->n + rows - 1) / rows;
    }
    for (int i = count; i <= kMaxGroups; ++i) grp.tile0[i] = tiles;
    if (tiles == 0) return ok();
    ok();   // clears the message that a refused LDS request would leave
    NVFP4_TILE_SWITCH(launch_gemv_cfg, MT, tc, dim3(tiles), gemv_lds_bytes(MT, k, tc), s, x, m, grp, k, bf16);
    if (nvfp4_mtp_last_error()[0]) return NVFP4_ERR_UNSUPPORTED;   // allow_lds refused
    return check_launch("w4a16_gemv");
}

// Grid of the persistent LM-head kernel: every workgroup that is resident at
// once (normally one per CU), never more than the workspace has partials for.
// Returns NVFP4_OK or the status of a refusal (nothing launched).
template <int MT, int CPL, bool BK, bool LP, bool MF = false>
static int launch_lm_kernel(size_t lds, hipStream_t s, const uint16_t *h, int m, const nvfp4_weight *w, int v,
                            char *ws, size_t wsb, int32_t *oi, float *om, float *olp, const uint32_t *mask,
                            int mask_words, const EmbedOut &emb) {
    constexpr int NW = MF ? kLmMfWaves : lm_waves<MT, CPL>();
    auto kern = mask != nullptr ? k_lmhead<MT, lm_rows_per_slot<MT>(), CPL, BK, LP, NW, MF, true>
                                : k_lmhead<MT, lm_rows_per_slot<MT>(), CPL, BK, LP, NW, MF, false>;
    const int rc = allow_lds(reinterpret_cast<const void *>(kern), lds, "lmhead_gemv_argmax");
    if (rc) return rc;
    const int per_cu = blocks_per_cu(reinterpret_cast<const void *>(kern), 64 * NW, lds);
    if (per_cu < 1)
        return fail(NVFP4_ERR_UNSUPPORTED, "lmhead_gemv_argmax: a %d-thread workgroup does not fit on a CU", 64 * NW);
    const int cap = num_cus() * per_cu, nparts = (v + 15) / 16, grid = cap < nparts ? cap : nparts;
    const size_t need = (size_t)kLmParts + sizeof(ArgPart) * MT * (size_t)grid;   // what this grid touches
    if (need > wsb)
        return fail(NVFP4_ERR_WORKSPACE, "lmhead_gemv_argmax: %d workgroups need %zu bytes of workspace, %zu available",
                    grid, need, wsb);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * NW), lds, s, h, m, w->codes, w->scales, w->global, v, w->k, ws, oi,
                       om, olp, mask, mask_words, emb, nullptr, 0, FcNext{});
    return check_launch("lmhead_gemv_argmax");
}

// The four key / log-probability variants of one unit shape.
template <int MT, int CPL, bool MF = false>
static int launch_lm_variant(bool bk, bool lp, size_t lds, hipStream_t s, const uint16_t *h, int m,
                             const nvfp4_weight *w, int v, char *ws, size_t wsb, int32_t *oi, float *om, float *olp,
                             const uint32_t *mask, int mask_words, const EmbedOut &emb) {
    if (bk)
        return lp ? launch_lm_kernel<MT, CPL, true, true, MF>(lds, s, h, m, w, v, ws, wsb, oi, om, olp, mask, mask_words, emb)
                  : launch_lm_kernel<MT, CPL, true, false, MF>(lds, s, h, m, w, v, ws, wsb, oi, om, olp, mask, mask_words, emb);
    return lp ? launch_lm_kernel<MT, CPL, false, true, MF>(lds, s, h, m, w, v, ws, wsb, oi, om, olp, mask, mask_words, emb)
              : launch_lm_kernel<MT, CPL, false, false, MF>(lds, s, h, m, w, v, ws, wsb, oi, om, olp, mask, mask_words, emb);
}

// Persistent streaming GEMV (the LM-head loop with plain outputs) for one
// weight.  One and two rows: when there are kPersistUnits or more units per
// wavefront of the chip (with about one per wavefront the per-tile grid is as
// fast).  Four to eight rows: the MFMA units whenever K allows them, as long
// as every fourth wavefront gets a unit (at 151936 x 2048: 35.8 and 37.9 us
// at M = 4 and 8, against 50.5 and 127 us on the per-tile grid).  Returns
// false (nothing launched) when the persistent grid is not used.
constexpr int kPersistUnits = 2;

template <int MT, int CPL, bool MF>
static bool launch_gemv_persist_k(size_t lds, hipStream_t s, const XRows &x, int m, const nvfp4_weight *w, void *y,
                                  int bf16) {
    constexpr int NW = MF ? kLmMfWaves : lm_waves<MT, CPL>();
    constexpr int rows = MF ? 16 : 4 * lm_rows_per_slot<MT>();
    auto kern = k_lmhead<MT, lm_rows_per_slot<MT>(), CPL, false, false, NW, MF, false, true>;
    const int per_cu = blocks_per_cu(reinterpret_cast<const void *>(kern), 64 * NW, lds);
    const long units = (w->n + rows - 1) / rows, waves = (long)num_cus() * per_cu * NW;
    if (per_cu < 1 || (MF ? 4 * units < waves : units < kPersistUnits * waves)) return false;
    if (allow_lds(reinterpret_cast<const void *>(kern), lds, "w4a16_gemv")) return false;
    hipLaunchKernelGGL(kern, dim3(num_cus() * per_cu), dim3(64 * NW), lds, s, x.x, m, w->codes, w->scales, w->global,
                       w->n, w->k, nullptr, nullptr, nullptr, nullptr, nullptr, 0, EmbedOut{}, y, bf16, FcNext{});
    return true;
}

template <int MT>
static bool launch_gemv_persist(hipStream_t s, const XRows &x, int m, const nvfp4_weight *w, void *y, int bf16) {
    if (x.kt > 0) return false;   // gathered rows: the per-tile grid
    const TileChoice tc{2, 1, w->k == 2048 ? 4 : 0};
    const size_t lds = gemv_lds_bytes(MT, w->k, tc);
    if (lds > kMaxLds) return false;
    if (lm_mf_fits(MT, w->k)) {
        if constexpr (MT >= kLmMfMinRows)
            return launch_gemv_persist_k<MT, 0, true>((size_t)MT * w->k * 2 + (size_t)kLmMfWaves * kMfStageBytes, s, x,
                                                      m, w, y, bf16);
    }
    if constexpr (MT >= kLmMfMinRows) {
        return false;   // K does not allow the MFMA units: the per-tile grid
    } else {
        if constexpr (MT == 1) {
            if (tc.CPL == 4) return launch_gemv_persist_k<MT, 4, false>(lds, s, x, m, w, y, bf16);
        }
        return launch_gemv_persist_k<MT, 0, false>(lds, s, x, m, w, y, bf16);
    }
}

// The one-row LM head (4 chunks a lane) with the next step's fc fused
// (FCPL chunks a lane), on the same persistent grid as launch_lm_kernel.
template <bool BK, int FCPL>
static int launch_lm_fc_k(size_t lds, hipStream_t s, const uint16_t *h, const nvfp4_weight *w, int v, char *ws,
                          size_t wsb, int32_t *oi, float *om, const FcNext &fc) {
    constexpr int NW = lm_waves<1, 4>();
    auto kern = k_lmhead<1, lm_rows_per_slot<1>(), 4, BK, false, NW, false, false, false, FCPL>;
    const size_t l = lds;
    const int rc = allow_lds(reinterpret_cast<const void *>(kern), l, "lmhead_gemv_argmax_fc");
    if (rc) return rc;
    const int per_cu = blocks_per_cu(reinterpret_cast<const void *>(kern), 64 * NW, l);
    if (per_cu < 1)
        return fail(NVFP4_ERR_UNSUPPORTED, "lmhead_gemv_argmax_fc: a %d-thread workgroup does not fit on a CU", 64 * NW);
    // every workgroup resident at once: all but the last wait for its draft id
    const int cap = num_cus() * per_cu, nparts = (v + 15) / 16, grid = cap < nparts ? cap : nparts;
    if ((long)(NW - 1) * grid * kLmFcRows < fc.n) return kLmFcNoFit;   // rows past the wavefronts' share
    const size_t need = (size_t)kLmParts + sizeof(ArgPart) * (size_t)grid;
    if (need > wsb)
        return fail(NVFP4_ERR_WORKSPACE, "lmhead_gemv_argmax_fc: %d workgroups need %zu bytes of workspace, %zu available",
                    grid, need, wsb);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * NW), l, s, h, 1, w->codes, w->scales, w->global, v, w->k, ws, oi, om,
                       nullptr, nullptr, 0, EmbedOut{}, nullptr, 0, fc);
    return check_launch("lmhead_gemv_argmax_fc");
}
template <bool BK>
static int launch_lm_fc(size_t lds, hipStream_t s, const uint16_t *h, const nvfp4_weight *w, int v, char *ws,
                        size_t wsb, int32_t *oi, float *om, const FcNext &fc) {
    if (fc.k == 2048) return launch_lm_fc_k<BK, 1>(lds, s, h, w, v, ws, wsb, oi, om, fc);
    if (fc.k == 4096) return launch_lm_fc_k<BK, 2>(lds, s, h, w, v, ws, wsb, oi, om, fc);
    return fail(NVFP4_ERR_UNSUPPORTED, "lmhead_gemv_argmax_fc: fused fc needs k = 2048 or 4096, got %d", fc.k);
}

// The LM head keeps KS = 1 and R = 2 (8-row wavefront units); there are at
// most ceil(V / 16) partials.  A fixed chunk count when K = 2048.  fcn: the
// next step's fc fused into the one-row argmax (lmhead_gemv_argmax_fc).
template <int MT>
static int launch_lmhead_m(const uint16_t *h, int m, const nvfp4_weight *w, int v, char *ws, size_t wsb, int32_t *oi,
                           float *om, float *olp, const uint32_t *mask, int mask_words, const EmbedOut &emb, bool bk,
                           hipStream_t s, const FcNext *fcn = nullptr) {
    const TileChoice tc{2, 1, w->k == 2048 ? 4 : 0};
    const size_t lds = gemv_lds_bytes(MT, w->k, tc);
    const bool lp = olp != nullptr;
    if constexpr (MT == 1) {
        if (fcn != nullptr) {
            if (tc.CPL != 4 || lp || mask != nullptr || emb.table != nullptr)
                return fail(NVFP4_ERR_UNSUPPORTED, "lmhead_gemv_argmax_fc: the fused fc follows a plain one-row argmax "
                            "at k = 2048");
            return bk ? launch_lm_fc<true>(lds, s, h, w, v, ws, wsb, oi, om, *fcn)
                      : launch_lm_fc<false>(lds, s, h, w, v, ws, wsb, oi, om, *fcn);
        }
    }
    if (lm_mf_fits(MT, w->k)) {
        if constexpr (MT >= kLmMfMinRows) {
            const size_t lmf = (size_t)MT * w->k * 2 + (size_t)kLmMfWaves * kMfStageBytes;
            return launch_lm_variant<MT, 0, true>(bk, lp, lmf, s, h, m, w, v, ws, wsb, oi, om, olp, mask, mask_words, emb);
        }
    }
    if (tc.CPL == 4)
        return launch_lm_variant<MT, 4>(bk, lp, lds, s, h, m, w, v, ws, wsb, oi, om, olp, mask, mask_words, emb);
    return launch_lm_variant<MT, 0>(bk, lp, lds, s, h, m, w, v, ws, wsb, oi, om, olp, mask, mask_words, emb);
}

}  // namespace nvfp4

using namespace nvfp4;

static int gemv_common(const XRows &x, int32_t m, const nvfp4_weight *const *w, void *const *y, int count,
                       int32_t y_dtype, void *stream, const char *who) {
    if (count < 1 || count > kMaxGroups) return fail(NVFP4_ERR_ARG, "%s: count=%d outside 1..%d", who, count, kMaxGroups);
    if (!w) return fail(NVFP4_ERR_ARG, "%s: NULL weight list", who);
    if (m < 1 || m > 8) return fail(NVFP4_ERR_SHAPE, "%s: m=%d outside 1..8", who, m);
    if (y_dtype != NVFP4_OUT_F32 && y_dtype != NVFP4_OUT_BF16)
        return fail(NVFP4_ERR_ARG, "%s: unknown y_dtype %d", who, y_dtype);
    int total_n = 0;
    for (int i = 0; i < count; ++i) {
        int rc = validate_weight(w[i], who);
        if (rc) return rc;
        if (w[i]->k != w[0]->k)
            return fail(NVFP4_ERR_SHAPE, "%s: weight %d has k=%d, weight 0 has k=%d", who, i, w[i]->k, w[0]->k);
        if (w[i]->n > 0 && (!y || !y[i])) return fail(NVFP4_ERR_ARG, "%s: NULL output %d", who, i);
        if (w[i]->n > 0 && !aligned(y[i], 4)) return fail(NVFP4_ERR_ALIGN, "%s: output %d not 4-byte aligned", who, i);
        total_n += w[i]->n;
    }
    if (total_n == 0) return ok();   // empty outputs: nothing to read or write
    const int k = w[0]->k;
    if (x.kt > k) return fail(NVFP4_ERR_SHAPE, "%s: gathered prefix of %d elements exceeds k=%d", who, x.kt, k);
    if (x.kt < k && !x.x) return fail(NVFP4_ERR_ARG, "%s: NULL x", who);
    if (!aligned(x.x, 16)) return fail(NVFP4_ERR_ALIGN, "%s: x not 16-byte aligned", who);
    if ((size_t)k * 2 > kMaxLds)
        return fail(NVFP4_ERR_UNSUPPORTED, "%s: one activation row of k=%d exceeds the LDS", who, k);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const int bf16 = y_dtype == NVFP4_OUT_BF16;
    // activation rows are staged in LDS: rows that do not fit at once go in
    // groups of the most that do (each group streams the weights again)
    int grp = round_up_mt(m);
    while ((size_t)grp * k * 2 > kMaxLds) grp >>= 1;
    for (int r0 = 0; r0 < m; r0 += grp) {
        const int mg = m - r0 < grp ? m - r0 : grp;
        void *yg[kMaxGroups];
        for (int i = 0; i < count; ++i)
            yg[i] = w[i]->n > 0 ? static_cast<char *>(y[i]) + (size_t)r0 * w[i]->n * (bf16 ? 2 : 4) : nullptr;
        XRows xg = x;
        if (xg.x) xg.x += (size_t)r0 * (k - x.kt);
        if (xg.idx) xg.idx += r0;
        int rc;
        switch (round_up_mt(mg)) {
            case 1: rc = launch_gemv_m<1>(xg, mg, w, yg, count, bf16, s); break;
            case 2: rc = launch_gemv_m<2>(xg, mg, w, yg, count, bf16, s); break;
            case 4: rc = launch_gemv_m<4>(xg, mg, w, yg, count, bf16, s); break;
            default: rc = launch_gemv_m<8>(xg, mg, w, yg, count, bf16, s); break;
        }
        if (rc) return rc;
    }
    return NVFP4_OK;
}

extern "C" int w4a16_gemv(const uint16_t *x_bf16, int32_t m, const nvfp4_weight *w, void *y, int32_t y_dtype,
                          void *stream) {
    const nvfp4_weight *ws[1] = {w};
    void *ys[1] = {y};
    return gemv_common(xrows_plain(x_bf16), m, ws, ys, 1, y_dtype, stream, "w4a16_gemv");
}

extern "C" int w4a16_gemv_grouped(const uint16_t *x_bf16, int32_t m, const nvfp4_weight *const *w, void *const *y,
                                  int32_t count, int32_t y_dtype, void *stream) {
    return gemv_common(xrows_plain(x_bf16), m, w, y, count, y_dtype, stream, "w4a16_gemv_grouped");
}

extern "C" int w4a16_gemv_embed(const int32_t *idx, const uint16_t *table_bf16, int32_t table_vocab, int32_t hidden,
                                const uint16_t *x_rest_bf16, int32_t m, const nvfp4_weight *w, void *y,
                                int32_t y_dtype, void *stream) {
    const char *who = "w4a16_gemv_embed";
    if (!idx || !table_bf16) return fail(NVFP4_ERR_ARG, "%s: NULL idx or table", who);
    if (table_vocab < 1 || hidden < 32 || hidden % 32)
        return fail(NVFP4_ERR_SHAPE, "%s: need table_vocab >= 1 and hidden a positive multiple of 32 (vocab=%d "
                    "hidden=%d)", who, table_vocab, hidden);
    if (!aligned(table_bf16, 16) || !aligned(idx, 4))
        return fail(NVFP4_ERR_ALIGN, "%s: table needs 16-byte, idx 4-byte alignment", who);
    const nvfp4_weight *ws[1] = {w};
    void *ys[1] = {y};
    const XRows x{x_rest_bf16, idx, table_bf16, table_vocab, hidden};
    return gemv_common(x, m, ws, ys, 1, y_dtype, stream, who);
}

extern "C" size_t lmhead_gemv_argmax_workspace_bytes(int32_t m, int32_t vocab_rows) {
    if (vocab_rows < 1) return 0;
    const int mt = round_up_mt(m < 1 ? 1 : (m > 8 ? 8 : m));
    return (size_t)kLmParts + (size_t)sizeof(ArgPart) * mt * (size_t)((vocab_rows + 15) / 16);
}

static int lmhead_common(const uint16_t *h_bf16, int32_t m, const nvfp4_weight *w, int32_t vocab_rows,
                         int32_t *out_idx, float *out_max, float *out_lp, const uint32_t *mask, int32_t mask_words,
                         const EmbedOut &emb, void *workspace, size_t ws_bytes, uint32_t flags, void *stream,
                         const char *who, bool sized_by_grid = false, const FcNext *fcn = nullptr) {
    int rc = validate_weight(w, who);
    if (rc) return rc;
    if (!h_bf16 || !out_idx || !out_max) return fail(NVFP4_ERR_ARG, "%s: NULL h/out_idx/out_max", who);
    if (m < 1 || m > 8) return fail(NVFP4_ERR_SHAPE, "%s: m=%d outside 1..8", who, m);
    if (vocab_rows < 0) return fail(NVFP4_ERR_ARG, "%s: vocab_rows=%d < 0", who, vocab_rows);
    if (flags & ~NVFP4_ARGMAX_BF16_KEYS) return fail(NVFP4_ERR_ARG, "%s: unknown flags 0x%x", who, flags);
    const int v = (vocab_rows == 0 || vocab_rows > w->n) ? w->n : vocab_rows;
    if (v < 1) return fail(NVFP4_ERR_SHAPE, "%s: empty vocabulary", who);
    if (!aligned(h_bf16, 16) || !aligned(out_idx, 4) || !aligned(out_max, 4) || (out_lp && !aligned(out_lp, 4)))
        return fail(NVFP4_ERR_ALIGN, "%s: h needs 16-byte, outputs 4-byte alignment", who);
    const int mt = round_up_mt(m);
    if ((size_t)mt * w->k * 2 > kMaxLds)
        return fail(NVFP4_ERR_UNSUPPORTED, "%s: %d (rounded-up) rows x k=%d activations exceed LDS", who, mt, w->k);
    // the documented size covers any grid; a fixed scratch is checked
    // against the grid actually launched
    const size_t need = lmhead_gemv_argmax_workspace_bytes(m, v);
    if (!workspace || (!sized_by_grid && ws_bytes < need))
        return fail(NVFP4_ERR_WORKSPACE, "%s: workspace needs %zu bytes for %d rows", who, need, v);
    if (!aligned(workspace, 256)) return fail(NVFP4_ERR_ALIGN, "%s: workspace not 256-byte aligned", who);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    char *ws = reinterpret_cast<char *>(workspace);
    const bool bk = (flags & NVFP4_ARGMAX_BF16_KEYS) != 0;
    switch (mt) {
        case 1: return launch_lmhead_m<1>(h_bf16, m, w, v, ws, ws_bytes, out_idx, out_max, out_lp, mask, mask_words, emb, bk, s, fcn);
        case 2: return launch_lmhead_m<2>(h_bf16, m, w, v, ws, ws_bytes, out_idx, out_max, out_lp, mask, mask_words, emb, bk, s);
        case 4: return launch_lmhead_m<4>(h_bf16, m, w, v, ws, ws_bytes, out_idx, out_max, out_lp, mask, mask_words, emb, bk, s);
        default: return launch_lmhead_m<8>(h_bf16, m, w, v, ws, ws_bytes, out_idx, out_max, out_lp, mask, mask_words, emb, bk, s);
    }
}

extern "C" int lmhead_gemv_argmax(const uint16_t *h_bf16, int32_t m, const nvfp4_weight *w, int32_t vocab_rows,
                                  int32_t *out_idx, float *out_max, void *workspace, size_t ws_bytes,
                                  uint32_t flags, void *stream) {
    return lmhead_common(h_bf16, m, w, vocab_rows, out_idx, out_max, nullptr, nullptr, 0, EmbedOut{}, workspace, ws_bytes,
                         flags, stream, "lmhead_gemv_argmax");
}

extern "C" int lmhead_gemv_argmax_fc(const uint16_t *h_bf16, int32_t m, const nvfp4_weight *w, int32_t vocab_rows,
                                     int32_t *out_idx, float *out_max, void *workspace, size_t ws_bytes,
                                     uint32_t flags, const uint16_t *table_bf16, int32_t table_vocab, int32_t hidden,
                                     const uint16_t *x_rest_bf16, const nvfp4_weight *fc, void *y, int32_t y_dtype,
                                     void *stream) {
    const char *who = "lmhead_gemv_argmax_fc";
    int rc = validate_weight(fc, who);
    if (rc) return rc;
    const bool fuse = m == 1 && w != nullptr && w->k == 2048 && (fc->k == 2048 || fc->k == 4096) && fc->n > 0;
    if (!fuse) {
        // the two calls it stands for
        rc = lmhead_common(h_bf16, m, w, vocab_rows, out_idx, out_max, nullptr, nullptr, 0, EmbedOut{}, workspace,
                           ws_bytes, flags, stream, who);
        if (rc) return rc;
        return w4a16_gemv_embed(out_idx, table_bf16, table_vocab, hidden, x_rest_bf16, m, fc, y, y_dtype, stream);
    }
    // the fc's checks of w4a16_gemv_embed
    if (!table_bf16 || !y) return fail(NVFP4_ERR_ARG, "%s: NULL table or y", who);
    if (table_vocab < 1 || hidden < 32 || hidden % 32 || hidden > fc->k)
        return fail(NVFP4_ERR_SHAPE, "%s: need table_vocab >= 1 and hidden a positive multiple of 32 up to the fc's k "
                    "(vocab=%d hidden=%d k=%d)", who, table_vocab, hidden, fc->k);
    if (hidden < fc->k && !x_rest_bf16) return fail(NVFP4_ERR_ARG, "%s: NULL x_rest", who);
    if (y_dtype != NVFP4_OUT_F32 && y_dtype != NVFP4_OUT_BF16) return fail(NVFP4_ERR_ARG, "%s: unknown y_dtype %d", who, y_dtype);
    if (!aligned(table_bf16, 16) || !aligned(x_rest_bf16, 16) || !aligned(y, 4))
        return fail(NVFP4_ERR_ALIGN, "%s: table and x_rest need 16-byte, y 4-byte alignment", who);
    const FcNext f{fc->codes, fc->scales, fc->global, fc->n, fc->k, table_bf16, table_vocab, hidden, x_rest_bf16, y,
                   y_dtype == NVFP4_OUT_BF16 ? 1 : 0};
    rc = lmhead_common(h_bf16, m, w, vocab_rows, out_idx, out_max, nullptr, nullptr, 0, EmbedOut{}, workspace, ws_bytes,
                       flags, stream, who, false, &f);
    if (rc != kLmFcNoFit) return rc;
    // more fc rows than the LM head's grid serves: the two calls
    rc = lmhead_common(h_bf16, m, w, vocab_rows, out_idx, out_max, nullptr, nullptr, 0, EmbedOut{}, workspace, ws_bytes,
                       flags, stream, who);
    if (rc) return rc;
    return w4a16_gemv_embed(out_idx, table_bf16, table_vocab, hidden, x_rest_bf16, m, fc, y, y_dtype, stream);
}

extern "C" int lmhead_gemv_argmax_logprob(const uint16_t *h_bf16, int32_t m, const nvfp4_weight *w,
                                          int32_t vocab_rows, int32_t *out_idx, float *out_max, float *out_logprob,
                                          void *workspace, size_t ws_bytes, uint32_t flags, void *stream) {
    if (!out_logprob) return fail(NVFP4_ERR_ARG, "lmhead_gemv_argmax_logprob: NULL out_logprob");
    return lmhead_common(h_bf16, m, w, vocab_rows, out_idx, out_max, out_logprob, nullptr, 0, EmbedOut{}, workspace,
                         ws_bytes, flags, stream, "lmhead_gemv_argmax_logprob");
}

extern "C" int lmhead_gemv_argmax_masked(const uint16_t *h_bf16, int32_t m, const nvfp4_weight *w,
                                         int32_t vocab_rows, const uint32_t *allow_mask, int32_t mask_words,
                                         int32_t *out_idx, float *out_max, float *out_logprob, void *workspace,
                                         size_t ws_bytes, uint32_t flags, void *stream) {
    if (!allow_mask) return fail(NVFP4_ERR_ARG, "lmhead_gemv_argmax_masked: NULL allow_mask");
    if (mask_words < 0) return fail(NVFP4_ERR_ARG, "lmhead_gemv_argmax_masked: mask_words=%d < 0", mask_words);
    if (!aligned(allow_mask, 4)) return fail(NVFP4_ERR_ALIGN, "lmhead_gemv_argmax_masked: mask not 4-byte aligned");
    return lmhead_common(h_bf16, m, w, vocab_rows, out_idx, out_max, out_logprob, allow_mask, mask_words, EmbedOut{},
                         workspace, ws_bytes, flags, stream, "lmhead_gemv_argmax_masked");
}

extern "C" int lmhead_gemv_argmax_embed(const uint16_t *h_bf16, int32_t m, const nvfp4_weight *w, int32_t vocab_rows,
                                        const uint32_t *allow_mask, int32_t mask_words, int32_t *out_idx,
                                        float *out_max, float *out_logprob, const uint16_t *table_bf16,
                                        int32_t table_vocab, int32_t hidden, uint16_t *out_embed, int64_t out_stride,
                                        int32_t *id_log, void *workspace, size_t ws_bytes, uint32_t flags,
                                        void *stream) {
    const char *who = "lmhead_gemv_argmax_embed";
    if (!table_bf16 || !out_embed) return fail(NVFP4_ERR_ARG, "%s: NULL table or out_embed", who);
    if (table_vocab < 1 || hidden < 8 || hidden % 8)
        return fail(NVFP4_ERR_SHAPE, "%s: need table_vocab >= 1 and hidden %% 8 == 0 (vocab=%d hidden=%d)", who,
                    table_vocab, hidden);
    if (out_stride < hidden || out_stride % 8)
        return fail(NVFP4_ERR_SHAPE, "%s: out_stride=%lld must be >= hidden and a multiple of 8", who,
                    (long long)out_stride);
    if (!aligned(table_bf16, 16) || !aligned(out_embed, 16) || (id_log && !aligned(id_log, 4)))
        return fail(NVFP4_ERR_ALIGN, "%s: table/out_embed need 16-byte, id_log 4-byte alignment", who);
    if (allow_mask && (mask_words < 0 || !aligned(allow_mask, 4)))
        return fail(NVFP4_ERR_ARG, "%s: bad allow_mask (mask_words=%d)", who, mask_words);
    const EmbedOut emb{reinterpret_cast<const uint4 *>(table_bf16), reinterpret_cast<uint4 *>(out_embed), id_log,
                       out_stride / 8, table_vocab, hidden / 8};
    return lmhead_common(h_bf16, m, w, vocab_rows, out_idx, out_max, out_logprob, allow_mask,
                         allow_mask ? mask_words : 0, emb, workspace, ws_bytes, flags, stream, who);
}

// ------------------------------------------------------- no-allocation ----
// lmhead_gemv_argmax for callers that cannot allocate a workspace (graph
// capture, serving loops, harnesses that forbid allocation): the same
// kernels with their workspace in this static device array, one copy per
// device, held until the process ends.  Its counters (ticket, per-row packed
// maxima) are zero when the code object is loaded, cleared once more at
// set-up, and returned to zero by every call.
static __device__ __align__(256) unsigned char scratch[NVFP4_NOALLOC_SCRATCH_BYTES];

namespace {
struct ScratchTable {
    std::mutex mu;
    char *ptr[64] = {};   // device address of `scratch` per device (null until set up)
};
ScratchTable &scratch_table() {
    static ScratchTable t;
    return t;
}
}  // namespace

__global__ void k_scratch_clear(unsigned int *p, int words) {
    for (int i = threadIdx.x; i < words; i += blockDim.x) p[i] = 0u;
}

// Device address of this device's scratch: looked up once per device with
// that device current (the host-side name of the array is not a device
// address), its counters cleared on `s` by a fill kernel.
static int scratch_ptr(hipStream_t s, char **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(NVFP4_ERR_HIP, "lmhead_gemv_argmax_noalloc: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= 64) return fail(NVFP4_ERR_UNSUPPORTED, "lmhead_gemv_argmax_noalloc: device %d", dev);
    ScratchTable &t = scratch_table();
    std::lock_guard<std::mutex> lock(t.mu);
    if (!t.ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr)
            return fail(NVFP4_ERR_HIP, "lmhead_gemv_argmax_noalloc: scratch address: %s", hipGetErrorString(e));
        hipLaunchKernelGGL(k_scratch_clear, dim3(1), dim3(64), 0, s, reinterpret_cast<unsigned int *>(p), kLmParts / 4);
        const int rc = check_launch("lmhead_gemv_argmax_noalloc(clear)");
        if (rc) return rc;
        t.ptr[dev] = reinterpret_cast<char *>(p);
    }
    *out = t.ptr[dev];
    return NVFP4_OK;
}

extern "C" int lmhead_gemv_argmax_noalloc(const uint16_t *h_bf16, int32_t m, const nvfp4_weight *w,
                                          int32_t vocab_rows, int32_t *out_idx, float *out_max, uint32_t flags,
                                          void *stream) {
    char *p = nullptr;
    const int rc = scratch_ptr(reinterpret_cast<hipStream_t>(stream), &p);
    if (rc) return rc;
    return lmhead_common(h_bf16, m, w, vocab_rows, out_idx, out_max, nullptr, nullptr, 0, EmbedOut{}, p,
                         NVFP4_NOALLOC_SCRATCH_BYTES, flags, stream, "lmhead_gemv_argmax_noalloc", true);
}
