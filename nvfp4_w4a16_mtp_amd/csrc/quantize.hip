// NVFP4 quantizer: the global-absmax pass and the block-encode pass that
// new.rs (`MtpHead::new`) resolves as `nvfp4_global_absmax` and
// `quantize_bf16_to_nvfp4` and runs once per weight matrix at load time.
//
// Pass 1 streams the bf16 tensor once (16-byte loads, four in flight per
// thread), keeps the largest |w| as an integer (non-negative bf16
// magnitudes order like unsigned integers) and folds it into the global
// struct with one atomic max per workgroup (at most four workgroups per CU,
// each striding over the tensor).  Pass 2 streams it again: one thread
// encodes 32 consecutive elements of a row (two 16-element blocks) from four
// 16-byte loads into one 16-byte code store and one 2-byte scale store.
// Every fp32 operation is a single correctly rounded IEEE operation (no
// contraction, division is the correctly rounded one), and the E2M1
// rounding is the hardware convert, which equals the threshold rounding on
// every finite input, so the result is bit-identical to the definition.
#include "common.hpp"

#pragma clang fp contract(off)

namespace nvfp4 {

// Clears the global struct (a kernel instead of a memset so that the call
// can be captured in a graph).
__global__ void k_quant_clear(nvfp4_global *g) {
    if (threadIdx.x == 0) {
        g->dec = 0.0f;
        g->enc = 0.0f;
        g->amax = 0.0f;
        g->flags = 0u;
    }
}

constexpr int kAbsmaxLoads = 4;

__global__ __launch_bounds__(256) void k_quant_absmax(const uint4 *__restrict__ w, int64_t nvec,
                                                     nvfp4_global *g) {
    uint32_t mx = 0;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    // kAbsmaxLoads loads in flight per thread; an index past the end re-reads
    // the round's first vector (harmless for a maximum) instead of branching
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nvec; i += kAbsmaxLoads * stride) {
        uint4 v[kAbsmaxLoads];
#pragma unroll
        for (int u = 0; u < kAbsmaxLoads; ++u) {
            const int64_t j = i + u * stride;
            v[u] = w[j < nvec ? j : i];
        }
#pragma unroll
        for (int u = 0; u < kAbsmaxLoads; ++u) {
            const uint32_t a = v[u].x & 0x7FFF7FFFu, b = v[u].y & 0x7FFF7FFFu, c = v[u].z & 0x7FFF7FFFu,
                           d = v[u].w & 0x7FFF7FFFu;
            mx = max(mx, max(max(a & 0xFFFFu, a >> 16), max(b & 0xFFFFu, b >> 16)));
            mx = max(mx, max(max(c & 0xFFFFu, c >> 16), max(d & 0xFFFFu, d >> 16)));
        }
    }
    // wave max, workgroup max, then one atomic per workgroup on the fp32 bit
    // pattern of amax (atomics on one word serialize: keep them few)
    __shared__ uint32_t wmax[4];
    for (int off = 32; off > 0; off >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, off, 64));
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = mx;
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t m4 = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
        if (m4) atomicMax(reinterpret_cast<unsigned int *>(&g->amax), m4 << 16);
    }
}

// Nearest E4M3FN byte to s >= 0: ties to even mantissa, subnormals kept,
// saturating at 448 (0x7E), never NaN.  Integer rounding of the fp32
// mantissa for normals, an exact power-of-two rescale plus rint below 2^-6.
__device__ __forceinline__ uint32_t e4m3_rne_sat(float s) {
    if (!(s > 0.0f)) return 0u;
    if (s >= 448.0f) return 0x7Eu;
    uint32_t u = __float_as_uint(s);
    int e = (int)(u >> 23) - 127;
    if (e < -6) return (uint32_t)__builtin_rintf(s * 512.0f);   // multiples of 2^-9, result <= 8
    uint32_t mant = u & 0x7FFFFFu;
    uint32_t keep = mant >> 20, rest = mant & 0xFFFFFu;
    keep += (rest > 0x80000u) || (rest == 0x80000u && (keep & 1u));
    uint32_t code = ((uint32_t)(e + 7) << 3) + keep;            // a carry moves into the exponent
    return code > 0x7Eu ? 0x7Eu : code;
}

// Nearest E2M1 codes to two fp32 values, written as byte SEL of `into` (low
// nibble = a): v_cvt_scalef32_pk_fp4_f32 with scale 1 rounds to nearest
// with ties to the even code, saturates at 6 and keeps the sign bit of a
// zero result.  Compared on the GPU for every non-NaN fp32 bit pattern
// (and both operand positions) with the threshold form
//   |v| > 0.25, >= 0.75, > 1.25, >= 1.75, > 2.5, >= 3.5, > 5  (count = magnitude code)
// plus the sign bit of v: no difference.  NaN inputs differ; they arise only
// from an infinite input times a zero factor, which encode_block handles
// apart.
template <int SEL>
__device__ __forceinline__ uint32_t e2m1_pair(uint32_t into, float a, float b) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(into, a, b, 1.0f, SEL);
}

__device__ __forceinline__ void global_scales(const nvfp4_global *g, float &enc, float &dec) {
    float amax = __builtin_nontemporal_load(&g->amax);
    enc = 0.0f;
    if (amax > 0.0f) {
        enc = 2688.0f / amax;
        if (enc > 3.402823466e38f) enc = 3.402823466e38f;
    }
    dec = amax / 2688.0f;
}

// Encodes one 16-element block held as eight bf16 pairs; returns the 8 code
// bytes (two dwords) and the scale byte.
__device__ __forceinline__ uint32_t encode_block(const uint32_t (&p)[8], float enc, uint32_t &lo, uint32_t &hi) {
    uint32_t bm = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t a = p[i] & 0x7FFF7FFFu;
        bm = max(bm, max(a & 0xFFFFu, a >> 16));
    }
    float bmax = bf16_bits_to_f32(bm);
    float t = bmax * enc;
    float s32 = t / 6.0f;
    uint32_t se = e4m3_rne_sat(s32);
    float sf = e4m3_to_f32(se);
    float inv = 0.0f;
    if (sf > 0.0f) {
        inv = enc / sf;
        if (inv > 3.402823466e38f) inv = 3.402823466e38f;
    }
    float v[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        v[2 * i] = bf16_bits_to_f32(p[i] & 0xFFFFu) * inv;
        v[2 * i + 1] = bf16_bits_to_f32(p[i] >> 16) * inv;
    }
    uint32_t out[2];
    if (inv == 0.0f) {
        // every product is a zero, or NaN for an infinite input (outside the
        // quantizer's domain): the code is the sign nibble alone, as the
        // threshold rounding gives it, NaN included
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            uint32_t o = 0u;
#pragma unroll
            for (int i = 0; i < 8; ++i) o |= ((__float_as_uint(v[8 * h + i]) >> 28) & 8u) << (4 * i);
            out[h] = o;
        }
    } else {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            uint32_t o = 0u;
            o = e2m1_pair<0>(o, v[8 * h + 0], v[8 * h + 1]);
            o = e2m1_pair<1>(o, v[8 * h + 2], v[8 * h + 3]);
            o = e2m1_pair<2>(o, v[8 * h + 4], v[8 * h + 5]);
            o = e2m1_pair<3>(o, v[8 * h + 6], v[8 * h + 7]);
            out[h] = o;
        }
    }
    lo = out[0];
    hi = out[1];
    return se;
}

__global__ __launch_bounds__(256) void k_quant_encode(const uint4 *__restrict__ w, int64_t nthreads,
                                                     uint4 *__restrict__ codes, uint16_t *__restrict__ scales,
                                                     nvfp4_global *g) {
    float enc, dec;
    global_scales(g, enc, dec);
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t first = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (first == 0) {
        g->enc = enc;
        g->dec = dec;
    }
    for (int64_t t = first; t < nthreads; t += stride) {
        // 32 consecutive elements of one row (k % 32 == 0): four 16-byte loads
        uint4 v0 = w[4 * t], v1 = w[4 * t + 1], v2 = w[4 * t + 2], v3 = w[4 * t + 3];
        uint32_t b0[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
        uint32_t b1[8] = {v2.x, v2.y, v2.z, v2.w, v3.x, v3.y, v3.z, v3.w};
        uint4 c;
        uint32_t s0 = encode_block(b0, enc, c.x, c.y);
        uint32_t s1 = encode_block(b1, enc, c.z, c.w);
        codes[t] = c;
        scales[t] = (uint16_t)(s0 | (s1 << 8));
    }
}

constexpr int kAbsmaxPerCu = 4;

static int grid_for(int64_t items, int per_cu) {
    int64_t blocks = (items + 255) / 256;
    int64_t cap = (int64_t)num_cus() * per_cu;
    if (blocks > cap) blocks = cap;
    return (int)(blocks < 1 ? 1 : blocks);
}

}  // namespace nvfp4

using namespace nvfp4;

extern "C" int nvfp4_quantize(const uint16_t *w_bf16, int32_t n, int32_t k, uint8_t *codes,
                              uint8_t *scales, nvfp4_global *global, void *stream) {
    if (!w_bf16 || !codes || !scales || !global) return fail(NVFP4_ERR_ARG, "nvfp4_quantize: NULL pointer");
    if (n < 1 || k < 32 || k % 32) return fail(NVFP4_ERR_SHAPE, "nvfp4_quantize: need n >= 1, k >= 32, k %% 32 == 0 (n=%d k=%d)", n, k);
    if ((int64_t)n * k >= ((int64_t)1 << 40)) return fail(NVFP4_ERR_SHAPE, "nvfp4_quantize: tensor too large");
    if (!aligned(w_bf16, 16) || !aligned(codes, 16) || !aligned(scales, 2) || !aligned(global, 16))
        return fail(NVFP4_ERR_ALIGN, "nvfp4_quantize: w/codes/global need 16-byte and scales 2-byte alignment");
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const int64_t count = (int64_t)n * k;
    hipLaunchKernelGGL(k_quant_clear, dim3(1), dim3(64), 0, s, global);
    int rc = check_launch("nvfp4_quantize(clear)");
    if (rc) return rc;
    const int64_t nvec = count / 8;
    hipLaunchKernelGGL(k_quant_absmax, dim3(grid_for(nvec, kAbsmaxPerCu)), dim3(256), 0, s,
                       reinterpret_cast<const uint4 *>(w_bf16), nvec, global);
    rc = check_launch("nvfp4_quantize(absmax)");
    if (rc) return rc;
    const int64_t nthreads = count / 32;
    hipLaunchKernelGGL(k_quant_encode, dim3(grid_for(nthreads, 16)), dim3(256), 0, s,
                       reinterpret_cast<const uint4 *>(w_bf16), nthreads, reinterpret_cast<uint4 *>(codes),
                       reinterpret_cast<uint16_t *>(scales), global);
    return check_launch("nvfp4_quantize(encode)");
}
