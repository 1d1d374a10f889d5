// Embedding rows of the draft tokens: the `embed_from_argmax` step of
// mtp_head.rs (`MtpHead` fields: the kernel that turns the device-side argmax
// into the next draft step's input and stores the draft id on the device for
// deferred readback), so a chain of draft steps runs without a host round
// trip.  One workgroup per token copies its bf16 row in 16-byte units.
#include "common.hpp"

namespace nvfp4 {

__global__ __launch_bounds__(256) void k_embed(const int32_t *__restrict__ idx, const uint4 *__restrict__ table,
                                              int vocab, int units, uint4 *__restrict__ out, int64_t out_stride_units,
                                              int32_t *__restrict__ id_log) {
    const int i = blockIdx.x;
    const int id = idx[i];
    const bool in = id >= 0 && id < vocab;
    const uint4 *src = table + (size_t)(in ? id : 0) * units;
    uint4 *dst = out + (size_t)i * out_stride_units;
    for (int u = threadIdx.x; u < units; u += blockDim.x) dst[u] = in ? src[u] : make_uint4(0, 0, 0, 0);
    if (threadIdx.x == 0 && id_log != nullptr) id_log[i] = id;
}

}  // namespace nvfp4

using namespace nvfp4;

extern "C" int embed_from_argmax(const int32_t *idx, int32_t m, const uint16_t *table_bf16, int32_t vocab,
                                 int32_t hidden, uint16_t *out_bf16, int64_t out_stride, int32_t *id_log,
                                 void *stream) {
    if (m == 0) return ok();
    if (!idx || !table_bf16 || !out_bf16) return fail(NVFP4_ERR_ARG, "embed_from_argmax: NULL idx/table/out");
    if (m < 0 || vocab < 1 || hidden < 8 || hidden % 8)
        return fail(NVFP4_ERR_SHAPE, "embed_from_argmax: need m >= 0, vocab >= 1, hidden %% 8 == 0 (m=%d vocab=%d "
                    "hidden=%d)", m, vocab, hidden);
    if (out_stride < hidden || out_stride % 8)
        return fail(NVFP4_ERR_SHAPE, "embed_from_argmax: out_stride=%lld must be >= hidden and a multiple of 8",
                    (long long)out_stride);
    if (!aligned(table_bf16, 16) || !aligned(out_bf16, 16) || !aligned(idx, 4) || (id_log && !aligned(id_log, 4)))
        return fail(NVFP4_ERR_ALIGN, "embed_from_argmax: table/out need 16-byte, idx/id_log 4-byte alignment");
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(k_embed, dim3(m), dim3(256), 0, s, idx, reinterpret_cast<const uint4 *>(table_bf16), vocab,
                       hidden / 8, reinterpret_cast<uint4 *>(out_bf16), out_stride / 8, id_log);
    return check_launch("embed_from_argmax");
}
