// Microbenchmarks for the attainable MFMA and HBM peaks of one gfx950 GPU
// (declared in include/atf_probes.h).  Not part of the attention path.
#include <hip/hip_runtime.h>

#include "../../include/atf_probes.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// 8 independent accumulator chains per wave: the MFMA pipe never waits for a
// result, so the rate is the matrix unit's own.
__global__ __launch_bounds__(256) void mfma_probe_kernel(const u32x4 *operands, float *sink, int iters) {
    const bf16x8_t a = __builtin_bit_cast(bf16x8_t, operands[0]);
    const bf16x8_t b = __builtin_bit_cast(bf16x8_t, operands[1]);
    f32x16_t acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[j][r];
    sink[(long long)blockIdx.x * 256 + threadIdx.x] = s;
}

// One pass over the buffer, 16-byte loads, 4 in flight per thread.
__global__ __launch_bounds__(256) void hbm_read_probe_kernel(const u32x4 *buf, long long n16, unsigned *sink) {
    const long long stride = (long long)gridDim.x * 256;
    u32x4 x = (u32x4){0u, 0u, 0u, 0u};
    long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4 v0 = buf[i], v1 = buf[i + stride], v2 = buf[i + 2 * stride], v3 = buf[i + 3 * stride];
        x ^= v0 ^ v1 ^ v2 ^ v3;
    }
    for (; i < n16; i += stride) x ^= buf[i];
    sink[(long long)blockIdx.x * 256 + threadIdx.x] = x.x ^ x.y ^ x.z ^ x.w;
}

}  // namespace

extern "C" {

int atf_probe_mfma_bf16(const void *operands, float *sink, int32_t n_wg, int32_t iters,
                        atf_probe_stream_t stream) {
    if (!operands || !sink || n_wg < 1 || iters < 1 || ((uintptr_t)operands & 15u)) return 1;
    mfma_probe_kernel<<<n_wg, 256, 0, (hipStream_t)stream>>>((const u32x4 *)operands, sink, iters);
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

int atf_probe_hbm_read(const void *buf, size_t bytes, uint32_t *sink, int32_t n_wg, atf_probe_stream_t stream) {
    if (!buf || !sink || n_wg < 1 || ((uintptr_t)buf & 15u) || bytes == 0 || bytes % (64 * 256 * 16) != 0)
        return 1;
    hbm_read_probe_kernel<<<n_wg, 256, 0, (hipStream_t)stream>>>((const u32x4 *)buf, (long long)(bytes / 16),
                                                                  (unsigned *)sink);
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // extern "C"
