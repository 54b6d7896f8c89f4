// mlp.hip -- the activation between the coded gate/up projections and the
// coded down projection of a SwiGLU MLP ("Unweight: Compressing LLM Weights
// for Faster Inference", section "Overlapping Work Across Transformer
// Layers": the down projection consumes gate, activation and up).
//
// h = fp16(silu(g) * u) with silu(z) = z / (1 + e^-z), in fp32, rounded to
// nearest even: the fp32 outputs of the two GEMVs become the fp16
// activations the down projection reads.  Elementwise, four per thread when
// the buffers allow 16-byte accesses.
#include "kernels.h"

namespace {

__device__ __forceinline__ _Float16 swiglu1(float g, float u)
{
    return (_Float16)(g / (1.0f + __expf(-g)) * u);
}

__global__ __launch_bounds__(256) void k_swiglu4(const float4 *g, const float4 *u, uint2 *h, int64_t n4)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n4) return;
    const float4 a = g[i], b = u[i];
    const _Float16 r0 = swiglu1(a.x, b.x), r1 = swiglu1(a.y, b.y), r2 = swiglu1(a.z, b.z), r3 = swiglu1(a.w, b.w);
    h[i] = make_uint2((uint32_t)__builtin_bit_cast(uint16_t, r0) | ((uint32_t)__builtin_bit_cast(uint16_t, r1) << 16),
                      (uint32_t)__builtin_bit_cast(uint16_t, r2) | ((uint32_t)__builtin_bit_cast(uint16_t, r3) << 16));
}

__global__ __launch_bounds__(256) void k_swiglu1(const float *g, const float *u, uint16_t *h, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    h[i] = __builtin_bit_cast(uint16_t, swiglu1(g[i], u[i]));
}

}  // namespace

hipError_t lw_launch_swiglu(const float *g, const float *u, uint16_t *h, int64_t n, hipStream_t s)
{
    const bool vec = n % 4 == 0 && reinterpret_cast<uintptr_t>(g) % 16 == 0 &&
                     reinterpret_cast<uintptr_t>(u) % 16 == 0 && reinterpret_cast<uintptr_t>(h) % 8 == 0;
    if (vec) {
        const int64_t n4 = n / 4;
        hipLaunchKernelGGL(k_swiglu4, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s,
                           reinterpret_cast<const float4 *>(g), reinterpret_cast<const float4 *>(u),
                           reinterpret_cast<uint2 *>(h), n4);
    } else {
        hipLaunchKernelGGL(k_swiglu1, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, g, u, h, n);
    }
    return hipGetLastError();
}
