// Peak-rate probes: the measured denominators reported beside the published
// MI355X figures (dense bf16 and f32 MFMA rate, HBM read bandwidth).  C ABI
// in include/convprobe.h.
//
// MFMA probe: every wave runs CH independent accumulator chains of one MFMA
// shape back to back, its operands held in registers (taken from a kernel
// argument so the compiler cannot fold them), and writes the sum of its
// accumulators once at the end.  Useful work = 2 * M * N * K per
// instruction.  HBM probe: a grid-stride streaming read of 16-byte vectors,
// eight in flight per lane, folded into one word per lane.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/convprobe.h"

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

constexpr int kThreads = 256;

template <int CH>
__global__ __launch_bounds__(kThreads) void mfma_bf16_probe(int iters, float v, float *sink)
{
    bf16x8_t a, b;
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)(v * (float)(threadIdx.x & 7));
        b[e] = (__bf16)(v * (float)(e + 1));
    }
    f32x16_t acc[CH];
    for (int c = 0; c < CH; ++c)
        for (int e = 0; e < 16; ++e) acc[c][e] = 0.0f;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int c = 0; c < CH; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    }
    float s = 0.0f;
    for (int c = 0; c < CH; ++c)
        for (int e = 0; e < 16; ++e) s += acc[c][e];
    sink[blockIdx.x * kThreads + threadIdx.x] = s;
}

template <int CH>
__global__ __launch_bounds__(kThreads) void mfma_bf16_16x16_probe(int iters, float v, float *sink)
{
    bf16x8_t a, b;
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)(v * (float)(threadIdx.x & 7));
        b[e] = (__bf16)(v * (float)(e + 1));
    }
    f32x4_t acc[CH];
    for (int c = 0; c < CH; ++c)
        for (int e = 0; e < 4; ++e) acc[c][e] = 0.0f;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int c = 0; c < CH; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
    }
    float s = 0.0f;
    for (int c = 0; c < CH; ++c)
        for (int e = 0; e < 4; ++e) s += acc[c][e];
    sink[blockIdx.x * kThreads + threadIdx.x] = s;
}

// LDS read rate: every lane reads 16 bytes per instruction from a 16 KB
// region, consecutive lanes consecutive 16-byte slots (no bank conflict),
// eight reads in flight.
__global__ __launch_bounds__(kThreads) void lds_read_probe(int iters, float *sink)
{
    __shared__ __attribute__((aligned(16))) float buf[4096];
    for (int i = threadIdx.x; i < 4096; i += kThreads) buf[i] = (float)i;
    __syncthreads();
    typedef __attribute__((ext_vector_type(4))) float v4;
    const v4 *p = reinterpret_cast<const v4 *>(buf);
    v4 acc = {0.f, 0.f, 0.f, 0.f};
    int idx = threadIdx.x & 63;
    for (int i = 0; i < iters; ++i) {
        v4 r[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) r[u] = p[(idx + u * 64) & 1023];
#pragma unroll
        for (int u = 0; u < 8; ++u) acc += r[u];
        idx = (idx + 7 * 64) & 1023;
    }
    sink[blockIdx.x * kThreads + threadIdx.x] = acc.x + acc.y + acc.z + acc.w;
}

template <int CH>
__global__ __launch_bounds__(kThreads) void mfma_f32_probe(int iters, float v, float *sink)
{
    const float a = v * (float)(threadIdx.x & 7), b = v * 0.5f;
    f32x4_t acc[CH];
    for (int c = 0; c < CH; ++c)
        for (int e = 0; e < 4; ++e) acc[c][e] = 0.0f;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int c = 0; c < CH; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[c], 0, 0, 0);
    }
    float s = 0.0f;
    for (int c = 0; c < CH; ++c)
        for (int e = 0; e < 4; ++e) s += acc[c][e];
    sink[blockIdx.x * kThreads + threadIdx.x] = s;
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void hbm_read_probe(const u32x4_t *p, int64_t n, uint32_t *sink)
{
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    uint32_t h = 0;
    for (; i + 7 * stride < n; i += 8 * stride) {
        u32x4_t v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
        for (int u = 0; u < 8; ++u) h ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n; i += stride) {
        const u32x4_t a = p[i];
        h ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    sink[blockIdx.x * kThreads + threadIdx.x] = h;
}

constexpr int kChainsBf16 = 8;
constexpr int kChainsF32 = 8;

}  // namespace

extern "C" {

int32_t conv_probe_threads(void) { return kThreads; }

int32_t conv_probe_mfma(int32_t kind, int32_t iters, int32_t grid, void *sink, void *stream, double *flop)
{
    if (kind < 0 || kind > 3 || iters < 1 || grid < 1 || !sink) return (int32_t)hipErrorInvalidValue;
    (void)hipGetLastError();
    const double waves = (double)grid * (kThreads / 64);
    if (kind == 2) {
        hipLaunchKernelGGL(mfma_bf16_16x16_probe<kChainsBf16>, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream,
                           iters, 0.0f, (float *)sink);
        if (flop) *flop = waves * iters * kChainsBf16 * (2.0 * 16 * 16 * 32);
    } else if (kind == 3) {
        hipLaunchKernelGGL(lds_read_probe, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream, iters, (float *)sink);
        if (flop) *flop = waves * iters * 8 * 1024.0;   // bytes read from LDS
    } else if (kind == 0) {
        hipLaunchKernelGGL(mfma_bf16_probe<kChainsBf16>, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream, iters,
                           0.0f, (float *)sink);
        if (flop) *flop = waves * iters * kChainsBf16 * (2.0 * 32 * 32 * 16);
    } else {
        hipLaunchKernelGGL(mfma_f32_probe<kChainsF32>, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream, iters,
                           0.0f, (float *)sink);
        if (flop) *flop = waves * iters * kChainsF32 * (2.0 * 16 * 16 * 4);
    }
    return (int32_t)hipGetLastError();
}

int32_t conv_probe_hbm_read(const void *buf, int64_t bytes, int32_t grid, void *sink, void *stream)
{
    if (!buf || !sink || bytes < 16 || (bytes & 15) || ((uintptr_t)buf & 15) || grid < 1)
        return (int32_t)hipErrorInvalidValue;
    (void)hipGetLastError();
    hipLaunchKernelGGL(hbm_read_probe, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream, (const u32x4_t *)buf,
                       bytes / 16, (uint32_t *)sink);
    return (int32_t)hipGetLastError();
}

}  // extern "C"
