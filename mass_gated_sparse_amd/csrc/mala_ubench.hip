// Microbenchmarks of the ceilings the MALA kernels run against on gfx950:
// dense bf16 MFMA rate, LDS read bandwidth (plain 16-byte reads and the
// transposing 8-byte reads), HBM streaming read bandwidth, and the rate of
// the hardware exp2 (the transcendental behind every kept score).  Built into a
// separate library (libmala_ubench.so); not part of the operator.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mala_device.hpp"

using namespace mala;

// 8 independent 32x32x16 accumulation chains per wave.
__global__ __launch_bounds__(256) void ub_mfma(const uint32_t* __restrict__ seed, float* __restrict__ out, int iters) {
    const int lane = threadIdx.x & 63;
    u32x4 a = {seed[lane], seed[lane + 1], seed[lane + 2], seed[lane + 3]};
    u32x4 b = {seed[lane + 4], seed[lane + 5], seed[lane + 6], seed[lane + 7]};
    f32x16 acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] = mfma32(a, b, acc[c]);
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[c][r];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Each wave reads 16 B per lane per instruction from a 64 KiB LDS buffer in a
// conflict-free pattern (16 consecutive lanes cover 256 contiguous bytes).
__global__ __launch_bounds__(256) void ub_lds(uint32_t* __restrict__ out, int iters) {
    __shared__ __attribute__((aligned(16))) uint8_t buf[65536];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int i = tid; i < 65536 / 4; i += 256) reinterpret_cast<uint32_t*>(buf)[i] = i;
    __syncthreads();
    u32x4 x = {0u, 0u, 0u, 0u};
    int off = wave * 4096 + lane * 16;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const u32x4 y = *reinterpret_cast<const u32x4*>(buf + ((off + u * 1024) & 65535));
            x[0] ^= y[0]; x[1] ^= y[1]; x[2] ^= y[2]; x[3] ^= y[3];
        }
        off += 8192;
    }
    out[blockIdx.x * blockDim.x + tid] = x[0] ^ x[1] ^ x[2] ^ x[3];
}

// Transposing 8-byte reads in the operand pattern used for V^T / K^T / Q^T / dO^T.
__global__ __launch_bounds__(256) void ub_lds_tr(uint32_t* __restrict__ out, int iters) {
    __shared__ __attribute__((aligned(1024))) uint8_t buf[65536];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int i = tid; i < 65536 / 4; i += 256) reinterpret_cast<uint32_t*>(buf)[i] = i;
    __syncthreads();
    uint32_t x = 0;
    for (int i = 0; i < iters; ++i) {
        const uint8_t* tile = buf + (((i + wave) & 3) << 14);  // four 16 KiB tiles of 64 rows
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const u32x4 y = tr_operand(tile, 16 * u, u, lane);
            x ^= y[0] ^ y[1] ^ y[2] ^ y[3];
        }
    }
    out[blockIdx.x * blockDim.x + tid] = x;
}

// Streaming read of n 16-byte vectors, grid-stride.
__global__ __launch_bounds__(256) void ub_hbm(const u32x4* __restrict__ src, long n, uint32_t* __restrict__ out) {
    uint32_t x = 0;
    for (long i = long(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += long(gridDim.x) * blockDim.x) {
        const u32x4 y = __builtin_nontemporal_load(src + i);
        x ^= y[0] ^ y[1] ^ y[2] ^ y[3];
    }
    out[blockIdx.x * blockDim.x + threadIdx.x] = x;
}

// Streaming read with U independent 16-byte loads in flight per thread: each
// thread reads vectors i, i + S, ..., i + (U-1) S of a chunk (S = threads in
// the grid), then moves U*S on; n must be a multiple of U*S.
template <int U>
__global__ __launch_bounds__(256) void ub_hbm_unroll(const u32x4* __restrict__ src, long n, uint32_t* __restrict__ out) {
    const long S = long(gridDim.x) * blockDim.x;
    uint32_t x = 0;
    for (long base = long(blockIdx.x) * blockDim.x + threadIdx.x; base < n; base += U * S) {
        u32x4 y[U];
#pragma unroll
        for (int u = 0; u < U; ++u) y[u] = __builtin_nontemporal_load(src + base + u * S);
#pragma unroll
        for (int u = 0; u < U; ++u) x ^= y[u][0] ^ y[u][1] ^ y[u][2] ^ y[u][3];
    }
    out[blockIdx.x * blockDim.x + threadIdx.x] = x;
}

// 8 independent chains of x = exp2(-x) per thread: one v_exp_f32 per step
// (the negation is a source modifier); x stays in (0.5, 1).
__global__ __launch_bounds__(256) void ub_exp(const uint32_t* __restrict__ seed, float* __restrict__ out, int iters) {
    const int tid = threadIdx.x;
    float x[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) x[c] = 0.5f + float(seed[(tid + c) & 255] & 0xffffu) * (0.5f / 65536.f);
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int c = 0; c < 8; ++c) x[c] = fast_exp2(-x[c]);
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) s += x[c];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

extern "C" {
// Each runs the kernel once on `stream`; sizes are validated by the caller.
int ubench_mfma(const void* seed, void* out, int blocks, int iters, void* stream) {
    hipLaunchKernelGGL(ub_mfma, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const uint32_t*)seed, (float*)out,
                       iters);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}
int ubench_lds(void* out, int blocks, int iters, void* stream) {
    hipLaunchKernelGGL(ub_lds, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (uint32_t*)out, iters);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}
int ubench_lds_tr(void* out, int blocks, int iters, void* stream) {
    hipLaunchKernelGGL(ub_lds_tr, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (uint32_t*)out, iters);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}
int ubench_exp(const void* seed, void* out, int blocks, int iters, void* stream) {
    hipLaunchKernelGGL(ub_exp, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const uint32_t*)seed, (float*)out,
                       iters);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}
// unroll 4 or 8; n16 must be a multiple of unroll * blocks * 256
int ubench_hbm_unroll(const void* src, long n16, void* out, int blocks, int unroll, void* stream) {
    if (unroll == 4)
        hipLaunchKernelGGL(ub_hbm_unroll<4>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const u32x4*)src, n16,
                           (uint32_t*)out);
    else if (unroll == 8)
        hipLaunchKernelGGL(ub_hbm_unroll<8>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const u32x4*)src, n16,
                           (uint32_t*)out);
    else
        return int(hipErrorInvalidValue);
    return int(hipGetLastError());
}

int ubench_hbm(const void* src, long n16, void* out, int blocks, void* stream) {
    hipLaunchKernelGGL(ub_hbm, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const u32x4*)src, n16,
                       (uint32_t*)out);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}
}
