// bw_read.hip -- the bandwidth reference of the benchmark: a plain read of a device buffer with
// 16-byte non-temporal loads and nothing else (an xor of the words, one store per wave so the
// loads are kept), in two orders: grid-stride (the grid sweeps the buffer as one window) and
// contiguous chunks (workgroup b reads the b-th 1/grid of the buffer; measured a few per cent
// faster on MI355X).  It is not part of the GEMV library; bench.py times it beside the GEMV
// kernels, at several launch shapes, to state how much of the attainable HBM read rate they
// reach.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kUnroll = 4;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ void k_read(const u32x4 *__restrict__ p, int64_t n16, uint32_t *__restrict__ out)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    for (; i < n16; i += stride) {
        const u32x4 v = __builtin_nontemporal_load(p + i);
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    // fold the wave's words so every lane's loads feed the one store of its wave
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        acc ^= __shfl_xor(acc, off);
    if ((threadIdx.x & 63) == 0)
        out[(int64_t)blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64] = acc;
}

// workgroup b reads words [b per, (b + 1) per) with per = ceil(n16 / grid)
__global__ void k_read_chunk(const u32x4 *__restrict__ p, int64_t n16, uint32_t *__restrict__ out)
{
    const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const int64_t b0 = (int64_t)blockIdx.x * per, b1 = b0 + per < n16 ? b0 + per : n16;
    const int64_t nt = blockDim.x;
    int64_t i = b0 + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (kUnroll - 1) * nt < b1; i += kUnroll * nt) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            v[u] = __builtin_nontemporal_load(p + i + u * nt);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    for (; i < b1; i += nt) {
        const u32x4 v = __builtin_nontemporal_load(p + i);
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        acc ^= __shfl_xor(acc, off);
    if ((threadIdx.x & 63) == 0)
        out[(int64_t)blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64] = acc;
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16) from buf with a grid of `grid` workgroups of `threads` threads
// (a multiple of 64, at most 1024), in grid-stride order (chunked = 0) or in contiguous chunks
// per workgroup (chunked = 1).  out must hold grid * threads / 64 words.  Returns a hipError_t
// value (0 = launched).
int qgbw_read(const void *buf, int64_t bytes, void *out, int grid, int threads, int chunked,
              void *stream)
{
    if (!buf || !out || bytes <= 0 || bytes % 16 || grid < 1 || threads < 64 || threads > 1024 ||
        threads % 64 || (chunked != 0 && chunked != 1))
        return (int)hipErrorInvalidValue;
    if (chunked)
        hipLaunchKernelGGL(k_read_chunk, dim3(grid), dim3(threads), 0,
                           static_cast<hipStream_t>(stream), static_cast<const u32x4 *>(buf),
                           bytes / 16, static_cast<uint32_t *>(out));
    else
        hipLaunchKernelGGL(k_read, dim3(grid), dim3(threads), 0, static_cast<hipStream_t>(stream),
                           static_cast<const u32x4 *>(buf), bytes / 16,
                           static_cast<uint32_t *>(out));
    return (int)hipGetLastError();
}

}  // extern "C"
