// rd_ceiling.hip -- measurement probes, not part of the reduction library:
// the bandwidth a trivial kernel reaches on this GPU, reported beside the
// reductions' fraction of the published 8 TB/s.
//
//   read:  every lane streams 16-byte nontemporal loads in grid-stride
//          order, 4 in flight, and writes one float (its sum) at the end so
//          that the loads are not dead code;
//   read_pieces: workgroup b reads the b-th piece of steps x 4096 chunks
//          (16 loads in flight per lane, each load instruction of the
//          workgroup 4 KB of adjacent chunks), then writes one float --
//          many short-lived workgroups each streaming one contiguous piece,
//          the shape of the library's row reduction; steps = 1 is one
//          16-load step per lane;
//   copy:  every lane copies 16-byte chunks with nontemporal loads and
//          stores, grid-stride; or (copy_flat) one chunk per lane, a grid of
//          as many lanes as chunks -- on MI355X the faster of the two by far
//          (measured 6.5-6.8 TB/s with 64-thread workgroups against 5.1-5.4
//          grid-stride).
// Only whole float4s are touched: n is rounded down to a multiple of 4.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rd_ceiling.h"

namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void read_kernel(const v4f* __restrict__ x, int64_t n4,
                                                   float* __restrict__ sink) {
    const int64_t tid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t stride = int64_t(gridDim.x) * blockDim.x;
    v4f a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
    int64_t i = tid;
    for (; i + 3 * stride < n4; i += 4 * stride) {
        const v4f v0 = __builtin_nontemporal_load(x + i);
        const v4f v1 = __builtin_nontemporal_load(x + i + stride);
        const v4f v2 = __builtin_nontemporal_load(x + i + 2 * stride);
        const v4f v3 = __builtin_nontemporal_load(x + i + 3 * stride);
        a += v0 + v2;
        b += v1 + v3;
    }
    for (; i < n4; i += stride) a += __builtin_nontemporal_load(x + i);
    a += b;
    sink[tid] = (a.x + a.y) + (a.z + a.w);
}

__global__ __launch_bounds__(256) void copy_kernel(const v4f* __restrict__ x, v4f* __restrict__ y,
                                                   int64_t n4) {
    const int64_t stride = int64_t(gridDim.x) * blockDim.x;
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n4; i += stride)
        __builtin_nontemporal_store(__builtin_nontemporal_load(x + i), y + i);
}

// workgroup b: chunks [b*P, (b+1)*P), P = steps * 16 * 256, 16 loads in
// flight per lane; every load is checked against n4
__global__ __launch_bounds__(256) void read_pieces_kernel(const v4f* __restrict__ x, int64_t n4,
                                                          int32_t steps,
                                                          float* __restrict__ sink) {
    constexpr int U = 16;
    const int64_t base = int64_t(blockIdx.x) * steps * (U * 256) + threadIdx.x;
    v4f a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < steps; ++s) {
        const int64_t i0 = base + int64_t(s) * (U * 256);
        v4f v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = i0 + u * 256;
            v[u] = i < n4 ? __builtin_nontemporal_load(x + i) : v4f{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int u = 0; u < U; u += 2) {
            a += v[u];
            b += v[u + 1];
        }
    }
    a += b;
    float t = (a.x + a.y) + (a.z + a.w);
    // one value per workgroup (any lane's would do; lane 0's keeps it simple)
    if (threadIdx.x == 0) sink[blockIdx.x] = t;
}

// one 16-byte chunk per lane; the grid covers n4 chunks
template <int T>
__global__ __launch_bounds__(T) void copy_flat_kernel(const v4f* __restrict__ x,
                                                      v4f* __restrict__ y, int64_t n4) {
    const int64_t i = int64_t(blockIdx.x) * T + threadIdx.x;
    if (i < n4) __builtin_nontemporal_store(__builtin_nontemporal_load(x + i), y + i);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" {

int rd_ceiling_read(const float* x, int64_t n, int32_t blocks, float* sink, hipStream_t stream) {
    if (!x || !sink || n < 4 || blocks < 1 || blocks > (1 << 20) || !aligned16(x)) return 1;
    read_kernel<<<dim3(uint32_t(blocks)), dim3(256), 0, stream>>>(
        reinterpret_cast<const v4f*>(x), n / 4, sink);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

int rd_ceiling_read_pieces(const float* x, int64_t n, int32_t steps, float* sink,
                           hipStream_t stream) {
    if (!x || !sink || n < 4 || steps < 1 || steps > 1024 || !aligned16(x)) return 1;
    const int64_t n4 = n / 4;
    const int64_t piece = int64_t(steps) * 16 * 256;
    const int64_t blocks = (n4 + piece - 1) / piece;
    if (blocks > int64_t(UINT32_MAX) / 256) return 1;
    read_pieces_kernel<<<dim3(uint32_t(blocks)), dim3(256), 0, stream>>>(
        reinterpret_cast<const v4f*>(x), n4, steps, sink);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

int rd_ceiling_copy(const float* x, float* y, int64_t n, int32_t blocks, hipStream_t stream) {
    if (!x || !y || n < 4 || blocks < 1 || blocks > (1 << 20) || !aligned16(x) || !aligned16(y))
        return 1;
    const uintptr_t a = reinterpret_cast<uintptr_t>(x), b = reinterpret_cast<uintptr_t>(y);
    const uintptr_t bytes = uintptr_t(n / 4) * 16u;
    if (a < b + bytes && b < a + bytes) return 1;  // overlap
    copy_kernel<<<dim3(uint32_t(blocks)), dim3(256), 0, stream>>>(
        reinterpret_cast<const v4f*>(x), reinterpret_cast<v4f*>(y), n / 4);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

int rd_ceiling_copy_flat(const float* x, float* y, int64_t n, int32_t threads,
                         hipStream_t stream) {
    if (!x || !y || n < 4 || !aligned16(x) || !aligned16(y)) return 1;
    const uintptr_t a = reinterpret_cast<uintptr_t>(x), b = reinterpret_cast<uintptr_t>(y);
    const uintptr_t bytes = uintptr_t(n / 4) * 16u;
    if (a < b + bytes && b < a + bytes) return 1;  // overlap
    const int64_t n4 = n / 4;
    const int64_t blocks = (n4 + threads - 1) / threads;
    if (blocks > int64_t(UINT32_MAX) / threads) return 1;  // the grid's lanes within 2^32
    const dim3 grid(static_cast<uint32_t>(blocks));
    const v4f* xs = reinterpret_cast<const v4f*>(x);
    v4f* ys = reinterpret_cast<v4f*>(y);
    switch (threads) {
        case 64: copy_flat_kernel<64><<<grid, dim3(64), 0, stream>>>(xs, ys, n4); break;
        case 256: copy_flat_kernel<256><<<grid, dim3(256), 0, stream>>>(xs, ys, n4); break;
        case 1024: copy_flat_kernel<1024><<<grid, dim3(1024), 0, stream>>>(xs, ys, n4); break;
        default: return 1;
    }
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
