// rd_kernels.hip -- gfx950 (CDNA4) kernels of the fp32 sum reduction.
//
// Prior art on the pages, and what is kept of it here:
//  * "Seven-step reduction: 30x from one kernel", V4/V6/V7: add while loading,
//    grid-stride loop, a register-only reduction inside a warp, one value per
//    warp staged in shared memory, one result per block.  Kept as structure;
//    the warp is a 64-lane wavefront here and its reduction a DPP/swizzle
//    butterfly, and the block results go to a second, fixed-order pass (no
//    float atomics), so results are bitwise reproducible.
//  * "High-Performance Reduction Kernels" README, ILP4 section: several
//    independent accumulators and several 128-bit loads in flight per thread.
//    Kept as U loads in flight per lane.  What limits loads in flight on
//    CDNA is not the add chain (loads never depend on the sum) but where the
//    s_waitcnt lands, which follows from the register budget.
//  * POPCORNBENCH problem-47 trace: lanes run along the contiguous inner
//    axis so a wave's loads are coalesced, and one thread owns 4 adjacent
//    columns read with one 16-byte load per row.  Kept for the column kernel;
//    the trace's worry that rows of 4095 floats break float4 alignment does
//    not apply, because CDNA's global_load_dwordx4 only needs dword alignment.
//
// Loads.  Every 16-byte load is issued from a 4-byte-aligned address through
// a 4-byte-aligned vector type (memcpy), which the compiler emits as one
// global_load_dwordx4.  No head peeling: element k of a row always lands in
// the same lane and accumulator, whatever the base address modulo 16, which
// keeps the result independent of the input's address.
//
// Summation order (fixed for a given plan; every add is IEEE fp32):
//  ROWS      a lane adds its k-th 16-byte chunk (interleaved or blocked
//            order, see rows_kernel) into float4 accumulator (k mod 2); the
//            R % 4 tail elements go to acc[0].x of the row's lanes 0..2;
//            a = acc[0] + acc[1], lane total = (a.x + a.y) + (a.z + a.w); then
//            the wave butterfly, then the wave sums in wave order; then (if
//            the row has several pieces) combine_row over the piece sums, in
//            a second kernel or in the last workgroup of the first.
//  COLS      wave (cw, rw) adds its k-th row, r0 + rw + k*RW, into float4
//            accumulator (k mod 2); acc[0] + acc[1]; then the row phases in
//            rw order; then (if split) the slabs in slab order.
// U, the number of 16-byte loads a lane keeps in flight, is even and does not
// change the order.  Two accumulators rather than U keep the kernels within
// 64 VGPRs (8 waves per SIMD) while all U loads are issued before the first
// add waits on one.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "rd_internal.h"

namespace rd {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

typedef float v4f_a4 __attribute__((ext_vector_type(4), aligned(4)));

// Four floats from a 4-byte-aligned address: one global_load_dwordx4, with
// the nontemporal (streaming) hint when NT.
template <bool NT>
__device__ __forceinline__ v4f load4(const float* p) {
    if constexpr (NT) {
        return __builtin_nontemporal_load(reinterpret_cast<const v4f_a4*>(p));
    } else {
        v4f v;
        __builtin_memcpy(&v, p, sizeof(v));
        return v;
    }
}

template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl,
                                           0xF, 0xF, false));
}

// Sum of v over the 64 lanes of a wavefront; every lane must be active.
// Butterfly: lane pairs at distance 1 and 2 (DPP quad_perm), quads paired by
// mirroring 8 lanes (row_half_mirror), 8-lane halves paired by mirroring 16
// lanes (row_mirror), 16-lane rows paired by a swizzle swap of 16, and the
// two 32-lane halves added through lanes 0 and 32.  Each step adds a lane's
// value to an equal-rank partner's, so every lane ends with the same bits.
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp<0x141>(v);  // row_half_mirror
    v += dpp<0x140>(v);  // row_mirror
    v += __builtin_bit_cast(
        float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
    const float lo = __builtin_bit_cast(
        float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const float hi = __builtin_bit_cast(
        float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    return lo + hi;
}

// Sum over a kBlock-thread workgroup, valid in thread 0: wave butterflies,
// then the wave sums in wave order.  The caller syncs before reusing `lds`.
__device__ __forceinline__ float block_sum(float v, float* lds) {
    v = wave_sum(v);
    if (threadIdx.x % kWave == 0) lds[threadIdx.x / kWave] = v;
    __syncthreads();
    float t = 0.f;
    if (threadIdx.x == 0) {
        t = lds[0];
#pragma unroll
        for (int k = 1; k < kBlock / kWave; ++k) t += lds[k];
    }
    return t;
}

// Workgroups are handed to the XCDs round-robin (hardware id b runs on XCD
// b % nxcd).  Renumber them so that each XCD receives one contiguous run of
// logical ids; neighbouring tiles, which share cache lines at their edges,
// then sit behind the same L2.  A bijection of [0, gridDim.x).
__device__ __forceinline__ int64_t xcd_block(uint32_t nxcd) {
    const uint32_t b = blockIdx.x;
    if (nxcd <= 1) return b;
    const uint32_t n = gridDim.x;
    const uint32_t x = b % nxcd, i = b / nxcd, q = n / nxcd, r = n % nxcd;
    return int64_t(x) * q + (x < r ? x : r) + i;
}

// out_o = the sum of the P piece sums of one row: lane t adds pieces t,
// t + 256, ... in order, then the workgroup reduction.  Used by the second
// pass and by the last workgroup of a fused first pass, so both give the same
// bits.  Every thread of the workgroup must call it.
__device__ __forceinline__ void combine_row(const float* __restrict__ part, int64_t P,
                                            float* __restrict__ out_o, float* lds) {
    float t = 0.f;
    for (int64_t k = threadIdx.x; k < P; k += kBlock) t += part[k];
    t = block_sum(t, lds);
    if (threadIdx.x == 0) *out_o = t;
    __syncthreads();
}

// ----------------------------------------------------------------- ROWS
// Each group of G lanes (one wave, or the whole workgroup) reduces one row
// piece: segment seg = (row o, piece p), o = seg / P, p = seg % P.  With
// P == 1, dst is the output (one value per row); otherwise dst holds the
// outer x P piece sums for rows_combine_kernel.  The full 1D reduce is the
// case outer == 1.
// Chunk order of the pieces of a row (16-byte chunks, nvec = R / 4 of them):
//   interleaved  lane g = p * G + lane takes chunks g, g + P*G, g + 2*P*G, ...
//   blocked      piece p owns the contiguous chunks [p*C, (p+1)*C) with
//                C = ceil(nvec / P) rounded up to a multiple of G, and its
//                lane takes p*C + lane, p*C + lane + G, ... (each group streams
//                one contiguous stretch of memory)
// Fused combine (ticket != null, P > 1): after storing its piece sums, each
// workgroup publishes them (device-scope release) and takes a ticket from an
// integer counter; the workgroup that draws the last ticket acquires, sums
// every row's pieces with combine_row into out[0 .. outer), and resets the
// counter to 0 for the next call on the same stream.  The counter must be 0
// at launch.  No float atomics: only the ticket is atomic, and the combine
// order is the second pass's.
template <int G, int U, bool NT>
__global__ __launch_bounds__(kBlock) void rows_kernel(const float* __restrict__ x,
                                                      int64_t R, int64_t nseg,
                                                      int64_t P, int32_t blocked,
                                                      float* __restrict__ dst,
                                                      uint32_t nxcd,
                                                      uint32_t* __restrict__ ticket,
                                                      float* __restrict__ out) {
    static_assert(G == kWave || G == kBlock, "group is a wave or a workgroup");
    constexpr int kGroups = kBlock / G;
    __shared__ float lds[kBlock / kWave];
    const int gl = threadIdx.x % G;
    const int64_t nvec = R >> 2;
    const int64_t tail = R & 3;
    const int64_t span = ((nvec + P - 1) / P + G - 1) / G * G;  // blocked: chunks per piece
    const int64_t L = blocked ? int64_t(G) : P * G;            // a lane's chunk stride
    const int64_t gstride = int64_t(gridDim.x) * kGroups;
    for (int64_t first = xcd_block(nxcd) * kGroups; first < nseg; first += gstride) {
        const int64_t seg = first + threadIdx.x / G;  // uniform per group
        float total = 0.f;
        if (seg < nseg) {
            const int64_t o = seg / P;
            const int64_t piece = seg - o * P;
            const int64_t g = piece * G + gl;
            const float* row = x + o * R;
            int64_t j = blocked ? piece * span + gl : g;
            int64_t end = nvec;
            if (blocked && piece * span + span < nvec) end = piece * span + span;
            v4f acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
            for (; j + (U - 1) * L < end; j += U * L) {
                v4f v[U];
#pragma unroll
                for (int u = 0; u < U; ++u) v[u] = load4<NT>(row + 4 * (j + u * L));
#pragma unroll
                for (int u = 0; u < U; ++u) acc[u & 1] += v[u];
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (j + u * L < end) acc[u & 1] += load4<NT>(row + 4 * (j + u * L));
            if (g < tail) acc[0].x += row[4 * nvec + g];
            const v4f a = acc[0] + acc[1];
            total = (a.x + a.y) + (a.z + a.w);
        }
        if constexpr (G == kBlock) {
            total = block_sum(total, lds);
            if (threadIdx.x == 0) dst[seg] = total;
            __syncthreads();
        } else {
            total = wave_sum(total);
            if (gl == 0 && seg < nseg) dst[seg] = total;
        }
    }
    if (ticket != nullptr) {
        // One release per workgroup, one acquire in the last one: a full
        // fence in every wave would write back and invalidate the L2 of
        // each XCD thousands of times under the still-running stream.
        __shared__ uint32_t last;
        __syncthreads();  // the workgroup's piece sums are stored
        if (threadIdx.x == 0)
            last = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELEASE,
                                          __HIP_MEMORY_SCOPE_AGENT) == gridDim.x - 1;
        __syncthreads();
        if (last) {
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            const int64_t outer = nseg / P;
            for (int64_t o = 0; o < outer; ++o) combine_row(dst + o * P, P, out + o, lds);
            if (threadIdx.x == 0)
                __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// Rows shorter than a wave's worth of chunks: one lane per row, 16-byte
// loads along the row, then the R % 4 tail in order.
__global__ __launch_bounds__(kBlock) void rows_short_kernel(const float* __restrict__ x,
                                                            int64_t outer, int64_t R,
                                                            float* __restrict__ out) {
    const int64_t stride = int64_t(gridDim.x) * kBlock;
    for (int64_t o = int64_t(blockIdx.x) * kBlock + threadIdx.x; o < outer; o += stride) {
        const float* row = x + o * R;
        v4f acc = {0.f, 0.f, 0.f, 0.f};
        int64_t k = 0;
        for (; k + 4 <= R; k += 4) acc += load4<false>(row + k);
        float t = (acc.x + acc.y) + (acc.z + acc.w);
        for (; k < R; ++k) t += row[k];
        out[o] = t;
    }
}

// Second pass of ROWS: out[o] = combine_row over the P piece sums of row o.
__global__ __launch_bounds__(kBlock) void rows_combine_kernel(const float* __restrict__ part,
                                                              int64_t outer, int64_t P,
                                                              float* __restrict__ out) {
    __shared__ float lds[kBlock / kWave];
    for (int64_t o = blockIdx.x; o < outer; o += gridDim.x)
        combine_row(part + o * P, P, out + o, lds);
}

// ----------------------------------------------------------------- COLS
// A workgroup is CW x RW waves and covers a tile of CW * 64 lane-columns of
// one outer index o and one slab s of R.  Lane-column lc owns the 4 adjacent
// columns c = 4*lc .. 4*lc + 3; per row it makes one 16-byte load.  The lane
// that holds the last 1..3 columns of a row loads the row's last 4 floats
// instead (start inner - 4) and keeps only its own, so no load leaves the
// row and no lane diverges.  Wave (cw, rw) takes the rows r0 + rw + k*RW of
// the slab, U rows in flight; the RW partial sums meet in LDS.  With S == 1,
// dst is the output; otherwise dst is [S][outer][inner] for
// slab_combine_kernel.  Needs inner >= 4.
template <int CW, int RW, int U, bool NT>
__global__ __launch_bounds__(kWave* CW* RW) void cols_kernel(
    const float* __restrict__ x, int64_t outer, int64_t R, int64_t inner, int64_t ntiles,
    int64_t S, int64_t rps, float* __restrict__ dst, uint32_t nxcd) {
    __shared__ v4f lds[RW > 1 ? (RW - 1) * CW * kWave : 1];
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int cw = wave % CW;
    const int rw = wave / CW;
    const int64_t nitems = ntiles * S * outer;
    for (int64_t item = xcd_block(nxcd); item < nitems; item += gridDim.x) {
        const int64_t tile = item % ntiles;
        const int64_t rest = item / ntiles;
        const int64_t s = rest % S;
        const int64_t o = rest / S;
        const int64_t c = 4 * ((tile * CW + cw) * kWave + lane);
        const bool active = c < inner;
        const int64_t cl = c + 4 <= inner ? c : inner - 4;
        const int64_t r0 = s * rps + rw;
        const int64_t r1 = (s + 1) * rps < R ? (s + 1) * rps : R;
        const int64_t m = r0 < r1 ? (r1 - r0 + RW - 1) / RW : 0;
        v4f acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        if (active) {
            const float* p = x + (o * R + r0) * inner + cl;
            const int64_t step = RW * inner;
            int64_t k = 0;
            for (; k + U <= m; k += U) {
                v4f v[U];
#pragma unroll
                for (int u = 0; u < U; ++u) v[u] = load4<NT>(p + u * step);
#pragma unroll
                for (int u = 0; u < U; ++u) acc[u & 1] += v[u];
                p += U * step;
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (k + u < m) acc[u & 1] += load4<NT>(p + u * step);
        }
        v4f a = acc[0] + acc[1];
        if constexpr (RW > 1) {
            if (rw > 0) lds[((rw - 1) * CW + cw) * kWave + lane] = a;
            __syncthreads();
            if (rw == 0) {
#pragma unroll
                for (int q = 1; q < RW; ++q) a += lds[((q - 1) * CW + cw) * kWave + lane];
            }
            __syncthreads();
        }
        if (rw == 0 && active) {
            float* d = dst + (s * outer + o) * inner + cl;
            const int keep = int(c - cl);  // 0, or 1..3 for the row's last lane
            for (int q = keep; q < 4; ++q) d[q] = a[q];
        }
    }
}

// inner in {2, 3} (or any inner): one lane per output of one slab, rows taken
// round robin into 4 accumulators, the slab's last R % 4 rows into the first.
__global__ __launch_bounds__(kBlock) void cols_narrow_kernel(const float* __restrict__ x,
                                                             int64_t outer, int64_t R,
                                                             int64_t inner, int64_t S,
                                                             int64_t rps,
                                                             float* __restrict__ dst) {
    const int64_t per_slab = outer * inner;
    const int64_t total = S * per_slab;
    const int64_t stride = int64_t(gridDim.x) * kBlock;
    for (int64_t e = int64_t(blockIdx.x) * kBlock + threadIdx.x; e < total; e += stride) {
        const int64_t s = e / per_slab;
        const int64_t oi = e - s * per_slab;
        const int64_t o = oi / inner;
        const int64_t i = oi - o * inner;
        const int64_t r0 = s * rps;
        const int64_t r1 = r0 + rps < R ? r0 + rps : R;
        const float* p = x + (o * R + r0) * inner + i;
        float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
        int64_t r = r0;
        for (; r + 4 <= r1; r += 4) {
            a0 += p[0];
            a1 += p[inner];
            a2 += p[2 * inner];
            a3 += p[3 * inner];
            p += 4 * inner;
        }
        for (; r < r1; ++r) {
            a0 += p[0];
            p += inner;
        }
        dst[e] = (a0 + a1) + (a2 + a3);
    }
}

// Second pass of a split along R: out[e] = slab[0][e] + slab[1][e] + ...
__global__ __launch_bounds__(kBlock) void slab_combine_kernel(const float* __restrict__ slab,
                                                              int64_t S, int64_t n,
                                                              float* __restrict__ out) {
    const int64_t stride = int64_t(gridDim.x) * kBlock;
    for (int64_t e = int64_t(blockIdx.x) * kBlock + threadIdx.x; e < n; e += stride) {
        float t = slab[e];
        for (int64_t s = 1; s < S; ++s) t += slab[s * n + e];
        out[e] = t;
    }
}

__global__ __launch_bounds__(kBlock) void fill_zero_kernel(float* __restrict__ out,
                                                           int64_t n) {
    const int64_t stride = int64_t(gridDim.x) * kBlock;
    for (int64_t e = int64_t(blockIdx.x) * kBlock + threadIdx.x; e < n; e += stride)
        out[e] = 0.f;
}

// ------------------------------------------------------------- launching
template <typename T>
struct same {
    using type = T;
};

// hipLaunchKernel with the kernel's own parameter types; returns its error.
template <typename... K>
hipError_t launch(void (*kernel)(K...), int64_t blocks, int threads, hipStream_t s,
                  typename same<K>::type... args) {
    void* argv[] = {static_cast<void*>(&args)...};
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel),
                           dim3(static_cast<uint32_t>(blocks)), dim3(threads), argv, 0, s);
}

int64_t grid_for(int64_t items) {
    int64_t b = (items + kBlock - 1) / kBlock;
    if (b < 1) b = 1;
    return b > kMaxBlocks ? kMaxBlocks : b;
}

// Instantiated kernel shapes.
constexpr int kRowGroups[] = {64, 256};
constexpr int kUnrolls[] = {2, 4, 8, 16};
struct ColShape {
    int cw, rw;
};
constexpr ColShape kColShapes[] = {{1, 1}, {1, 2}, {1, 4}, {1, 8}, {1, 16}, {2, 1},
                                   {2, 2}, {2, 4}, {2, 8}, {4, 1}, {4, 2}, {4, 4},
                                   {8, 1}, {8, 2}, {16, 1}};

template <int G, int U, bool NT>
hipError_t rows_dispatch_u(const rd_plan& p, const float* x, int64_t outer, int64_t R,
                           float* dst, uint32_t* ticket, float* out, hipStream_t s) {
    return launch(rows_kernel<G, U, NT>, p.blocks, kBlock, s, x, R, outer * p.split,
                  p.split, int32_t(p.order == RD_ORDER_BLOCKED), dst, uint32_t(p.nxcd),
                  ticket, out);
}

template <int G, bool NT>
hipError_t rows_dispatch(const rd_plan& p, const float* x, int64_t outer, int64_t R,
                         float* dst, uint32_t* ticket, float* out, hipStream_t s) {
    switch (p.unroll) {
        case 2: return rows_dispatch_u<G, 2, NT>(p, x, outer, R, dst, ticket, out, s);
        case 4: return rows_dispatch_u<G, 4, NT>(p, x, outer, R, dst, ticket, out, s);
        case 8: return rows_dispatch_u<G, 8, NT>(p, x, outer, R, dst, ticket, out, s);
        case 16: return rows_dispatch_u<G, 16, NT>(p, x, outer, R, dst, ticket, out, s);
        default: return hipErrorInvalidValue;
    }
}

template <int CW, int RW, int U, bool NT>
hipError_t cols_dispatch_u(const rd_plan& p, const float* x, int64_t outer, int64_t R,
                           int64_t inner, float* dst, hipStream_t s) {
    const int64_t ntiles = ((inner + 3) / 4 + CW * kWave - 1) / (CW * kWave);
    return launch(cols_kernel<CW, RW, U, NT>, p.blocks, kWave * CW * RW, s, x, outer, R,
                  inner, ntiles, p.split, p.rows_per_split, dst, uint32_t(p.nxcd));
}

template <int CW, int RW, bool NT>
hipError_t cols_dispatch_nt(const rd_plan& p, const float* x, int64_t outer, int64_t R,
                            int64_t inner, float* dst, hipStream_t s) {
    switch (p.unroll) {
        case 2: return cols_dispatch_u<CW, RW, 2, NT>(p, x, outer, R, inner, dst, s);
        case 4: return cols_dispatch_u<CW, RW, 4, NT>(p, x, outer, R, inner, dst, s);
        case 8: return cols_dispatch_u<CW, RW, 8, NT>(p, x, outer, R, inner, dst, s);
        case 16: return cols_dispatch_u<CW, RW, 16, NT>(p, x, outer, R, inner, dst, s);
        default: return hipErrorInvalidValue;
    }
}

template <int CW, int RW>
hipError_t cols_dispatch(const rd_plan& p, const float* x, int64_t outer, int64_t R,
                         int64_t inner, float* dst, hipStream_t s) {
    if (p.nontemporal) return cols_dispatch_nt<CW, RW, true>(p, x, outer, R, inner, dst, s);
    return cols_dispatch_nt<CW, RW, false>(p, x, outer, R, inner, dst, s);
}

}  // namespace

bool rows_shape_supported(int group, int unroll) {
    bool g = false, u = false;
    for (int v : kRowGroups) g |= v == group;
    for (int v : kUnrolls) u |= v == unroll;
    return g && u;
}

bool cols_shape_supported(int col_waves, int row_waves, int unroll) {
    bool c = false, u = false;
    for (const ColShape& v : kColShapes) c |= v.cw == col_waves && v.rw == row_waves;
    for (int v : kUnrolls) u |= v == unroll;
    return c && u;
}

hipError_t launch_fill_zero(float* out, int64_t n, hipStream_t s) {
    return launch(fill_zero_kernel, grid_for(n), kBlock, s, out, n);
}

hipError_t launch_rows(const rd_plan& p, const float* x, int64_t outer, int64_t R,
                       float* dst, uint32_t* ticket, float* out, hipStream_t s) {
    if (p.group == kBlock)
        return p.nontemporal
                   ? rows_dispatch<kBlock, true>(p, x, outer, R, dst, ticket, out, s)
                   : rows_dispatch<kBlock, false>(p, x, outer, R, dst, ticket, out, s);
    if (p.group == kWave)
        return p.nontemporal
                   ? rows_dispatch<kWave, true>(p, x, outer, R, dst, ticket, out, s)
                   : rows_dispatch<kWave, false>(p, x, outer, R, dst, ticket, out, s);
    return hipErrorInvalidValue;
}

hipError_t launch_rows_short(const float* x, int64_t outer, int64_t R, float* out,
                             hipStream_t s) {
    return launch(rows_short_kernel, grid_for(outer), kBlock, s, x, outer, R, out);
}

hipError_t launch_rows_combine(const float* part, int64_t outer, int64_t P, float* out,
                               hipStream_t s) {
    const int64_t blocks = outer < kMaxBlocks ? outer : kMaxBlocks;
    return launch(rows_combine_kernel, blocks, kBlock, s, part, outer, P, out);
}

hipError_t launch_cols(const rd_plan& p, const float* x, int64_t outer, int64_t R,
                       int64_t inner, float* dst, hipStream_t s) {
#define RD_COLS_CASE(CW, RW) \
    if (p.col_waves == CW && p.row_waves == RW) \
        return cols_dispatch<CW, RW>(p, x, outer, R, inner, dst, s);
    RD_COLS_CASE(1, 1)
    RD_COLS_CASE(1, 2)
    RD_COLS_CASE(1, 4)
    RD_COLS_CASE(1, 8)
    RD_COLS_CASE(1, 16)
    RD_COLS_CASE(2, 1)
    RD_COLS_CASE(2, 2)
    RD_COLS_CASE(2, 4)
    RD_COLS_CASE(2, 8)
    RD_COLS_CASE(4, 1)
    RD_COLS_CASE(4, 2)
    RD_COLS_CASE(4, 4)
    RD_COLS_CASE(8, 1)
    RD_COLS_CASE(8, 2)
    RD_COLS_CASE(16, 1)
#undef RD_COLS_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_cols_narrow(const rd_plan& p, const float* x, int64_t outer, int64_t R,
                              int64_t inner, float* dst, hipStream_t s) {
    return launch(cols_narrow_kernel, p.blocks, kBlock, s, x, outer, R, inner, p.split,
                  p.rows_per_split, dst);
}

hipError_t launch_slab_combine(const float* slab, int64_t S, int64_t n, float* out,
                               hipStream_t s) {
    return launch(slab_combine_kernel, grid_for(n), kBlock, s, slab, S, n, out);
}

}  // namespace rd
