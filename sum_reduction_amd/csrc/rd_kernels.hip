// rd_kernels.hip -- gfx950 (CDNA4) kernels of the fp32 reductions.
//
// Prior art on the pages, and what is kept of it here:
//  * "Seven-step reduction: 30x from one kernel", V4/V6/V7: add while loading,
//    grid-stride loop, a register-only reduction inside a warp, one value per
//    warp staged in shared memory, one result per block.  Kept as structure;
//    the warp is a 64-lane wavefront here and its reduction a DPP/swizzle
//    butterfly, and the block results go to a second, fixed-order pass (no
//    float atomics), so results are bitwise reproducible.  The same page
//    names sum, max and the L2 norm as one primitive: the kernels take the
//    operator (sum, sum of squares, maximum, minimum) as a parameter.
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
// a 4-byte-aligned vector type, which the compiler emits as one
// global_load_dwordx4.  No head peeling: element k of a row always lands in
// the same lane and accumulator, whatever the base address modulo 16, which
// keeps the result independent of the input's address.
//
// Order of the operations (fixed for a given plan; "fold" adds a term,
// "join" combines two partial results, see Op below):
//  ROWS      a lane folds its k-th 16-byte chunk (interleaved or blocked
//            order, see rows_kernel) into float4 accumulator (k mod 2); the
//            R % 4 tail elements go to acc[0].x of the row's lanes 0..2;
//            a = join(acc[0], acc[1]), lane result = join(join(a.x, a.y),
//            join(a.z, a.w)); then the wave butterfly, then the wave results
//            in wave order; then (if the row has several pieces) combine_row
//            over the piece results, in a second kernel or in the last
//            workgroup of the first.
//  COLS      wave (cw, rw) folds its k-th row, r0 + rw + k*RW, into float4
//            accumulator (k mod 2); join(acc[0], acc[1]); then the row phases
//            in rw order; then (if split) the slabs in slab order.
//  COLS_SMALL  row phase rho folds its k-th row into accumulator (k mod 2);
//            join(acc[0], acc[1]); then the row phases by a fixed tree (see
//            cols_small_kernel); then (if split) the slabs in slab order.
// U, the number of 16-byte loads a lane keeps in flight, is even and does not
// change the order.  Two accumulators rather than U keep the kernels within
// 64 VGPRs (8 waves per SIMD) while all U loads are issued before the first
// fold waits on one.
#include <hip/hip_runtime.h>

#include "rd_device.h"
#include "rd_internal.h"

namespace rd {
namespace {

// ------------------------------------------------------------- operators
// start: the value of an empty reduction; fold: one more term into a
// partial result; join: two partial results into one.
//  sum      0,     a + v,           a + b
//  sum sq   0,     fma(v, v, a),    a + b      (one rounding per term)
//  max      -Inf,  maximum(a, v),   maximum(a, b)
//  min      +Inf,  minimum(a, v),   minimum(a, b)
// maximum / minimum are IEEE 754-2019 (v_maximum3_f32 / v_minimum3_f32 on
// gfx950): a NaN operand gives NaN and -0 < +0, so their result does not
// depend on the order of the terms.
template <int OP>
struct Op;

template <>
struct Op<RD_OP_SUM> {
    static __device__ __forceinline__ float start() { return 0.f; }
    static __device__ __forceinline__ v4f fold(v4f a, v4f v) { return a + v; }
    static __device__ __forceinline__ float fold(float a, float v) { return a + v; }
    static __device__ __forceinline__ v4f join(v4f a, v4f b) { return a + b; }
    static __device__ __forceinline__ float join(float a, float b) { return a + b; }
};

template <>
struct Op<RD_OP_SUMSQ> {
    static __device__ __forceinline__ float start() { return 0.f; }
    static __device__ __forceinline__ v4f fold(v4f a, v4f v) {
        return __builtin_elementwise_fma(v, v, a);
    }
    static __device__ __forceinline__ float fold(float a, float v) {
        return __builtin_fmaf(v, v, a);
    }
    static __device__ __forceinline__ v4f join(v4f a, v4f b) { return a + b; }
    static __device__ __forceinline__ float join(float a, float b) { return a + b; }
};

template <>
struct Op<RD_OP_MAX> {
    static __device__ __forceinline__ float start() { return -__builtin_inff(); }
    static __device__ __forceinline__ v4f fold(v4f a, v4f v) {
        return __builtin_elementwise_maximum(a, v);
    }
    static __device__ __forceinline__ float fold(float a, float v) {
        return __builtin_elementwise_maximum(a, v);
    }
    static __device__ __forceinline__ v4f join(v4f a, v4f b) { return fold(a, b); }
    static __device__ __forceinline__ float join(float a, float b) { return fold(a, b); }
};

template <>
struct Op<RD_OP_MIN> {
    static __device__ __forceinline__ float start() { return __builtin_inff(); }
    static __device__ __forceinline__ v4f fold(v4f a, v4f v) {
        return __builtin_elementwise_minimum(a, v);
    }
    static __device__ __forceinline__ float fold(float a, float v) {
        return __builtin_elementwise_minimum(a, v);
    }
    static __device__ __forceinline__ v4f join(v4f a, v4f b) { return fold(a, b); }
    static __device__ __forceinline__ float join(float a, float b) { return fold(a, b); }
};

template <int OP>
__device__ __forceinline__ v4f start4() {
    const float s = Op<OP>::start();
    return v4f{s, s, s, s};
}

// The four lanes of a float4 partial result joined in a fixed order.
template <int OP>
__device__ __forceinline__ float join_lanes(v4f a) {
    return Op<OP>::join(Op<OP>::join(a.x, a.y), Op<OP>::join(a.z, a.w));
}

// ------------------------------------------------- wave and block steps
template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl,
                                           0xF, 0xF, false));
}

// Join of v over the 64 lanes of a wavefront; every lane must be active.
// Butterfly: lane pairs at distance 1 and 2 (DPP quad_perm), quads paired by
// mirroring 8 lanes (row_half_mirror), 8-lane halves paired by mirroring 16
// lanes (row_mirror), 16-lane rows paired by a swizzle swap of 16, and the
// two 32-lane halves joined through lanes 0 and 32.  Each step joins a
// lane's value with an equal-rank partner's, and every join is commutative,
// so every lane ends with the same bits.
template <int OP>
__device__ __forceinline__ float wave_reduce(float v) {
    v = Op<OP>::join(v, dpp<0xB1>(v));   // quad_perm [1,0,3,2]
    v = Op<OP>::join(v, dpp<0x4E>(v));   // quad_perm [2,3,0,1]
    v = Op<OP>::join(v, dpp<0x141>(v));  // row_half_mirror
    v = Op<OP>::join(v, dpp<0x140>(v));  // row_mirror
    v = Op<OP>::join(v, __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(
                                                      __builtin_bit_cast(int, v), 0x401F)));
    const float lo = __builtin_bit_cast(
        float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const float hi = __builtin_bit_cast(
        float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    return Op<OP>::join(lo, hi);
}

// The value v of lane `src` (ds_bpermute).  v is taken by value: a bit cast
// applied to a vector element in place was miscompiled into one permute of
// element 0 for all four.
__device__ __forceinline__ float lane_value(int src, float v) {
    return __builtin_bit_cast(float,
                              __builtin_amdgcn_ds_bpermute(4 * src, __builtin_bit_cast(int, v)));
}

// Join over a kBlock-thread workgroup, valid in thread 0: wave butterflies,
// then the wave results in wave order.  The caller syncs before reusing lds.
template <int OP>
__device__ __forceinline__ float block_reduce(float v, float* lds) {
    v = wave_reduce<OP>(v);
    if (threadIdx.x % kWave == 0) lds[threadIdx.x / kWave] = v;
    __syncthreads();
    float t = Op<OP>::start();
    if (threadIdx.x == 0) {
        t = lds[0];
#pragma unroll
        for (int k = 1; k < kBlock / kWave; ++k) t = Op<OP>::join(t, lds[k]);
    }
    return t;
}

// out_o = the join of the P piece results of one row: lane t joins pieces
// t, t + 256, ... in order, then the workgroup reduction.  Used by the
// second pass and by the last workgroup of a fused first pass, so both give
// the same bits.  Every thread of the workgroup must call it.
template <int OP>
__device__ __forceinline__ void combine_row(const float* __restrict__ part, int64_t P,
                                            float* __restrict__ out_o, float* lds) {
    float t = Op<OP>::start();
    for (int64_t k = threadIdx.x; k < P; k += kBlock) t = Op<OP>::join(t, part[k]);
    t = block_reduce<OP>(t, lds);
    if (threadIdx.x == 0) *out_o = t;
    __syncthreads();
}

// ----------------------------------------------------------------- ROWS
// Each group of G lanes (one wave, or the whole workgroup) reduces one row
// piece: segment seg = (row o, piece p), o = seg / P, p = seg % P.  With
// P == 1, dst is the output (one value per row); otherwise dst holds the
// outer x P piece results for rows_combine_kernel.  The full 1D reduce is
// the case outer == 1.
// Chunk order of the pieces of a row (16-byte chunks, nvec = R / 4 of them):
//   interleaved  lane g = p * G + lane takes chunks g, g + P*G, g + 2*P*G, ...
//   blocked      piece p owns the contiguous chunks [p*C, (p+1)*C) with
//                C = ceil(nvec / P) rounded up to a multiple of G, and its
//                lane takes p*C + lane, p*C + lane + G, ... (each group streams
//                one contiguous stretch of memory)
// Fused combine (ticket != null, P > 1): after storing its piece results,
// each workgroup publishes them (device-scope release) and takes a ticket
// from an integer counter; the workgroup that draws the last ticket acquires,
// joins every row's pieces with combine_row into out[0 .. outer), and resets
// the counter to 0 for the next call on the same stream.  The counter must
// be 0 at launch.  Only the ticket is atomic, and the combine order is the
// second pass's.
template <int OP, int G, int U, bool NT>
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
        float total = Op<OP>::start();
        if (seg < nseg) {
            const int64_t o = seg / P;
            const int64_t piece = seg - o * P;
            const int64_t g = piece * G + gl;
            const float* row = x + o * R;
            int64_t j = blocked ? piece * span + gl : g;
            int64_t end = nvec;
            if (blocked && piece * span + span < nvec) end = piece * span + span;
            v4f acc[2] = {start4<OP>(), start4<OP>()};
            for (; j + (U - 1) * L < end; j += U * L) {
                v4f v[U];
#pragma unroll
                for (int u = 0; u < U; ++u) v[u] = load4<NT>(row + 4 * (j + u * L));
#pragma unroll
                for (int u = 0; u < U; ++u) acc[u & 1] = Op<OP>::fold(acc[u & 1], v[u]);
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (j + u * L < end)
                    acc[u & 1] = Op<OP>::fold(acc[u & 1], load4<NT>(row + 4 * (j + u * L)));
            if (g < tail) acc[0].x = Op<OP>::fold(acc[0].x, row[4 * nvec + g]);
            total = join_lanes<OP>(Op<OP>::join(acc[0], acc[1]));
        }
        if constexpr (G == kBlock) {
            total = block_reduce<OP>(total, lds);
            if (threadIdx.x == 0) dst[seg] = total;
            __syncthreads();
        } else {
            total = wave_reduce<OP>(total);
            if (gl == 0 && seg < nseg) dst[seg] = total;
        }
    }
    if (ticket != nullptr) {
        // One release per workgroup, one acquire in the last one: a full
        // fence in every wave would write back and invalidate the L2 of
        // each XCD thousands of times under the still-running stream.
        __shared__ uint32_t last;
        __syncthreads();  // the workgroup's piece results are stored
        if (threadIdx.x == 0)
            last = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELEASE,
                                          __HIP_MEMORY_SCOPE_AGENT) == gridDim.x - 1;
        __syncthreads();
        if (last) {
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            const int64_t outer = nseg / P;
            for (int64_t o = 0; o < outer; ++o)
                combine_row<OP>(dst + o * P, P, out + o, lds);
            if (threadIdx.x == 0)
                __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// Rows shorter than a wave's worth of chunks: one lane per row, 16-byte
// loads along the row, then the R % 4 tail in order.
template <int OP>
__global__ __launch_bounds__(kBlock) void rows_short_kernel(const float* __restrict__ x,
                                                            int64_t outer, int64_t R,
                                                            float* __restrict__ out) {
    const int64_t stride = int64_t(gridDim.x) * kBlock;
    for (int64_t o = int64_t(blockIdx.x) * kBlock + threadIdx.x; o < outer; o += stride) {
        const float* row = x + o * R;
        v4f acc = start4<OP>();
        int64_t k = 0;
        for (; k + 4 <= R; k += 4) acc = Op<OP>::fold(acc, load4<false>(row + k));
        float t = join_lanes<OP>(acc);
        for (; k < R; ++k) t = Op<OP>::fold(t, row[k]);
        out[o] = t;
    }
}

// Second pass of ROWS: out[o] = combine_row over the P piece results of row o.
template <int OP>
__global__ __launch_bounds__(kBlock) void rows_combine_kernel(const float* __restrict__ part,
                                                              int64_t outer, int64_t P,
                                                              float* __restrict__ out) {
    __shared__ float lds[kBlock / kWave];
    for (int64_t o = blockIdx.x; o < outer; o += gridDim.x)
        combine_row<OP>(part + o * P, P, out + o, lds);
}

// ----------------------------------------------------------------- COLS
// A workgroup is CW x RW waves and covers a tile of CW * 64 lane-columns of
// one outer index o and one slab s of R.  Lane-column lc owns the 4 adjacent
// columns c = 4*lc .. 4*lc + 3; per row it makes one 16-byte load.  The lane
// that holds the last 1..3 columns of a row loads the row's last 4 floats
// instead (start inner - 4) and keeps only its own, so no load leaves the
// row and no lane diverges.  Wave (cw, rw) takes the rows r0 + rw + k*RW of
// the slab, U rows in flight; the RW partial results meet in LDS.  With
// S == 1, dst is the output; otherwise dst is [S][outer][inner] for
// slab_combine_kernel.  Needs inner >= 4.
template <int OP, int CW, int RW, int U, bool NT>
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
        v4f acc[2] = {start4<OP>(), start4<OP>()};
        if (active) {
            const float* p = x + (o * R + r0) * inner + cl;
            const int64_t step = RW * inner;
            int64_t k = 0;
            for (; k + U <= m; k += U) {
                v4f v[U];
#pragma unroll
                for (int u = 0; u < U; ++u) v[u] = load4<NT>(p + u * step);
#pragma unroll
                for (int u = 0; u < U; ++u) acc[u & 1] = Op<OP>::fold(acc[u & 1], v[u]);
                p += U * step;
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (k + u < m) acc[u & 1] = Op<OP>::fold(acc[u & 1], load4<NT>(p + u * step));
        }
        v4f a = Op<OP>::join(acc[0], acc[1]);
        if constexpr (RW > 1) {
            if (rw > 0) lds[((rw - 1) * CW + cw) * kWave + lane] = a;
            __syncthreads();
            if (rw == 0) {
#pragma unroll
                for (int q = 1; q < RW; ++q)
                    a = Op<OP>::join(a, lds[((q - 1) * CW + cw) * kWave + lane]);
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

// Small inner (2 <= inner <= 128): several rows of one outer index per load
// instruction.  The rows of one outer index are adjacent in memory, so a wave
// covers RPW consecutive rows at once: lane = (row phase rho, lane-column lc)
// with LC = ceil(inner / 4) lane-columns per row and RPW = 64 / LC row
// phases (lanes from RPW * LC on idle); each instruction reads RPW * inner
// contiguous floats.  Lane-column lc owns columns 4*lc .. 4*lc + 3 (the
// row's last lane-column loads the row's last 4 floats and keeps its own,
// as in cols_kernel); with inner < 4 (V = inner) a lane loads its whole row.
// Each wave works on one item (outer index o, slab s of R) at a time: row
// phase rho folds rows r0 + rho + k*RPW into accumulator (k mod 2), U rows in
// flight; then the row phases of each lane-column are joined by a fixed
// tree (LC == 1: the wave butterfly; else pairs rho, rho + d for d = 1, 2,
// 4, ... through ds_bpermute) and the rho == 0 lanes write.  With S == 1,
// dst is the output; otherwise dst is [S][outer][inner] for
// slab_combine_kernel.
template <int OP, int V, int U, bool NT>
__global__ __launch_bounds__(kBlock) void cols_small_kernel(
    const float* __restrict__ x, int64_t outer, int64_t R, int64_t inner, int64_t S,
    int64_t rps, int32_t LC, float* __restrict__ dst, uint32_t nxcd) {
    constexpr int kWaves = kBlock / kWave;
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int RPW = kWave / LC;
    const int rho = lane / LC;
    const int lc = lane - rho * LC;
    const bool active = rho < RPW;
    const int64_t c = 4 * int64_t(lc);
    const int64_t cl = (V == 4 && c + 4 > inner) ? inner - 4 : c;
    const int keep = int(c - cl);  // 0, or 1..3 for the row's last lane-column
    const int64_t nitems = S * outer;
    const int64_t wstride = int64_t(gridDim.x) * kWaves;
    for (int64_t item = xcd_block(nxcd) * kWaves + wave; item < nitems; item += wstride) {
        const int64_t o = item / S;
        const int64_t s = item - o * S;
        const int64_t r0 = s * rps + rho;
        const int64_t r1 = (s + 1) * rps < R ? (s + 1) * rps : R;
        const int64_t m = r0 < r1 ? (r1 - r0 + RPW - 1) / RPW : 0;
        v4f acc[2] = {start4<OP>(), start4<OP>()};
        if (active) {
            const float* p = x + (o * R + r0) * inner + cl;
            const int64_t step = int64_t(RPW) * inner;
            const float fill = Op<OP>::start();
            int64_t k = 0;
            for (; k + U <= m; k += U) {
                v4f v[U];
#pragma unroll
                for (int u = 0; u < U; ++u) v[u] = loadv<V, NT>(p + u * step, fill);
#pragma unroll
                for (int u = 0; u < U; ++u) acc[u & 1] = Op<OP>::fold(acc[u & 1], v[u]);
                p += U * step;
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (k + u < m)
                    acc[u & 1] = Op<OP>::fold(acc[u & 1], loadv<V, NT>(p + u * step, fill));
        }
        // join the row phases of each lane-column by a fixed tree
        v4f a = Op<OP>::join(acc[0], acc[1]);
        if (LC == 1) {
#pragma unroll
            for (int j = 0; j < V; ++j) a[j] = wave_reduce<OP>(a[j]);
        } else {
            for (int d = 1; d < RPW; d *= 2) {
                const int src = lane + d * LC < kWave ? lane + d * LC : lane;
                v4f t;
#pragma unroll
                for (int j = 0; j < 4; ++j) t[j] = lane_value(src, a[j]);
                if ((rho & (2 * d - 1)) == 0 && rho + d < RPW) a = Op<OP>::join(a, t);
            }
        }
        if (rho == 0) {
            float* d = dst + (s * outer + o) * inner + cl;
            if constexpr (V == 4) {
                for (int q = keep; q < 4; ++q) d[q] = a[q];
            } else {
                for (int q = 0; q < V; ++q) d[q] = a[q];
            }
        }
    }
}

// Second pass of a split along R: out[e] = join of slab[0][e], slab[1][e], ...
template <int OP>
__global__ __launch_bounds__(kBlock) void slab_combine_kernel(const float* __restrict__ slab,
                                                              int64_t S, int64_t n,
                                                              float* __restrict__ out) {
    const int64_t stride = int64_t(gridDim.x) * kBlock;
    for (int64_t e = int64_t(blockIdx.x) * kBlock + threadIdx.x; e < n; e += stride) {
        float t = slab[e];
        for (int64_t s = 1; s < S; ++s) t = Op<OP>::join(t, slab[s * n + e]);
        out[e] = t;
    }
}

// R == 0: every output is the operator's start value.
template <int OP>
__global__ __launch_bounds__(kBlock) void fill_start_kernel(float* __restrict__ out,
                                                            int64_t n) {
    const int64_t stride = int64_t(gridDim.x) * kBlock;
    for (int64_t e = int64_t(blockIdx.x) * kBlock + threadIdx.x; e < n; e += stride)
        out[e] = Op<OP>::start();
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

// Instantiated kernel shapes.  The sum has every tuning shape; the other
// operators have the shapes the planner picks by default (U = 8 or 16 on
// ROWS, one row phase and U = 4 on COLS), each with and without the
// streaming hint.
constexpr bool unroll_built(int u) { return u == 2 || u == 4 || u == 8 || u == 16; }

constexpr bool rows_built(int op, int g, int u) {
    if (g != kWave && g != kBlock) return false;
    return op == RD_OP_SUM ? unroll_built(u) : (u == 8 || u == 16);
}

constexpr bool col_shape_built(int cw, int rw) {
    return (cw == 1 && (rw == 1 || rw == 2 || rw == 4 || rw == 8 || rw == 16)) ||
           (cw == 2 && (rw == 1 || rw == 2 || rw == 4 || rw == 8)) ||
           (cw == 4 && (rw == 1 || rw == 2 || rw == 4)) || (cw == 8 && (rw == 1 || rw == 2)) ||
           (cw == 16 && rw == 1);
}

constexpr bool cols_built(int op, int cw, int rw, int u) {
    if (op == RD_OP_SUM) return col_shape_built(cw, rw) && unroll_built(u);
    return rw == 1 && (cw == 1 || cw == 2 || cw == 4 || cw == 8) && u == 4;
}

constexpr bool op_valid(int op) {
    return op == RD_OP_SUM || op == RD_OP_SUMSQ || op == RD_OP_MAX || op == RD_OP_MIN;
}

struct RowsArgs {
    const float* x;
    int64_t outer, R;
    float* dst;
    uint32_t* ticket;
    float* out;
};

template <int OP, int G, int U, bool NT>
hipError_t rows_go(const rd_plan& p, const RowsArgs& a, hipStream_t s) {
    if constexpr (rows_built(OP, G, U)) {
        return launch(rows_kernel<OP, G, U, NT>, p.blocks, kBlock, s, a.x, a.R,
                      a.outer * p.split, p.split, int32_t(p.order == RD_ORDER_BLOCKED), a.dst,
                      uint32_t(p.nxcd), a.ticket, a.out);
    } else {
        return hipErrorInvalidValue;
    }
}

template <int OP, int G, bool NT>
hipError_t rows_u(const rd_plan& p, const RowsArgs& a, hipStream_t s) {
    switch (p.unroll) {
        case 2: return rows_go<OP, G, 2, NT>(p, a, s);
        case 4: return rows_go<OP, G, 4, NT>(p, a, s);
        case 8: return rows_go<OP, G, 8, NT>(p, a, s);
        case 16: return rows_go<OP, G, 16, NT>(p, a, s);
        default: return hipErrorInvalidValue;
    }
}

template <int OP>
hipError_t rows_op(const rd_plan& p, const RowsArgs& a, hipStream_t s) {
    if (p.group == kBlock)
        return p.nontemporal ? rows_u<OP, kBlock, true>(p, a, s)
                             : rows_u<OP, kBlock, false>(p, a, s);
    if (p.group == kWave)
        return p.nontemporal ? rows_u<OP, kWave, true>(p, a, s)
                             : rows_u<OP, kWave, false>(p, a, s);
    return hipErrorInvalidValue;
}

struct ColsArgs {
    const float* x;
    int64_t outer, R, inner;
    float* dst;
};

template <int OP, int CW, int RW, int U, bool NT>
hipError_t cols_go(const rd_plan& p, const ColsArgs& a, hipStream_t s) {
    if constexpr (cols_built(OP, CW, RW, U)) {
        const int64_t ntiles = ((a.inner + 3) / 4 + CW * kWave - 1) / (CW * kWave);
        return launch(cols_kernel<OP, CW, RW, U, NT>, p.blocks, kWave * CW * RW, s, a.x,
                      a.outer, a.R, a.inner, ntiles, p.split, p.rows_per_split, a.dst,
                      uint32_t(p.nxcd));
    } else {
        return hipErrorInvalidValue;
    }
}

template <int OP, int CW, int RW, bool NT>
hipError_t cols_u(const rd_plan& p, const ColsArgs& a, hipStream_t s) {
    switch (p.unroll) {
        case 2: return cols_go<OP, CW, RW, 2, NT>(p, a, s);
        case 4: return cols_go<OP, CW, RW, 4, NT>(p, a, s);
        case 8: return cols_go<OP, CW, RW, 8, NT>(p, a, s);
        case 16: return cols_go<OP, CW, RW, 16, NT>(p, a, s);
        default: return hipErrorInvalidValue;
    }
}

template <int OP, int CW, int RW>
hipError_t cols_nt(const rd_plan& p, const ColsArgs& a, hipStream_t s) {
    return p.nontemporal ? cols_u<OP, CW, RW, true>(p, a, s)
                         : cols_u<OP, CW, RW, false>(p, a, s);
}

template <int OP>
hipError_t cols_op(const rd_plan& p, const ColsArgs& a, hipStream_t s) {
#define RD_COLS_CASE(CW, RW) \
    if (p.col_waves == CW && p.row_waves == RW) return cols_nt<OP, CW, RW>(p, a, s);
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

// Calls F<OP>(args...) for the runtime operator op.
#define RD_BY_OP(op, F, ...)                                  \
    switch (op) {                                             \
        case RD_OP_SUM: return F<RD_OP_SUM>(__VA_ARGS__);     \
        case RD_OP_SUMSQ: return F<RD_OP_SUMSQ>(__VA_ARGS__); \
        case RD_OP_MAX: return F<RD_OP_MAX>(__VA_ARGS__);     \
        case RD_OP_MIN: return F<RD_OP_MIN>(__VA_ARGS__);     \
        default: return hipErrorInvalidValue;                 \
    }

template <int OP>
hipError_t fill_go(float* out, int64_t n, hipStream_t s) {
    return launch(fill_start_kernel<OP>, grid_for(n), kBlock, s, out, n);
}

template <int OP>
hipError_t rows_short_go(const float* x, int64_t outer, int64_t R, float* out,
                         hipStream_t s) {
    return launch(rows_short_kernel<OP>, grid_for(outer), kBlock, s, x, outer, R, out);
}

template <int OP>
hipError_t rows_combine_go(const float* part, int64_t outer, int64_t P, float* out,
                           hipStream_t s) {
    const int64_t blocks = outer < kMaxBlocks ? outer : kMaxBlocks;
    return launch(rows_combine_kernel<OP>, blocks, kBlock, s, part, outer, P, out);
}

constexpr bool small_built(int op, int v, int u) {
    if (v != 2 && v != 3 && v != 4) return false;
    return op == RD_OP_SUM ? (u == 2 || u == 4 || u == 8) : u == 4;
}

template <int OP, int V, int U, bool NT>
hipError_t small_go(const rd_plan& p, const ColsArgs& a, hipStream_t s) {
    if constexpr (small_built(OP, V, U)) {
        const int32_t lc = int32_t((a.inner + 3) / 4);
        return launch(cols_small_kernel<OP, V, U, NT>, p.blocks, kBlock, s, a.x, a.outer, a.R,
                      a.inner, p.split, p.rows_per_split, lc, a.dst, uint32_t(p.nxcd));
    } else {
        return hipErrorInvalidValue;
    }
}

template <int OP, int V, bool NT>
hipError_t small_u(const rd_plan& p, const ColsArgs& a, hipStream_t s) {
    switch (p.unroll) {
        case 2: return small_go<OP, V, 2, NT>(p, a, s);
        case 4: return small_go<OP, V, 4, NT>(p, a, s);
        case 8: return small_go<OP, V, 8, NT>(p, a, s);
        default: return hipErrorInvalidValue;
    }
}

template <int OP, int V>
hipError_t small_nt(const rd_plan& p, const ColsArgs& a, hipStream_t s) {
    return p.nontemporal ? small_u<OP, V, true>(p, a, s) : small_u<OP, V, false>(p, a, s);
}

template <int OP>
hipError_t cols_small_go(const rd_plan& p, const ColsArgs& a, hipStream_t s) {
    if (a.inner == 2) return small_nt<OP, 2>(p, a, s);
    if (a.inner == 3) return small_nt<OP, 3>(p, a, s);
    return small_nt<OP, 4>(p, a, s);
}

template <int OP>
hipError_t slab_combine_go(const float* slab, int64_t S, int64_t n, float* out,
                           hipStream_t s) {
    return launch(slab_combine_kernel<OP>, grid_for(n), kBlock, s, slab, S, n, out);
}

}  // namespace

bool rows_shape_supported(int op, int group, int unroll) {
    return op_valid(op) && rows_built(op, group, unroll);
}

bool cols_shape_supported(int op, int col_waves, int row_waves, int unroll) {
    return op_valid(op) && cols_built(op, col_waves, row_waves, unroll);
}

bool small_shape_supported(int op, int unroll) {
    return op_valid(op) && small_built(op, 4, unroll);
}

hipError_t launch_fill_start(int op, float* out, int64_t n, hipStream_t s) {
    RD_BY_OP(op, fill_go, out, n, s)
}

hipError_t launch_rows(int op, const rd_plan& p, const float* x, int64_t outer, int64_t R,
                       float* dst, uint32_t* ticket, float* out, hipStream_t s) {
    const RowsArgs a{x, outer, R, dst, ticket, out};
    RD_BY_OP(op, rows_op, p, a, s)
}

hipError_t launch_rows_short(int op, const float* x, int64_t outer, int64_t R, float* out,
                             hipStream_t s) {
    RD_BY_OP(op, rows_short_go, x, outer, R, out, s)
}

hipError_t launch_rows_combine(int op, const float* part, int64_t outer, int64_t P,
                               float* out, hipStream_t s) {
    RD_BY_OP(op, rows_combine_go, part, outer, P, out, s)
}

hipError_t launch_cols(int op, const rd_plan& p, const float* x, int64_t outer, int64_t R,
                       int64_t inner, float* dst, hipStream_t s) {
    const ColsArgs a{x, outer, R, inner, dst};
    RD_BY_OP(op, cols_op, p, a, s)
}

hipError_t launch_cols_small(int op, const rd_plan& p, const float* x, int64_t outer,
                             int64_t R, int64_t inner, float* dst, hipStream_t s) {
    const ColsArgs a{x, outer, R, inner, dst};
    RD_BY_OP(op, cols_small_go, p, a, s)
}

hipError_t launch_slab_combine(int op, const float* slab, int64_t S, int64_t n, float* out,
                               hipStream_t s) {
    RD_BY_OP(op, slab_combine_go, slab, S, n, out, s)
}

}  // namespace rd
