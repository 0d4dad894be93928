// rd_kernels.hip -- gfx950 (CDNA4) kernels of the fp32 reductions.
//
// Prior art on the pages, and what is kept of it here:
//  * "Seven-step reduction: 30x from one kernel", V4/V6/V7: add while loading,
//    grid-stride loop, a register-only reduction inside a warp, one value per
//    warp staged in shared memory, one result per block.  Kept as structure;
//    the warp is a 64-lane wavefront here and its reduction a DPP/swizzle
//    butterfly, and the block results go to a second, fixed-order pass (no
//    float atomics), so results are bitwise reproducible.  The same page
//    names sum, max, the L2 norm and the softmax denominator as one
//    primitive: the kernels take the operator (sum, sum of squares, maximum,
//    minimum, the softmax pair) as a parameter, through the state layer St.
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
//            in rw order; then (if split) the slabs in slab order -- or, with
//            64 slabs or more and at most 256 outputs, lane l of a wave joins
//            slabs l, l + 64, ... and the wave butterfly joins the lanes (the
//            same for COLS_SMALL and STRIDED slabs).
//  COLS_SMALL  row phase rho folds its k-th row into accumulator (k mod 2);
//            join(acc[0], acc[1]); then the row phases by a fixed tree (see
//            cols_small_kernel); then (if split) the slabs in slab order.
//  ROWS_SHORT  a thread folds its row's float4 groups into one float4
//            accumulator, joins its lanes, then folds the R % 4 tail
//            (rows_short_tile_kernel reads the row from LDS, rows_short_kernel
//            from memory: the same order).
//  STRIDED   lane (slab, output) folds its terms in r order; then the slabs
//            in slab order.
// U, the number of 16-byte loads a lane keeps in flight, is even and does not
// change the order.  Two accumulators rather than U keep the kernels within
// 64 VGPRs (8 waves per SIMD) while all U loads are issued before the first
// fold waits on one.  (The softmax pair folds a step's U loads at once into
// accumulator 0: the group's maximum, a lazy re-centring, then the group's
// exponentials summed by a pairwise tree -- see St<RD_OP_SOFTMAX_DENOM>.)
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

// The softmax denominator ("Seven-step reduction: 30x from one kernel",
// opening section, lists it beside the sum and the maximum): per output the
// maximum m of its terms and s = sum exp(x - c) with c = m when m is finite,
// else 0, so that softmax(x) = exp(x - c) / s.  It is one pass over x: the
// maximum and the sum of exponentials are folded together ("online"
// softmax), e^y being computed as 2^(y log2 e) by the hardware exp2.
//  * A lane's running state is (m, c, s) with s = sum exp(x - c) over the
//    terms it has seen.  The shift c is moved only when the running maximum
//    leaves [c, c + kLazy] (lazy re-centring): s is then multiplied by
//    e^(c_old - c_new) <= e^-kLazy, so the rounding of each re-centring
//    weighs on terms that the next one shrinks by e^-kLazy again, and the
//    errors cannot pile up however slowly the maximum creeps up; every term
//    stays at or below e^kLazy.
//  * Joined states, and stored ones, are re-centred on their maximum
//    exactly (c = m, or 0 when m is not finite), which the pair (m, s)
//    implies; a join multiplies by e^(c - m) with the exponent's rounding
//    compensated (2^(zh + zl) = 2^zh (1 + zl ln 2) with zh + zl = d log2 e
//    to ~2^-48).  Joins of a finite maximum re-centre both sides; joins of
//    an infinite or NaN maximum add the s values (+Inf, NaN propagate).
//  * Terms x = -Inf add exp(-Inf) = 0; +Inf makes m = +Inf and s = +Inf; a
//    NaN makes both NaN; no terms give (-Inf, 0).
constexpr float kLog2e = 1.44269502f;        // log2(e) rounded to fp32
constexpr float kLog2eLo = 1.925963e-8f;     // log2(e) - kLog2e
constexpr float kLn2 = 0.693147182f;
constexpr float kLazy = 8.f;

__device__ __forceinline__ float sm_exp(float y) {
    return __builtin_amdgcn_exp2f(y * kLog2e);
}

__device__ __forceinline__ v4f sm_exp(v4f y) {
    return v4f{sm_exp(y.x), sm_exp(y.y), sm_exp(y.z), sm_exp(y.w)};
}

__device__ __forceinline__ bool sm_finite(float m) { return __builtin_isfinite(m); }

// The shift a maximum implies: m when finite, else 0.
__device__ __forceinline__ float sm_shift(float m) { return sm_finite(m) ? m : 0.f; }

// e^(a - b) for finite a, b, with the exponent's rounding compensated: the
// difference is split exactly into dh + dl (two-sum), d log2 e into zh + zl,
// and 2^(zh + zl) = 2^zh (1 + zl ln 2).
__device__ __forceinline__ float sm_factor(float a, float b) {
    const float dh = a - b;
    const float bv = dh - a;
    const float dl = (a - (dh - bv)) - (b + bv);
    const float zh = dh * kLog2e;
    const float zl = (__builtin_fmaf(dh, kLog2e, -zh) + dh * kLog2eLo) + dl * kLog2e;
    const float e = __builtin_amdgcn_exp2f(zh);
    return __builtin_fmaf(e, zl * kLn2, e);
}

// s * e^(a - b) for finite a, b; s == 0 stays 0 whatever the factor, and
// a == b leaves s as it is.  No branch: both sides are computed.
__device__ __forceinline__ float sm_rescale(float s, float a, float b) {
    const float f = sm_factor(a, b);
    return ((s == 0.f) | (a == b)) ? s : s * f;
}

struct SmPair {   // (m, s), s relative to sm_shift(m)
    float m, s;
};
struct SmState4 {  // four independent running states
    v4f m, c, s;
};
struct SmOut {    // where pairs are stored: the maxima, the sums
    float* __restrict__ m;
    float* __restrict__ s;
};

__device__ __forceinline__ SmPair sm_join(SmPair a, SmPair b) {
    const float m = __builtin_elementwise_maximum(a.m, b.m);
    if (!sm_finite(m)) return SmPair{m, a.s + b.s};
    return SmPair{m, sm_rescale(a.s, sm_shift(a.m), m) + sm_rescale(b.s, sm_shift(b.m), m)};
}

// ------------------------------------------------------------- states
// St<OP> is how the kernels hold, move and store partial results:
//   S1 / S4   one partial result / four independent ones (float4 lanes)
//   Out       where results are stored (an array, or a pair of arrays)
//   start1/4  the empty result;  fold(S4, v4f) adds one term per lane;
//   fold_x    adds one term to lane x only;  fold_all<U> adds U float4s of
//   terms into acc[0..1];  join (S1 or S4);  lane / set_lane move one lane
//   of an S4;  get / put / at read, write and offset an Out, get4 reads
//   four consecutive results as an S4;  fill is the value of a load lane
//   that holds no term (neutral for fold).
// For sum, sum of squares, maximum and minimum a result is one float and
// every step is the Op<OP> arithmetic above.
template <int OP>
struct St {
    typedef float S1;
    typedef v4f S4;
    typedef float* __restrict__ Out;
    static __device__ __forceinline__ S1 start1() { return Op<OP>::start(); }
    static __device__ __forceinline__ S4 start4() {
        const float s = Op<OP>::start();
        return v4f{s, s, s, s};
    }
    static __device__ __forceinline__ float fill() { return Op<OP>::start(); }
    static __device__ __forceinline__ S4 fold(S4 a, v4f v) { return Op<OP>::fold(a, v); }
    static __device__ __forceinline__ S1 fold(S1 a, float v) { return Op<OP>::fold(a, v); }
    static __device__ __forceinline__ S4 fold_x(S4 a, float v) {
        a.x = Op<OP>::fold(a.x, v);
        return a;
    }
    template <int U>
    static __device__ __forceinline__ void fold_all(S4 (&acc)[2], const v4f (&v)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) acc[u & 1] = Op<OP>::fold(acc[u & 1], v[u]);
    }
    static __device__ __forceinline__ S4 join(S4 a, S4 b) { return Op<OP>::join(a, b); }
    static __device__ __forceinline__ S1 join(S1 a, S1 b) { return Op<OP>::join(a, b); }
    static __device__ __forceinline__ S1 lane(S4 a, int q) { return a[q]; }
    static __device__ __forceinline__ void set_lane(S4& a, int q, S1 v) { a[q] = v; }
    static __device__ __forceinline__ S1 get(Out o, int64_t e) { return o[e]; }
    static __device__ __forceinline__ S4 get4(Out o, int64_t e) { return load4<false>(o + e); }
    static __device__ __forceinline__ void put(Out o, int64_t e, S1 v) { o[e] = v; }
    static __device__ __forceinline__ Out at(Out o, int64_t e) { return o + e; }
    static Out make_out(float* a, float*) { return a; }
};

template <>
struct St<RD_OP_SOFTMAX_DENOM> {
    typedef SmPair S1;
    typedef SmState4 S4;
    typedef SmOut Out;
    static __device__ __forceinline__ S1 start1() { return SmPair{-__builtin_inff(), 0.f}; }
    static __device__ __forceinline__ S4 start4() {
        const float n = -__builtin_inff();
        return SmState4{v4f{n, n, n, n}, v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}};
    }
    static __device__ __forceinline__ float fill() { return -__builtin_inff(); }
    // U float4s of terms into acc[0]: the new maxima first, a lazy re-centring
    // of the lanes whose finite maximum left [c, c + kLazy] (or that hold
    // nothing yet, s == 0, where it costs no rounding), then the sum of the
    // exponentials.
    template <int U>
    static __device__ __forceinline__ void fold_all(S4 (&acc)[2], const v4f (&v)[U]) {
        S4& a = acc[0];
        v4f mb = a.m;
#pragma unroll
        for (int u = 0; u < U; ++u) mb = __builtin_elementwise_maximum(mb, v[u]);
        // A lane whose state holds a sum (s != 0) has c <= m: c was a
        // maximum of its terms.  Re-centre where the maximum is finite and
        // either nothing is held yet or it passed c + kLazy; the test takes
        // no branch per lane, the (rare) re-centring one for all four.
        bool need[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
            need[q] = sm_finite(mb[q]) & ((a.s[q] == 0.f) | (mb[q] > a.c[q] + kLazy));
        if (need[0] | need[1] | need[2] | need[3]) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float r = sm_rescale(a.s[q], a.c[q], mb[q]);
                a.s[q] = need[q] ? r : a.s[q];
                a.c[q] = need[q] ? mb[q] : a.c[q];
            }
        }
        a.m = mb;
        // the U exponentials summed by a pairwise tree, then added to s: the
        // long-running sum takes one rounding per U terms
        v4f t[U];
#pragma unroll
        for (int u = 0; u < U; ++u) t[u] = sm_exp(v[u] - a.c);
#pragma unroll
        for (int w = 1; w < U; w *= 2)
#pragma unroll
            for (int u = 0; u + w < U; u += 2 * w) t[u] = t[u] + t[u + w];
        a.s = a.s + t[0];
    }
    static __device__ __forceinline__ S4 fold(S4 a, v4f v) {
        S4 acc[2] = {a, a};
        const v4f w[1] = {v};
        fold_all<1>(acc, w);
        return acc[0];
    }
    static __device__ __forceinline__ S4 fold_x(S4 a, float v) {
        const float n = -__builtin_inff();
        return fold(a, v4f{v, n, n, n});
    }
    static __device__ __forceinline__ S1 fold(S1 a, float v) {
        const bool f = sm_finite(v);
        return sm_join(a, SmPair{v, f ? 1.f : sm_exp(v)});
    }
    // one lane of a running state, re-centred on its maximum
    static __device__ __forceinline__ S1 lane(S4 a, int q) {
        const float m = a.m[q];
        return SmPair{m, sm_finite(m) ? sm_rescale(a.s[q], a.c[q], m) : a.s[q]};
    }
    static __device__ __forceinline__ void set_lane(S4& a, int q, S1 v) {
        a.m[q] = v.m;
        a.c[q] = sm_shift(v.m);
        a.s[q] = v.s;
    }
    static __device__ __forceinline__ S4 join(S4 a, S4 b) {
        S4 r;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float m = __builtin_elementwise_maximum(a.m[q], b.m[q]);
            r.m[q] = m;
            if (sm_finite(m)) {
                r.c[q] = m;
                r.s[q] = sm_rescale(a.s[q], a.c[q], m) + sm_rescale(b.s[q], b.c[q], m);
            } else {
                r.c[q] = 0.f;
                r.s[q] = a.s[q] + b.s[q];
            }
        }
        return r;
    }
    static __device__ __forceinline__ S1 join(S1 a, S1 b) { return sm_join(a, b); }
    static __device__ __forceinline__ S1 get(Out o, int64_t e) { return SmPair{o.m[e], o.s[e]}; }
    // four stored pairs as running states: each sum is relative to its
    // pair's shift
    static __device__ __forceinline__ S4 get4(Out o, int64_t e) {
        S4 r;
        r.m = load4<false>(o.m + e);
        r.s = load4<false>(o.s + e);
#pragma unroll
        for (int q = 0; q < 4; ++q) r.c[q] = sm_shift(r.m[q]);
        return r;
    }
    static __device__ __forceinline__ void put(Out o, int64_t e, S1 v) {
        o.m[e] = v.m;
        o.s[e] = v.s;
    }
    static __device__ __forceinline__ Out at(Out o, int64_t e) { return SmOut{o.m + e, o.s + e}; }
    static Out make_out(float* a, float* b) { return SmOut{a, b}; }
};

// The four lanes of an S4 joined in a fixed order.
template <int OP>
__device__ __forceinline__ typename St<OP>::S1 join_lanes(typename St<OP>::S4 a) {
    typedef St<OP> T;
    return T::join(T::join(T::lane(a, 0), T::lane(a, 1)), T::join(T::lane(a, 2), T::lane(a, 3)));
}

// ------------------------------------------------- wave and block steps
template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl,
                                           0xF, 0xF, false));
}

template <int kCtrl>
__device__ __forceinline__ SmPair dpp(SmPair v) {
    return SmPair{dpp<kCtrl>(v.m), dpp<kCtrl>(v.s)};
}

// ds_swizzle swap of 16 lanes, and v_readlane, for each kind of result
__device__ __forceinline__ float swap16(float v) {
    return __builtin_bit_cast(float,
                              __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
}

__device__ __forceinline__ SmPair swap16(SmPair v) { return SmPair{swap16(v.m), swap16(v.s)}; }

__device__ __forceinline__ float read_lane(float v, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

__device__ __forceinline__ SmPair read_lane(SmPair v, int l) {
    return SmPair{read_lane(v.m, l), read_lane(v.s, l)};
}

// Join of v over the 64 lanes of a wavefront; every lane must be active.
// Butterfly: lane pairs at distance 1 and 2 (DPP quad_perm), quads paired by
// mirroring 8 lanes (row_half_mirror), 8-lane halves paired by mirroring 16
// lanes (row_mirror), 16-lane rows paired by a swizzle swap of 16, and the
// two 32-lane halves joined through lanes 0 and 32.  Each step joins a
// lane's value with an equal-rank partner's, and every join is commutative,
// so every lane ends with the same bits.
// The softmax pair takes the same butterfly twice instead of joining pairs:
// first the maximum m, then every lane's sum re-centred on m once and the
// sums added -- one exp2 per lane rather than a rescale at every step.
__device__ __forceinline__ float wave_max(float m) {
    m = __builtin_elementwise_maximum(m, dpp<0xB1>(m));
    m = __builtin_elementwise_maximum(m, dpp<0x4E>(m));
    m = __builtin_elementwise_maximum(m, dpp<0x141>(m));
    m = __builtin_elementwise_maximum(m, dpp<0x140>(m));
    m = __builtin_elementwise_maximum(m, swap16(m));
    return __builtin_elementwise_maximum(read_lane(m, 0), read_lane(m, 32));
}

__device__ __forceinline__ float wave_add(float s) {
    s = s + dpp<0xB1>(s);
    s = s + dpp<0x4E>(s);
    s = s + dpp<0x141>(s);
    s = s + dpp<0x140>(s);
    s = s + swap16(s);
    return read_lane(s, 0) + read_lane(s, 32);
}

template <int OP>
__device__ __forceinline__ typename St<OP>::S1 wave_reduce(typename St<OP>::S1 v) {
    typedef St<OP> T;
    if constexpr (OP == RD_OP_SOFTMAX_DENOM) {
        const float m = wave_max(v.m);
        // a finite maximum: each sum re-centred on it (a lane that holds
        // nothing has s = 0 and stays 0); otherwise the sums are added as
        // they are (+Inf, NaN propagate; all -Inf gives 0)
        const float s = sm_finite(m) ? sm_rescale(v.s, sm_shift(v.m), m) : v.s;
        return SmPair{m, wave_add(s)};
    }
    v = T::join(v, dpp<0xB1>(v));   // quad_perm [1,0,3,2]
    v = T::join(v, dpp<0x4E>(v));   // quad_perm [2,3,0,1]
    v = T::join(v, dpp<0x141>(v));  // row_half_mirror
    v = T::join(v, dpp<0x140>(v));  // row_mirror
    v = T::join(v, swap16(v));
    return T::join(read_lane(v, 0), read_lane(v, 32));
}

// The value v of lane `src` (ds_bpermute).  v is taken by value: a bit cast
// applied to a vector element in place was miscompiled into one permute of
// element 0 for all four.
__device__ __forceinline__ float lane_value(int src, float v) {
    return __builtin_bit_cast(float,
                              __builtin_amdgcn_ds_bpermute(4 * src, __builtin_bit_cast(int, v)));
}

// All four lanes of lane `src`'s partial results, one permute per float.
__device__ __forceinline__ v4f lane_value(int src, v4f a) {
    v4f t;
#pragma unroll
    for (int j = 0; j < 4; ++j) t[j] = lane_value(src, a[j]);
    return t;
}

__device__ __forceinline__ SmState4 lane_value(int src, SmState4 a) {
    return SmState4{lane_value(src, a.m), lane_value(src, a.c), lane_value(src, a.s)};
}

// Join over a kBlock-thread workgroup, valid in thread 0: wave butterflies,
// then the wave results in wave order.  The caller syncs before reusing lds.
template <int OP>
__device__ __forceinline__ typename St<OP>::S1 block_reduce(typename St<OP>::S1 v,
                                                            typename St<OP>::S1* lds) {
    typedef St<OP> T;
    v = wave_reduce<OP>(v);
    if (threadIdx.x % kWave == 0) lds[threadIdx.x / kWave] = v;
    __syncthreads();
    typename T::S1 t = T::start1();
    if (threadIdx.x == 0) {
        t = lds[0];
#pragma unroll
        for (int k = 1; k < kBlock / kWave; ++k) t = T::join(t, lds[k]);
    }
    return t;
}

// out_o = the join of the P piece results of one row.  Lane t keeps four
// running results, the pieces 4q .. 4q + 3 for q = t, t + 256, ... joined
// lane-wise in that order (16-byte loads, kCombineLoads of them issued before
// the first join, so tens of thousands of pieces cost a few memory round
// trips); its four lanes are then joined (join_lanes), the P % 4 last pieces
// joined by threads 0 .. 2, then the workgroup reduction.  Used by the second
// pass and by the last workgroup of a fused first pass, so both give the same
// bits.  Every thread of the workgroup must call it.
constexpr int kCombineLoads = 16;

template <int OP>
__device__ __forceinline__ void combine_row(typename St<OP>::Out part, int64_t P,
                                            typename St<OP>::Out out_o,
                                            typename St<OP>::S1* lds) {
    typedef St<OP> T;
    const int64_t nq = P >> 2;
    typename T::S4 acc = T::start4();
    for (int64_t q = threadIdx.x; q < nq; q += kCombineLoads * kBlock) {
        typename T::S4 v[kCombineLoads];
#pragma unroll
        for (int u = 0; u < kCombineLoads; ++u)
            if (q + u * kBlock < nq) v[u] = T::get4(part, 4 * (q + u * kBlock));
#pragma unroll
        for (int u = 0; u < kCombineLoads; ++u)
            if (q + u * kBlock < nq) acc = T::join(acc, v[u]);
    }
    typename T::S1 t = join_lanes<OP>(acc);
    if (threadIdx.x < (P & 3)) t = T::join(t, T::get(part, 4 * nq + threadIdx.x));
    t = block_reduce<OP>(t, lds);
    if (threadIdx.x == 0) T::put(out_o, 0, t);
    __syncthreads();
}

// Where the rows of the ROWS kernels start.  Row o (o < rows) is the pair
// (o / ninner, o % ninner) of a view whose reduced axis is contiguous; it
// starts at (o / ninner) * so + (o % ninner) * si floats from x.  A
// contiguous [outer, R] array is ninner = 1, so = R.
struct RowMap {
    int64_t so, si, ninner;
};

__device__ __forceinline__ int64_t row_start(const RowMap& m, int64_t o) {
    if (m.ninner == 1) return o * m.so;
    const int64_t a = o / m.ninner;
    return a * m.so + (o - a * m.ninner) * m.si;
}

constexpr int kPubLoads = 16;

// A piece result: stored to dst, or published -- the softmax pair as two
// words, its maximum at seg and its sum at nseg + seg.
template <int OP>
__device__ __forceinline__ void put_piece(typename St<OP>::Out dst, const Published& pub,
                                          int64_t seg, int64_t nseg, typename St<OP>::S1 v) {
    if (pub.words != nullptr) {
        if constexpr (OP == RD_OP_SOFTMAX_DENOM) {
            publish_word(pub.words + seg, pub.epoch, v.m);
            publish_word(pub.words + nseg + seg, pub.epoch, v.s);
        } else {
            publish_word(pub.words + seg, pub.epoch, v);
        }
        return;
    }
    St<OP>::put(dst, seg, v);
}

// The published values copied to vals, as piece results (words per piece:
// 1, or 2 for the softmax pair).
template <int OP>
constexpr int kPieceWords = OP == RD_OP_SOFTMAX_DENOM ? 2 : 1;

template <int OP>
__device__ __forceinline__ typename St<OP>::Out vals_out(float* vals, int64_t nseg) {
    if constexpr (OP == RD_OP_SOFTMAX_DENOM)
        return SmOut{vals, vals + nseg};
    else
        return vals;
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
// Single-launch combine (pub.words != null, P > 1, one-float operators):
// each piece result is published as a tagged word instead of stored to dst,
// and the grid's last workgroup (hardware id gridDim.x - 1), once its own
// pieces are done, waits for every word, copies the values to pub.vals and
// joins every row's pieces with combine_row into out[0 .. outer) -- the
// second kernel's code, so the same bits.  No other workgroup waits on
// anything, so the one that waits can always be outlasted: however the
// workgroups are scheduled, the others finish and publish.  No fence and no
// counter: the tag (the launch's epoch) travels with each value.
// At most 5 waves per SIMD: the U loads of a step are all issued before the
// first fold waits (about 90 VGPRs at U = 16).  Left free to aim at 8 waves,
// the compiler squeezed the kernel into 64 VGPRs by waiting after every
// other load, and the 1D reduce of 1e9 floats -- 1 wave per SIMD -- lost
// 1.2 % (measured on MI355X).
template <int OP, int G, int U, bool NT>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(1, 5)))
void rows_kernel(const float* __restrict__ x,
                                                      RowMap map, int64_t R, int64_t nseg,
                                                      int64_t P, int32_t blocked,
                                                      typename St<OP>::Out dst,
                                                      uint32_t nxcd, Published pub,
                                                      typename St<OP>::Out out) {
    static_assert(G == kWave || G == kBlock, "group is a wave or a workgroup");
    typedef St<OP> T;
    constexpr int kGroups = kBlock / G;
    __shared__ typename T::S1 lds[kBlock / kWave];
    const int gl = threadIdx.x % G;
    const int64_t nvec = R >> 2;
    const int64_t tail = R & 3;
    const int64_t span = ((nvec + P - 1) / P + G - 1) / G * G;  // blocked: chunks per piece
    const int64_t L = blocked ? int64_t(G) : P * G;            // a lane's chunk stride
    const int64_t gstride = int64_t(gridDim.x) * kGroups;
    for (int64_t first = xcd_block(nxcd) * kGroups; first < nseg; first += gstride) {
        const int64_t seg = first + threadIdx.x / G;  // uniform per group
        typename T::S1 total = T::start1();
        if (seg < nseg) {
            const int64_t o = seg / P;
            const int64_t piece = seg - o * P;
            const int64_t g = piece * G + gl;
            const float* row = x + row_start(map, o);
            int64_t j = blocked ? piece * span + gl : g;
            int64_t end = nvec;
            if (blocked && piece * span + span < nvec) end = piece * span + span;
            typename T::S4 acc[2] = {T::start4(), T::start4()};
            for (; j + (U - 1) * L < end; j += U * L) {
                v4f v[U];
#pragma unroll
                for (int u = 0; u < U; ++u) v[u] = load4<NT>(row + 4 * (j + u * L));
                T::template fold_all<U>(acc, v);
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (j + u * L < end)
                    acc[u & 1] = T::fold(acc[u & 1], load4<NT>(row + 4 * (j + u * L)));
            if (g < tail) acc[0] = T::fold_x(acc[0], row[4 * nvec + g]);
            total = join_lanes<OP>(T::join(acc[0], acc[1]));
        }
        if constexpr (G == kBlock) {
            total = block_reduce<OP>(total, lds);
            if (threadIdx.x == 0) put_piece<OP>(dst, pub, seg, nseg, total);
            __syncthreads();
        } else {
            total = wave_reduce<OP>(total);
            if (gl == 0 && seg < nseg) put_piece<OP>(dst, pub, seg, nseg, total);
        }
    }
    if (pub.words != nullptr && blockIdx.x == gridDim.x - 1) {
        __syncthreads();  // lds is free again
        // kPubLoads words in flight per thread; a word not yet tagged with
        // this launch's epoch is then polled on its own
        const int64_t nw = kPieceWords<OP> * nseg;
        for (int64_t i0 = threadIdx.x; i0 < nw; i0 += kPubLoads * kBlock) {
            uint64_t w[kPubLoads];
#pragma unroll
            for (int u = 0; u < kPubLoads; ++u) {
                const int64_t i = i0 + u * kBlock;
                w[u] = i < nw ? __hip_atomic_load(pub.words + i, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT)
                              : 0;
            }
#pragma unroll
            for (int u = 0; u < kPubLoads; ++u) {
                const int64_t i = i0 + u * kBlock;
                if (i < nw)
                    pub.vals[i] = uint32_t(w[u] >> 32) == pub.epoch
                                      ? __builtin_bit_cast(float, uint32_t(w[u]))
                                      : await_word(pub.words + i, pub.epoch, pub.spin_limit);
            }
        }
        __syncthreads();  // every value is in vals
        const typename T::Out part = vals_out<OP>(pub.vals, nseg);
        const int64_t outer = nseg / P;
        for (int64_t o = 0; o < outer; ++o) combine_row<OP>(T::at(part, o * P), P, T::at(out, o), lds);
    }
}

// Rows shorter than a wave's worth of chunks: one lane per row, 16-byte
// loads along the row, then the R % 4 tail in order.
template <int OP>
__global__ __launch_bounds__(kBlock) void rows_short_kernel(const float* __restrict__ x,
                                                            RowMap map, int64_t outer,
                                                            int64_t R,
                                                            typename St<OP>::Out out) {
    typedef St<OP> T;
    const int64_t stride = int64_t(gridDim.x) * kBlock;
    for (int64_t o = int64_t(blockIdx.x) * kBlock + threadIdx.x; o < outer; o += stride) {
        const float* row = x + row_start(map, o);
        typename T::S4 acc = T::start4();
        int64_t k = 0;
        for (; k + 4 <= R; k += 4) acc = T::fold(acc, load4<false>(row + k));
        typename T::S1 t = join_lanes<OP>(acc);
        for (; k < R; ++k) t = T::fold(t, row[k]);
        T::put(out, o, t);
    }
}

// Short rows that are adjacent in memory (row o at o*R, R < 64): a lane per
// row reads 16 bytes from each of 64 rows R floats apart per load, so a
// workgroup instead stages 256 rows at a time through LDS.  The tile's 256*R
// floats are read with coalesced 16-byte loads (thread t takes float4s
// t, t + 256, ...) and each float is put at (row, column) of an LDS tile
// whose pitch is odd (R, or R + 1 for even R), so that thread t then reads
// row t without bank conflicts.  Thread t folds its row in the order of
// rows_short_kernel (float4 groups into four accumulators, their join, the
// R % 4 tail), so both give the same bits.  The (row, column) of a float is
// the same in every tile and is advanced incrementally (1024 floats per
// step), with no division per element.  Dynamic LDS: 256 * pitch floats.
template <int OP>
__global__ __launch_bounds__(kBlock) void rows_short_tile_kernel(const float* __restrict__ x,
                                                                 int64_t outer, int32_t R,
                                                                 int32_t pitch, int32_t TR,
                                                                 typename St<OP>::Out out) {
    typedef St<OP> T;
    extern __shared__ float tile[];
    const int t = threadIdx.x;
    // the float4 a thread loads first starts at float 4t of the tile
    const int row0 = (4 * t) / R;
    const int col0 = 4 * t - row0 * R;
    const int drow = (4 * kBlock) / R;  // one step: 1024 floats further
    const int dcol = 4 * kBlock - drow * R;
    const int64_t ntiles = (outer + TR - 1) / TR;
    for (int64_t tb = blockIdx.x; tb < ntiles; tb += gridDim.x) {
        const int64_t o0 = tb * TR;
        const int rows = outer - o0 < TR ? int(outer - o0) : TR;
        const int nf = rows * R;  // floats of this tile (< 16384)
        const float* base = x + o0 * R;
        __syncthreads();  // the previous tile's rows have been read
        int row = row0, col = col0;
        for (int j = t; 4 * j + 3 < nf; j += kBlock) {
            const v4f v = load4<true>(base + 4 * j);
            int r = row, c = col;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                tile[r * pitch + c] = v[q];
                if (++c == R) {
                    c = 0;
                    ++r;
                }
            }
            row += drow;
            col += dcol;
            if (col >= R) {
                col -= R;
                ++row;
            }
        }
        for (int g = (nf & ~3) + t; g < nf; g += kBlock) {  // nf % 4 last floats
            const int r = g / R;
            tile[r * pitch + (g - r * R)] = base[g];
        }
        __syncthreads();
        if (t < rows) {
            const float* rw = tile + t * pitch;
            typename T::S4 acc = T::start4();
            int k = 0;
            for (; k + 4 <= R; k += 4) acc = T::fold(acc, v4f{rw[k], rw[k + 1], rw[k + 2], rw[k + 3]});
            typename T::S1 v = join_lanes<OP>(acc);
            for (; k < R; ++k) v = T::fold(v, rw[k]);
            T::put(out, o0 + t, v);
        }
    }
}

// Rows per LDS tile of rows_short_tile_kernel: 256, 128 or 64, the most
// whose tile fits 22 KB.  Measured on MI355X, the tile size is what matters
// (smaller tiles, more workgroups per CU): [4194304, 8] 62 % of peak with 256
// rows vs 46 % with 128; [2097152, 40] 80 % with 128 vs 54 % with 256;
// [1048576, 63] 81 % with 64 vs 41 % with 256.
int32_t short_tile_rows(int64_t R) {
    const int64_t pitch = R | 1;
    for (int32_t tr = kBlock; tr > 64; tr /= 2)
        if (tr * pitch * int64_t(sizeof(float)) <= 22528) return tr;
    return 64;
}

// Second pass of ROWS: out[o] = combine_row over the P piece results of row o.
template <int OP>
__global__ __launch_bounds__(kBlock) void rows_combine_kernel(typename St<OP>::Out part,
                                                              int64_t outer, int64_t P,
                                                              typename St<OP>::Out out) {
    typedef St<OP> T;
    __shared__ typename T::S1 lds[kBlock / kWave];
    for (int64_t o = blockIdx.x; o < outer; o += gridDim.x)
        combine_row<OP>(T::at(part, o * P), P, T::at(out, o), lds);
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
// slab_combine_kernel.  Needs inner >= 4.  Element (o, r, c) is read at
// x + o*so + r*sr + c: columns are contiguous, rows and outer indices may be
// any distance apart (a contiguous array has so = R*inner, sr = inner).
// Column c goes to output c / cstride of its outer index (inner_out per outer
// index) when c % cstride == 0: cstride == 1 for an array; a strided view whose
// terms are cstride floats apart along its kept inner axis is read as the dense
// span of its rows and only every cstride-th column is kept (each column has
// accumulator lanes of its own, so the floats in between never reach a kept
// result).
// pub.words != nullptr (one-wave tiles with row waves, one float per result,
// at most kPubColMaxSlabs slabs, a workgroup per item, all resident): the
// slabs are joined in the same launch.  The workgroups of slabs 0 .. S-2
// publish their results as tagged words at pub.words[(s*outer + o)*inner_out
// + k]; in the workgroup of the last slab, wave rw fetches slabs rw, rw + RW,
// ... of its tile's columns into LDS (a wait that runs out gives NaN), and
// wave 0 joins slab 0, 1, ..., S-2 and its own result in that order into out
// -- slab_combine_kernel's order, so the same bits.
template <int CW, int RW, int OP>
constexpr bool cols_pub_shape() {
    return CW == 1 && RW > 1 && OP != RD_OP_SOFTMAX_DENOM;
}

template <int OP, int CW, int RW>
constexpr int cols_lds_slots() {
    if constexpr (cols_pub_shape<CW, RW, OP>())
        return (RW - 1 > kPubColMaxSlabs - 1 ? RW - 1 : int(kPubColMaxSlabs) - 1) * kWave;
    return RW > 1 ? (RW - 1) * CW * kWave : 1;
}

// The four tagged words at base + idx[q] (idx[q] < 0: none, its lane 0),
// polled together until each carries `tag`, at most spin_limit + 1 times; a
// word that never comes gives NaN.
__device__ __forceinline__ v4f await_words4(const uint64_t* base, const int64_t (&idx)[4],
                                            uint32_t tag, uint32_t spin_limit) {
    v4f r = {0.f, 0.f, 0.f, 0.f};
    for (uint32_t it = 0;; ++it) {
        uint64_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
            w[q] = idx[q] >= 0 ? __hip_atomic_load(base + idx[q], __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT)
                               : uint64_t(tag) << 32;
        bool all = true;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const bool ok = uint32_t(w[q] >> 32) == tag;
            all = all && ok;
            r[q] = ok ? __builtin_bit_cast(float, uint32_t(w[q]))
                      : (it >= spin_limit ? __builtin_nanf("") : r[q]);
        }
        if (all || it >= spin_limit) return r;
        __builtin_amdgcn_s_sleep(1);
    }
}

template <int OP, int CW, int RW, int U, bool NT>
__global__ __launch_bounds__(kWave* CW* RW) void cols_kernel(
    const float* __restrict__ x, int64_t outer, int64_t R, int64_t inner, int64_t so,
    int64_t sr, int64_t ntiles, int64_t S, int64_t rps, int64_t cstride, int64_t inner_out,
    typename St<OP>::Out dst, uint32_t nxcd, Published pub, typename St<OP>::Out out) {
    typedef St<OP> T;
    __shared__ typename T::S4 lds[cols_lds_slots<OP, CW, RW>()];
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
        typename T::S4 acc[2] = {T::start4(), T::start4()};
        if (active) {
            const float* p = x + o * so + r0 * sr + cl;
            const int64_t step = RW * sr;
            int64_t k = 0;
            if constexpr (OP == RD_OP_SOFTMAX_DENOM) {
                // Software-pipelined: the next U rows are loaded before the
                // exponentials of the current U are taken, so the loads stay
                // in flight across the arithmetic (two waves per SIMD do not
                // hide it otherwise).  Same order of the folds.
                if (k + U <= m) {
                    v4f cur[U];
#pragma unroll
                    for (int u = 0; u < U; ++u) cur[u] = load4<NT>(p + u * step);
                    p += U * step;
                    for (; k + 2 * U <= m; k += U) {
                        v4f nxt[U];
#pragma unroll
                        for (int u = 0; u < U; ++u) nxt[u] = load4<NT>(p + u * step);
                        T::template fold_all<U>(acc, cur);
#pragma unroll
                        for (int u = 0; u < U; ++u) cur[u] = nxt[u];
                        p += U * step;
                    }
                    T::template fold_all<U>(acc, cur);
                    k += U;
                }
            } else {
                for (; k + U <= m; k += U) {
                    v4f v[U];
#pragma unroll
                    for (int u = 0; u < U; ++u) v[u] = load4<NT>(p + u * step);
                    T::template fold_all<U>(acc, v);
                    p += U * step;
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (k + u < m) acc[u & 1] = T::fold(acc[u & 1], load4<NT>(p + u * step));
        }
        typename T::S4 a = T::join(acc[0], acc[1]);
        if constexpr (RW > 1) {
            if (rw > 0) lds[((rw - 1) * CW + cw) * kWave + lane] = a;
            __syncthreads();
            if (rw == 0) {
#pragma unroll
                for (int q = 1; q < RW; ++q)
                    a = T::join(a, lds[((q - 1) * CW + cw) * kWave + lane]);
            }
            __syncthreads();
        }
        if constexpr (cols_pub_shape<CW, RW, OP>()) {
            if (pub.words) {
                // this lane's kept columns: their result index in o's row, or -1
                int64_t idx[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int64_t col = cl + q;
                    const int64_t k = cstride == 1 ? col : col / cstride;
                    idx[q] = active && col >= c && k * cstride == col ? k : -1;
                }
                if (s + 1 < S) {
                    if (rw == 0) {
                        uint64_t* w = pub.words + (s * outer + o) * inner_out;
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            if (idx[q] >= 0) publish_word(w + idx[q], pub.epoch, T::lane(a, q));
                    }
                    continue;
                }
                for (int64_t j = rw; j < S - 1; j += RW)
                    lds[j * kWave + lane] = await_words4(pub.words + (j * outer + o) * inner_out,
                                                         idx, pub.epoch, pub.spin_limit);
                __syncthreads();
                if (rw == 0) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        if (idx[q] < 0) continue;
                        float t = lds[lane][q];
                        for (int64_t j = 1; j < S - 1; ++j) t = T::join(t, lds[j * kWave + lane][q]);
                        T::put(out, o * inner_out + idx[q], T::join(t, T::lane(a, q)));
                    }
                }
                __syncthreads();
                continue;
            }
        }
        if (rw == 0 && active) {
            const int keep = int(c - cl);  // 0, or 1..3 for the row's last lane
            if (cstride == 1) {
                const int64_t e = (s * outer + o) * inner + cl;
                for (int q = keep; q < 4; ++q) T::put(dst, e + q, T::lane(a, q));
            } else {
                const int64_t e = (s * outer + o) * inner_out;
                for (int q = keep; q < 4; ++q) {
                    const int64_t col = cl + q;
                    const int64_t k = col / cstride;
                    if (k * cstride == col) T::put(dst, e + k, T::lane(a, q));
                }
            }
        }
    }
}

// Small inner (2 <= inner <= 128): several rows of one outer index per load
// instruction.  Element (o, r, c) is at x + o*so + r*sr + c as in cols_kernel.
// In a contiguous array (sr = inner) the rows of one outer index are
// adjacent in memory, so a wave
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
    const float* __restrict__ x, int64_t outer, int64_t R, int64_t inner, int64_t so,
    int64_t sr, int64_t S, int64_t rps, int32_t LC, typename St<OP>::Out dst,
    uint32_t nxcd) {
    typedef St<OP> T;
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
    const int64_t step = int64_t(RPW) * sr;
    const float fill = T::fill();

    // the row phases of each lane-column joined by a fixed tree, then stored
    auto finish = [&](int64_t item, typename T::S4 (&acc)[2]) {
        const int64_t o = item / S;
        const int64_t s = item - o * S;
        typename T::S4 a = T::join(acc[0], acc[1]);
        if (LC == 1) {
#pragma unroll
            for (int j = 0; j < V; ++j) T::set_lane(a, j, wave_reduce<OP>(T::lane(a, j)));
        } else {
            for (int d = 1; d < RPW; d *= 2) {
                const int src = lane + d * LC < kWave ? lane + d * LC : lane;
                const typename T::S4 t = lane_value(src, a);
                if ((rho & (2 * d - 1)) == 0 && rho + d < RPW) a = T::join(a, t);
            }
        }
        if (rho == 0) {
            const int64_t e = (s * outer + o) * inner + cl;
            if constexpr (V == 4) {
                for (int q = keep; q < 4; ++q) T::put(dst, e + q, T::lane(a, q));
            } else {
                for (int q = 0; q < V; ++q) T::put(dst, e + q, T::lane(a, q));
            }
        }
    };

    if (rps <= int64_t(RPW) * U && nitems > wstride) {
        // Every item is one step of at most U load instructions and a wave
        // has several: it issues the next item's loads before it folds,
        // joins and stores the current one, so short items (a few KB) do not
        // each wait out a memory round trip.  Instructions past the item's
        // rows load the neutral fill, which every fold leaves unchanged.
        auto load_item = [&](int64_t item, v4f (&v)[U]) {
            const int64_t o = item / S;
            const int64_t s = item - o * S;
            const int64_t r0 = s * rps + rho;
            const int64_t r1 = (s + 1) * rps < R ? (s + 1) * rps : R;
            const int64_t m = active && r0 < r1 ? (r1 - r0 + RPW - 1) / RPW : 0;
            const float* p = x + o * so + r0 * sr + cl;
#pragma unroll
            for (int u = 0; u < U; ++u)
                v[u] = u < m ? loadv<V, NT>(p + u * step, fill) : v4f{fill, fill, fill, fill};
        };
        int64_t item = xcd_block(nxcd) * kWaves + wave;
        if (item >= nitems) return;
        v4f cur[U], nxt[U];
        load_item(item, cur);
        for (;;) {
            const int64_t next = item + wstride;
            const bool more = next < nitems;
            if (more) load_item(next, nxt);
            __builtin_amdgcn_sched_barrier(0);  // the next item's loads go out first
            typename T::S4 acc[2] = {T::start4(), T::start4()};
            T::template fold_all<U>(acc, cur);
            finish(item, acc);
            if (!more) break;
#pragma unroll
            for (int u = 0; u < U; ++u) cur[u] = nxt[u];
            item = next;
        }
        return;
    }

    for (int64_t item = xcd_block(nxcd) * kWaves + wave; item < nitems; item += wstride) {
        const int64_t o = item / S;
        const int64_t s = item - o * S;
        const int64_t r0 = s * rps + rho;
        const int64_t r1 = (s + 1) * rps < R ? (s + 1) * rps : R;
        const int64_t m = r0 < r1 ? (r1 - r0 + RPW - 1) / RPW : 0;
        typename T::S4 acc[2] = {T::start4(), T::start4()};
        if (active) {
            const float* p = x + o * so + r0 * sr + cl;
            int64_t k = 0;
            for (; k + U <= m; k += U) {
                v4f v[U];
#pragma unroll
                for (int u = 0; u < U; ++u) v[u] = loadv<V, NT>(p + u * step, fill);
                T::template fold_all<U>(acc, v);
                p += U * step;
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (k + u < m)
                    acc[u & 1] = T::fold(acc[u & 1], loadv<V, NT>(p + u * step, fill));
        }
        finish(item, acc);
    }
}

// Views with no unit stride along the reduced axis or the kept inner axis:
// one lane per (slab s, output e), e fastest, so a wave's lanes read
// neighbouring outputs.  Lane (s, e) folds the terms x[o*so + r*sr + i*si]
// of rows r in [s*rps, min(R, (s+1)*rps)) in r order, 8 loads in flight.
// With S == 1 dst is the output; otherwise dst is [S][outer*inner] for
// slab_combine_kernel.  Correct for any strides; as fast as scattered
// 4-byte loads allow.
template <int OP>
__global__ __launch_bounds__(kBlock) void strided_kernel(const float* __restrict__ x,
                                                         int64_t outer, int64_t R,
                                                         int64_t inner, int64_t so,
                                                         int64_t sr, int64_t si, int64_t S,
                                                         int64_t rps,
                                                         typename St<OP>::Out dst) {
    typedef St<OP> T;
    constexpr int kIn = 8;
    const int64_t n = outer * inner;
    const int64_t items = n * S;
    const int64_t stride = int64_t(gridDim.x) * kBlock;
    for (int64_t it = int64_t(blockIdx.x) * kBlock + threadIdx.x; it < items; it += stride) {
        const int64_t s = it / n;
        const int64_t e = it - s * n;
        const int64_t o = e / inner;
        const int64_t r0 = s * rps;
        const int64_t r1 = r0 + rps < R ? r0 + rps : R;
        const float* p = x + o * so + (e - o * inner) * si + r0 * sr;
        typename T::S1 t = T::start1();
        int64_t r = r0;
        for (; r + kIn <= r1; r += kIn) {
            float v[kIn];
#pragma unroll
            for (int u = 0; u < kIn; ++u) v[u] = p[u * sr];
#pragma unroll
            for (int u = 0; u < kIn; ++u) t = T::fold(t, v[u]);
            p += kIn * sr;
        }
        for (; r < r1; ++r, p += sr) t = T::fold(t, *p);
        T::put(dst, it, t);
    }
}

// Second pass of a split along R: out[e] = join of slab[0][e], slab[1][e], ...
// in that order; the slabs are loaded kSlabAhead at a time, so that many are
// in flight per thread.
constexpr int kSlabAhead = 8;

template <int OP>
__global__ __launch_bounds__(kBlock) void slab_combine_kernel(typename St<OP>::Out slab,
                                                              int64_t S, int64_t n,
                                                              typename St<OP>::Out out) {
    typedef St<OP> T;
    const int64_t stride = int64_t(gridDim.x) * kBlock;
    for (int64_t e = int64_t(blockIdx.x) * kBlock + threadIdx.x; e < n; e += stride) {
        typename T::S1 t = T::get(slab, e);
        int64_t s = 1;
        for (; s + kSlabAhead <= S; s += kSlabAhead) {
            typename T::S1 v[kSlabAhead];
#pragma unroll
            for (int u = 0; u < kSlabAhead; ++u) v[u] = T::get(slab, (s + u) * n + e);
#pragma unroll
            for (int u = 0; u < kSlabAhead; ++u) t = T::join(t, v[u]);
        }
        for (; s < S; ++s) t = T::join(t, T::get(slab, s * n + e));
        T::put(out, e, t);
    }
}

// The same for few outputs and many slabs (kSlabWaveMinS or more): a wave
// per output, lane l joining slabs l, l + 64, l + 128, ... in that order,
// then the wave's butterfly (wave_reduce) -- a fixed order, with every lane
// holding at least one slab.  A thread per output would walk all S slabs
// one after another.
constexpr int64_t kSlabWaveMinS = kWave;
constexpr int64_t kSlabWaveMaxN = 65536;

template <int OP>
__global__ __launch_bounds__(kBlock) void slab_combine_wave_kernel(typename St<OP>::Out slab,
                                                                   int64_t S, int64_t n,
                                                                   typename St<OP>::Out out) {
    typedef St<OP> T;
    const int lane = threadIdx.x % kWave;
    const int64_t waves = int64_t(gridDim.x) * (kBlock / kWave);
    for (int64_t e = int64_t(blockIdx.x) * (kBlock / kWave) + wave_in_block(); e < n;
         e += waves) {
        typename T::S1 t = T::get(slab, int64_t(lane) * n + e);
        for (int64_t s = lane + kWave; s < S; s += kWave) t = T::join(t, T::get(slab, s * n + e));
        t = wave_reduce<OP>(t);
        if (lane == 0) T::put(out, e, t);
    }
}

// R == 0: every output is the operator's start value.
template <int OP>
__global__ __launch_bounds__(kBlock) void fill_start_kernel(typename St<OP>::Out out,
                                                            int64_t n) {
    typedef St<OP> T;
    const int64_t stride = int64_t(gridDim.x) * kBlock;
    for (int64_t e = int64_t(blockIdx.x) * kBlock + threadIdx.x; e < n; e += stride)
        T::put(out, e, T::start1());
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

// The same with `lds` bytes of dynamic LDS.
template <typename... K>
hipError_t launch_lds(void (*kernel)(K...), int64_t blocks, int threads, size_t lds,
                      hipStream_t s, typename same<K>::type... args) {
    void* argv[] = {static_cast<void*>(&args)...};
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel),
                           dim3(static_cast<uint32_t>(blocks)), dim3(threads), argv, lds, s);
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
    if (op == RD_OP_SUM) return unroll_built(u);
    // the other one-float operators also take the shallow 256-lane shapes
    // the planner gives small inputs
    if (op != RD_OP_SOFTMAX_DENOM && g == kBlock && (u == 2 || u == 4)) return true;
    return u == 8 || u == 16;
}

constexpr bool col_shape_built(int cw, int rw) {
    return (cw == 1 && (rw == 1 || rw == 2 || rw == 4 || rw == 8 || rw == 16)) ||
           (cw == 2 && (rw == 1 || rw == 2 || rw == 4 || rw == 8)) ||
           (cw == 4 && (rw == 1 || rw == 2 || rw == 4)) || (cw == 8 && (rw == 1 || rw == 2)) ||
           (cw == 16 && rw == 1);
}

constexpr bool cols_built(int op, int cw, int rw, int u) {
    if (op == RD_OP_SUM) return col_shape_built(cw, rw) && unroll_built(u);
    // the planner's shapes: wide tiles, or one tile with 8 row waves in slabs
    if (cw == 1 && rw == 8 && u == 4) return true;
    if (op == RD_OP_SOFTMAX_DENOM)
        return rw == 1 && (cw == 1 || cw == 2 || cw == 4 || cw == 8) && (u == 4 || u == 8);
    return rw == 1 && (cw == 1 || cw == 2 || cw == 4 || cw == 8) && u == 4;
}

constexpr bool op_valid(int op) {
    return op == RD_OP_SUM || op == RD_OP_SUMSQ || op == RD_OP_MAX || op == RD_OP_MIN ||
           op == RD_OP_SOFTMAX_DENOM;
}

template <int OP>
typename St<OP>::Out out_of(Results r) {
    return St<OP>::make_out(r.a, r.b);
}

struct RowsArgs {
    const float* x;
    RowMap map;
    int64_t outer, R;
    Results dst;
    Published pub;
    Results out;
};

template <int OP, int G, int U, bool NT>
hipError_t rows_go(const rd_plan& p, const RowsArgs& a, hipStream_t s) {
    if constexpr (rows_built(OP, G, U)) {
        return launch(rows_kernel<OP, G, U, NT>, p.blocks, kBlock, s, a.x, a.map, a.R,
                      a.outer * p.split, p.split, int32_t(p.order == RD_ORDER_BLOCKED),
                      out_of<OP>(a.dst), uint32_t(p.nxcd), a.pub, out_of<OP>(a.out));
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

// inner: the floats read per row; cstride, inner_out: see cols_kernel (1 and
// inner for an array).
struct ColsArgs {
    const float* x;
    int64_t outer, R, inner, so, sr;
    Results dst;
    int64_t cstride, inner_out;
    Published pub;  // words == nullptr: no single-launch combine
    Results out;
};

template <int OP, int CW, int RW, int U, bool NT>
hipError_t cols_go(const rd_plan& p, const ColsArgs& a, hipStream_t s) {
    if constexpr (cols_built(OP, CW, RW, U)) {
        const int64_t ntiles = ((a.inner + 3) / 4 + CW * kWave - 1) / (CW * kWave);
        if (a.pub.words) {
            // every item a workgroup of its own (none waits for itself), the
            // shape and sizes the single-launch combine is built for
            if (!cols_pub_shape<CW, RW, OP>() || p.split < 2 || p.split > kPubColMaxSlabs ||
                p.blocks < ntiles * p.split * a.outer ||
                (p.split - 1) * a.outer * a.inner_out > kPubColWords)
                return hipErrorInvalidValue;
        }
        return launch(cols_kernel<OP, CW, RW, U, NT>, p.blocks, kWave * CW * RW, s, a.x,
                      a.outer, a.R, a.inner, a.so, a.sr, ntiles, p.split, p.rows_per_split,
                      a.cstride, a.inner_out, out_of<OP>(a.dst), uint32_t(p.nxcd), a.pub,
                      out_of<OP>(a.out));
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
        case RD_OP_SOFTMAX_DENOM:                             \
            return F<RD_OP_SOFTMAX_DENOM>(__VA_ARGS__);       \
        default: return hipErrorInvalidValue;                 \
    }

template <int OP>
hipError_t fill_go(Results out, int64_t n, hipStream_t s) {
    return launch(fill_start_kernel<OP>, grid_for(n), kBlock, s, out_of<OP>(out), n);
}

template <int OP>
hipError_t rows_short_go(const float* x, RowMap map, int64_t outer, int64_t R, Results out,
                         hipStream_t s) {
    if (map.ninner == 1 && map.so == R && R >= 1 && R < kShortRow) {
        // adjacent rows: staged through LDS, TR rows per tile
        const int32_t pitch = int32_t(R | 1);
        const int32_t TR = short_tile_rows(R);
        const int64_t tiles = (outer + TR - 1) / TR;
        return launch_lds(rows_short_tile_kernel<OP>, tiles < kMaxBlocks ? tiles : kMaxBlocks,
                          kBlock, size_t(TR) * pitch * sizeof(float), s, x, outer, int32_t(R),
                          pitch, TR, out_of<OP>(out));
    }
    return launch(rows_short_kernel<OP>, grid_for(outer), kBlock, s, x, map, outer, R,
                  out_of<OP>(out));
}

template <int OP>
hipError_t strided_go(const rd_plan& p, const float* x, const Strides& v, Results dst,
                      hipStream_t s) {
    return launch(strided_kernel<OP>, p.blocks, kBlock, s, x, v.outer, v.R, v.inner, v.so, v.sr,
                  v.si, p.split, p.rows_per_split, out_of<OP>(dst));
}

template <int OP>
hipError_t rows_combine_go(Results part, int64_t outer, int64_t P, Results out,
                           hipStream_t s) {
    const int64_t blocks = outer < kMaxBlocks ? outer : kMaxBlocks;
    return launch(rows_combine_kernel<OP>, blocks, kBlock, s, out_of<OP>(part), outer, P,
                  out_of<OP>(out));
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
                      a.inner, a.so, a.sr, p.split, p.rows_per_split, lc, out_of<OP>(a.dst),
                      uint32_t(p.nxcd));
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
hipError_t slab_combine_go(Results slab, int64_t S, int64_t n, Results out, hipStream_t s) {
    if (S >= kSlabWaveMinS && n <= kSlabWaveMaxN)
        return launch(slab_combine_wave_kernel<OP>, (n + kBlock / kWave - 1) / (kBlock / kWave),
                      kBlock, s, out_of<OP>(slab), S, n, out_of<OP>(out));
    return launch(slab_combine_kernel<OP>, grid_for(n), kBlock, s, out_of<OP>(slab), S, n,
                  out_of<OP>(out));
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

hipError_t launch_fill_start(int op, Results out, int64_t n, hipStream_t s) {
    RD_BY_OP(op, fill_go, out, n, s)
}

// The rows of a ROWS plan: v.outer * v.inner rows of v.R contiguous floats
// (v.sr == 1), row (o, i) starting at o*so + i*si.
RowMap row_map(const Strides& v) {
    return v.inner == 1 ? RowMap{v.so, 0, 1} : RowMap{v.so, v.si, v.inner};
}

hipError_t launch_rows(int op, const rd_plan& p, const float* x, const Strides& v,
                       Results dst, const Published* pub, Results out, hipStream_t s) {
    if (pub && (p.split < 2 || !pub->words || !pub->vals)) return hipErrorInvalidValue;
    const RowsArgs a{x, row_map(v), v.outer * v.inner, v.R, dst, pub ? *pub : Published{}, out};
    RD_BY_OP(op, rows_op, p, a, s)
}

hipError_t launch_rows_short(int op, const float* x, const Strides& v, Results out,
                             hipStream_t s) {
    RD_BY_OP(op, rows_short_go, x, row_map(v), v.outer * v.inner, v.R, out, s)
}

hipError_t launch_strided(int op, const rd_plan& p, const float* x, const Strides& v,
                          Results dst, hipStream_t s) {
    RD_BY_OP(op, strided_go, p, x, v, dst, s)
}

hipError_t launch_rows_combine(int op, Results part, int64_t outer, int64_t P, Results out,
                               hipStream_t s) {
    RD_BY_OP(op, rows_combine_go, part, outer, P, out, s)
}

hipError_t launch_cols(int op, const rd_plan& p, const float* x, const Strides& v,
                       Results dst, const Published* pub, Results out, hipStream_t s) {
    if (v.si != 1 && !dense_columns(v)) return hipErrorInvalidValue;
    const int64_t span = (v.inner - 1) * v.si + 1;  // v.inner for an array
    const ColsArgs a{x, v.outer, v.R, span, v.so, v.sr, dst, v.si, v.inner,
                     pub ? *pub : Published{}, out};
    RD_BY_OP(op, cols_op, p, a, s)
}

hipError_t launch_cols_small(int op, const rd_plan& p, const float* x, const Strides& v,
                             Results dst, hipStream_t s) {
    if (v.si != 1) return hipErrorInvalidValue;
    const ColsArgs a{x, v.outer, v.R, v.inner, v.so, v.sr, dst, 1, v.inner, Published{}, Results{}};
    RD_BY_OP(op, cols_small_go, p, a, s)
}

hipError_t launch_slab_combine(int op, Results slab, int64_t S, int64_t n, Results out,
                               hipStream_t s) {
    RD_BY_OP(op, slab_combine_go, slab, S, n, out, s)
}

}  // namespace rd
