// rd_device.h -- device helpers shared by the reduction and the scan kernels:
// 16-byte (and 8/12-byte) loads and stores at 4-byte alignment, DPP moves,
// floats published between the workgroups of a launch, and the XCD-aware
// workgroup numbering.
#pragma once

#include <hip/hip_runtime.h>

namespace rd {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v4f_a4 __attribute__((ext_vector_type(4), aligned(4)));

// The calling wave's index in its workgroup (64-lane waves) as a scalar.
// threadIdx.x / 64 is the same on every lane of a wave, but the compiler
// cannot tell, and otherwise keeps whatever is computed from it -- a wave's
// row pointer, its window of positions -- in vector registers, one copy per
// lane (in the row scans, enough to spill them to scratch memory).
__device__ __forceinline__ int wave_in_block() {
    return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x / 64));
}

// Four floats from a 4-byte-aligned address: one global_load_dwordx4, with
// the nontemporal (streaming) hint when NT.  CDNA's multi-dword global loads
// need only dword alignment.
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

// V = 2, 3 or 4 floats from a 4-byte-aligned address (global_load_dwordx2 /
// dwordx3 / dwordx4) into the first V lanes of a float4; the other lanes get
// `fill`.
template <int V, bool NT>
__device__ __forceinline__ v4f loadv(const float* p, float fill) {
    if constexpr (V == 4) {
        return load4<NT>(p);
    } else {
        typedef float vNf __attribute__((ext_vector_type(V), aligned(4)));
        vNf w;
        if constexpr (NT)
            w = __builtin_nontemporal_load(reinterpret_cast<const vNf*>(p));
        else
            __builtin_memcpy(&w, p, sizeof(w));
        v4f v = {fill, fill, fill, fill};
        v.x = w.x;
        v.y = w.y;
        if constexpr (V == 3) v.z = w.z;
        return v;
    }
}

// Four floats to a 4-byte-aligned address: one global_store_dwordx4, with
// the nontemporal (streaming) hint when NT.
template <bool NT>
__device__ __forceinline__ void store4(float* p, v4f v) {
    if constexpr (NT)
        __builtin_nontemporal_store(v, reinterpret_cast<v4f_a4*>(p));
    else
        __builtin_memcpy(p, &v, sizeof(v));
}

// v moved between lanes by a DPP control (gfx9 encoding); lanes whose source
// is outside the pattern, or whose row is masked off, get 0.
template <int kCtrl, int kRowMask = 0xF>
__device__ __forceinline__ float dpp_or_zero(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, kRowMask,
                                           0xF, true));
}

// A float published to other workgroups of the same launch as one 64-bit
// word, `tag` in the high half and the float's bits in the low half, stored
// and loaded by relaxed device-scope atomics (with an L2 per XCD these go to
// memory, sc1): the value travels with its tag, so a reader that sees the tag
// has the value, and no release / acquire fence -- an L2 write-back per
// workgroup on MI355X -- is needed.  await_word polls until the word carries
// `tag`, at most spin_limit + 1 times; a wait that runs out returns NaN.
__device__ __forceinline__ void publish_word(uint64_t* w, uint32_t tag, float v) {
    const uint64_t word = (uint64_t(tag) << 32) | uint64_t(__builtin_bit_cast(uint32_t, v));
    __hip_atomic_store(w, word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float await_word(uint64_t* w, uint32_t tag, uint32_t spin_limit) {
    for (uint32_t it = 0;; ++it) {
        const uint64_t word = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (uint32_t(word >> 32) == tag) return __builtin_bit_cast(float, uint32_t(word));
        if (it >= spin_limit) return __builtin_nanf("");
        __builtin_amdgcn_s_sleep(1);
    }
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

}  // namespace rd
