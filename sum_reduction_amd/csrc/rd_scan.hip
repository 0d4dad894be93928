// rd_scan.hip -- gfx950 kernels of the fp32 cumulative sum along an axis.
//
// The POPCORNBENCH level-1 problem 91 trace computes a reverse cumulative sum
// over the rows of a [32768, 32768] array, y = cumsum(x.flip(1), 1).flip(1),
// i.e. y[i][j] = x[i][j] + ... + x[i][N-1], and notes that the flips of the
// library formulation cost two extra passes; its own kernel gives each row to
// one block that walks tiles from the right with a running carry and scans
// each tile in the block.  Kept here: rows walked in processing order with a
// running carry, each element read once and written once.  Changed for
// wave64: a row (or row piece) belongs to one wave, not to a block, so there
// is no barrier and no LDS -- the 64 lanes walk the row in chunks of
// 256*K elements, every load and store a full 1 KB wave access, and the next
// chunk's loads are issued before the current chunk is scanned and stored.
// Loads and stores both carry the nontemporal hint (measured on MI355X:
// hinting both was the fastest of the four combinations, up to 10% ahead of
// hinting the loads alone).
// Positions are counted in processing order q (q = 0 is the first element
// the sum takes: the row's last one for the reverse sum).
//
// Order of the adds within a chunk (fixed for a given plan): slice k of the
// chunk holds q = 256k + 4l + j in lane l (j = 0..3);
//   lane       s_j = ((x_0 + x_1) + ...) + x_j over its 4 elements
//   wave       inclusive DPP scan of the lane totals s_3 (row_shr 1, 2, 4, 8,
//              then row_bcast 15 and 31), shifted one lane for the exclusive e
//   output     (carry + e) + s_j
//   carry      carry + (the slice total, lane 63's inclusive value)
// Long rows among few run in one launch by a fixed-order look-back (a
// workgroup per piece; scan_rows_lookback_kernel).  Shorter rows among very
// few are cut into pieces and run in three kernels: the piece totals (the
// same chunks, carry only), their exclusive scan in piece order, and the
// scan of each piece from its carry.  The column scans (inner > 1) keep the
// running sums of 4 adjacent columns in a lane and walk R in processing
// order, advancing the running sums once per group of rows: 256 columns a
// wave for wide rows (scan_cols_kernel, or scan_cols_rounds_kernel with the
// waves of a block taking turns on one tile's rows), several whole rows a
// load instruction for inner <= 128 (scan_small_kernel).  Too few tiles for
// the chip are cut into slabs of R: the slab totals (for row rounds, by the
// column reduction's own kernel), their exclusive scan in slab order, and the
// scan of each slab from its carry.
#include <hip/hip_runtime.h>

#include "rd_device.h"
#include "rd_internal.h"

namespace rd {
namespace {

// Inclusive scan of v over the 64 lanes of a wave (lane 0 first); every lane
// must be active.
__device__ __forceinline__ float wave_scan_inclusive(float v) {
    v += dpp_or_zero<0x111>(v);         // row_shr:1
    v += dpp_or_zero<0x112>(v);         // row_shr:2
    v += dpp_or_zero<0x114>(v);         // row_shr:4
    v += dpp_or_zero<0x118>(v);         // row_shr:8
    v += dpp_or_zero<0x142, 0xA>(v);    // row_bcast:15 into rows 1 and 3
    v += dpp_or_zero<0x143, 0xC>(v);    // row_bcast:31 into rows 2 and 3
    return v;
}

__device__ __forceinline__ float lane63(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// The 4 elements at processing positions q .. q + 3 of a row of R, in
// processing order, from one 16-byte load (REV: memory R - 4 - q .. R - 1 - q,
// reversed).
template <bool REV, bool NT>
__device__ __forceinline__ v4f load_q4(const float* row, int64_t R, int64_t q) {
    if constexpr (REV) {
        const v4f m = load4<NT>(row + (R - 4 - q));
        return v4f{m.w, m.z, m.y, m.x};
    } else {
        return load4<NT>(row + q);
    }
}

template <bool REV, bool NT>
__device__ __forceinline__ void store_q4(float* row, int64_t R, int64_t q, v4f y) {
    if constexpr (REV)
        store4<NT>(row + (R - 4 - q), v4f{y.w, y.z, y.y, y.x});
    else
        store4<NT>(row + q, y);
}

// Positions q .. q + 3, those below q_end only (the others read as 0 / are
// not written): the partial chunk of a row piece.  A lane whose 4 positions
// are all below q_end makes one 16-byte access, the lane across q_end one
// access per position.
template <bool REV, bool NT>
__device__ __forceinline__ v4f load_q4_part(const float* row, int64_t R, int64_t q,
                                            int64_t q_end) {
    if (q + 4 <= q_end) return load_q4<REV, NT>(row, R, q);
    v4f v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j)
        if (q + j < q_end) v[j] = row[REV ? R - 1 - (q + j) : q + j];
    return v;
}

template <bool REV, bool NT>
__device__ __forceinline__ void store_q4_part(float* row, int64_t R, int64_t q, int64_t q_end,
                                              v4f y) {
    if (q + 4 <= q_end) {
        store_q4<REV, NT>(row, R, q, y);
        return;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
        if (q + j < q_end) row[REV ? R - 1 - (q + j) : q + j] = y[j];
}

// Scan of one chunk held as K slices (v[k]: this lane's 4 elements of slice
// k, processing order); y[k] receives the outputs.  Returns the new carry.
template <int K, bool OUT>
__device__ __forceinline__ float scan_chunk(const v4f (&v)[K], v4f (&y)[K], float carry) {
    float e[K], tot[K];
    v4f s[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        s[k].x = v[k].x;
        s[k].y = s[k].x + v[k].y;
        s[k].z = s[k].y + v[k].z;
        s[k].w = s[k].z + v[k].w;
        const float incl = wave_scan_inclusive(s[k].w);
        e[k] = dpp_or_zero<0x138>(incl);  // wave_shr:1
        tot[k] = lane63(incl);
    }
#pragma unroll
    for (int k = 0; k < K; ++k) {
        if constexpr (OUT) {
            const float pre = carry + e[k];
            y[k] = v4f{pre + s[k].x, pre + s[k].y, pre + s[k].z, pre + s[k].w};
        }
        carry = carry + tot[k];
    }
    return carry;
}

// ------------------------------------------------------------ rows
// One chunk step of a row: issue the loads of chunk q_load into `next`, then
// scan chunk `cur` (already in flight) at q_cur and store it.  The two
// buffers alternate between steps, so no register copy waits on a load.
template <bool REV, int K, bool NT, bool OUT>
__device__ __forceinline__ float rows_step(const float* row, float* orow, int64_t R,
                                           int64_t q_cur, int64_t q_load, int64_t lq,
                                           const v4f (&cur)[K], v4f (&next)[K], float carry) {
#pragma unroll
    for (int k = 0; k < K; ++k) next[k] = load_q4<REV, NT>(row, R, q_load + 256 * k + lq);
    __builtin_amdgcn_sched_barrier(0);  // the loads go out before any of the scan
    v4f y[K];
    carry = scan_chunk<K, OUT>(cur, y, carry);
    if constexpr (OUT) {
#pragma unroll
        for (int k = 0; k < K; ++k) store_q4<REV, NT>(orow, R, q_cur + 256 * k + lq, y[k]);
    }
    // keep the next step's scan below these stores: hoisted above them it
    // would wait on the loads just issued
    __builtin_amdgcn_sched_barrier(0);
    return carry;
}

// nfull full chunks from position qf, the first already loaded into a; two
// buffers in turn, every load fetches a chunk that is then scanned.
template <bool REV, int K, bool NT, bool OUT>
__device__ __forceinline__ float rows_full(const float* row, float* orow, int64_t R, int64_t qf,
                                           int64_t nfull, int64_t lq, v4f (&a)[K], v4f (&b)[K],
                                           float carry) {
    constexpr int64_t kChunk = 256 * K;
    int64_t c = 0;
    for (; c + 2 < nfull; c += 2) {  // chunks c, c + 1; loads c + 1, c + 2
        const int64_t q0 = qf + c * kChunk;
        carry = rows_step<REV, K, NT, OUT>(row, orow, R, q0, q0 + kChunk, lq, a, b, carry);
        carry = rows_step<REV, K, NT, OUT>(row, orow, R, q0 + kChunk, q0 + 2 * kChunk, lq, b, a,
                                           carry);
    }
    // one or two chunks left, the first in a
    const int64_t q0 = qf + c * kChunk;
    v4f y[K];
    if (c + 1 < nfull) {
        carry = rows_step<REV, K, NT, OUT>(row, orow, R, q0, q0 + kChunk, lq, a, b, carry);
        carry = scan_chunk<K, OUT>(b, y, carry);
        if constexpr (OUT) {
#pragma unroll
            for (int k = 0; k < K; ++k) store_q4<REV, NT>(orow, R, q0 + kChunk + 256 * k + lq, y[k]);
        }
    } else {
        carry = scan_chunk<K, OUT>(a, y, carry);
        if constexpr (OUT) {
#pragma unroll
            for (int k = 0; k < K; ++k) store_q4<REV, NT>(orow, R, q0 + 256 * k + lq, y[k]);
        }
    }
    return carry;
}

// The positions [q_begin, q_end) of a row piece, walked by one wave.  When
// the piece is no whole number of chunks, its partial chunk comes first: its
// loads go out together with those of the first full chunk, and the piece
// ends on a full chunk (a partial chunk at the end would wait for its loads
// after all the others, one memory latency per piece).
template <bool REV, int K, bool NT, bool OUT>
__device__ __forceinline__ float rows_piece(const float* row, float* orow, int64_t R,
                                            int64_t q_begin, int64_t q_end, int lane,
                                            float carry) {
    constexpr int64_t kChunk = 256 * K;
    const int64_t lq = 4 * lane;
    const int64_t n = q_end > q_begin ? q_end - q_begin : 0;
    const int64_t nfull = n / kChunk;
    const int64_t qf = q_begin + (n - nfull * kChunk);  // the first full chunk
    v4f a[K], b[K];
    if (qf > q_begin) {
#pragma unroll
        for (int k = 0; k < K; ++k) a[k] = load_q4_part<REV, NT>(row, R, q_begin + 256 * k + lq, qf);
        if (nfull > 0) {
#pragma unroll
            for (int k = 0; k < K; ++k) b[k] = load_q4<REV, NT>(row, R, qf + 256 * k + lq);
        }
        __builtin_amdgcn_sched_barrier(0);
        v4f y[K];
        carry = scan_chunk<K, OUT>(a, y, carry);
        if constexpr (OUT) {
#pragma unroll
            for (int k = 0; k < K; ++k)
                store_q4_part<REV, NT>(orow, R, q_begin + 256 * k + lq, qf, y[k]);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (nfull > 0) carry = rows_full<REV, K, NT, OUT>(row, orow, R, qf, nfull, lq, b, a, carry);
    } else if (nfull > 0) {
#pragma unroll
        for (int k = 0; k < K; ++k) a[k] = load_q4<REV, NT>(row, R, qf + 256 * k + lq);
        carry = rows_full<REV, K, NT, OUT>(row, orow, R, qf, nfull, lq, a, b, carry);
    }
    return carry;
}

// Waves per SIMD the row scan is compiled for, 8 with 4-slice chunks (a
// register budget of 512 / 8 = 64 VGPRs; the few spills sit outside the
// chunk loop): the 32768 rows of the [32768, 32768] scan then fill the chip's
// 256 * 4 * 8 wave slots in exactly 4 rounds.  8-slice chunks need 4.
template <int K>
constexpr int scan_rows_waves_per_simd() { return K <= 4 ? 8 : 4; }

// Item = (row o, piece p): processing positions [p*L, min(R, (p+1)*L)), L a
// multiple of the chunk.  One wave per item; the block's waves take
// consecutive items.  totals != null: only the piece total (the final carry)
// goes to totals[item]; otherwise the piece is scanned from carry
// carry_in[item] (0 when carry_in is null) into out.  Row o of x starts at
// x + o*so (so = R for a contiguous array), row o of out at out + o*R.  x and
// out may be the same array: every element is loaded, then stored, by the
// same lane.
template <bool REV, int K, bool NT>
__global__ __launch_bounds__(kBlock, scan_rows_waves_per_simd<K>()) void scan_rows_kernel(
    const float* x, float* out, int64_t outer, int64_t R, int64_t so,
    int64_t P, int64_t L, const float* __restrict__ carry_in, float* __restrict__ totals) {
    constexpr int kWaves = kBlock / kWave;
    const int wave = wave_in_block();
    const int lane = threadIdx.x % kWave;
    const int64_t nitems = outer * P;
    const int64_t wstride = int64_t(gridDim.x) * kWaves;
    for (int64_t item = int64_t(blockIdx.x) * kWaves + wave; item < nitems; item += wstride) {
        const int64_t o = item / P;
        const int64_t p = item - o * P;
        const int64_t q_begin = p * L;
        const int64_t q_end = q_begin + L < R ? q_begin + L : R;
        if (totals == nullptr) {
            const float carry = carry_in != nullptr ? carry_in[item] : 0.f;
            rows_piece<REV, K, NT, true>(x + o * so, out + o * R, R, q_begin, q_end, lane, carry);
        } else {
            const float t = rows_piece<REV, K, NT, false>(x + o * so, nullptr, R, q_begin, q_end,
                                                          lane, 0.f);
            if (lane == 0) totals[item] = t;
        }
    }
}

// The row scan with a workgroup of NW waves per item instead of a wave.  The
// item's positions are walked in block chunks of NW waves x K slices: wave w
// scans the K slices [c0 + w*256K, c0 + (w+1)*256K) of chunk c0 as a wave
// does above (in-lane sums of 4, DPP across the wave), the NW wave totals
// meet in LDS (two slot sets in turn, so one barrier per chunk suffices), and
// wave w's outputs start from the block carry plus the totals of the waves
// before it; the block carry then grows by the NW totals in wave order.
// Adjacent waves stream adjacent 1-8 KB of one row, which HBM serves faster
// than rows apart, and the wider the block chunk the faster (copies of
// 128 KB rows, a workgroup per row, measured on MI355X: 4 waves x 8 KB
// steps 5.57 TB/s, 16 waves taking the whole row at once 6.0 TB/s).  The
// next chunk's loads are issued before the current chunk is scanned (a
// barrier does not wait for them).
template <bool REV, int NW, int K, bool NT, bool OUT>
__device__ __forceinline__ float block_chunk(const float* row, float* orow, int64_t R,
                                             int64_t qw, int64_t q_end, bool part,
                                             int64_t lq, const v4f (&v)[K], float carry,
                                             float* slots, int wave) {
    float e[K], tot[K];
    v4f s[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        s[k].x = v[k].x;
        s[k].y = s[k].x + v[k].y;
        s[k].z = s[k].y + v[k].z;
        s[k].w = s[k].z + v[k].w;
        const float incl = wave_scan_inclusive(s[k].w);
        e[k] = dpp_or_zero<0x138>(incl);  // wave_shr:1
        tot[k] = lane63(incl);
    }
    float wt = tot[0];
#pragma unroll
    for (int k = 1; k < K; ++k) wt = wt + tot[k];
    if (threadIdx.x % kWave == 0) slots[wave] = wt;
    __syncthreads();
    float mine = carry, next = carry;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const float t = slots[w];
        if (w < wave) mine = mine + t;
        next = next + t;
    }
    if constexpr (OUT) {
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const float pre = mine + e[k];
            const v4f y = v4f{pre + s[k].x, pre + s[k].y, pre + s[k].z, pre + s[k].w};
            mine = mine + tot[k];
            if (part)
                store_q4_part<REV, NT>(orow, R, qw + 256 * k + lq, q_end, y);
            else
                store_q4<REV, NT>(orow, R, qw + 256 * k + lq, y);
        }
    }
    return next;
}

// nfull full block chunks from position qf, the first already loaded into a
// (this wave's window of it); two buffers in turn.
template <bool REV, int NW, int K, bool NT, bool OUT>
__device__ __forceinline__ float block_full(const float* row, float* orow, int64_t R,
                                            int64_t qf, int64_t nfull, float carry,
                                            v4f (&a)[K], v4f (&b)[K], float (&slots)[2][NW],
                                            int& parity) {
    constexpr int64_t kSpan = 256 * K;         // a wave's positions per chunk
    constexpr int64_t kChunk = NW * kSpan;     // the block's positions per chunk
    const int wave = wave_in_block();
    const int64_t lq = 4 * (threadIdx.x % kWave);
    const int64_t qw = qf + wave * kSpan;  // this wave's window in the first chunk
    // full chunks two at a time (a, then b), the next chunk's loads first
    int64_t c = 0;
    for (; c + 2 <= nfull; c += 2) {
        const int64_t q0 = qw + c * kChunk;
#pragma unroll
        for (int k = 0; k < K; ++k) b[k] = load_q4<REV, NT>(row, R, q0 + kChunk + 256 * k + lq);
        __builtin_amdgcn_sched_barrier(0);
        carry = block_chunk<REV, NW, K, NT, OUT>(row, orow, R, q0, 0, false, lq, a, carry,
                                                 slots[parity], wave);
        parity ^= 1;
        __builtin_amdgcn_sched_barrier(0);
        if (c + 2 < nfull) {
#pragma unroll
            for (int k = 0; k < K; ++k)
                a[k] = load_q4<REV, NT>(row, R, q0 + 2 * kChunk + 256 * k + lq);
        }
        __builtin_amdgcn_sched_barrier(0);
        carry = block_chunk<REV, NW, K, NT, OUT>(row, orow, R, q0 + kChunk, 0, false, lq, b,
                                                 carry, slots[parity], wave);
        parity ^= 1;
        __builtin_amdgcn_sched_barrier(0);
    }
    if (c < nfull) {  // one full chunk left, in a
        carry = block_chunk<REV, NW, K, NT, OUT>(row, orow, R, qw + c * kChunk, 0, false, lq, a,
                                                 carry, slots[parity], wave);
        parity ^= 1;
    }
    return carry;
}

// One item's positions [q_begin, q_end) from carry (OUT: outputs stored;
// otherwise only the total is computed).  Every thread of the block calls it.
// As in rows_piece, a partial chunk comes first, loaded together with the
// first full chunk.
template <bool REV, int NW, int K, bool NT, bool OUT>
__device__ __forceinline__ float block_piece(const float* row, float* orow, int64_t R,
                                             int64_t q_begin, int64_t q_end, float carry,
                                             float (&slots)[2][NW], int& parity) {
    constexpr int64_t kSpan = 256 * K;         // a wave's positions per chunk
    constexpr int64_t kChunk = NW * kSpan;     // the block's positions per chunk
    const int wave = wave_in_block();
    const int64_t lq = 4 * (threadIdx.x % kWave);
    const int64_t n = q_end - q_begin;
    const int64_t nfull = n / kChunk;
    const int64_t qf = q_begin + (n - nfull * kChunk);  // the first full chunk
    v4f a[K], b[K];
    if (qf > q_begin) {
        const int64_t qh = q_begin + wave * kSpan;  // this wave's window of the partial chunk
#pragma unroll
        for (int k = 0; k < K; ++k) a[k] = load_q4_part<REV, NT>(row, R, qh + 256 * k + lq, qf);
        if (nfull > 0) {
#pragma unroll
            for (int k = 0; k < K; ++k)
                b[k] = load_q4<REV, NT>(row, R, qf + wave * kSpan + 256 * k + lq);
        }
        __builtin_amdgcn_sched_barrier(0);
        carry = block_chunk<REV, NW, K, NT, OUT>(row, orow, R, qh, qf, true, lq, a, carry,
                                                 slots[parity], wave);
        parity ^= 1;
        __builtin_amdgcn_sched_barrier(0);
        if (nfull > 0)
            carry = block_full<REV, NW, K, NT, OUT>(row, orow, R, qf, nfull, carry, b, a, slots,
                                                    parity);
    } else if (nfull > 0) {
#pragma unroll
        for (int k = 0; k < K; ++k) a[k] = load_q4<REV, NT>(row, R, qf + wave * kSpan + 256 * k + lq);
        carry = block_full<REV, NW, K, NT, OUT>(row, orow, R, qf, nfull, carry, a, b, slots,
                                                parity);
    }
    return carry;
}

// Item = (row o, piece p) as in scan_rows_kernel, one workgroup of NW waves
// per item.
template <bool REV, int NW, int K, bool NT>
__global__ __launch_bounds__(NW * kWave, scan_rows_waves_per_simd<K>()) void
scan_rows_block_kernel(const float* x, float* out, int64_t outer, int64_t R, int64_t so,
                       int64_t P, int64_t L, const float* __restrict__ carry_in,
                       float* __restrict__ totals) {
    __shared__ float slots[2][NW];
    const int64_t nitems = outer * P;
    int parity = 0;
    for (int64_t item = blockIdx.x; item < nitems; item += gridDim.x) {
        const int64_t o = item / P;
        const int64_t p = item - o * P;
        const int64_t q_begin = p * L;
        const int64_t q_end = q_begin + L < R ? q_begin + L : R;
        if (totals == nullptr) {
            const float carry = carry_in != nullptr ? carry_in[item] : 0.f;
            block_piece<REV, NW, K, NT, true>(x + o * so, out + o * R, R, q_begin, q_end, carry,
                                          slots, parity);
        } else {
            const float t = block_piece<REV, NW, K, NT, false>(x + o * so, nullptr, R, q_begin,
                                                           q_end, 0.f, slots, parity);
            if (threadIdx.x == 0) totals[item] = t;
        }
    }
}

// Few long rows in one pass: a decoupled look-back in a fixed order.  Row o
// is cut into P pieces of one block chunk each (L = NW*256*K processing
// positions, the row's last piece partial), a workgroup per piece.  A
// workgroup takes piece t = o*P + j by a ticket drawn at its start, so every
// piece it waits for belongs to a workgroup that started before it (and is
// resident or done), and none of those waits for a later piece: no wait can
// close a cycle.  The workgroup loads its chunk, adds it up in the order of
// block_chunk, publishes the chunk total a_j, then forms its carry from what
// earlier pieces of the row published.  Pieces form groups of kLookGroup;
// the last piece of a group that has a successor also publishes the group
// total T_g = (a_gG + ... + a_{j-1}) + a_j, and piece j of group g takes
//   carry = (T_0 + ... + T_{g-1}) + (a_gG + ... + a_{j-1}),
// each run of terms summed by a wave scan in index order (T's 64 at a time,
// the batches added in order).  The terms and their order depend on the
// plan and the data alone, never on which piece finished first, so every
// run gives the same bits.  A published value is one 64-bit word, 1 in the
// high half and the float's bits in the low half, stored and loaded by
// relaxed device-scope atomics: the value travels with its flag, so no fence
// is needed.  The flag is `tag`: 1 in a workspace zeroed before the launch,
// or the launch's epoch in a buffer its stream keeps (where earlier launches
// left words of other epochs).  The ticket starts at 0, and the workgroup
// that draws the last one sets it back to 0 for the next launch (every
// workgroup of this one has drawn by then).  With one piece per row nothing
// is published.  A wait gives up after spin_limit polls and returns NaN, so
// a piece that could not get its carry writes NaN, never a wrong finite sum.
// x and out may be the same array (each element is loaded and stored by the
// same lane).
template <bool REV, int NW, int K, bool NT>
__global__ __launch_bounds__(NW * kWave, scan_rows_waves_per_simd<K>()) void
scan_rows_lookback_kernel(const float* x, float* out, int64_t outer, int64_t R, int64_t so,
                          int64_t P, int64_t NG, uint32_t* __restrict__ ticket, uint64_t* agg,
                          uint64_t* gsum, uint32_t tag, uint32_t spin_limit) {
    constexpr int64_t kSpan = 256 * K;      // a wave's positions
    constexpr int64_t kChunk = NW * kSpan;  // the piece's positions
    __shared__ float slots[NW];
    __shared__ uint32_t s_item;
    __shared__ float s_carry;
    const int wave = wave_in_block();
    const int lane = threadIdx.x % kWave;
    if (threadIdx.x == 0) {
        const uint32_t t = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
        if (int64_t(t) == outer * P - 1)
            __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_item = t;
    }
    __syncthreads();
    const int64_t item = s_item;
    if (item >= outer * P) return;  // only if the ticket was not 0: never wait on it
    const int64_t o = item / P;
    const int64_t j = item - o * P;
    const float* row = x + o * so;
    float* orow = out + o * R;
    const int64_t q_begin = j * kChunk;
    const int64_t q_end = q_begin + kChunk < R ? q_begin + kChunk : R;
    const bool part = q_end - q_begin < kChunk;
    const int64_t lq = 4 * lane;
    const int64_t qw = q_begin + wave * kSpan;  // this wave's window
    v4f v[K];
    if (part) {
#pragma unroll
        for (int k = 0; k < K; ++k) v[k] = load_q4_part<REV, NT>(row, R, qw + 256 * k + lq, q_end);
    } else {
#pragma unroll
        for (int k = 0; k < K; ++k) v[k] = load_q4<REV, NT>(row, R, qw + 256 * k + lq);
    }
    float e[K], tot[K];
    v4f sv[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        sv[k].x = v[k].x;
        sv[k].y = sv[k].x + v[k].y;
        sv[k].z = sv[k].y + v[k].z;
        sv[k].w = sv[k].z + v[k].w;
        const float incl = wave_scan_inclusive(sv[k].w);
        e[k] = dpp_or_zero<0x138>(incl);  // wave_shr:1
        tot[k] = lane63(incl);
    }
    float wt = tot[0];
#pragma unroll
    for (int k = 1; k < K; ++k) wt = wt + tot[k];
    if (lane == 0) slots[wave] = wt;
    __syncthreads();
    if (wave == 0) {
        float a = 0.f;  // the chunk total, 0 + t_0 + ... + t_{NW-1}
#pragma unroll
        for (int w = 0; w < NW; ++w) a = a + slots[w];
        if (lane == 0 && j + 1 < P) publish_word(agg + item, tag, a);
        const int64_t g = j / kLookGroup;
        const int64_t first = g * kLookGroup;
        // this group's earlier chunk totals, lane i <- piece first + i
        const float ai = first + lane < j ? await_word(agg + o * P + first + lane, tag, spin_limit) : 0.f;
        const float in_group = lane63(wave_scan_inclusive(ai));
        if (j == first + kLookGroup - 1 && j + 1 < P && lane == 0)
            publish_word(gsum + o * NG + g, tag, in_group + a);
        float before = 0.f;  // the earlier groups' totals
        for (int64_t h0 = 0; h0 < g; h0 += kWave) {
            const float th = h0 + lane < g ? await_word(gsum + o * NG + h0 + lane, tag, spin_limit) : 0.f;
            before = before + lane63(wave_scan_inclusive(th));
        }
        if (lane == 0) s_carry = before + in_group;
    }
    __syncthreads();
    float mine = s_carry;
#pragma unroll
    for (int w = 0; w < NW; ++w)
        if (w < wave) mine = mine + slots[w];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const float pre = mine + e[k];
        const v4f y = v4f{pre + sv[k].x, pre + sv[k].y, pre + sv[k].z, pre + sv[k].w};
        mine = mine + tot[k];
        if (part)
            store_q4_part<REV, NT>(orow, R, qw + 256 * k + lq, q_end, y);
        else
            store_q4<REV, NT>(orow, R, qw + 256 * k + lq, y);
    }
}

// Whole rows (no pieces) by persistent workgroups of NW waves: workgroup b
// takes rows b, b + G, b + 2G, ... (G = gridDim.x) and walks their chunks as
// one stream -- each row's partial chunk, if any, then its full chunks, the
// order of block_piece -- loading chunk g + 1 (the next row's first one
// included) while chunk g is scanned, so no row starts on a memory latency
// of its own.  Same chunks, same order, same bits as scan_rows_block_kernel.
template <bool REV, int NW, int K, bool NT>
__device__ __forceinline__ void stream_load(const float* xr, int64_t R, int64_t c0, int64_t c1,
                                            bool part, int64_t lq, int wave, v4f (&v)[K]) {
    const int64_t q0 = c0 + int64_t(wave) * 256 * K;
    if (part) {
#pragma unroll
        for (int k = 0; k < K; ++k) v[k] = load_q4_part<REV, NT>(xr, R, q0 + 256 * k + lq, c1);
    } else {
#pragma unroll
        for (int k = 0; k < K; ++k) v[k] = load_q4<REV, NT>(xr, R, q0 + 256 * k + lq);
    }
}

template <bool REV, int NW, int K, bool NT>
__global__ __launch_bounds__(NW * kWave, scan_rows_waves_per_simd<K>()) void
scan_rows_stream_kernel(const float* x, float* out, int64_t outer, int64_t R, int64_t so) {
    __shared__ float slots[2][NW];
    constexpr int64_t kChunk = NW * 256 * K;
    const int wave = wave_in_block();
    const int64_t lq = 4 * (threadIdx.x % kWave);
    const int64_t G = gridDim.x;
    const int64_t o0 = blockIdx.x;
    if (o0 >= outer || R <= 0) return;
    const int64_t nfull = R / kChunk;
    const int64_t h = R - nfull * kChunk;              // the partial chunk's length
    const int64_t hp = h > 0 ? 1 : 0;
    const int64_t nch = nfull + hp;                     // chunks per row
    const int64_t total = ((outer - 1 - o0) / G + 1) * nch;
    // chunk j of a row covers [c0(j), c1(j)); only j == 0 can be partial
    auto c0 = [&](int64_t jj) { return jj == 0 ? int64_t(0) : h + (jj - hp) * kChunk; };
    auto c1 = [&](int64_t jj) { return hp ? h + jj * kChunk : (jj + 1) * kChunk; };
    int64_t o = o0, j = 0;  // the chunk being scanned: row o, chunk j
    v4f a[K], b[K];
    stream_load<REV, NW, K, NT>(x + o * so, R, c0(0), c1(0), hp != 0, lq, wave, a);
    float carry = 0.f;
    int parity = 0;
    // one step: load chunk g + 1 into nxt, scan chunk g (held in cur)
    auto step = [&](int64_t g, v4f (&cur)[K], v4f (&nxt)[K]) {
        const int64_t jn = j + 1 == nch ? 0 : j + 1;
        const int64_t on = j + 1 == nch ? o + G : o;
        if (g + 1 < total)
            stream_load<REV, NW, K, NT>(x + on * so, R, c0(jn), c1(jn), jn == 0 && hp != 0, lq,
                                        wave, nxt);
        __builtin_amdgcn_sched_barrier(0);
        if (j == 0) carry = 0.f;
        carry = block_chunk<REV, NW, K, NT, true>(x + o * so, out + o * R, R,
                                                  c0(j) + int64_t(wave) * 256 * K, c1(j),
                                                  j == 0 && hp != 0, lq, cur, carry,
                                                  slots[parity], wave);
        parity ^= 1;
        __builtin_amdgcn_sched_barrier(0);
        o = on;
        j = jn;
    };
    for (int64_t g = 0; g < total; g += 2) {
        step(g, a, b);
        if (g + 1 < total) step(g + 1, b, a);
    }
}

// Exclusive scan of the P piece totals of each row, in piece order:
// carries[o*P + p] = totals[o*P] + ... + totals[o*P + p - 1] (summed as the
// chunks are: lane-sequential within 4, DPP across the wave, a carry across
// 256-total chunks).  One wave per row.
__global__ __launch_bounds__(kBlock) void scan_carries_kernel(const float* __restrict__ totals,
                                                              float* __restrict__ carries,
                                                              int64_t rows, int64_t P) {
    constexpr int kWaves = kBlock / kWave;
    const int wave = wave_in_block();
    const int lane = threadIdx.x % kWave;
    const int64_t wstride = int64_t(gridDim.x) * kWaves;
    for (int64_t o = int64_t(blockIdx.x) * kWaves + wave; o < rows; o += wstride) {
        const float* t = totals + o * P;
        float* c = carries + o * P;
        float carry = 0.f;
        for (int64_t base = 0; base < P; base += 4 * kWave) {
            const int64_t p0 = base + 4 * lane;
            float v[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] = p0 + j < P ? t[p0 + j] : 0.f;
            const float s0 = v[0], s1 = s0 + v[1], s2 = s1 + v[2], s3 = s2 + v[3];
            const float incl = wave_scan_inclusive(s3);
            const float pre = carry + dpp_or_zero<0x138>(incl);  // wave_shr:1
            const float ex[4] = {pre, pre + s0, pre + s1, pre + s2};
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (p0 + j < P) c[p0 + j] = ex[j];
            carry = carry + lane63(incl);
        }
    }
}

// ------------------------------------------------------------ columns
// The running sums of a lane-column to one row: all 4 with one 16-byte store,
// else only components keep .. V-1 (the row's last lane-column, or V < 4).
template <int V, bool NT>
__device__ __forceinline__ void store_cols(float* q, int keep, v4f acc) {
    if (V == 4 && keep == 0) {
        store4<NT>(q, acc);
    } else {
#pragma unroll
        for (int j = 0; j < V; ++j)
            if (j >= keep) q[j] = acc[j];
    }
}

// The U rows of a group g (in processing order) added to the running sums
// acc: row u's outputs are acc + (g[0] + ... + g[u]), stored when scan_out,
// and the new running sums are acc + (g[0] + ... + g[U-1]).  The running sums
// take one add per group, not per row, so the rounding they carry down a tall
// column grows with R/U additions rather than R.
template <int V, int U, bool NT>
__device__ __forceinline__ v4f cols_group(float* qc, int64_t qstep, int keep, bool scan_out,
                                          const v4f (&g)[U], v4f acc) {
    v4f run = g[0];
    if (scan_out) store_cols<V, NT>(qc, keep, acc + run);
#pragma unroll
    for (int u = 1; u < U; ++u) {
        run += g[u];
        if (scan_out) store_cols<V, NT>(qc + u * qstep, keep, acc + run);
    }
    return acc + run;
}

// One group step of a lane-column: issue the loads of the U rows at element
// offset off_load into `next`, then add the U rows of `cur` (rows at off_cur)
// to the running sums (cols_group) and store them; then meet the block's
// other waves.  pl: the first row of the group to load (rows pstep floats
// apart in x); qc: the first output row of the group in `cur` (qstep floats
// apart in out).
template <int V, int U, bool NT>
__device__ __forceinline__ v4f cols_step(const float* pl, float* qc, int64_t pstep,
                                         int64_t qstep, int keep, bool scan_out,
                                         const v4f (&cur)[U], v4f (&next)[U], v4f acc) {
#pragma unroll
    for (int u = 0; u < U; ++u) next[u] = loadv<V, NT>(pl + u * pstep, 0.f);
    __builtin_amdgcn_sched_barrier(0);  // the loads go out before the adds (as in rows_step)
    acc = cols_group<V, U, NT>(qc, qstep, keep, scan_out, cur, acc);
    __syncthreads();
    return acc;
}

// A lane owns lane-column lc: the V = min(4, inner) columns from 4*lc (the
// row's last lane-column loads the row's last 4 floats and keeps only its
// own, as the column reduction does).  A wave holds 64 lane-columns (a tile,
// 1 KB of a row); a block holds BW adjacent tiles of one outer index o and one
// slab s of R (block items are numbered tile group fastest, then slab, then
// o), and its waves walk the slab's rows in processing order (REV: from the
// last row) in lockstep, U rows per step with a barrier after each step.  In
// lockstep, the cache lines two neighbouring tiles share at their edge (rows
// need not be line-aligned) are written by both within one step, not rows
// apart, so they leave the L2 whole.  Each step issues the next group's loads
// before adding and storing the current group (cols_group; two buffers in
// turn).  totals != null: only the slab totals go to totals[s][o][i]; otherwise the
// slab is scanned from carry_in[s][o][i] (0 when null) into out.  Element
// (o, r, c) of x is at x + o*so + r*sr + c (a contiguous array: so = R*inner,
// sr = inner); out is contiguous.  x and out may be the same array.
template <bool REV, int V, int U, int BW, bool NT>
__global__ __launch_bounds__(BW * kWave) void scan_cols_kernel(
    const float* x, float* out, int64_t outer, int64_t R,
    int64_t inner, int64_t so, int64_t sr, int64_t ntiles, int64_t S, int64_t rps,
    const float* __restrict__ carry_in, float* __restrict__ totals, uint32_t nxcd) {
    constexpr int kWaves = BW;
    const int wave = wave_in_block();
    const int lane = threadIdx.x % kWave;
    const bool scan_out = totals == nullptr;
    const int64_t ngt = (ntiles + kWaves - 1) / kWaves;  // tile groups per row
    const int64_t nitems = ngt * S * outer;
    for (int64_t item = xcd_block(nxcd); item < nitems; item += gridDim.x) {
        const int64_t tg = item % ngt;
        const int64_t rest = item / ngt;
        const int64_t s = rest % S;
        const int64_t o = rest / S;
        const int64_t r_begin = s * rps;
        const int64_t r_end = r_begin + rps < R ? r_begin + rps : R;
        const int64_t m = r_end > r_begin ? r_end - r_begin : 0;
        const int64_t ngroups = m / U;  // steps (and barriers) of every wave
        const int64_t tile = tg * kWaves + wave;
        if (tile >= ntiles) {  // a wave past the row's end only keeps step
            for (int64_t g = 0; g < ngroups; ++g) __syncthreads();
            continue;
        }
        // lanes past the row's end shadow the last lane-column and store nothing
        const int64_t c = 4 * (tile * kWave + lane);
        const bool live = c < inner;
        const int64_t cl = V == 4 ? (c + 4 > inner ? inner - 4 : c) : 0;
        const int keep = live ? int(c - cl) : V;
        const int64_t cbase = (s * outer + o) * inner + cl;
        v4f acc = {0.f, 0.f, 0.f, 0.f};
        if (live && scan_out && carry_in != nullptr) acc = loadv<V, false>(carry_in + cbase, 0.f);
        // the k-th row in processing order is x row first + k*dir: pstep
        // floats apart in x, qstep in out
        const int64_t first = REV ? r_end - 1 : r_begin;
        const int64_t pstep = REV ? -sr : sr;
        const int64_t qstep = REV ? -inner : inner;
        const float* p = x + o * so + first * sr + cl;
        float* q = out + (o * R + first) * inner + cl;
        if (ngroups > 0) {
            v4f a[U], b[U];
#pragma unroll
            for (int u = 0; u < U; ++u) a[u] = loadv<V, NT>(p + u * pstep, 0.f);
            int64_t g = 0;
            for (; g + 2 < ngroups; g += 2) {  // groups g, g + 1; loads g + 1, g + 2
                const float* p1 = p + (g + 1) * U * pstep;
                float* q0 = q + g * U * qstep;
                acc = cols_step<V, U, NT>(p1, q0, pstep, qstep, keep, scan_out, a, b, acc);
                acc = cols_step<V, U, NT>(p1 + U * pstep, q0 + U * qstep, pstep, qstep, keep,
                                          scan_out, b, a, acc);
            }
            // one or two groups left, the first in a (a barrier after each)
            float* q0 = q + g * U * qstep;
            if (g + 1 < ngroups) {
                acc = cols_step<V, U, NT>(p + (g + 1) * U * pstep, q0, pstep, qstep, keep,
                                          scan_out, a, b, acc);
                acc = cols_group<V, U, NT>(q0 + U * qstep, qstep, keep, scan_out, b, acc);
            } else {
                acc = cols_group<V, U, NT>(q0, qstep, keep, scan_out, a, acc);
            }
            __syncthreads();
            p += ngroups * U * pstep;
            q += ngroups * U * qstep;
        }
        for (int64_t k = ngroups * U; k < m; ++k) {
            acc += loadv<V, NT>(p, 0.f);
            if (scan_out) store_cols<V, NT>(q, keep, acc);
            p += pstep;
            q += qstep;
        }
        if (!scan_out)
            for (int j = keep; j < V; ++j) totals[cbase + j] = acc[j];
    }
}

// Few tiles, tall columns: a block of RW waves on one tile (64 lane-columns,
// 256 columns) of one outer index and one slab s of R (S == 1: the whole of
// R, one pass, x read once).  Wave w takes the groups of U rows w, w + RW,
// w + 2RW, ... of the slab in processing order; per round of RW groups each
// wave adds its group up (running sums pre_u in processing order, group
// total t_w), the totals meet in LDS (two slot sets in turn: one barrier a
// round), wave w's outputs are (carry + t_0 + ... + t_{w-1}) + pre_u, and the
// carry of the next round is carry + t_0 + ... + t_{RW-1} -- a fixed order, so
// the results do not depend on timing.  The slab's first carry is
// carry_in[s][o][i] (0 when null).  Items are numbered tile fastest, then
// slab, then o.  The next round's loads go out before the current round is
// added up.  inner >= 4; element (o, r, c) at x + o*so + r*sr + c as in
// scan_cols_kernel, out contiguous.
template <bool REV, int U, int RW, bool NT>
__global__ __launch_bounds__(RW * kWave) void scan_cols_rounds_kernel(
    const float* x, float* out, int64_t outer, int64_t R, int64_t inner, int64_t so,
    int64_t sr, int64_t ntiles, int64_t S, int64_t rps, const float* __restrict__ carry_in,
    uint32_t nxcd) {
    __shared__ v4f slots[2][RW][kWave];
    const int wave = wave_in_block();
    const int lane = threadIdx.x % kWave;
    const int64_t nitems = ntiles * S * outer;
    const int64_t per_round = int64_t(RW) * U;
    int parity = 0;
    for (int64_t item = xcd_block(nxcd); item < nitems; item += gridDim.x) {
        const int64_t tile = item % ntiles;
        const int64_t rest = item / ntiles;
        const int64_t sl = rest % S;
        const int64_t o = rest / S;
        const int64_t r_begin = sl * rps;
        const int64_t r_end = r_begin + rps < R ? r_begin + rps : R;
        const int64_t m = r_end > r_begin ? r_end - r_begin : 0;  // rows of the slab
        const int64_t nrounds = (m + per_round - 1) / per_round;
        const int64_t c = 4 * (tile * kWave + lane);
        const bool live = c < inner;
        const int64_t cl = c + 4 > inner ? inner - 4 : c;
        const int keep = live ? int(c - cl) : 4;
        const int64_t first = REV ? r_end - 1 : r_begin;
        const int64_t pstep = REV ? -sr : sr;
        const int64_t qstep = REV ? -inner : inner;
        const float* p = x + o * so + first * sr + cl;
        float* q = out + (o * R + first) * inner + cl;
        // the group of round g: processing positions g*per_round + wave*U + u
        auto load_group = [&](int64_t g, v4f (&v)[U]) {
            const int64_t k0 = g * per_round + int64_t(wave) * U;
#pragma unroll
            for (int u = 0; u < U; ++u)
                v[u] = live && k0 + u < m ? load4<NT>(p + (k0 + u) * pstep) : v4f{0.f, 0.f, 0.f, 0.f};
        };
        auto round = [&](int64_t g, v4f (&v)[U], v4f& carry) {
            const int64_t k0 = g * per_round + int64_t(wave) * U;
            v4f t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int u = 0; u < U; ++u) {
                t += v[u];
                v[u] = t;
            }
            slots[parity][wave][lane] = t;
            __syncthreads();
            v4f mine = carry, next = carry;
#pragma unroll
            for (int w = 0; w < RW; ++w) {
                const v4f sw = slots[parity][w][lane];
                if (w < wave) mine += sw;
                next += sw;
            }
            carry = next;
            parity ^= 1;
            if (live) {
#pragma unroll
                for (int u = 0; u < U; ++u)
                    if (k0 + u < m) store_cols<4, NT>(q + (k0 + u) * qstep, keep, mine + v[u]);
            }
        };
        v4f carry = {0.f, 0.f, 0.f, 0.f};
        if (live && carry_in != nullptr)
            carry = load4<false>(carry_in + (sl * outer + o) * inner + cl);
        v4f a[U], b[U];
        load_group(0, a);
        for (int64_t g = 0; g < nrounds; g += 2) {
            if (g + 1 < nrounds) load_group(g + 1, b);
            __builtin_amdgcn_sched_barrier(0);  // the next round's loads go out first
            round(g, a, carry);
            __builtin_amdgcn_sched_barrier(0);
            if (g + 1 >= nrounds) break;
            if (g + 2 < nrounds) load_group(g + 2, a);
            __builtin_amdgcn_sched_barrier(0);
            round(g + 1, b, carry);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// ------------------------------------------------------------ small inner
// Inclusive scan over the row phases of a wave: lane l = rho*LC + lc receives
// the sum of the lanes rho' <= rho of its lane-column lc (Hillis-Steele steps
// of d*LC lanes through ds_bpermute; the sources of a lane with rho < RPW
// all have rho' < RPW).  LC == 1 (inner <= 4) takes the DPP wave scan.
__device__ __forceinline__ float phase_scan(float v, int lane, int rho, int LC, int RPW) {
    if (LC == 1) return wave_scan_inclusive(v);
    for (int d = 1; d < RPW; d *= 2) {
        const int src = lane - d * LC;
        const float t = __builtin_bit_cast(
            float, __builtin_amdgcn_ds_bpermute(4 * (src < 0 ? lane : src),
                                                __builtin_bit_cast(int, v)));
        v += rho >= d ? t : 0.f;
    }
    return v;
}

// The value lane (RPW - 1)*LC + lc holds, in every lane of lane-column lc.
__device__ __forceinline__ float phase_last(float v, int lc, int LC, int RPW) {
    if (LC == 1) return lane63(v);
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(
                                         4 * ((RPW - 1) * LC + lc), __builtin_bit_cast(int, v)));
}

// inner <= 128: a lane is (row phase rho, lane-column lc), LC = ceil(inner/4)
// lane-columns per row and RPW = 64 / LC rows per load instruction, so one
// instruction reads RPW adjacent rows of one outer index (RPW*inner
// contiguous floats; inner 2-3: one row per lane, 8- or 12-byte loads).  A
// wave owns one item (outer index, slab of R) at a time and walks it in
// processing order, RPW rows per instruction and U instructions per step:
// each instruction is scanned across its row phases (phase_scan) and added to
// the running sums carried from the instruction before; the next step's loads
// are issued before the current one is scanned and stored.  Lanes past RPW*LC
// shadow the last row phase (valid loads) and store nothing.  Order of the
// adds: Hillis-Steele over the phases, then carry + that.
// Element (o, r, c) of x is at x + o*so + r*sr + c (a contiguous array: so =
// R*inner, sr = inner, when each instruction reads RPW*inner contiguous
// floats); out is contiguous.
template <bool REV, int V, int U, bool NT>
__global__ __launch_bounds__(kBlock) void scan_small_kernel(
    const float* x, float* out, int64_t outer, int64_t R, int64_t inner, int64_t so,
    int64_t sr, int64_t S, int64_t rps, int32_t LC, const float* __restrict__ carry_in,
    float* __restrict__ totals, uint32_t nxcd) {
    constexpr int kWaves = kBlock / kWave;
    const int wave = wave_in_block();
    const int lane = threadIdx.x % kWave;
    const int RPW = kWave / LC;
    const int rho_raw = lane / LC;
    const bool active = rho_raw < RPW;
    const int rho = active ? rho_raw : RPW - 1;
    const int lc = lane - rho_raw * LC;
    const int64_t c = 4 * int64_t(lc);
    const int64_t cl = V == 4 ? (c + 4 > inner ? inner - 4 : c) : 0;
    const int keep = active ? int(c - cl) : V;  // V: store nothing
    const bool scan_out = totals == nullptr;
    const int64_t nitems = S * outer;
    const int64_t wstride = int64_t(gridDim.x) * kWaves;
    for (int64_t item = xcd_block(nxcd) * kWaves + wave; item < nitems; item += wstride) {
        const int64_t o = item / S;
        const int64_t s = item - o * S;
        const int64_t r_begin = s * rps;
        const int64_t r_end = r_begin + rps < R ? r_begin + rps : R;
        const int64_t m = r_end > r_begin ? r_end - r_begin : 0;
        const int64_t cbase = (s * outer + o) * inner + cl;
        v4f carry = {0.f, 0.f, 0.f, 0.f};
        if (scan_out && carry_in != nullptr) carry = loadv<V, false>(carry_in + cbase, 0.f);
        // processing position k of this lane in instruction g: g*RPW + rho;
        // its row is first + k*dir
        const int64_t first = REV ? r_end - 1 : r_begin;
        const int64_t pstep = REV ? -sr : sr;        // rows apart in x
        const int64_t qstep = REV ? -inner : inner;  // rows apart in out
        const float* p = x + o * so + first * sr + cl + int64_t(rho) * pstep;
        float* q = out + (o * R + first) * inner + cl + int64_t(rho) * qstep;
        const int64_t istep = int64_t(RPW) * pstep;  // x elements per instruction
        const int64_t ostep = int64_t(RPW) * qstep;  // out elements per instruction
        const int64_t nfull = m / RPW;               // instructions with every phase valid
        const int64_t nsteps = nfull / U;

        auto scan_one = [&](v4f v, float* qq, bool store) {
            v4f y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < V; ++j) y[j] = carry[j] + phase_scan(v[j], lane, rho, LC, RPW);
            if (scan_out && store) store_cols<V, NT>(qq, keep, y);
#pragma unroll
            for (int j = 0; j < V; ++j) carry[j] = phase_last(y[j], lc, LC, RPW);
        };

        if (nsteps > 0) {
            v4f a[U], b[U];
#pragma unroll
            for (int u = 0; u < U; ++u) a[u] = loadv<V, NT>(p + u * istep, 0.f);
            int64_t g = 0;
            for (; g + 2 < nsteps; g += 2) {  // steps g, g + 1; loads g + 1, g + 2
#pragma unroll
                for (int u = 0; u < U; ++u) b[u] = loadv<V, NT>(p + ((g + 1) * U + u) * istep, 0.f);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int u = 0; u < U; ++u) scan_one(a[u], q + (g * U + u) * ostep, true);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int u = 0; u < U; ++u) a[u] = loadv<V, NT>(p + ((g + 2) * U + u) * istep, 0.f);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int u = 0; u < U; ++u) scan_one(b[u], q + ((g + 1) * U + u) * ostep, true);
                __builtin_amdgcn_sched_barrier(0);
            }
            if (g + 1 < nsteps) {  // two steps left
#pragma unroll
                for (int u = 0; u < U; ++u) b[u] = loadv<V, NT>(p + ((g + 1) * U + u) * istep, 0.f);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int u = 0; u < U; ++u) scan_one(a[u], q + (g * U + u) * ostep, true);
#pragma unroll
                for (int u = 0; u < U; ++u) scan_one(b[u], q + ((g + 1) * U + u) * ostep, true);
            } else {
#pragma unroll
                for (int u = 0; u < U; ++u) scan_one(a[u], q + (g * U + u) * ostep, true);
            }
        }
        // the remaining instructions, the last one possibly partial
        for (int64_t g = nsteps * U; g * RPW < m; ++g) {
            const bool valid = g * RPW + rho < m;
            const v4f v = valid ? loadv<V, NT>(p + g * istep, 0.f) : v4f{0.f, 0.f, 0.f, 0.f};
            scan_one(v, q + g * ostep, valid);
        }
        if (!scan_out && rho_raw == 0)
            for (int j = keep; j < V; ++j) totals[cbase + j] = carry[j];
    }
}

// The slab carries when there are many slabs: one wave per (o, i), the S
// totals scanned in processing order in 256-total chunks (as
// scan_carries_kernel), the reverse sum taking the last slab first.
template <bool REV>
__global__ __launch_bounds__(kBlock) void scan_slab_carries_wave_kernel(
    const float* __restrict__ totals, float* __restrict__ carries, int64_t S, int64_t n) {
    constexpr int kWaves = kBlock / kWave;
    const int wave = wave_in_block();
    const int lane = threadIdx.x % kWave;
    const int64_t wstride = int64_t(gridDim.x) * kWaves;
    for (int64_t e = int64_t(blockIdx.x) * kWaves + wave; e < n; e += wstride) {
        float carry = 0.f;
        for (int64_t base = 0; base < S; base += 4 * kWave) {
            const int64_t k0 = base + 4 * lane;
            float v[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t k = k0 + j;
                v[j] = k < S ? totals[(REV ? S - 1 - k : k) * n + e] : 0.f;
            }
            const float s0 = v[0], s1 = s0 + v[1], s2 = s1 + v[2], s3 = s2 + v[3];
            const float incl = wave_scan_inclusive(s3);
            const float pre = carry + dpp_or_zero<0x138>(incl);  // wave_shr:1
            const float ex[4] = {pre, pre + s0, pre + s1, pre + s2};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t k = k0 + j;
                if (k < S) carries[(REV ? S - 1 - k : k) * n + e] = ex[j];
            }
            carry = carry + lane63(incl);
        }
    }
}

// Exclusive scan over the S slabs of each (o, i), in processing order:
// the reverse sum takes the last slab first.
template <bool REV>
__global__ __launch_bounds__(kBlock) void scan_slab_carries_kernel(
    const float* __restrict__ totals, float* __restrict__ carries, int64_t S, int64_t n) {
    const int64_t stride = int64_t(gridDim.x) * kBlock;
    for (int64_t e = int64_t(blockIdx.x) * kBlock + threadIdx.x; e < n; e += stride) {
        float run = 0.f;
        for (int64_t k = 0; k < S; ++k) {
            const int64_t s = REV ? S - 1 - k : k;
            carries[s * n + e] = run;
            run = run + totals[s * n + e];
        }
    }
}

// Views with no unit stride along the columns (nor, when inner == 1, along
// R): a lane per (slab s, output column e = o*inner + i), columns fastest.
// The lane adds the slab's terms x[o*so + r*sr + i*si] one after the other in
// processing order (REV: from the slab's last row), 8 loads in flight, and
// stores each prefix at out[(o*R + r)*inner + i].  totals != null: only the
// slab total goes to totals[s*n + e]; otherwise the slab is scanned from
// carry_in[s*n + e] (0 when null).  Plain loads and stores: the lines a lane
// touches are often the ones its neighbours touch next, or itself at the
// next row, and are found again in the cache.
template <bool REV>
__global__ __launch_bounds__(kBlock) void scan_strided_kernel(
    const float* x, float* out, int64_t outer, int64_t R,
    int64_t inner, int64_t so, int64_t sr, int64_t si, int64_t S, int64_t rps,
    const float* __restrict__ carry_in, float* __restrict__ totals) {
    constexpr int kLoads = 8;
    const bool scan_out = totals == nullptr;
    const int64_t n = outer * inner;
    const int64_t nitems = S * n;
    const int64_t stride = int64_t(gridDim.x) * kBlock;
    for (int64_t item = int64_t(blockIdx.x) * kBlock + threadIdx.x; item < nitems;
         item += stride) {
        const int64_t s = item / n;
        const int64_t e = item - s * n;
        const int64_t o = e / inner;
        const int64_t i = e - o * inner;
        const int64_t r_begin = s * rps;
        const int64_t r_end = r_begin + rps < R ? r_begin + rps : R;
        const int64_t m = r_end > r_begin ? r_end - r_begin : 0;
        const int64_t first = REV ? r_end - 1 : r_begin;
        const int64_t pstep = REV ? -sr : sr;
        const int64_t qstep = REV ? -inner : inner;
        const float* p = x + o * so + first * sr + i * si;
        float* q = out + (o * R + first) * inner + i;
        float acc = scan_out && carry_in != nullptr ? carry_in[item] : 0.f;
        int64_t k = 0;
        for (; k + kLoads <= m; k += kLoads) {
            float v[kLoads];
#pragma unroll
            for (int u = 0; u < kLoads; ++u) v[u] = p[u * pstep];
#pragma unroll
            for (int u = 0; u < kLoads; ++u) {
                acc += v[u];
                if (scan_out) q[u * qstep] = acc;
            }
            p += kLoads * pstep;
            q += kLoads * qstep;
        }
        for (; k < m; ++k) {
            acc += *p;
            if (scan_out) *q = acc;
            p += pstep;
            q += qstep;
        }
        if (!scan_out) totals[item] = acc;
    }
}

// A view with no unit stride along its kept inner axis and enough columns for
// the chip, in one pass: a block of RW waves on 64 columns (a lane each,
// column e = 64*item + lane of the outer*inner columns), over the whole of R.
// Wave w takes the groups of U rows w, w + RW, ... in processing order; per
// round each wave adds its group up (running sums pre_u, group total t_w),
// the totals meet in LDS, wave w's outputs are (carry + t_0 + ... + t_{w-1})
// + pre_u and the next round's carry is carry + t_0 + ... + t_{RW-1} -- the
// order of scan_cols_rounds_kernel, one column a lane.  Lanes past the last
// column load and store nothing.  Element (o, r, i) at x + o*so + r*sr + i*si,
// out contiguous.
template <bool REV, int U, int RW>
__global__ __launch_bounds__(RW * kWave) void scan_strided_rounds_kernel(
    const float* x, float* out, int64_t outer, int64_t R, int64_t inner, int64_t so,
    int64_t sr, int64_t si, int64_t ngroups, uint32_t nxcd) {
    __shared__ float slots[2][RW][kWave];
    const int wave = wave_in_block();
    const int lane = threadIdx.x % kWave;
    const int64_t n = outer * inner;
    const int64_t per_round = int64_t(RW) * U;
    const int64_t nrounds = (R + per_round - 1) / per_round;
    int parity = 0;
    for (int64_t item = xcd_block(nxcd); item < ngroups; item += gridDim.x) {
        const int64_t e0 = item * kWave + lane;
        const bool live = e0 < n;
        const int64_t e = live ? e0 : n - 1;
        const int64_t o = e / inner;
        const int64_t i = e - o * inner;
        const int64_t first = REV ? R - 1 : 0;
        const int64_t pstep = REV ? -sr : sr;
        const int64_t qstep = REV ? -inner : inner;
        const float* p = x + o * so + first * sr + i * si;
        float* q = out + (o * R + first) * inner + i;
        auto load_group = [&](int64_t g, float (&v)[U]) {
            const int64_t k0 = g * per_round + int64_t(wave) * U;
#pragma unroll
            for (int u = 0; u < U; ++u) v[u] = live && k0 + u < R ? p[(k0 + u) * pstep] : 0.f;
        };
        auto round = [&](int64_t g, float (&v)[U], float& carry) {
            const int64_t k0 = g * per_round + int64_t(wave) * U;
            float t = 0.f;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                t += v[u];
                v[u] = t;
            }
            slots[parity][wave][lane] = t;
            __syncthreads();
            float mine = carry, next = carry;
#pragma unroll
            for (int w = 0; w < RW; ++w) {
                const float sw = slots[parity][w][lane];
                if (w < wave) mine += sw;
                next += sw;
            }
            carry = next;
            parity ^= 1;
            if (live) {
#pragma unroll
                for (int u = 0; u < U; ++u)
                    if (k0 + u < R) q[(k0 + u) * qstep] = mine + v[u];
            }
        };
        float carry = 0.f;
        float a[U], b[U];
        load_group(0, a);
        for (int64_t g = 0; g < nrounds; g += 2) {
            if (g + 1 < nrounds) load_group(g + 1, b);
            __builtin_amdgcn_sched_barrier(0);  // the next round's loads go out first
            round(g, a, carry);
            __builtin_amdgcn_sched_barrier(0);
            if (g + 1 >= nrounds) break;
            if (g + 2 < nrounds) load_group(g + 2, a);
            __builtin_amdgcn_sched_barrier(0);
            round(g + 1, b, carry);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// Two layouts of scan_strided_kernel's lanes have one unit-stride side that
// the lanes do not follow; a block then stages that side through LDS.  A
// block is kStageWaves waves on kStageCols adjacent columns (lane l of every
// wave keeps column c0 + l), so a [32768, 32768] transpose has 512 blocks and
// needs no slabs (x read once).  The block walks its slab in rounds of
// kStageWaves chunks of kTileRows rows, in processing order; wave w takes the
// round's w-th chunk:
//   - it loads its chunk's terms and adds them up in processing order into
//     running sums pre_j (chunk-local prefixes) and the chunk total t_w;
//   - the totals meet in LDS (two slot sets in turn: one barrier a round);
//   - its outputs are (carry + t_0 + ... + t_{w-1}) + pre_j, the brackets
//     summed left to right, and the next round's carry is carry + t_0 + ... +
//     t_{kStageWaves-1}, the same sum in every wave;
// so a column's results do not depend on timing (a different, equally fixed
// order from scan_strided_kernel's one term after the other).  Items: (slab
// s, block of kStageCols columns), columns fastest.  totals != null: only the
// slab totals (the final carries) go to totals[s*n + e].
constexpr int kTileRows = 32;
constexpr int kTilePitch = kTileRows + 1;  // odd: column-wise and row-wise LDS walks hit distinct banks
constexpr int kStageWaves = 4;
constexpr int kStageCols = kWave;

// The rows [lo, lo + kc) of chunk c (c0 = c*kTileRows processing positions
// into a slab [r_begin, r_end)): REV walks the slab from its end.
template <bool REV>
__device__ __forceinline__ int64_t chunk_lo(int64_t r_begin, int64_t r_end, int64_t c0, int kc) {
    return REV ? r_end - c0 - kc : r_begin + c0;
}

// The round's chunk totals t (this lane's column, this wave's chunk) joined:
// returns carry + t_0 + ... + t_{w-1} and sets carry to the sum over every
// wave.  Every thread of the block calls it once a round.
__device__ __forceinline__ float stage_carry(float t, float& carry,
                                             float (&slots)[2][kStageWaves][kStageCols],
                                             int& parity, int wave, int lane) {
    slots[parity][wave][lane] = t;
    __syncthreads();
    float mine = carry, next = carry;
#pragma unroll
    for (int w = 0; w < kStageWaves; ++w) {
        const float v = slots[parity][w][lane];
        if (w < wave) mine = mine + v;
        next = next + v;
    }
    carry = next;
    parity ^= 1;
    return mine;
}

// inner == 1: column o's outputs are out[o*R + r], R floats apart from the
// next column's, so lanes storing their own prefixes would each write 4
// bytes of a different line.  Lane l keeps column o = o0 + l: it loads its
// chunk's terms x[o*so + r*sr] (adjacent across lanes when so == 1), adds
// them, and parks each output at tile[l][r - lo] of its wave's tile; then the
// wave writes the tile out row by row of out (kTileRows consecutive floats of
// one column per 32 lanes).
template <bool REV>
__global__ __launch_bounds__(kStageWaves * kWave) void scan_tile_out_kernel(
    const float* x, float* out, int64_t outer, int64_t R, int64_t so, int64_t sr, int64_t S,
    int64_t rps, const float* __restrict__ carry_in, float* __restrict__ totals) {
    __shared__ float tile[kStageWaves][kStageCols * kTilePitch];
    __shared__ float slots[2][kStageWaves][kStageCols];
    const int wave = wave_in_block();
    const int lane = threadIdx.x % kWave;
    const bool scan_out = totals == nullptr;
    float* wt = tile[wave];
    const int64_t nblk = (outer + kStageCols - 1) / kStageCols;
    const int64_t nitems = nblk * S;
    int parity = 0;
    for (int64_t item = blockIdx.x; item < nitems; item += gridDim.x) {
        const int64_t s = item / nblk;
        const int64_t o0 = (item - s * nblk) * kStageCols;
        const int ncols = outer - o0 < kStageCols ? int(outer - o0) : kStageCols;
        const bool live = lane < ncols;
        const int64_t r_begin = s * rps;
        const int64_t r_end = r_begin + rps < R ? r_begin + rps : R;
        const int64_t m = r_end - r_begin;  // >= 1: no slab is empty
        const float* p = x + (live ? (o0 + lane) * so : 0);
        float carry = live && scan_out && carry_in != nullptr ? carry_in[s * outer + o0 + lane] : 0.f;
        for (int64_t c0 = 0; c0 < m; c0 += kStageWaves * kTileRows) {
            const int64_t cw = c0 + int64_t(wave) * kTileRows;  // this wave's chunk
            const int kc = cw >= m ? 0 : (m - cw < kTileRows ? int(m - cw) : kTileRows);
            const int64_t lo = chunk_lo<REV>(r_begin, r_end, cw, kc);
            float v[kTileRows];
            float t = 0.f;
            if (live && kc == kTileRows) {
#pragma unroll
                for (int j = 0; j < kTileRows; ++j)
                    v[j] = p[(lo + (REV ? kTileRows - 1 - j : j)) * sr];
#pragma unroll
                for (int j = 0; j < kTileRows; ++j) {
                    t += v[j];
                    v[j] = t;
                }
            } else if (live) {
#pragma unroll
                for (int j = 0; j < kTileRows; ++j) {
                    if (j < kc) {
                        t += p[(lo + (REV ? kc - 1 - j : j)) * sr];
                        v[j] = t;
                    }
                }
            }
            const float mine = stage_carry(t, carry, slots, parity, wave, lane);
            if (scan_out && kc > 0) {
                if (live) {
#pragma unroll
                    for (int j = 0; j < kTileRows; ++j)
                        if (j < kc) wt[lane * kTilePitch + (REV ? kc - 1 - j : j)] = mine + v[j];
                }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                if (kc == kTileRows) {
#pragma unroll 8
                    for (int mm = 0; mm < kStageCols / 2; ++mm) {
                        const int col = 2 * mm + lane / kTileRows;
                        const int k = lane % kTileRows;
                        if (col < ncols) out[(o0 + col) * R + lo + k] = wt[col * kTilePitch + k];
                    }
                } else {
                    for (int f = lane; f < ncols * kc; f += kWave) {
                        const int col = f / kc;
                        const int k = f - col * kc;
                        out[(o0 + col) * R + lo + k] = wt[col * kTilePitch + k];
                    }
                }
                // the wave's tile is refilled next round only after these
                // reads: its own later LDS writes follow them in order
                __builtin_amdgcn_wave_barrier();
            }
        }
        if (!scan_out && live && wave == 0) totals[s * outer + o0 + lane] = carry;
    }
}

// stride_r == 1, inner > 1 (columns e = o*inner + i at x[o*so + i*si], their
// terms adjacent): lanes own adjacent outputs, so their stores are adjacent,
// but their loads are si floats apart.  Each wave first reads its chunk's
// kTileRows terms of the block's columns, 32 lanes per column run (128
// contiguous bytes), into its tile[col][r - lo]; then lane l adds column
// e0 + l's terms from the tile and stores each output at
// out[(o*R + r)*inner + i].
template <bool REV>
__global__ __launch_bounds__(kStageWaves * kWave) void scan_tile_in_kernel(
    const float* x, float* out, int64_t outer, int64_t R, int64_t inner, int64_t so,
    int64_t si, int64_t S, int64_t rps, const float* __restrict__ carry_in,
    float* __restrict__ totals) {
    __shared__ float tile[kStageWaves][kStageCols * kTilePitch];
    __shared__ float slots[2][kStageWaves][kStageCols];
    __shared__ int64_t base[kStageCols];  // where each column's terms start in x
    const int wave = wave_in_block();
    const int lane = threadIdx.x % kWave;
    const bool scan_out = totals == nullptr;
    float* wt = tile[wave];
    const int64_t n = outer * inner;
    const int64_t nblk = (n + kStageCols - 1) / kStageCols;
    const int64_t nitems = nblk * S;
    int parity = 0;
    for (int64_t item = blockIdx.x; item < nitems; item += gridDim.x) {
        const int64_t s = item / nblk;
        const int64_t e0 = (item - s * nblk) * kStageCols;
        const int ncols = n - e0 < kStageCols ? int(n - e0) : kStageCols;
        const bool live = lane < ncols;
        const int64_t e = e0 + lane;
        const int64_t o = live ? e / inner : 0;
        const int64_t i = live ? e - o * inner : 0;
        const int64_t r_begin = s * rps;
        const int64_t r_end = r_begin + rps < R ? r_begin + rps : R;
        const int64_t m = r_end - r_begin;  // >= 1: no slab is empty
        float* q = out + o * R * inner + i;
        float carry = live && scan_out && carry_in != nullptr ? carry_in[s * n + e] : 0.f;
        __syncthreads();  // the previous item is done with base
        if (wave == 0) base[lane] = o * so + i * si;
        __syncthreads();
        const float* wr = wt + lane * kTilePitch;
        for (int64_t c0 = 0; c0 < m; c0 += kStageWaves * kTileRows) {
            const int64_t cw = c0 + int64_t(wave) * kTileRows;  // this wave's chunk
            const int kc = cw >= m ? 0 : (m - cw < kTileRows ? int(m - cw) : kTileRows);
            const int64_t lo = chunk_lo<REV>(r_begin, r_end, cw, kc);
            if (kc == kTileRows) {  // all loads in flight, then the tile
                float v[kStageCols / 2];
#pragma unroll
                for (int mm = 0; mm < kStageCols / 2; ++mm) {
                    const int col = 2 * mm + lane / kTileRows;
                    v[mm] = col < ncols ? x[base[col] + lo + lane % kTileRows] : 0.f;
                }
#pragma unroll
                for (int mm = 0; mm < kStageCols / 2; ++mm) {
                    const int col = 2 * mm + lane / kTileRows;
                    wt[col * kTilePitch + lane % kTileRows] = v[mm];
                }
            } else {
                for (int f = lane; f < ncols * kc; f += kWave) {
                    const int col = f / kc;
                    const int k = f - col * kc;
                    wt[col * kTilePitch + k] = x[base[col] + lo + k];
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            float v[kTileRows];
            float t = 0.f;
#pragma unroll
            for (int j = 0; j < kTileRows; ++j) {
                if (j < kc) {
                    t += wr[REV ? kc - 1 - j : j];
                    v[j] = t;
                }
            }
            if (!live) t = 0.f;
            const float mine = stage_carry(t, carry, slots, parity, wave, lane);
            if (scan_out && live) {
#pragma unroll
                for (int j = 0; j < kTileRows; ++j)
                    if (j < kc) q[(lo + (REV ? kc - 1 - j : j)) * inner] = mine + v[j];
            }
            // the wave's tile is refilled next round only after these reads
            __builtin_amdgcn_wave_barrier();
        }
        if (!scan_out && live && wave == 0) totals[s * n + e] = carry;
    }
}

// ------------------------------------------------------------ launching
template <typename T>
struct same {
    using type = T;
};

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

template <bool REV, int NW, int K>
hipError_t rows_block_k(const rd_plan& p, const float* x, float* out, const Strides& v,
                        const float* carry_in, float* totals, hipStream_t s) {
    if (p.order == RD_ORDER_INTERLEAVED) {  // persistent workgroups streaming whole rows
        if (p.split != 1 || carry_in || totals) return hipErrorInvalidValue;
        if (p.nontemporal)
            return launch(scan_rows_stream_kernel<REV, NW, K, true>, p.blocks, NW * kWave, s, x,
                          out, v.outer, v.R, v.so);
        return launch(scan_rows_stream_kernel<REV, NW, K, false>, p.blocks, NW * kWave, s, x,
                      out, v.outer, v.R, v.so);
    }
    if (p.nontemporal)
        return launch(scan_rows_block_kernel<REV, NW, K, true>, p.blocks, NW * kWave, s, x, out,
                      v.outer, v.R, v.so, p.split, p.rows_per_split, carry_in, totals);
    return launch(scan_rows_block_kernel<REV, NW, K, false>, p.blocks, NW * kWave, s, x, out,
                  v.outer, v.R, v.so, p.split, p.rows_per_split, carry_in, totals);
}

template <bool REV, int K>
hipError_t rows_k(const rd_plan& p, const float* x, float* out, const Strides& v,
                  const float* carry_in, float* totals, hipStream_t s) {
    // a workgroup of group / 64 waves per item, or a wave per item
    switch (p.group) {
        case 4 * kWave: return rows_block_k<REV, 4, K>(p, x, out, v, carry_in, totals, s);
        case 8 * kWave: return rows_block_k<REV, 8, K>(p, x, out, v, carry_in, totals, s);
        case 16 * kWave: return rows_block_k<REV, 16, K>(p, x, out, v, carry_in, totals, s);
        case kWave: break;
        default: return hipErrorInvalidValue;
    }
    if (p.nontemporal)
        return launch(scan_rows_kernel<REV, K, true>, p.blocks, kBlock, s, x, out, v.outer, v.R,
                      v.so, p.split, p.rows_per_split, carry_in, totals);
    return launch(scan_rows_kernel<REV, K, false>, p.blocks, kBlock, s, x, out, v.outer, v.R,
                  v.so, p.split, p.rows_per_split, carry_in, totals);
}

template <bool REV>
hipError_t rows_go(const rd_plan& p, const float* x, float* out, const Strides& v,
                   const float* carry_in, float* totals, hipStream_t s) {
    if (p.unroll == 8) return rows_k<REV, 8>(p, x, out, v, carry_in, totals, s);
    return rows_k<REV, 4>(p, x, out, v, carry_in, totals, s);
}

template <bool REV, int V, int BW, bool NT>
hipError_t cols_bw(const rd_plan& p, const float* x, float* out, const Strides& v,
                   int64_t ntiles, const float* carry_in, float* totals, hipStream_t s) {
    const uint32_t nx = uint32_t(p.nxcd);
    if (p.unroll == 16)
        return launch(scan_cols_kernel<REV, V, 16, BW, NT>, p.blocks, BW * kWave, s, x, out,
                      v.outer, v.R, v.inner, v.so, v.sr, ntiles, p.split, p.rows_per_split,
                      carry_in, totals, nx);
    if (p.unroll == 8)
        return launch(scan_cols_kernel<REV, V, 8, BW, NT>, p.blocks, BW * kWave, s, x, out,
                      v.outer, v.R, v.inner, v.so, v.sr, ntiles, p.split, p.rows_per_split,
                      carry_in, totals, nx);
    return launch(scan_cols_kernel<REV, V, 4, BW, NT>, p.blocks, BW * kWave, s, x, out, v.outer,
                  v.R, v.inner, v.so, v.sr, ntiles, p.split, p.rows_per_split, carry_in, totals,
                  nx);
}

template <bool REV, int RW, bool NT>
hipError_t rounds_go(const rd_plan& p, const float* x, float* out, const Strides& v,
                     int64_t ntiles, const float* carry_in, hipStream_t s) {
    const uint32_t nx = uint32_t(p.nxcd);
    if (p.unroll == 8)
        return launch(scan_cols_rounds_kernel<REV, 8, RW, NT>, p.blocks, RW * kWave, s, x, out,
                      v.outer, v.R, v.inner, v.so, v.sr, ntiles, p.split, p.rows_per_split,
                      carry_in, nx);
    if (p.unroll == 4)
        return launch(scan_cols_rounds_kernel<REV, 4, RW, NT>, p.blocks, RW * kWave, s, x, out,
                      v.outer, v.R, v.inner, v.so, v.sr, ntiles, p.split, p.rows_per_split,
                      carry_in, nx);
    return hipErrorInvalidValue;
}

// The slab totals of a row-rounds plan cut into slabs: totals[s][o][i] = the
// sum of slab s of column (o, i), by the column reduction (one-wave tiles,
// kScanSlabTotalsRowWaves waves taking turns on the rows, the same slabs) --
// a fixed order of its own; the carries and the scan pass follow.
hipError_t slab_totals(const rd_plan& p, const float* x, const Strides& v, float* totals,
                       hipStream_t s) {
    rd_plan q = p;
    q.path = RD_PATH_COLS;
    q.col_waves = 1;
    q.row_waves = kScanSlabTotalsRowWaves;
    q.unroll = kScanSlabTotalsUnroll;
    q.block_threads = kWave * q.row_waves;
    const int64_t tiles = ((v.inner + 3) / 4 + kWave - 1) / kWave;
    q.blocks = tiles * p.split * v.outer;
    if (q.blocks > kMaxBlocks) q.blocks = kMaxBlocks;
    return launch_cols(RD_OP_SUM, q, x, v, Results{totals, nullptr}, nullptr, Results{}, s);
}

template <bool REV, int V, bool NT>
hipError_t cols_go(const rd_plan& p, const float* x, float* out, const Strides& v,
                   const float* carry_in, float* totals, hipStream_t s) {
    const int64_t lane_cols = v.inner >= 4 ? (v.inner + 3) / 4 : 1;
    const int64_t ntiles = (lane_cols + kWave - 1) / kWave;
    if (p.row_waves > 1) {  // waves of a block taking turns in R
        if constexpr (V == 4) {
            if (p.col_waves != 1 || (p.split == 1 && (carry_in || totals)))
                return hipErrorInvalidValue;
            if (totals) return slab_totals(p, x, v, totals, s);
            switch (p.row_waves) {
                case 2: return rounds_go<REV, 2, NT>(p, x, out, v, ntiles, carry_in, s);
                case 4: return rounds_go<REV, 4, NT>(p, x, out, v, ntiles, carry_in, s);
                case 8: return rounds_go<REV, 8, NT>(p, x, out, v, ntiles, carry_in, s);
                case 16: return rounds_go<REV, 16, NT>(p, x, out, v, ntiles, carry_in, s);
                default: return hipErrorInvalidValue;
            }
        }
        return hipErrorInvalidValue;
    }
    if (p.col_waves == 16)
        return cols_bw<REV, V, 16, NT>(p, x, out, v, ntiles, carry_in, totals, s);
    if (p.col_waves == 8)
        return cols_bw<REV, V, 8, NT>(p, x, out, v, ntiles, carry_in, totals, s);
    if constexpr (V == 4) {
        if (p.col_waves == 2)
            return cols_bw<REV, V, 2, NT>(p, x, out, v, ntiles, carry_in, totals, s);
        if (p.col_waves == 1)
            return cols_bw<REV, V, 1, NT>(p, x, out, v, ntiles, carry_in, totals, s);
    }
    if (p.col_waves != 4) return hipErrorInvalidValue;
    return cols_bw<REV, V, 4, NT>(p, x, out, v, ntiles, carry_in, totals, s);
}

template <bool REV, bool NT>
hipError_t cols_v(const rd_plan& p, const float* x, float* out, const Strides& v,
                  const float* carry_in, float* totals, hipStream_t s) {
    if (v.si != 1) return hipErrorInvalidValue;
    if (v.inner == 2) return cols_go<REV, 2, NT>(p, x, out, v, carry_in, totals, s);
    if (v.inner == 3) return cols_go<REV, 3, NT>(p, x, out, v, carry_in, totals, s);
    return cols_go<REV, 4, NT>(p, x, out, v, carry_in, totals, s);
}

template <bool REV, int V, bool NT>
hipError_t small_go(const rd_plan& p, const float* x, float* out, const Strides& v,
                    const float* carry_in, float* totals, hipStream_t s) {
    const int32_t lc = v.inner >= 4 ? int32_t((v.inner + 3) / 4) : 1;
    const uint32_t nx = uint32_t(p.nxcd);
    if (p.unroll == 8)
        return launch(scan_small_kernel<REV, V, 8, NT>, p.blocks, kBlock, s, x, out, v.outer, v.R,
                      v.inner, v.so, v.sr, p.split, p.rows_per_split, lc, carry_in, totals, nx);
    return launch(scan_small_kernel<REV, V, 4, NT>, p.blocks, kBlock, s, x, out, v.outer, v.R,
                  v.inner, v.so, v.sr, p.split, p.rows_per_split, lc, carry_in, totals, nx);
}

template <bool REV, bool NT>
hipError_t small_v(const rd_plan& p, const float* x, float* out, const Strides& v,
                   const float* carry_in, float* totals, hipStream_t s) {
    if (v.inner == 2) return small_go<REV, 2, NT>(p, x, out, v, carry_in, totals, s);
    if (v.inner == 3) return small_go<REV, 3, NT>(p, x, out, v, carry_in, totals, s);
    return small_go<REV, 4, NT>(p, x, out, v, carry_in, totals, s);
}

}  // namespace

hipError_t launch_scan_small(const rd_plan& p, bool reverse, const float* x, float* out,
                             const Strides& v, const float* carry_in, float* totals,
                             hipStream_t s) {
    if (reverse)
        return p.nontemporal ? small_v<true, true>(p, x, out, v, carry_in, totals, s)
                             : small_v<true, false>(p, x, out, v, carry_in, totals, s);
    return p.nontemporal ? small_v<false, true>(p, x, out, v, carry_in, totals, s)
                         : small_v<false, false>(p, x, out, v, carry_in, totals, s);
}

hipError_t launch_scan_rows(const rd_plan& p, bool reverse, const float* x, float* out,
                            const Strides& v, const float* carry_in, float* totals,
                            hipStream_t s) {
    return reverse ? rows_go<true>(p, x, out, v, carry_in, totals, s)
                   : rows_go<false>(p, x, out, v, carry_in, totals, s);
}

struct LookArgs {
    uint32_t* ticket;
    uint64_t* agg;
    uint64_t* gsum;
    int64_t NG;
    uint32_t tag, spin_limit;
};

template <bool REV, int NW, int K>
hipError_t lookback_k(const rd_plan& p, const float* x, float* out, const Strides& v,
                      const LookArgs& a, hipStream_t s) {
    if (p.nontemporal)
        return launch(scan_rows_lookback_kernel<REV, NW, K, true>, p.blocks, NW * kWave, s, x,
                      out, v.outer, v.R, v.so, p.split, a.NG, a.ticket, a.agg, a.gsum, a.tag,
                      a.spin_limit);
    return launch(scan_rows_lookback_kernel<REV, NW, K, false>, p.blocks, NW * kWave, s, x, out,
                  v.outer, v.R, v.so, p.split, a.NG, a.ticket, a.agg, a.gsum, a.tag,
                  a.spin_limit);
}

template <bool REV, int NW>
hipError_t lookback_go(const rd_plan& p, const float* x, float* out, const Strides& v,
                       const LookArgs& a, hipStream_t s) {
    if (p.unroll == 4) return lookback_k<REV, NW, 4>(p, x, out, v, a, s);
    return lookback_k<REV, NW, 8>(p, x, out, v, a, s);
}

hipError_t launch_scan_rows_lookback(const rd_plan& p, bool reverse, const float* x, float* out,
                                     const Strides& v, void* ws, const Published* pub,
                                     uint32_t spin_limit, hipStream_t s) {
    const int64_t NG = lookback_groups(p.split);
    const int nw = p.group / kWave;
    if (p.combine != RD_COMBINE_LOOKBACK || (p.unroll != 4 && p.unroll != 8) ||
        (nw != 4 && nw != 8 && nw != 16) ||
        p.rows_per_split != int64_t(nw) * 256 * p.unroll || p.blocks != v.outer * p.split ||
        p.blocks > int64_t(UINT32_MAX) ||
        p.workspace_bytes != lookback_workspace_bytes(v.outer, p.split))
        return hipErrorInvalidValue;
    LookArgs a{};
    a.NG = NG;
    a.spin_limit = spin_limit;
    if (pub) {
        if (!pub->ticket || !pub->words || pub->epoch == 0 ||
            lookback_words(v.outer, p.split) > kPubColWords)
            return hipErrorInvalidValue;
        a.ticket = pub->ticket;
        a.agg = pub->words;
        a.tag = pub->epoch;
    } else {
        if (ws == nullptr) return hipErrorInvalidValue;
        hipError_t e = hipMemsetAsync(ws, 0, size_t(p.workspace_bytes), s);
        if (e != hipSuccess) return e;
        char* base = static_cast<char*>(ws);
        a.ticket = reinterpret_cast<uint32_t*>(base);
        a.agg = reinterpret_cast<uint64_t*>(base + kLookTicketBytes);
        a.tag = 1;
    }
    a.gsum = a.agg + v.outer * p.split;
    switch ((reverse ? 100 : 0) + nw) {
        case 104: return lookback_go<true, 4>(p, x, out, v, a, s);
        case 108: return lookback_go<true, 8>(p, x, out, v, a, s);
        case 116: return lookback_go<true, 16>(p, x, out, v, a, s);
        case 4: return lookback_go<false, 4>(p, x, out, v, a, s);
        case 8: return lookback_go<false, 8>(p, x, out, v, a, s);
        default: return lookback_go<false, 16>(p, x, out, v, a, s);
    }
}

hipError_t launch_scan_carries(const float* totals, float* carries, int64_t rows, int64_t P,
                               hipStream_t s) {
    int64_t blocks = (rows + kBlock / kWave - 1) / (kBlock / kWave);  // a wave per row
    blocks = blocks > kMaxBlocks ? kMaxBlocks : blocks;
    return launch(scan_carries_kernel, blocks, kBlock, s, totals, carries, rows, P);
}

hipError_t launch_scan_cols(const rd_plan& p, bool reverse, const float* x, float* out,
                            const Strides& v, const float* carry_in, float* totals,
                            hipStream_t s) {
    if (reverse)
        return p.nontemporal ? cols_v<true, true>(p, x, out, v, carry_in, totals, s)
                             : cols_v<true, false>(p, x, out, v, carry_in, totals, s);
    return p.nontemporal ? cols_v<false, true>(p, x, out, v, carry_in, totals, s)
                         : cols_v<false, false>(p, x, out, v, carry_in, totals, s);
}

template <int RW>
hipError_t strided_rounds_go(const rd_plan& p, bool reverse, const float* x, float* out,
                             const Strides& v, int64_t ngroups, hipStream_t s) {
    constexpr int U = kStridedRoundsUnroll;
    const uint32_t nx = uint32_t(p.nxcd);
    if (reverse)
        return launch(scan_strided_rounds_kernel<true, U, RW>, p.blocks, RW * kWave, s, x, out,
                      v.outer, v.R, v.inner, v.so, v.sr, v.si, ngroups, nx);
    return launch(scan_strided_rounds_kernel<false, U, RW>, p.blocks, RW * kWave, s, x, out,
                  v.outer, v.R, v.inner, v.so, v.sr, v.si, ngroups, nx);
}

hipError_t launch_scan_strided(const rd_plan& p, bool reverse, const float* x, float* out,
                               const Strides& v, const float* carry_in, float* totals,
                               hipStream_t s) {
    const int64_t blocks = p.blocks;
    if (v.inner == 1) {  // stage the outputs: a block per (slab, kStageCols columns)
        if (reverse)
            return launch(scan_tile_out_kernel<true>, blocks, kStageWaves * kWave, s, x, out,
                          v.outer, v.R, v.so, v.sr, p.split, p.rows_per_split, carry_in, totals);
        return launch(scan_tile_out_kernel<false>, blocks, kStageWaves * kWave, s, x, out, v.outer,
                      v.R, v.so, v.sr, p.split, p.rows_per_split, carry_in, totals);
    }
    if (v.sr == 1) {  // stage the inputs: a block per (slab, kStageCols columns)
        if (reverse)
            return launch(scan_tile_in_kernel<true>, blocks, kStageWaves * kWave, s, x, out,
                          v.outer, v.R, v.inner, v.so, v.si, p.split, p.rows_per_split, carry_in,
                          totals);
        return launch(scan_tile_in_kernel<false>, blocks, kStageWaves * kWave, s, x, out, v.outer,
                      v.R, v.inner, v.so, v.si, p.split, p.rows_per_split, carry_in, totals);
    }
    if (p.row_waves > 1) {  // one pass, RW waves a block taking turns on the rows
        if (p.split != 1 || carry_in || totals || p.unroll != kStridedRoundsUnroll)
            return hipErrorInvalidValue;
        const int64_t ngroups = (v.outer * v.inner + kWave - 1) / kWave;
        switch (p.row_waves) {
            case 2: return strided_rounds_go<2>(p, reverse, x, out, v, ngroups, s);
            case 4: return strided_rounds_go<4>(p, reverse, x, out, v, ngroups, s);
            case 8: return strided_rounds_go<8>(p, reverse, x, out, v, ngroups, s);
            default: return hipErrorInvalidValue;
        }
    }
    // a lane per (slab, column)
    if (reverse)
        return launch(scan_strided_kernel<true>, blocks, kBlock, s, x, out, v.outer, v.R,
                      v.inner, v.so, v.sr, v.si, p.split, p.rows_per_split, carry_in, totals);
    return launch(scan_strided_kernel<false>, blocks, kBlock, s, x, out, v.outer, v.R, v.inner,
                  v.so, v.sr, v.si, p.split, p.rows_per_split, carry_in, totals);
}

hipError_t launch_scan_slab_carries(bool reverse, const float* totals, float* carries, int64_t S,
                                    int64_t n, hipStream_t s) {
    if (S > kWave) {  // many slabs: a wave per (o, i)
        int64_t blocks = (n + kBlock / kWave - 1) / (kBlock / kWave);
        blocks = blocks > kMaxBlocks ? kMaxBlocks : blocks;
        if (reverse)
            return launch(scan_slab_carries_wave_kernel<true>, blocks, kBlock, s, totals, carries,
                          S, n);
        return launch(scan_slab_carries_wave_kernel<false>, blocks, kBlock, s, totals, carries, S,
                      n);
    }
    if (reverse)
        return launch(scan_slab_carries_kernel<true>, grid_for(n), kBlock, s, totals, carries, S, n);
    return launch(scan_slab_carries_kernel<false>, grid_for(n), kBlock, s, totals, carries, S, n);
}

}  // namespace rd
