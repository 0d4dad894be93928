// rd_internal.h -- declarations shared by the C ABI, the planner and the
// kernel launchers.  Not installed; the public boundary is include/rd.h.
#pragma once

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "rd.h"

namespace rd {

// Lanes per wavefront on CDNA.
constexpr int kWave = 64;
// Threads of every ROWS / combine / fill workgroup.
constexpr int kBlock = 256;
// Rows shorter than this take the lane-per-row path.
constexpr int64_t kShortRow = 64;
// Inner sizes up to this take the several-rows-per-load column path.
constexpr int64_t kSmallInner = 128;
// A strided view whose kept inner axis is 2 .. kDenseColumnStride floats apart
// (every 128-byte line of a row's span then holds one of its terms) and whose
// rows span more than kSmallInner floats is reduced by the column kernel over
// the dense span of its rows, keeping every si-th column (dense_columns).
constexpr int64_t kDenseColumnStride = 32;
// Upper bound on workgroups per launch; larger problems loop inside the
// kernels (a grid's total thread count must stay below 2^32 on AMD, and
// workgroups have up to 1024 threads).
constexpr int64_t kMaxBlocks = int64_t(1) << 20;
// Devices the library keeps state for (indices 0 .. kMaxDevices - 1).
constexpr int kMaxDevices = 64;


// Where a launch stores its results: `a` holds them (for the softmax
// denominator, the maxima), `b` the softmax denominator's sums (null for the
// other operators).  Workspaces of partial results are laid out the same way.
struct Results {
    float* a;
    float* b;
};

// The [outer, R, inner] view a reduction reads: element (o, r, i) at
// x[o*so + r*sr + i*si] (strides in floats).  A contiguous array has
// so = R*inner, sr = inner, si = 1.  The planner picks the kernel from the
// unit stride: si == 1 (columns contiguous) -> the column kernels;
// sr == 1 -> the row kernels over outer*inner rows; neither -> the
// lane-per-output kernel.
struct Strides {
    int64_t outer, R, inner, so, sr, si;
};

// Planner (rd_plan.cpp).  `tune` may be null; `op` is an rd_op (it only
// decides which kernel shapes exist).  plan_view first normalises *v (the
// strides of length-1 axes; a strided reduction with adjacent outputs becomes
// a column reduction), and the launch must use the normalised view.
rd_status plan_view(int cu_count, Strides* v, int op, const rd_tune* tune, rd_plan* plan);
// Non-negative sizes and strides whose furthest element, and outer*R*inner
// floats, are representable in bytes.
bool view_sizes_ok(const Strides& v);
// A view the column kernel reads as the dense span of its rows (see
// kDenseColumnStride): inner > 1, 2 <= si <= kDenseColumnStride, span wider
// than kSmallInner, rows that do not overlap (sr >= span, or R == 1).
// plan_view gives it a COLS plan; launch_cols keeps every si-th column.
bool dense_columns(const Strides& v);
// A contiguous [outer, R, inner] array.
rd_status plan_dim(int cu_count, int64_t outer, int64_t R, int64_t inner, int op,
                   const rd_tune* tune, rd_plan* plan);

// Kernel launchers (rd_kernels.hip).  Each enqueues on `s` and returns the
// error hipLaunchKernel reports for the launch; `op` is an rd_op.
hipError_t launch_fill_start(int op, Results out, int64_t n, hipStream_t s);
// The single-launch combine of a row reduce cut into pieces: every
// workgroup publishes its piece results as tagged words (publish_word, tag =
// epoch) at words[seg] (a softmax pair: its maximum there, its sum at
// words[nseg + seg]); the grid's last workgroup waits for all of them
// (await_word: NaN for one that never comes), copies them to vals in the
// same layout and combines each row's pieces into out as the second kernel
// does, with the same bits.  words holds no word tagged `epoch` when
// the kernel starts (the host gives each launch on a stream a new epoch and
// the stream its own buffer).
// Piece results a stream's buffer holds, and the most rows the planner
// gives the single-launch combine.
constexpr int64_t kPubWords = 8192;
constexpr int64_t kPubMaxRows = 4;
constexpr int64_t kPubRowsMaxWords = 512;  // the planner's default limit
// The same for a column reduce cut into a few slabs (at most kPubColMaxSlabs,
// the blocks within one per CU, so all of them run at once): every block
// but those of the last slab publishes its slab's column results as tagged
// words at words[(s*outer + o)*inner_out + k], and the last slab's block of
// each tile joins slabs 0 .. S-1 of its columns in that order (the second
// kernel's order, so the same bits) into out.  At most kPubColWords words.
constexpr int64_t kPubColWords = 65536;
constexpr int64_t kPubColMaxSlabs = 16;
struct Published {
    uint64_t* words = nullptr;
    float* vals = nullptr;
    uint32_t* ticket = nullptr;  // the look-back scan's ticket: 0 between launches
    uint32_t epoch = 0;
    uint32_t spin_limit = 0;
};
// Rows (v.sr == 1): v.outer * v.inner rows.  pub == nullptr: dst receives
// the piece results (or the row results when p.split == 1); otherwise they
// are published and the last workgroup combines them into out.
hipError_t launch_rows(int op, const rd_plan& p, const float* x, const Strides& v,
                       Results dst, const Published* pub, Results out, hipStream_t s);
hipError_t launch_rows_short(int op, const float* x, const Strides& v, Results out,
                             hipStream_t s);
hipError_t launch_rows_combine(int op, Results part, int64_t outer, int64_t P, Results out,
                               hipStream_t s);
// Columns (v.si == 1, or a dense_columns view).  pub == nullptr: dst
// receives the slab results (or the outputs when p.split == 1); otherwise
// the slabs are joined in the same launch into out (kPubColWords).
hipError_t launch_cols(int op, const rd_plan& p, const float* x, const Strides& v,
                       Results dst, const Published* pub, Results out, hipStream_t s);
hipError_t launch_cols_small(int op, const rd_plan& p, const float* x, const Strides& v,
                             Results dst, hipStream_t s);
// Any strides: one lane per (slab, output); dst is the output when
// p.split == 1, else [p.split][outer*inner] partial results.
hipError_t launch_strided(int op, const rd_plan& p, const float* x, const Strides& v,
                          Results dst, hipStream_t s);
hipError_t launch_slab_combine(int op, Results slab, int64_t S, int64_t n, Results out,
                               hipStream_t s);

// Cumulative sums (rd_scan.hip).  The input is a view (Strides: element
// (o, r, i) at x[o*so + r*sr + i*si]; a contiguous array has so = R*inner,
// sr = inner, si = 1); the output is the contiguous [outer, R, inner] array.
// Rows (inner == 1, sr == 1): item = (row, piece of p.rows_per_split
// processing positions); totals != nullptr writes only the piece totals,
// otherwise pieces are scanned from carry_in (nullptr: 0).
hipError_t launch_scan_rows(const rd_plan& p, bool reverse, const float* x, float* out,
                            const Strides& v, const float* carry_in, float* totals,
                            hipStream_t s);
hipError_t launch_scan_carries(const float* totals, float* carries, int64_t rows, int64_t P,
                               hipStream_t s);
// Rows in one pass by a fixed-order look-back (p.combine RD_COMBINE_LOOKBACK):
// p.split pieces of one block chunk per row, a workgroup each.  pub ==
// nullptr: ws holds p.workspace_bytes, which the call zeroes (in stream
// order) and the kernel uses for its ticket and the published totals (tag 1).
// Otherwise the stream's buffer serves, with nothing zeroed: its ticket (0
// between launches: the workgroup that draws the launch's last ticket sets it
// back to 0) and, with more than one piece per row, lookback_words(outer, P)
// of its words (at most kPubColWords), tagged with the launch's epoch.  A wait
// of the kernel ends after spin_limit polls (the piece's outputs are then
// NaN).
constexpr int64_t kLookGroup = 64;          // chunk totals per group total
constexpr int64_t kLookTicketBytes = 256;   // the ticket, padded
constexpr uint32_t kLookSpinLimit = 1u << 18;
inline int64_t lookback_groups(int64_t P) { return (P + kLookGroup - 1) / kLookGroup; }
inline int64_t lookback_workspace_bytes(int64_t outer, int64_t P) {
    return kLookTicketBytes + 8 * outer * (P + lookback_groups(P));
}
// Tagged words the look-back publishes: chunk totals and group totals, none
// with one piece per row (no piece has a successor).
inline int64_t lookback_words(int64_t outer, int64_t P) {
    return P > 1 ? outer * (P + lookback_groups(P)) : 0;
}
hipError_t launch_scan_rows_lookback(const rd_plan& p, bool reverse, const float* x, float* out,
                                     const Strides& v, void* ws, const Published* pub,
                                     uint32_t spin_limit, hipStream_t s);
// Columns (inner >= 2, si == 1): item = (64 lane-columns, slab of R, outer index).
hipError_t launch_scan_cols(const rd_plan& p, bool reverse, const float* x, float* out,
                            const Strides& v, const float* carry_in, float* totals,
                            hipStream_t s);
hipError_t launch_scan_small(const rd_plan& p, bool reverse, const float* x, float* out,
                             const Strides& v, const float* carry_in, float* totals,
                             hipStream_t s);
hipError_t launch_scan_slab_carries(bool reverse, const float* totals, float* carries, int64_t S,
                                    int64_t n, hipStream_t s);
// Any strides: a lane per (slab, output column); slab totals and carries
// laid out as those of launch_scan_cols.
hipError_t launch_scan_strided(const rd_plan& p, bool reverse, const float* x, float* out,
                               const Strides& v, const float* carry_in, float* totals,
                               hipStream_t s);

// Planner of the cumulative sum (rd_plan.cpp): plan_cumsum_view normalises
// the strides of length-1 axes in *v, then picks the rows scan (inner == 1,
// sr == 1), the column scans (inner > 1, si == 1) or the lane-per-column
// kernel; the launches must use the normalised view.
rd_status plan_cumsum_view(int cu_count, Strides* v, const rd_tune* tune, rd_plan* plan);
rd_status plan_cumsum(int cu_count, int64_t outer, int64_t R, int64_t inner,
                      const rd_tune* tune, rd_plan* plan);
// Row pieces of the row scan are whole multiples of kScanTile positions (a
// multiple of every wave chunk, 256 * slices, and of a workgroup's 4-slice
// chunk; a piece that is no multiple of the chunk ends with a partial one).
constexpr int64_t kScanTile = 4096;
// Row scans: 8-slice chunks (2048 positions a wave); rows longer than
// kScanRowsBlockMinR positions that are not cut into pieces take a workgroup
// of 8 waves (chunks of 16384 positions), from kScanRowsWideMinR on one of
// 16 (chunks of 32768).  A workgroup's chunk is 8 or 16 times a wave's, so
// a row of a chunk or less leaves no next chunk to load while one is
// scanned; 16 waves fill a CU alone, so they need rows of two chunks.
// Measured on MI355X (each line on one box, interleaved), forward / reverse,
// us:
//   R        wave        4 waves     8 waves     16 waves
//   4096     1580/1507   1396/1436   1820/2157   5542/6069
//   16384    1591/1571   1652/1604   1668/1675   1918/2037
//   20000    1511/1513   1487/1506   1446/1394   1589/1649
//   32768    1685/1669   1556/1566   1510/1539   1598/1679
//   68559    --          1550/1570   1512/1525   1434/1460
//   262144   1654/1638   1588/1580   1556/1554   1507/1503
// (1 GiB of input each; rows cut into pieces are faster by waves).
constexpr int kScanRowsChunkSlices = 8;
constexpr int64_t kScanRowsBlockMinR = 16384;
constexpr int64_t kScanRowsWideMinR = 65536;
// Few rows.  Rows are cut into pieces (piece totals, their scan, the scan
// from the carries: three launches, x read twice) only when there are fewer
// than a third as many rows as CUs and the rows hold at least
// kScanRowsCutMinR positions; otherwise every row is scanned in one pass,
// and with fewer than kScanRowWavesMin rows per CU a row of more than one
// tile takes a workgroup of 4 waves or more.  Measured on MI355X (one box,
// interleaved), us, pieces / one pass: [64, 65536] 18.9 / 14.4, [256, 65536]
// 39.7 / 24.7, [512, 16384] 21.8 / 14.6, [128, 131072] 39.8 / 29.0,
// [100, 1048576] 235.8 / 206.3; the other way round [64, 131072] 21.6 /
// 27.8, [64, 262144] 39.7 / 46.5, [64, 1048576] 131.9 / 179.8 (one
// workgroup streams a row at ~60 GB/s).  Rows of 4096 < R <= 16384 among
// few: a wave 7.5 -> 4 waves 6.2 us ([64, 8192]), 15.8 -> 9.2 ([256, 16384]).
// Longer rows among few -- at least kScanRowsLookMinR positions and
// kScanRowsLookMinN elements in all -- take the one-pass look-back instead
// (launch_scan_rows_lookback), pieces of 32768 positions: us, before -> after,
// [1, 2^28] 590.3 -> 397.5, [2, 2^26] 299.4 -> 206.5, [4, 2.5e7] 220.7 ->
// 161.9, [64, 2^20] 133.8 -> 110.6, [85, 2^20] 198.0 -> 142.4, [256, 2^20]
// 398.5 -> 381.0, [16, 2^20] 40.4 -> 39.6; shorter rows or smaller arrays
// lose the zeroing of its workspace (one more dispatch): [1, 2^22] 19.4 ->
// 21.1, [64, 2^17] 21.8 -> 25.3, [256, 2^18] 95.9 -> 104.7.
// Since the look-back takes the stream's buffer (nothing zeroed before the
// launch) it also replaces the three kernels for few rows of at least
// kScanRowsLookFewMinR positions (fewer rows than a third of the CUs): us,
// same box, A/B of the two libraries, three kernels (or one workgroup a row)
// -> look-back: [1, 1000003] 17.8 -> 9.4, [2, 131071] 15.8 -> 7.8, [16,
// 2^19] 22.0 -> 17.1, [64, 2^17] 21.9 -> 17.4, [80, 2^17] 29.5 -> 24.2, [7,
// 777777] 22.1 -> 19.3, [64, 2^16] 14.5 -> 12.3, [1, 65537] 12.7 -> 8.1; with
// more rows one workgroup a row stays ahead ([128, 2^17] 28.9 / 31.7,
// [256, 2^16] 25.0 / 31.2).  Up to kScanRowsLookSmallN elements the pieces
// are of 8 waves (16384 positions), twice the workgroups: us, 16 -> 8 waves,
// [1, 2^20] 9.4 -> 8.2, [1, 2^16] 7.7 -> 6.9, [2, 2^17] 8.3 -> 7.5; from
// 8 MB on 16 waves win ([8, 2^20] 17.6 / 21.4, [64, 2^16] 12.4 / 13.4).
constexpr int64_t kScanRowWavesMin = 4;
constexpr int64_t kScanRowsCutMinR = 131072;
constexpr int64_t kScanRowsLookMinR = int64_t(1) << 20;
constexpr int64_t kScanRowsLookMinN = int64_t(1) << 24;
constexpr int64_t kScanRowsLookFewMinR = 65536;
constexpr int64_t kScanRowsLookSmallN = int64_t(1) << 20;
// Arrays of at least kScanRowsTicketMinBytes whose rows fill an 8-wave
// chunk take the look-back kernel too: its workgroups take their pieces by a
// ticket, so all XCDs work on one narrow stretch of the array at a time,
// where block ids hand each XCD every eighth piece and the XCDs drift apart
// (same kernel, [32768, 32768]: 1321.5 us by ticket, 1478.5 us by block id;
// the block-per-row kernel 1524.8 us).  us, before -> after: [4096, 65536]
// 377.3 -> 348.5, [8192, 131072] 1570.7 -> 1351.9, [30000, 35791] 1663.2 ->
// 1513.8 (pieces of 16384), [1000, 262144] 367.2 -> 354.6; below 1 GB its
// fixed costs (zeroing the workspace, the tickets) lose: [256, 262144] 95.9
// -> 104.7, [512, 262144] 191.1 -> 191.7 -- except for rows of whole
// 32768-position pieces, which gain from 512 MB on ([4096, 32768] 188.9 ->
// 179.9, [1024, 131072] 196.3 -> 187.4; [2048, 32768] 94.9 -> 99.9).
constexpr int64_t kScanRowsTicketMinBytes = int64_t(1) << 30;
constexpr int64_t kScanRowWavesSplit = 16;  // pieces per CU once they are cut
constexpr int kScanColsUnroll = 8;        // rows per load group of the column scan,
// 16 for slabs of kScanColsDeepRows rows or more (same box, interleaved:
// [128, 4096, 4095] 3369 -> 3285 us, [16, 8192, 4096] 1073 -> 1055; short
// slabs -- [64, 512, 1024], 64 rows -- lose 3-5 % with 16)
constexpr int64_t kScanColsDeepRows = 1024;
// Column scans with between half and twice as many tiles (x outer) as CUs:
// a block per tile whose waves take turns on its row groups, at most
// kScanColsMaxRowWaves of them, aiming at kScanColsRoundWavesPerCu waves per CU.
constexpr int32_t kScanColsMaxRowWaves = 8;
constexpr int64_t kScanColsRoundWavesPerCu = 4;
// Fewer tiles (x outer) than half the CUs: slabs of R, as many as keep the
// blocks within one per CU; the slab totals by the column reduction (one-wave
// tiles, kScanSlabTotalsRowWaves row waves, kScanSlabTotalsUnroll rows in
// flight: the reduction's own plan for such columns), the scan pass a block
// of kScanSlabRowWaves waves per (tile, slab) taking turns on its rows from
// the slab's carry -- except for row strides that are a multiple of
// kScanSlabLockStride floats (8 KB) and at least twice that, which keep
// single-wave blocks walking the rows for both passes.  Measured on MI355X
// (same box, us, row rounds vs single waves, both with the reduction's
// totals): [1, 65536, 4095] 663 vs 714, [1, 131072, 4095] 1279 vs 1433,
// [1, 65536, 8000] 1021 vs 1065, [3, 100000, 300] 275 vs 316,
// [2, 100000, 129] 73 vs 104, [4, 8192, 2048] 127 vs 133; but
// [1, 65536, 4096] 618 vs 531, [1, 65536, 8192] 1157 vs 996,
// [1, 16384, 16384] 529 vs 498, [1, 65536, 6144] 835 vs 808.
// A lane-per-column strided scan with at least half as many groups of 64
// columns as CUs (and fewer than would fill the chip as single lanes): one
// pass, a block of row waves per group (the fewest of 2, 4, 8 that make about
// kStridedRoundsWavesPerCu waves per CU), kStridedRoundsUnroll rows a group.
constexpr int kStridedRoundsUnroll = 8;
constexpr int32_t kStridedRoundsMaxRowWaves = 8;
constexpr int64_t kStridedRoundsWavesPerCu = 4;
constexpr int32_t kScanSlabRowWaves = 8;
constexpr int32_t kScanSlabTotalsRowWaves = 8;
constexpr int32_t kScanSlabTotalsUnroll = 4;
constexpr int64_t kScanSlabLockStride = 2048;
constexpr int kScanSmallUnroll = 8;       // load instructions per step, small inner
constexpr int64_t kScanSmallWavesPerCu = 16;
// Inputs up to this size are read by a split scan's totals pass without the
// streaming hint (MI355X has a 256 MB last-level cache).
constexpr uint64_t kScanCachedTotalsBytes = uint64_t(256) << 20;

// The no-allocation sum (rd_api.cpp; its scratch buffer is in rd_noalloc.hip).
// ScratchFn gives the device's scratch buffer (device index in, pointer out);
// it is called once the arguments are valid and the device is set up, with
// that device current.  sum_dim_fixed is rd_sum_dim with that buffer, of
// scratch_bytes bytes, as the workspace: RD_ERR_WORKSPACE if the plan needs
// more; nothing allocated, the partial results combined by the second kernel.
typedef rd_status (*ScratchFn)(int device, float** ptr);
rd_status sum_dim_fixed(const float* x, int64_t outer, int64_t R, int64_t inner, float* out,
                        ScratchFn scratch, int64_t scratch_bytes, hipStream_t stream);
// Keeps e for rd_last_hip_error() on the calling thread.
void set_last_hip_error(hipError_t e);

// Which kernel shapes this build instantiates for an operator (rd_kernels.hip).
bool rows_shape_supported(int op, int group, int unroll);
bool cols_shape_supported(int op, int col_waves, int row_waves, int unroll);
bool small_shape_supported(int op, int unroll);

}  // namespace rd
