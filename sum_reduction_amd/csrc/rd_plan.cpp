// rd_plan.cpp -- how a reduction is cut into kernels (host logic, no HIP call).
//
// The pages size their grids from the SM count ("High-Performance Reduction
// Kernels" README, key design decisions: blocks = multiProcessorCount x
// max_blocks_per_SM) and worry that a grid of a few hundred blocks is too
// small for the chip (POPCORNBENCH problem-47 trace, grid sizing discussion).
//
// Measured on MI355X (256 CUs, HBM3E): a column reduction saturates HBM with
// every CU busy and a few waves per CU (about 8 MB of 16-byte loads in flight
// over the chip), so it is split along R only when its natural parallelism is
// below that.  Long rows read fastest as many short-lived workgroups, each
// streaming one piece of about 128 KB, rather than as a few long streams far
// apart in memory: the row planner cuts them into such pieces (and combines
// the piece results in a second pass).  Every path takes the streaming hint,
// which keeps a once-read stream from allocating in the caches (it was worth
// 10-15% on every path).
#include <string.h>

#include "rd_internal.h"

namespace rd {
namespace {

// Waves x loads-in-flight per lane to aim for, per CU (8 waves x 4 loads).
constexpr int64_t kLoadWavesPerCu = 32;
// Inputs in (kMidInputLo, kMidInputHi] bytes are cut into 8 pieces per CU.
constexpr int64_t kMidInputLo = int64_t(256) << 20;
constexpr int64_t kMidInputHi = int64_t(1) << 30;
// Few rows of at most kShallowMaxBytes take kShallowUnroll loads per step.
constexpr int64_t kShallowMaxBytes = int64_t(128) << 20;
constexpr int32_t kShallowUnroll = 4;
// Defaults measured on MI355X for the two kernels.
constexpr int kRowsUnrollBlock = 16;  // 256-lane groups
// Row pieces of about kPieceFloats floats (128 KB): long rows read by many
// workgroups of one such piece each, five resident per CU, move faster than
// by a few workgroups streaming far apart (measured on MI355X: the 1D sum of
// 1e9 floats 1.6 % faster than with one piece per CU, [100, 1e7] rows 27 %,
// [8192, 131072] 27 %; neutral at 1e8, where the pieces were already that
// short).  Rows that already give every CU a workgroup are cut only when the
// input reaches kPieceSplitBytes (at [1000, 100000], 400 MB, the second pass
// costs more than the pieces gain).  The softmax denominator's pieces are
// twice as long: its per-piece epilogue joins pairs, and 65536-float pieces
// measured best for it (1e9 floats: 576 us against 583 us with 32768; its
// [100, 1e7] rows 563 against 566 us).
constexpr int64_t kPieceFloats = 32768;
constexpr int64_t kPieceFloatsSoftmax = 65536;
constexpr int64_t kPieceSplitBytes = int64_t(1) << 30;
constexpr int kRowsUnrollWave = 8;    // 64-lane groups
constexpr int kColsUnroll = 4;
// Workgroups per CU for small-inner items of a single load step (a wave
// prefetches its next item).  Same box, A/B of 4, 8, 16, 64 and no cap:
// 64 was fastest on every such shape measured ([1048576, 256, 2] 408 ->
// 328 us, [2097152, 128, 2] 698 -> 514, [524288, 128, 4] 218 -> 182,
// [262144, 64, 8] 128 -> 115 against a wave per item).
constexpr int64_t kTinyItemBlocksPerCu = 64;
constexpr int kColsMaxColWaves = 8;
// Columns too few for single-wave tiles to give every CU a workgroup are cut
// into slabs of R; there, blocks of one tile and kColsSlabRowWaves waves
// taking turns on its rows, with no more blocks than CUs, beat wide tiles
// (measured on MI355X, us, wide 8-wave tiles in ~CU blocks -> one-wave tiles
// x 8 row waves in floor(CU / tiles) slabs: [1, 262144, 512] 301 -> 113,
// [2, 65536, 1024] 138 -> 95, [4, 8192, 2048] 67 -> 51, [1, 4096, 10922] 62
// -> 37, [1, 32768, 32768] 650 -> 622, [1, 1000000, 200] 136 -> 129; and a
// grid just past the CU count pays for a second round: [1, 4096, 10922] in
// 258 blocks 50 us against 37 in 215).
constexpr int kColsSlabRowWaves = 8;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// The streaming-hint choice: the tuning override's (1 = off, 2 = on) or the
// default.  False for an invalid request.
bool nontemporal_choice(const rd_tune* t, bool dflt, int32_t* out) {
    const int32_t v = t ? t->nontemporal : 0;
    if (v < 0 || v > 2) return false;
    *out = v == 0 ? int32_t(dflt) : int32_t(v == 2);
    return true;
}

// Bytes of one partial result: a float, or the softmax denominator's pair.
int64_t result_bytes(int op) {
    return int64_t(sizeof(float)) * (op == RD_OP_SOFTMAX_DENOM ? 2 : 1);
}

int32_t nxcd_for(int cu_count) {
    // MI355X: 8 XCDs of 32 CUs.  Only used to spread the workgroup numbering,
    // so a wrong guess costs locality, never correctness.
    return (cu_count >= 8 && cu_count % 8 == 0) ? 8 : 1;
}

rd_status plan_rows(int cu, int64_t outer, int64_t R, int op, const rd_tune* t,
                    rd_plan* p) {
    const bool forced = t && (t->group || t->unroll || t->split || t->order || t->combine);
    if (t && t->path) return RD_ERR_INVALID_ARG;  // inner == 1 has no column path
    if (R < kShortRow && !forced) {
        p->path = RD_PATH_ROWS_SHORT;
        p->block_threads = kBlock;
        p->group = 1;
        p->split = 1;
        p->passes = 1;
        p->blocks = ceil_div(outer, kBlock);
        if (p->blocks > kMaxBlocks) p->blocks = kMaxBlocks;
        return RD_OK;
    }
    p->path = RD_PATH_ROWS;
    p->block_threads = kBlock;
    p->group = (t && t->group) ? t->group : (R >= 4096 ? kBlock : kWave);
    p->unroll = (t && t->unroll) ? t->unroll
                                 : (p->group == kBlock ? kRowsUnrollBlock : kRowsUnrollWave);
    if (!rows_shape_supported(op, p->group, p->unroll)) return RD_ERR_INVALID_ARG;
    p->order = (t && t->order) ? t->order : RD_ORDER_BLOCKED;
    if (p->order != RD_ORDER_INTERLEAVED && p->order != RD_ORDER_BLOCKED)
        return RD_ERR_INVALID_ARG;
    if (!nontemporal_choice(t, true, &p->nontemporal)) return RD_ERR_INVALID_ARG;

    const int64_t nvec = R / 4;
    const int64_t groups_per_block = kBlock / p->group;
    // every lane gets at least one full unrolled step of loads
    int64_t cap = nvec / (int64_t(p->group) * p->unroll);
    if (cap < 1) cap = 1;
    const int64_t pieces =
        ceil_div(R, op == RD_OP_SOFTMAX_DENOM ? kPieceFloatsSoftmax : kPieceFloats);
    int64_t P = 1;
    if (t && t->split) {
        P = t->split;
        if (P < 1) return RD_ERR_INVALID_ARG;
    } else if (outer < int64_t(cu) * groups_per_block) {
        // fewer rows than one workgroup per CU: cut each row into pieces,
        // at least one per CU -- eight per CU for inputs between the
        // last-level cache's 256 MB and 1 GB, where the uneven finish of a
        // few long streams showed (n = 1e8 and 2e8 floats 6-9% faster with
        // 2048 pieces than 256) -- and pieces of at most about kPieceFloats
        const int64_t bytes = outer * R * int64_t(sizeof(float));
        const int64_t per_cu = (bytes > kMidInputLo && bytes <= kMidInputHi) ? 8 : 1;
        P = ceil_div(int64_t(cu) * per_cu * groups_per_block, outer);
        // A few rows too short to give every CU a piece at the default depth
        // (their pieces combined in the same launch), but long enough to at
        // a depth of 2 loads: the shallowest depth that does.  Measured on
        // MI355X, 1D sums, us: 1e6 floats 8.2 (61 pieces of depth 16) -> 7.1
        // (256 of depth 2), 4e6 8.6 (244, 16) -> 7.7 (256, 8); 1e7 keeps 306
        // pieces of 16.  The softmax denominator's shallowest built depth is
        // 8: 1e6 floats 13.3 (61 pieces of 16) -> 12.5 (122 of 8), 2e6 15.5
        // -> 12.6, 4e6 14.4 -> 13.5.
        if (!(t && t->unroll) && p->group == kBlock && outer <= kPubMaxRows &&
            nvec / (int64_t(p->group) * 2) >= P) {
            while (cap < P && p->unroll > 2 && rows_shape_supported(op, p->group, p->unroll / 2)) {
                p->unroll /= 2;
                cap = nvec / (int64_t(p->group) * p->unroll);
                if (cap < 1) cap = 1;
            }
        }
        // Up to kShallowMaxBytes, rows still at the default depth take 4
        // loads a step (pieces of the same length, more steps each): us,
        // same box, A/B, 70001 floats 8.8 -> 7.15 (17 pieces instead of 4),
        // 3e5 7.8 -> 7.15, 6e6 12.2 -> 11.55, 1e7 13.7 -> 13.0, 2e7 20.1 ->
        // 18.5; 3.4e7 and 4e7 level; [100, 3e5] 26.4 -> 24.4, [200, 1e5]
        // 21.5 -> 19.8, [5, 2e5] 9.1 -> 8.4, [8, 2e6] 15.1 -> 14.5, [32, 1e6]
        // and [10, 3e6] level.  (Where the rule above has already gone to 8
        // it stays: 4e6 8.4 at 8, 8.9 at 4.)
        if (!(t && t->unroll) && p->group == kBlock &&
            p->unroll == kRowsUnrollBlock && bytes <= kShallowMaxBytes &&
            rows_shape_supported(op, p->group, kShallowUnroll)) {
            p->unroll = kShallowUnroll;
            cap = nvec / (int64_t(p->group) * p->unroll);
            if (cap < 1) cap = 1;
        }
        if (P < pieces) P = pieces;
        if (P > cap) P = cap;
    } else if (pieces > 1 && outer * R >= kPieceSplitBytes / int64_t(sizeof(float))) {
        P = pieces < cap ? pieces : cap;
    }
    if (P > INT64_MAX / result_bytes(op) / outer) return RD_ERR_INVALID_ARG;
    p->split = P;
    const int64_t segs = outer * P;
    p->blocks = ceil_div(segs, groups_per_block);
    if (p->blocks > kMaxBlocks) p->blocks = kMaxBlocks;
    p->workspace_bytes = P > 1 ? segs * result_bytes(op) : 0;
    p->combine = RD_COMBINE_NONE;
    if (P > 1) {
        // A few rows (at most kPubWords piece words in all, two per softmax
        // pair):
        // the last workgroup combines the pieces in the same launch, from
        // results the others publish as tagged words (no fence, no counter;
        // launch_rows).  Measured on MI355X, us, second kernel -> one launch:
        // 1e6 floats 13.6 -> 7.8, 1e7 17.1 -> 11.6, 1e8 65.6 -> 63.2, [5,
        // 1000003] 14.2 -> 12.3.  More rows lose: the one workgroup combines
        // them one after another ([64, 262144]: 19.8 -> 69.3); so do more
        // pieces, whose words it reads a round at a time.  (A first version
        // published the results with a device-scope release, which writes back
        // an XCD's L2 -- about 47 ns per workgroup, serialized: 1e8 floats
        // 200 us.)  Since the second kernel's partial results live in the
        // stream's scratch (no pool allocation, ~5 us less), it wins again
        // from about a thousand piece words: us, one launch / two kernels,
        // same box, 1e6 floats (256 pieces) 7.4 / 8.5, 1e7 (306) 14.0 /
        // 14.1, 1e8 (3052) 64.4 / 62.8, [2, 2e7] (1222) 31.0 / 30.0, [4,
        // 2.5e7] (3052) 69.0 / 64.9: at most kPubRowsMaxWords words.
        const bool one = outer <= kPubMaxRows &&
                         (op == RD_OP_SOFTMAX_DENOM ? 2 : 1) * outer * P <= kPubRowsMaxWords;
        const int32_t c = (t && t->combine) ? t->combine
                                            : (one ? RD_COMBINE_LAST_BLOCK : RD_COMBINE_PASS);
        if (c != RD_COMBINE_PASS && c != RD_COMBINE_LAST_BLOCK) return RD_ERR_INVALID_ARG;
        p->combine = c;
    }
    p->passes = p->combine == RD_COMBINE_PASS ? 2 : 1;
    return RD_OK;
}

// Rows per slab for S slabs, and S again so that no slab is empty.
void split_rows(int64_t R, int64_t S, rd_plan* p) {
    if (S < 1) S = 1;
    if (S > R) S = R;
    const int64_t rps = ceil_div(R, S);
    p->rows_per_split = rps;
    p->split = ceil_div(R, rps);
}

// Columns: lanes along the contiguous inner axis.  inner is the width read
// per row and inner_out the outputs per outer index: the same for an array;
// a view whose kept inner axis has a small stride is read as the dense span
// of its rows (inner = (inner_out - 1) * stride + 1, the COLS kernel only).
rd_status plan_cols(int cu, int64_t outer, int64_t R, int64_t inner, int64_t inner_out,
                    int op, const rd_tune* t, rd_plan* p) {
    const int32_t forced = t ? t->path : 0;
    if (forced && forced != RD_PATH_COLS && forced != RD_PATH_COLS_SMALL)
        return RD_ERR_INVALID_ARG;
    if (inner != inner_out && (forced == RD_PATH_COLS_SMALL || inner <= kSmallInner))
        return RD_ERR_INVALID_ARG;
    if (forced == RD_PATH_COLS && inner < 4) return RD_ERR_INVALID_ARG;
    if (forced == RD_PATH_COLS_SMALL && inner > 2 * kSmallInner) return RD_ERR_INVALID_ARG;
    if (forced == RD_PATH_COLS_SMALL || (!forced && inner <= kSmallInner)) {
        // several adjacent rows per load instruction; a wave per item
        // (outer index, slab of R), the split along R only for few items
        p->path = RD_PATH_COLS_SMALL;
        p->block_threads = kBlock;
        p->unroll = (t && t->unroll) ? t->unroll : kColsUnroll;
        // few items, cut into slabs: twice the rows in flight per wave and
        // half the slabs (where that shape is built) -- [1, 2^28, 4] 771 ->
        // 699 us, [16, 4194304, 7] 303 -> 288 us on one box
        if (!(t && t->unroll) && outer < int64_t(cu) * kLoadWavesPerCu / kColsUnroll &&
            small_shape_supported(op, 2 * kColsUnroll))
            p->unroll = 2 * kColsUnroll;
        if (!small_shape_supported(op, p->unroll)) return RD_ERR_INVALID_ARG;
        if (!nontemporal_choice(t, true, &p->nontemporal)) return RD_ERR_INVALID_ARG;
        if (t && t->combine && t->combine != RD_COMBINE_PASS) return RD_ERR_INVALID_ARG;
        const int64_t lc = ceil_div(inner, 4);
        const int64_t rpw = kWave / lc;
        const int64_t waves_per_block = kBlock / kWave;
        const int64_t want = int64_t(cu) * kLoadWavesPerCu / p->unroll;  // waves
        int64_t S = 1;
        if (t && t->split) {
            S = t->split;
        } else if (outer < want) {
            S = ceil_div(want, outer);
            // every lane keeps at least one full unrolled step of rows per slab
            int64_t cap = R / (rpw * p->unroll);
            if (cap < 1) cap = 1;
            if (S > cap) S = cap;
        }
        if (S < 1) return RD_ERR_INVALID_ARG;
        split_rows(R, S, p);
        if (p->split > INT64_MAX / result_bytes(op) / (outer * inner)) return RD_ERR_INVALID_ARG;
        p->blocks = ceil_div(p->split * outer, waves_per_block);
        // items of one load step each: a wave takes many in turn, each
        // item's loads issued while the one before is joined and stored --
        // except full single steps of 12-byte rows, which measured faster
        // a wave per item ([1048576, 256, 3]: 434 us against 503; yet
        // [4194304, 32, 3], a partial step, 1209 -> 1031 us)
        const bool one_step = p->rows_per_split <= rpw * p->unroll;
        const bool full_step_of_3 = inner == 3 && p->rows_per_split == rpw * p->unroll;
        if (one_step && !full_step_of_3 && p->blocks > int64_t(cu) * kTinyItemBlocksPerCu)
            p->blocks = int64_t(cu) * kTinyItemBlocksPerCu;
        if (p->blocks > kMaxBlocks) p->blocks = kMaxBlocks;
        p->passes = p->split > 1 ? 2 : 1;
        p->combine = p->split > 1 ? RD_COMBINE_PASS : RD_COMBINE_NONE;
        p->workspace_bytes = p->split > 1 ? p->split * outer * inner * result_bytes(op) : 0;
        return RD_OK;
    }
    p->path = RD_PATH_COLS;
    const int64_t lane_cols = ceil_div(inner, 4);
    // Wide tiles: every tile edge inside a row is a cache line that two
    // workgroups fetch.  Take the widest tile the row has columns for (up to
    // 8 waves) that still gives every CU a workgroup; if no width does, the
    // split along R fills the chip (kColsSlabRowWaves).
    int32_t widest = kColsMaxColWaves;
    while (widest > 1 && lane_cols <= int64_t(widest / 2) * kWave) widest /= 2;
    int32_t cw = widest;
    while (cw > 1 && ceil_div(lane_cols, int64_t(cw) * kWave) * outer < cu) cw /= 2;
    int32_t rw = 1;
    // even single-wave tiles leave CUs without a workgroup: R is cut into
    // slabs, each block one tile with row waves (widest tiles if that shape
    // is not built for op)
    const bool slabs = ceil_div(lane_cols, int64_t(cw) * kWave) * outer < cu;
    if (slabs) {
        if (cols_shape_supported(op, 1, kColsSlabRowWaves, kColsUnroll))
            rw = kColsSlabRowWaves;
        else
            cw = widest;
    }
    const bool own_shape = !(t && (t->col_waves || t->row_waves || t->unroll));
    p->col_waves = (t && t->col_waves) ? t->col_waves : cw;
    p->row_waves = (t && t->row_waves) ? t->row_waves : rw;
    p->unroll = (t && t->unroll) ? t->unroll : kColsUnroll;
    if (!cols_shape_supported(op, p->col_waves, p->row_waves, p->unroll))
        return RD_ERR_INVALID_ARG;
    if (!nontemporal_choice(t, true, &p->nontemporal)) return RD_ERR_INVALID_ARG;
    p->block_threads = kWave * p->col_waves * p->row_waves;

    const int64_t tiles = ceil_div(lane_cols, int64_t(kWave) * p->col_waves);
    const int64_t base = tiles * outer;  // workgroups without a split
    int64_t S = 1;
    if (t && t->split) {
        S = t->split;
    } else if (slabs && own_shape && rw > 1) {
        // as many slabs as keep the blocks within one per CU, each with at
        // least one full step of U rows per row wave
        S = cu / base > 1 ? cu / base : 1;
        int64_t cap = R / (int64_t(rw) * p->unroll);
        if (cap < 1) cap = 1;
        if (S > cap) S = cap;
    } else {
        // loads in flight over the chip without a split, in lane-waves x U:
        // base * per, compared as base < ceil(want / per) so that the
        // product is only formed when it is small
        const int64_t per = int64_t(p->col_waves) * p->row_waves * p->unroll;
        const int64_t want = int64_t(cu) * kLoadWavesPerCu;
        if (base < ceil_div(want, per) || base < cu) {
            S = base < ceil_div(want, per) ? ceil_div(want, base * per) : 1;
            const int64_t fill = ceil_div(cu, base);
            if (S < fill) S = fill;
            // every wave keeps at least one full unrolled step of rows per slab
            int64_t cap = R / (int64_t(p->row_waves) * p->unroll);
            if (cap < 1) cap = 1;
            if (S > cap) S = cap;
        }
    }
    if (S < 1) return RD_ERR_INVALID_ARG;
    split_rows(R, S, p);
    if (p->split > INT64_MAX / result_bytes(op) / (outer * inner_out)) return RD_ERR_INVALID_ARG;
    p->blocks = base * p->split;
    if (p->blocks > kMaxBlocks) p->blocks = kMaxBlocks;
    p->combine = RD_COMBINE_NONE;
    if (p->split > 1) {
        // A few slabs of one-wave tiles, a workgroup per item and no more
        // workgroups than CUs: the last slab's workgroups join the others'
        // published results in the same launch (cols_kernel), which saves the
        // second kernel and the gap before it.  Limited to kPubColMaxSlabs,
        // as many as the last slab's waves fetch in two rounds.
        const bool one = op != RD_OP_SOFTMAX_DENOM && p->col_waves == 1 && p->row_waves > 1 &&
                         p->split <= kPubColMaxSlabs && p->blocks == base * p->split &&
                         p->blocks <= cu && (p->split - 1) * outer * inner_out <= kPubColWords;
        const int32_t c = (t && t->combine) ? t->combine
                                            : (one ? RD_COMBINE_LAST_BLOCK : RD_COMBINE_PASS);
        if (c != RD_COMBINE_PASS && !(c == RD_COMBINE_LAST_BLOCK && one))
            return RD_ERR_INVALID_ARG;
        p->combine = c;
    }
    p->passes = p->combine == RD_COMBINE_PASS ? 2 : 1;
    p->workspace_bytes = p->split > 1 ? p->split * outer * inner_out * result_bytes(op) : 0;
    return RD_OK;
}

// No unit stride: a lane per (slab, output).  Few outputs are split along R
// into slabs until about kStridedLanesPerCu lanes per CU are busy, each slab
// keeping at least kStridedMinRows rows.
constexpr int64_t kStridedLanesPerCu = 1024;
constexpr int64_t kStridedMinRows = 32;

rd_status plan_strided(int cu, int64_t outer, int64_t R, int64_t inner, int op,
                       const rd_tune* t, rd_plan* p) {
    if (t && (t->path || t->group || t->col_waves || t->row_waves || t->unroll || t->order ||
              t->combine))
        return RD_ERR_INVALID_ARG;
    const int64_t n = outer * inner;
    int64_t S = 1;
    if (t && t->split) {
        S = t->split;
    } else {
        const int64_t want = int64_t(cu) * kStridedLanesPerCu;
        if (n < want) {
            S = ceil_div(want, n);
            int64_t cap = R / kStridedMinRows;
            if (cap < 1) cap = 1;
            if (S > cap) S = cap;
        }
    }
    if (S < 1) return RD_ERR_INVALID_ARG;
    split_rows(R, S, p);
    if (p->split > INT64_MAX / result_bytes(op) / n) return RD_ERR_INVALID_ARG;
    p->path = RD_PATH_STRIDED;
    p->block_threads = kBlock;
    p->blocks = ceil_div(p->split * n, kBlock);
    if (p->blocks > kMaxBlocks) p->blocks = kMaxBlocks;
    p->passes = p->split > 1 ? 2 : 1;
    p->combine = p->split > 1 ? RD_COMBINE_PASS : RD_COMBINE_NONE;
    p->workspace_bytes = p->split > 1 ? p->split * n * result_bytes(op) : 0;
    return RD_OK;
}

}  // namespace

// Sizes of a view are valid when its furthest element, in bytes, and the
// outer*R*inner*4 bytes a contiguous copy would take are representable.
bool view_sizes_ok(const Strides& v) {
    if (v.outer < 0 || v.R < 0 || v.inner < 0 || v.so < 0 || v.sr < 0 || v.si < 0)
        return false;
    const int64_t lim = INT64_MAX / 4;
    if (v.outer && v.R && v.inner) {
        if (v.R > lim / v.outer || v.inner > lim / (v.outer * v.R)) return false;
    } else if (v.outer && v.inner && v.inner > lim / v.outer) {
        return false;
    }
    if (v.outer == 0 || v.R == 0 || v.inner == 0) return true;
    // (outer-1)*so + (R-1)*sr + (inner-1)*si must stay below lim
    int64_t left = lim;
    const int64_t n[3] = {v.outer - 1, v.R - 1, v.inner - 1};
    const int64_t st[3] = {v.so, v.sr, v.si};
    for (int k = 0; k < 3; ++k) {
        if (n[k] == 0 || st[k] == 0) continue;
        if (st[k] > left / n[k]) return false;
        left -= n[k] * st[k];
    }
    return true;
}

bool dense_columns(const Strides& v) {
    if (!(v.inner > 1 && v.si >= 2 && v.si <= kDenseColumnStride)) return false;
    const int64_t span = (v.inner - 1) * v.si + 1;
    // rows whose spans overlap (a transposed array, stride_r < span) would
    // read the same lines once per row: those keep the lane-per-output kernels
    return span > kSmallInner && (v.R == 1 || v.sr >= span);
}

void normalize_view(Strides* v) {
    // strides of axes of length 1 never move: give them the unit value
    if (v->inner == 1) v->si = 1;
    if (v->R == 1) v->sr = 1;
    if (v->outer == 1) v->so = 0;
    // a single kept axis whose elements are adjacent (outputs o at so == 1)
    // and a strided reduced axis: the same as a column reduction of
    // [1, R, outer], whose outputs keep their order
    if (v->inner == 1 && v->sr != 1 && v->so == 1 && v->outer > 1) {
        *v = Strides{1, v->R, v->outer, 0, v->sr, 1};
    }
}

rd_status plan_view(int cu_count, Strides* v, int op, const rd_tune* tune, rd_plan* plan) {
    if (!plan || !v || cu_count < 1 || !view_sizes_ok(*v)) return RD_ERR_INVALID_ARG;
    if (op < RD_OP_SUM || op > RD_OP_SOFTMAX_DENOM) return RD_ERR_INVALID_ARG;
    memset(plan, 0, sizeof(*plan));
    normalize_view(v);
    const int64_t outer = v->outer, R = v->R, inner = v->inner;
    plan->nxcd = nxcd_for(cu_count);
    plan->split = 1;
    plan->passes = 1;
    if (outer == 0 || inner == 0) {
        plan->path = RD_PATH_NONE;
        plan->passes = 0;
        return RD_OK;
    }
    if (R == 0) {
        plan->path = RD_PATH_ZERO;
        plan->block_threads = kBlock;
        plan->blocks = (outer * inner + kBlock - 1) / kBlock;
        if (plan->blocks > kMaxBlocks) plan->blocks = kMaxBlocks;
        return RD_OK;
    }
    if (inner == 1 && v->sr == 1) return plan_rows(cu_count, outer, R, op, tune, plan);
    if (inner > 1 && v->si == 1)
        return plan_cols(cu_count, outer, R, inner, inner, op, tune, plan);
    // the reduced axis contiguous, the kept ones strided: outer*inner rows
    if (v->sr == 1) return plan_rows(cu_count, outer * inner, R, op, tune, plan);
    // the kept inner axis a few floats apart: every cache line of a row's
    // span holds a term, so the dense span is read with the column kernel
    // (the same lines, in 16-byte loads) and every si-th column kept
    if (dense_columns(*v)) {
        const int64_t span = (inner - 1) * v->si + 1;
        if (!(tune && tune->path == RD_PATH_COLS_SMALL))
            return plan_cols(cu_count, outer, R, span, inner, op, tune, plan);
    }
    return plan_strided(cu_count, outer, R, inner, op, tune, plan);
}

rd_status plan_dim(int cu_count, int64_t outer, int64_t R, int64_t inner, int op,
                   const rd_tune* tune, rd_plan* plan) {
    if (!plan || cu_count < 1 || outer < 0 || R < 0 || inner < 0)
        return RD_ERR_INVALID_ARG;
    // outer * R * inner * 4 must be representable
    const int64_t lim = INT64_MAX / 4;
    if (outer && R && inner) {
        if (R > lim / outer || inner > lim / (outer * R)) return RD_ERR_INVALID_ARG;
    } else if (outer && inner && inner > lim / outer) {
        return RD_ERR_INVALID_ARG;
    }
    Strides v{outer, R, inner, R * inner, inner, 1};
    return plan_view(cu_count, &v, op, tune, plan);
}

namespace {

// The lane-per-column scan.  Views whose unit-stride side the lanes do not
// follow (inner == 1: the outputs are staged; stride_r == 1: the inputs) run
// in blocks of kStageWaves waves on kStageCols columns, which take turns on a
// slab's row chunks; columns are split along R into slabs (totals, their
// scan, the scan from the carries: x read twice) only when there are fewer
// than two such blocks per CU, with slabs of at least one round of the block
// (kStageWaves x 32 rows).  (The transposed [32768, 32768] array, 32768
// columns: 512 blocks, one pass.)  Other views take a lane per (slab,
// column), 256 columns a workgroup, split until about kStridedLanesPerCu
// lanes per CU are busy, each slab keeping at least kStridedMinRows rows.
constexpr int64_t kStageCols = 64;
constexpr int64_t kStageRound = 4 * 32;

rd_status plan_scan_strided(int64_t cu, const Strides& v, const rd_tune* t, rd_plan* p) {
    if (t && (t->group || t->col_waves || t->unroll || t->order || t->combine))
        return RD_ERR_INVALID_ARG;
    const int64_t outer = v.outer, R = v.R, inner = v.inner;
    const int64_t n = outer * inner;
    const bool staged = inner == 1 || v.sr == 1;
    // Between half a group of 64 columns per CU and enough single lanes for
    // the chip: one pass, row waves taking turns (scan_strided_rounds_kernel)
    // where slabs would read x twice.  Measured on MI355X: x[::8, ::3] of
    // [32768, 32768] (10922 columns, 171 groups), cumsum along dim 0:
    // 300 us in 25 slabs of a lane per column, 164 us in 8-wave rounds.
    const int64_t groups = ceil_div(n, kWave);
    int32_t rw = 1;
    if (t && t->row_waves) {
        rw = t->row_waves;
        if (staged || (rw != 2 && rw != 4 && rw != 8) || (t->split && t->split != 1))
            return RD_ERR_INVALID_ARG;
    } else if (!staged && !(t && t->split) && 2 * groups >= cu &&
               n < cu * kStridedLanesPerCu) {
        rw = 2;
        while (rw < kStridedRoundsMaxRowWaves && groups * rw < kStridedRoundsWavesPerCu * cu)
            rw *= 2;
    }
    if (rw > 1) {
        p->path = RD_PATH_SCAN_STRIDED;
        p->nontemporal = 0;  // neighbouring lanes share lines: keep them cached
        p->row_waves = rw;
        p->unroll = kStridedRoundsUnroll;
        p->block_threads = rw * kWave;
        p->blocks = groups < kMaxBlocks ? groups : kMaxBlocks;
        p->split = 1;
        p->rows_per_split = R;
        return RD_OK;
    }
    const int64_t cols = staged ? kStageCols : kBlock;  // columns per workgroup
    const int64_t nblk = ceil_div(n, cols);
    int64_t S = 1;
    if (t && t->split) {
        S = t->split;
    } else if (staged ? nblk < 2 * cu : n < cu * kStridedLanesPerCu) {
        S = staged ? ceil_div(2 * cu, nblk) : ceil_div(cu * kStridedLanesPerCu, n);
        int64_t cap = R / (staged ? kStageRound : kStridedMinRows);
        if (cap < 1) cap = 1;
        if (S > cap) S = cap;
    }
    if (S < 1) return RD_ERR_INVALID_ARG;
    split_rows(R, S, p);
    if (p->split > INT64_MAX / 8 / n) return RD_ERR_INVALID_ARG;
    p->path = RD_PATH_SCAN_STRIDED;
    p->nontemporal = 0;  // neighbouring lanes and rows share lines: keep them cached
    p->block_threads = kBlock;
    p->blocks = p->split * nblk;  // a workgroup per (slab, columns)
    if (p->blocks > kMaxBlocks) p->blocks = kMaxBlocks;
    if (p->split > 1) {
        p->passes = 3;
        p->combine = RD_COMBINE_PASS;
        p->workspace_bytes = 2 * p->split * n * int64_t(sizeof(float));
    }
    return RD_OK;
}

}  // namespace

rd_status plan_cumsum_view(int cu_count, Strides* v, const rd_tune* t, rd_plan* p) {
    if (!p || !v || cu_count < 1 || !view_sizes_ok(*v)) return RD_ERR_INVALID_ARG;
    memset(p, 0, sizeof(*p));
    // strides of axes of length 1 never move (the output is laid out in the
    // view's own order, so no axes are exchanged as for reductions)
    if (v->inner == 1) v->si = 1;
    if (v->R == 1) v->sr = 1;
    if (v->outer == 1) v->so = 0;
    const int64_t outer = v->outer, R = v->R, inner = v->inner;
    p->nxcd = nxcd_for(cu_count);
    p->split = 1;
    if (outer == 0 || R == 0 || inner == 0) {
        p->path = RD_PATH_NONE;
        return RD_OK;
    }
    if (!nontemporal_choice(t, true, &p->nontemporal)) return RD_ERR_INVALID_ARG;
    p->block_threads = kBlock;
    p->passes = 1;
    const int64_t cu = cu_count;
    const int32_t forced = t ? t->path : 0;
    const bool rows_ok = inner == 1 && v->sr == 1;
    const bool cols_ok = inner > 1 && v->si == 1;
    // (a kept inner axis of terms a few floats apart is not scanned over the
    // dense span of its rows as the reductions do: x[::8, ::3] of [32768,
    // 32768], whose 128 tiles need slabs, took 0.39 ms so against 0.30 ms
    // with a lane per column, measured on MI355X)
    if (forced == RD_PATH_SCAN_STRIDED || (!rows_ok && !cols_ok))
        return forced && forced != RD_PATH_SCAN_STRIDED
                   ? RD_ERR_INVALID_ARG
                   : plan_scan_strided(cu, *v, t, p);
    if (inner == 1 ? (forced && forced != RD_PATH_SCAN_ROWS)
                   : (forced && forced != RD_PATH_SCAN_COLS && forced != RD_PATH_SCAN_COLS_SMALL))
        return RD_ERR_INVALID_ARG;
    if (forced == RD_PATH_SCAN_COLS_SMALL && inner > 2 * kSmallInner) return RD_ERR_INVALID_ARG;
    if (inner == 1) {
        // a wave or a workgroup per row piece; pieces only for few long rows
        // (then: piece totals, their scan, the scan from the carries -- x is
        // read twice)
        p->path = RD_PATH_SCAN_ROWS;
        const int32_t comb = t ? t->combine : 0;
        if (comb != 0 && comb != RD_COMBINE_PASS && comb != RD_COMBINE_LOOKBACK)
            return RD_ERR_INVALID_ARG;
        // The look-back kernel (one launch, x read once, pieces taken in
        // ticket order) for long rows among few -- at least kScanRowsLookMinR
        // positions, fewer than kScanRowWavesMin rows per CU,
        // kScanRowsLookMinN elements in all -- and for every large array of
        // rows of at least one 8-wave chunk (kScanRowsTicketMinBytes; half of
        // that for rows of whole 32768-position pieces).
        // Pieces of 32768 positions (16 waves) for the long rows and for rows
        // made of whole such pieces, else of 16384 (8 waves): a row's partial
        // last piece idles fewer lanes in a smaller workgroup (measured on
        // MI355X, us, 8 / 16 waves: [53687, 20000] 1456 / 1882, [40000,
        // 24000] 1281 / 1524, [65536, 16384] 1359 / 2148; whole pieces:
        // [8192, 32768] 365 / 348, [2048, 131072] 369 / 356).
        const int64_t chunk8 = int64_t(8) * kWave * 4 * kScanRowsChunkSlices;
        const int64_t chunk16 = 2 * chunk8;
        const bool tuned = t && (t->split || t->order || t->group || t->unroll);
        const bool few_long = outer < cu * kScanRowWavesMin && R >= kScanRowsLookMinR &&
                              outer * R >= kScanRowsLookMinN;
        const bool large = R >= chunk8 && outer * R * int64_t(sizeof(float)) >=
                                              (R % chunk16 == 0 ? kScanRowsTicketMinBytes / 2
                                                                : kScanRowsTicketMinBytes);
        // fewer rows than a third of the CUs, each of two or more 32768-position
        // chunks: the look-back in place of the three-kernel scheme
        const bool few = 3 * outer < cu && R >= kScanRowsLookFewMinR;
        // (arrays of at most kScanRowsLookSmallN elements: 8-wave pieces, twice
        // as many workgroups)
        const int32_t look_group =
            (few_long || R % chunk16 == 0) && !(few && !large && outer * R <= kScanRowsLookSmallN)
                ? 16 * kWave
                : 8 * kWave;
        const bool look =
            comb == RD_COMBINE_LOOKBACK ||
            (comb == 0 && !tuned && (few_long || large || few) &&
             ceil_div(R, int64_t(look_group / kWave) * kWave * 4 * kScanRowsChunkSlices) <=
                 kMaxBlocks / outer);
        if (look) {
            // one launch, a workgroup of 4, 8 or 16 waves per piece of one
            // block chunk (4 or 8 slices a wave), the carries by look-back
            if (t && (t->split || t->order || (t->unroll && t->unroll != 4 && t->unroll != 8)))
                return RD_ERR_INVALID_ARG;
            const int32_t group = (t && t->group) ? t->group : look_group;
            const int32_t slices = (t && t->unroll) ? t->unroll : kScanRowsChunkSlices;
            if (group != 4 * kWave && group != 8 * kWave && group != 16 * kWave)
                return RD_ERR_INVALID_ARG;
            const int64_t L = int64_t(group / kWave) * kWave * 4 * slices;
            const int64_t P = ceil_div(R, L);
            if (P > kMaxBlocks / outer) return RD_ERR_INVALID_ARG;
            p->unroll = slices;
            p->group = group;
            p->block_threads = group;
            p->split = P;
            p->rows_per_split = L;
            p->blocks = outer * P;
            p->combine = RD_COMBINE_LOOKBACK;
            p->workspace_bytes = lookback_workspace_bytes(outer, P);
            return RD_OK;
        }
        p->unroll = (t && t->unroll) ? t->unroll : kScanRowsChunkSlices;
        if (p->unroll != 4 && p->unroll != 8) return RD_ERR_INVALID_ARG;
        if (t && t->group && t->group != kWave && t->group != kBlock &&
            t->group != 2 * kBlock && t->group != 4 * kBlock)
            return RD_ERR_INVALID_ARG;
        const int64_t tiles = ceil_div(R, kScanTile);
        int64_t P = 1;
        if (t && t->split) {
            P = t->split;
        } else if (3 * outer < cu && R >= kScanRowsCutMinR) {
            P = ceil_div(cu * kScanRowWavesSplit, outer);
        }
        if (P < 1) return RD_ERR_INVALID_ARG;
        if (P > tiles) P = tiles;
        const int64_t L = ceil_div(tiles, P) * kScanTile;
        P = ceil_div(R, L);
        p->split = P;
        p->rows_per_split = L;
        // long uncut rows: a workgroup per row (adjacent waves on adjacent
        // stretches of it) -- 8 waves, 16 for rows of two of their chunks or
        // more; with 4-slice chunks (kernels built for 8 waves a SIMD, where
        // wider workgroups spill) 4 waves --; uncut rows of more than a tile
        // among few rows: 4 waves; else a wave per item
        int32_t group = kWave;
        if (P == 1 && R > kScanRowsBlockMinR)
            group = p->unroll == 4 ? kBlock : R >= kScanRowsWideMinR ? 16 * kWave : 8 * kWave;
        else if (P == 1 && R > kScanTile && outer < cu * kScanRowWavesMin)
            group = kBlock;
        p->group = (t && t->group) ? t->group : group;
        // interleaved: persistent workgroups, each streaming the chunks of
        // rows b, b + blocks, ... (whole rows, a workgroup per row only)
        p->order = (t && t->order) ? t->order : 0;
        if (p->order && (p->order != RD_ORDER_INTERLEAVED || p->group == kWave || P != 1))
            return RD_ERR_INVALID_ARG;
        // a workgroup of 256 threads holds 4 wave items; a wider group is one
        // workgroup per item
        int64_t b = p->group == kWave ? ceil_div(outer * P, kBlock / kWave) : outer * P;
        if (p->order == RD_ORDER_INTERLEAVED) {
            // as many workgroups as the CUs hold at once: 4 SIMDs x the
            // waves a SIMD the kernel is built for, over the workgroup's waves
            const int64_t per_cu = 4 * int64_t(p->unroll == 4 ? 8 : 4) / (p->group / kWave);
            const int64_t resident = cu * (per_cu > 0 ? per_cu : 1);
            if (resident < b) b = resident;
        }
        p->blocks = b < kMaxBlocks ? b : kMaxBlocks;
        p->block_threads = p->group == kWave ? kBlock : p->group;
        if (P > 1) {
            p->passes = 3;
            p->combine = RD_COMBINE_PASS;
            p->workspace_bytes = 2 * outer * P * int64_t(sizeof(float));
        }
        return RD_OK;
    }
    if (forced == RD_PATH_SCAN_COLS_SMALL || (!forced && inner <= kSmallInner)) {
        // several rows per load instruction, a wave per (outer index, slab);
        // slabs when there are fewer than kScanSmallWavesPerCu waves per CU
        p->path = RD_PATH_SCAN_COLS_SMALL;
        p->unroll = (t && t->unroll) ? t->unroll : kScanSmallUnroll;
        if (p->unroll != 4 && p->unroll != 8) return RD_ERR_INVALID_ARG;
        const int64_t lc = inner >= 4 ? ceil_div(inner, 4) : 1;
        const int64_t rpw = kWave / lc;
        const int64_t want = cu * kScanSmallWavesPerCu;
        int64_t S = 1;
        if (t && t->split) {
            S = t->split;
        } else if (outer < want) {
            S = ceil_div(want, outer);
            // every slab keeps at least two full steps of loads
            int64_t cap = R / (2 * rpw * p->unroll);
            if (cap < 1) cap = 1;
            if (S > cap) S = cap;
        }
        if (S < 1) return RD_ERR_INVALID_ARG;
        split_rows(R, S, p);
        const int64_t b = ceil_div(p->split * outer, kBlock / kWave);
        p->blocks = b < kMaxBlocks ? b : kMaxBlocks;
        if (p->split > 1) {
            if (p->split > INT64_MAX / 8 / (outer * inner)) return RD_ERR_INVALID_ARG;
            p->passes = 3;
            p->combine = RD_COMBINE_PASS;
            p->workspace_bytes = 2 * p->split * outer * inner * int64_t(sizeof(float));
        }
        return RD_OK;
    }
    // a lane per 4 columns (per row of 2 or 3), a wave per 64 lane-columns;
    // slabs of R (totals, their scan, the scan from the carries: x is read
    // twice) only when there are fewer waves than CUs.  Measured on MI355X:
    // [16, 8192, 4096] (256 waves) 1074 us cut into 8 slabs of 8-wave
    // blocks, 713 us in one pass of single-wave blocks; [64, 512, 1024] 75 ->
    // 65 us; [1, 65536, 8192] (32 waves) 1171 -> 991 us in 8 slabs of
    // single-wave blocks.
    p->path = RD_PATH_SCAN_COLS;
    p->unroll = (t && t->unroll) ? t->unroll : kScanColsUnroll;
    if (p->unroll != 4 && p->unroll != 8 && p->unroll != 16) return RD_ERR_INVALID_ARG;
    const int64_t lane_cols = inner >= 4 ? ceil_div(inner, 4) : 1;
    const int64_t tiles = ceil_div(lane_cols, kWave);
    const int64_t waves = tiles * outer;
    // Between half and twice as many tiles (x outer) as CUs: a block per
    // tile whose rw waves take turns on its row groups (one pass), the fewest
    // that make about kScanColsRoundWavesPerCu waves per CU, at most
    // kScanColsMaxRowWaves (each block runs on one CU, so fewer tiles than
    // half the CUs would leave most of them idle: slabs then).  Measured on
    // MI355X: [1, 16384, 32768] (128 tiles) 1063 us in 2 slabs, 849 us with 8
    // row waves; [3, 16384, 16384] 1552 -> 1060 us (8); [64, 512, 1024] 64 ->
    // 50 us (4); [16, 8192, 4096] 707 us with single waves, 704 with 4.
    int32_t rw = 1;
    if (t && t->row_waves) {
        rw = t->row_waves;
        if (rw != 1 && rw != 2 && rw != 4 && rw != 8 && rw != 16) return RD_ERR_INVALID_ARG;
        if (rw > 1 && (inner < 4 || (t->col_waves && t->col_waves != 1)))
            return RD_ERR_INVALID_ARG;
    } else if (2 * waves >= cu && waves < 2 * cu && inner >= 4 &&
               !(t && (t->split || t->col_waves))) {
        while (rw < kScanColsMaxRowWaves && waves * rw < kScanColsRoundWavesPerCu * cu) rw *= 2;
    }
    int64_t S = 1;
    if (t && t->split) {
        S = t->split;
    } else if (2 * waves < cu && rw == 1 && inner >= 4 &&
               !(t && (t->col_waves || t->row_waves || t->unroll))) {
        // few tiles: slabs (the blocks within one per CU, at least a round
        // of kScanSlabRowWaves groups of U rows each) scanned in row rounds,
        // or by single waves for rows a multiple of 8 KB apart (from 16 KB)
        const int64_t sr = v->sr;
        const bool lock = sr >= 2 * kScanSlabLockStride && sr % kScanSlabLockStride == 0;
        rw = lock ? 1 : kScanSlabRowWaves;
        S = cu / waves;
        int64_t cap = R / (int64_t(kScanSlabRowWaves) * p->unroll);
        if (cap < 1) cap = 1;
        if (S > cap) S = cap;
    } else if (waves < cu && rw == 1) {
        S = ceil_div(cu, waves);
        int64_t cap = R / 64;
        if (cap < 1) cap = 1;
        if (S > cap) S = cap;
    }
    if (S < 1) return RD_ERR_INVALID_ARG;
    split_rows(R, S, p);
    // slabs of at least kScanColsDeepRows rows keep 16 rows in flight (the
    // row-round blocks take groups of 8)
    if (!(t && t->unroll) && rw == 1 && p->rows_per_split >= kScanColsDeepRows) p->unroll = 16;
    if (rw > 1 && p->unroll != 4 && p->unroll != 8) return RD_ERR_INVALID_ARG;
    p->row_waves = rw;
    // a block per (col_waves adjacent tiles, slab, outer index): the widest
    // of 16, 8, 4, 2, 1 tiles that still gives every CU a block (wide blocks
    // share fewer tile edges; [128, 4096, 4095]: 8 tiles, 3322 us against
    // 3960 with single-wave blocks)
    if (rw > 1) {
        p->col_waves = 1;
    } else if (t && t->col_waves) {
        p->col_waves = t->col_waves;
        if (p->col_waves != 4 && p->col_waves != 8 && p->col_waves != 16 &&
            !((p->col_waves == 1 || p->col_waves == 2) && inner >= 4))
            return RD_ERR_INVALID_ARG;
    } else {
        p->col_waves = inner >= 4 ? 1 : 4;
        for (int bw = 16; bw > p->col_waves; bw /= 2) {
            if (tiles >= bw && ceil_div(tiles, bw) * p->split * outer >= cu) {
                p->col_waves = bw;
                break;
            }
        }
    }
    p->block_threads = p->col_waves * rw * kWave;
    const int64_t block_items = ceil_div(tiles, p->col_waves) * p->split * outer;
    p->blocks = block_items < kMaxBlocks ? block_items : kMaxBlocks;
    if (p->split > 1) {
        if (p->split > INT64_MAX / 8 / (outer * inner)) return RD_ERR_INVALID_ARG;
        p->passes = 3;
        p->combine = RD_COMBINE_PASS;
        p->workspace_bytes = 2 * p->split * outer * inner * int64_t(sizeof(float));
    }
    return RD_OK;
}

rd_status plan_cumsum(int cu_count, int64_t outer, int64_t R, int64_t inner,
                      const rd_tune* t, rd_plan* p) {
    if (!p || cu_count < 1 || outer < 0 || R < 0 || inner < 0) return RD_ERR_INVALID_ARG;
    // outer * R * inner * 4 must be representable
    const int64_t lim = INT64_MAX / 4;
    if (outer && R && inner) {
        if (R > lim / outer || inner > lim / (outer * R)) return RD_ERR_INVALID_ARG;
    } else if (outer && inner && inner > lim / outer) {
        return RD_ERR_INVALID_ARG;
    }
    Strides v{outer, R, inner, R * inner, inner, 1};
    return plan_cumsum_view(cu_count, &v, t, p);
}

}  // namespace rd
