// Host-only fuzz of the launch planner (sum_reduction_amd/csrc/rd_plan.cpp),
// built with g++ under AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_plan_sanitized.py.  Random shapes (zeros, ones, small, huge,
// near the int64 limits), strides, operators and tuning overrides go
// through plan_view, plan_cumsum and plan_cumsum_view; every accepted plan
// must satisfy the
// invariants the launchers rely on.  Any signed overflow, out-of-bounds
// access or failed invariant ends the run with a nonzero status.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <random>

#include "rd_internal.h"

// Kernel-shape tables live with the kernels (rd_kernels.hip, not built
// here); every shape counts as built, so tuning requests reach the sizing.
namespace rd {
bool rows_shape_supported(int, int group, int unroll) {
    return (group == 64 || group == 256) && unroll > 0 && unroll <= 16;
}
bool cols_shape_supported(int, int cw, int rw, int unroll) {
    return cw > 0 && rw > 0 && cw * rw <= 16 && unroll > 0 && unroll <= 16;
}
bool small_shape_supported(int, int unroll) { return unroll > 0 && unroll <= 8; }
}  // namespace rd

namespace {

std::mt19937_64 rng;

int64_t pick_size() {
    switch (rng() % 8) {
        case 0: return 0;
        case 1: return 1;
        case 2: return int64_t(rng() % 8);
        case 3: return int64_t(rng() % 5000);
        case 4: return int64_t(1) << (rng() % 40);
        case 5: return (int64_t(1) << (rng() % 62)) + int64_t(rng() % 3) - 1;
        case 6: return int64_t(rng() >> 1);           // up to INT64_MAX
        default: return int64_t(rng() % 100000000);
    }
}

int64_t pick_stride(int64_t contiguous) {
    switch (rng() % 6) {
        case 0: return 0;
        case 1: return 1;
        case 2: return contiguous;
        case 3: return int64_t(rng() % 70000);
        case 4: return int64_t(rng() >> (1 + rng() % 62));
        default:
            return contiguous > 0 && contiguous < (int64_t(1) << 60)
                       ? contiguous * int64_t(1 + rng() % 3)
                       : 1;
    }
}

void fail(const char* what, const rd::Strides& v, int op, const rd_plan& p) {
    fprintf(stderr,
            "invariant failed: %s; view [%lld, %lld, %lld] strides (%lld, %lld, %lld) op %d; "
            "plan path %d split %lld rows_per_split %lld blocks %lld workspace %lld\n",
            what, (long long)v.outer, (long long)v.R, (long long)v.inner, (long long)v.so,
            (long long)v.sr, (long long)v.si, op, p.path, (long long)p.split,
            (long long)p.rows_per_split, (long long)p.blocks, (long long)p.workspace_bytes);
    exit(3);
}

void check_reduce_plan(const rd::Strides& v, int op, const rd_plan& p, int cu) {
    const int64_t max_blocks = rd::kMaxBlocks;
    if (p.path == RD_PATH_NONE) {
        if (v.outer * v.inner != 0) fail("NONE with outputs", v, op, p);
        return;
    }
    if (p.blocks < 1 || p.blocks > max_blocks) fail("blocks out of range", v, op, p);
    if (p.split < 1) fail("split < 1", v, op, p);
    if (p.workspace_bytes < 0) fail("negative workspace", v, op, p);
    if (p.passes != (p.split > 1 && p.combine != RD_COMBINE_LAST_BLOCK ? 2 : 1) &&
        p.path != RD_PATH_ZERO && p.path != RD_PATH_ROWS_SHORT)
        fail("passes", v, op, p);
    const int64_t bytes = op == RD_OP_SOFTMAX_DENOM ? 8 : 4;
    switch (p.path) {
        case RD_PATH_ROWS:
            if (v.inner != 1 && v.sr != 1) fail("rows path without unit stride", v, op, p);
            if (p.group != 64 && p.group != 256) fail("group", v, op, p);
            if (p.split > 1 && p.workspace_bytes / bytes != v.outer * v.inner * p.split)
                fail("rows workspace", v, op, p);
            break;
        case RD_PATH_COLS:
        case RD_PATH_COLS_SMALL:
            // a strided kept inner axis only as a dense span (every
            // si-th column of it kept), and only on the wide column path
            if (v.si != 1 && !(rd::dense_columns(v) && p.path == RD_PATH_COLS))
                fail("column path without unit inner stride", v, op, p);
            if (v.si != 1 && (v.inner - 1) * v.si + 1 <= rd::kSmallInner)
                fail("dense span too narrow for the column kernel", v, op, p);
            if (p.rows_per_split < 1 || p.split * p.rows_per_split < v.R ||
                (p.split - 1) * p.rows_per_split >= v.R)
                fail("slabs do not tile R", v, op, p);
            if (p.split > 1 && p.workspace_bytes / bytes != p.split * v.outer * v.inner)
                fail("slab workspace", v, op, p);
            if (p.combine == RD_COMBINE_LAST_BLOCK) {
                // the last slab's workgroups wait for the others: one item
                // each, all resident, within the words and LDS slots built
                const int64_t span = (v.inner - 1) * v.si + 1;
                const int64_t tiles_n = ((span + 3) / 4 + 63) / 64;
                if (p.path != RD_PATH_COLS || op == RD_OP_SOFTMAX_DENOM || p.col_waves != 1 ||
                    p.row_waves < 2 || p.split < 2 || p.split > rd::kPubColMaxSlabs ||
                    p.blocks != tiles_n * v.outer * p.split || p.blocks > cu ||
                    (p.split - 1) * v.outer * v.inner > rd::kPubColWords)
                    fail("column slabs joined in one launch", v, op, p);
            }
            break;
        case RD_PATH_STRIDED:
            if (v.sr == 1 || (v.si == 1 && v.inner > 1)) fail("strided path with a unit stride", v, op, p);
            if (p.rows_per_split < 1 || p.split * p.rows_per_split < v.R ||
                (p.split - 1) * p.rows_per_split >= v.R)
                fail("strided slabs do not tile R", v, op, p);
            if (p.split > 1 && p.workspace_bytes / bytes != p.split * v.outer * v.inner)
                fail("strided workspace", v, op, p);
            break;
        default:
            break;
    }
}

bool tiles(int64_t R, int64_t split, int64_t per) {
    return per >= 1 && split >= 1 && split * per >= R && (split - 1) * per < R;
}

void check_scan_plan(const rd::Strides& v, const rd_plan& p) {
    if (p.path == RD_PATH_NONE) {
        if (v.outer != 0 && v.R != 0 && v.inner != 0) fail("scan NONE with elements", v, -1, p);
        return;
    }
    if (p.blocks < 1 || p.blocks > rd::kMaxBlocks) fail("scan blocks out of range", v, -1, p);
    const bool look = p.combine == RD_COMBINE_LOOKBACK;
    if (p.passes != (p.split > 1 && !look ? 3 : 1)) fail("scan passes", v, -1, p);
    const int64_t n = v.outer * v.inner;
    if (look) {
        // one launch, a workgroup of 8 or 16 waves per piece of one block
        // chunk; workspace: ticket, chunk totals, group totals
        if (p.path != RD_PATH_SCAN_ROWS || v.inner != 1 || v.sr != 1)
            fail("look-back off the row path", v, -1, p);
        if ((p.group != 512 && p.group != 1024) || p.block_threads != p.group || p.unroll != 8 ||
            p.rows_per_split != p.group / 64 * 2048 || !tiles(v.R, p.split, p.rows_per_split) ||
            p.blocks != v.outer * p.split ||
            p.workspace_bytes != rd::lookback_workspace_bytes(v.outer, p.split))
            fail("look-back plan", v, -1, p);
        return;
    }
    switch (p.path) {
        case RD_PATH_SCAN_ROWS:
            if (v.inner != 1 || v.sr != 1) fail("scan rows without unit row stride", v, -1, p);
            if (!tiles(v.R, p.split, p.rows_per_split)) fail("pieces do not tile R", v, -1, p);
            if (p.workspace_bytes != (p.split > 1 ? 8 * v.outer * p.split : 0))
                fail("scan rows workspace", v, -1, p);
            // a wave per item (4 to a 256-thread workgroup) or a workgroup of
            // `group` threads per item
            if (p.group == 64) {
                if (p.block_threads != rd::kBlock ||
                    p.blocks != std::min(rd::kMaxBlocks, (v.outer * p.split + 3) / 4))
                    fail("scan rows wave grid", v, -1, p);
            } else if (p.group == 256 || p.group == 512 || p.group == 1024) {
                // persistent workgroups (interleaved rows) take at most one
                // row each at a time; otherwise one workgroup per item
                const bool streamed = p.order == RD_ORDER_INTERLEAVED;
                if (p.block_threads != p.group ||
                    (streamed ? p.split != 1 || p.blocks > std::min(rd::kMaxBlocks, v.outer)
                              : p.order != 0 ||
                                    p.blocks != std::min(rd::kMaxBlocks, v.outer * p.split)))
                    fail("scan rows workgroup grid", v, -1, p);
            } else {
                fail("scan rows group", v, -1, p);
            }
            break;
        case RD_PATH_SCAN_COLS:
        case RD_PATH_SCAN_COLS_SMALL:
        case RD_PATH_SCAN_STRIDED:
            if (p.path != RD_PATH_SCAN_STRIDED && (v.inner < 2 || v.si != 1))
                fail("column scan without unit inner stride", v, -1, p);
            if (!tiles(v.R, p.split, p.rows_per_split)) fail("scan slabs do not tile R", v, -1, p);
            if (p.workspace_bytes != (p.split > 1 ? 8 * p.split * n : 0))
                fail("scan slab workspace", v, -1, p);
            if (p.path == RD_PATH_SCAN_STRIDED && p.row_waves > 1) {
                // one pass in row rounds: a block of row waves per 64 columns
                if (p.split != 1 || p.block_threads != 64 * p.row_waves ||
                    p.blocks != std::min(rd::kMaxBlocks, (n + 63) / 64))
                    fail("scan strided rounds", v, -1, p);
            } else if (p.path == RD_PATH_SCAN_STRIDED) {
                // staged views: blocks of 64 columns; otherwise 256 columns
                const int64_t cols = (v.inner == 1 || v.sr == 1) ? 64 : rd::kBlock;
                if (p.blocks != std::min(rd::kMaxBlocks, p.split * ((n + cols - 1) / cols)))
                    fail("scan strided blocks", v, -1, p);
            }
            break;
            break;
        default:
            fail("unknown scan path", v, -1, p);
    }
}

}  // namespace

int main(int argc, char** argv) {
    const long iters = argc > 1 ? atol(argv[1]) : 200000;
    rng.seed(argc > 2 ? strtoull(argv[2], nullptr, 10) : 12345);
    long accepted = 0;
    for (long it = 0; it < iters; ++it) {
        const int cu = (rng() % 4 == 0) ? int(1 + rng() % 512) : 256;
        rd::Strides v;
        v.outer = pick_size();
        v.R = pick_size();
        v.inner = pick_size();
        const bool contiguous = rng() % 2 == 0;
        // contiguous strides only when they are representable
        const bool fits = v.inner < (int64_t(1) << 31) && v.R < (int64_t(1) << 31);
        v.so = contiguous && fits ? v.R * v.inner : pick_stride(v.R);
        v.sr = contiguous && fits ? v.inner : pick_stride(v.inner);
        v.si = contiguous ? 1 : pick_stride(1);
        const int op = int(rng() % 5);
        rd_tune t{};
        const bool tuned = rng() % 3 == 0;
        if (tuned) {
            static const int32_t groups[] = {0, 64, 256, 512, 1024};
            t.group = groups[rng() % 5];
            t.col_waves = int32_t(rng() % 5 == 0 ? 0 : 1 << (rng() % 5));
            t.row_waves = int32_t(rng() % 3 == 0 ? 0 : 1 << (rng() % 4));
            t.unroll = int32_t(rng() % 3 == 0 ? 0 : 1 << (rng() % 5));
            t.order = int32_t(rng() % 3);
            t.nontemporal = int32_t(rng() % 3);
            t.combine = int32_t(rng() % 3);
            static const int32_t paths[] = {RD_PATH_COLS, RD_PATH_COLS_SMALL, RD_PATH_SCAN_ROWS,
                                            RD_PATH_SCAN_COLS, RD_PATH_SCAN_COLS_SMALL,
                                            RD_PATH_SCAN_STRIDED};
            t.path = rng() % 4 == 0 ? paths[rng() % 6] : 0;
            t.split = rng() % 2 ? 0 : int64_t(rng() % 5000);
        }
        rd::Strides w = v;
        rd_plan p;
        if (rd::plan_view(cu, &w, op, tuned ? &t : nullptr, &p) == RD_OK) {
            ++accepted;
            check_reduce_plan(w, op, p, cu);
        }
        rd::Strides u = v;
        rd_plan q;
        if (rd::plan_cumsum_view(cu, &u, tuned ? &t : nullptr, &q) == RD_OK) {
            ++accepted;
            check_scan_plan(u, q);
        }
        if (contiguous && fits) {
            rd_plan c;
            const rd_status a = rd::plan_cumsum(cu, v.outer, v.R, v.inner, tuned ? &t : nullptr, &c);
            rd::Strides cv{v.outer, v.R, v.inner, v.R * v.inner, v.inner, 1};
            rd_plan d;
            const rd_status b = rd::plan_cumsum_view(cu, &cv, tuned ? &t : nullptr, &d);
            if (a != b || (a == RD_OK && memcmp(&c, &d, sizeof(c)) != 0))
                fail("contiguous view plans unlike the array", v, -1, c);
        }
    }
    printf("plan_fuzz: %ld iterations, %ld accepted plans, no finding\n", iters, accepted);
    return 0;
}
