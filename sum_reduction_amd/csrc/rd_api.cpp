// rd_api.cpp -- the C ABI of include/rd.h: argument validation, per-device
// state, the stream-ordered workspace and the launch sequence of a plan.
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <memory>
#include <mutex>
#include <unordered_map>

#include <hip/hip_runtime_api.h>

#include "rd_internal.h"

namespace {

thread_local int t_last_hip = 0;

// Per-device state.  The first call on a device reads its CU count (which
// fixes the plan, hence the summation order); the first call that needs a
// workspace also creates the library's memory pool for workspaces, which
// keeps its memory between calls; the first single-launch combine on a
// stream creates that stream's buffer.  Calls whose plan needs no
// workspace, and rd_sum_dim_noalloc, never allocate.
// Buffers of the single-launch combine: one per stream that has made such a
// call on the device (up to kPubStreams), each with room for kPubColWords
// tagged words (row pieces use the first kPubWords, with their values; slab
// results of a column reduce and the totals of a look-back row scan all of
// them), the look-back scan's ticket, the stream's last epoch, and
// kStreamScratchBytes of plain scratch: the workspace of a split plan that
// takes a second kernel, when it fits (calls on one stream never overlap, so
// one call's partial results are never another's).  The scratch is kept apart
// from the tagged words, so its floats can never pass for a published word.
// A launch publishes its words tagged with a new epoch of its stream; calls
// on one stream never overlap, so every word a launch finds tagged with its
// own epoch was written by that launch.  Zeroed when created, and again
// before an epoch is reused (after 2^32 - 1 launches).
constexpr int kPubStreams = 256;
constexpr size_t kStreamScratchBytes = size_t(1) << 20;
using rd::kPubWords;
using rd::kPubColWords;
struct StreamPub {
    uint64_t* words = nullptr;
    float* vals = nullptr;
    uint32_t* ticket = nullptr;
    float* scratch = nullptr;
    // held from a call's first launch that uses the scratch to its last, so
    // that calls from two host threads on one stream do not interleave their
    // kernels (the second call's first kernel would overwrite the first's
    // partial results before its second kernel reads them)
    std::shared_ptr<std::mutex> scratch_mu;
    uint32_t epoch = 0;
};
struct Device {
    std::once_flag once;
    std::atomic<bool> ready{false};  // set once the CU count is known
    int cu = 0;
    hipError_t err = hipSuccess;
    std::once_flag mem_once;  // the workspace pool, on the first workspace plan
    hipMemPool_t pool = nullptr;
    hipError_t mem_err = hipSuccess;
    std::mutex pub_mu;
    std::unordered_map<hipStream_t, StreamPub> pub_of;
};
Device g_devices[rd::kMaxDevices];

// A zeroed buffer of kPubColWords tagged words, kPubWords values and a
// ticket, or null if it cannot be had (then the call takes the two-kernel
// combine, or the zeroed workspace, with the same results).
StreamPub make_pub() {
    StreamPub b;
    void* mem = nullptr;
    const size_t vals_end = size_t(kPubColWords) * sizeof(uint64_t) + size_t(kPubWords) * sizeof(float);
    const size_t ticket_end = vals_end + size_t(rd::kLookTicketBytes);
    const size_t bytes = ticket_end + kStreamScratchBytes;
    if (hipMalloc(&mem, bytes) != hipSuccess) return b;
    hipStream_t s = nullptr;
    bool ok = hipStreamCreateWithFlags(&s, hipStreamNonBlocking) == hipSuccess;
    ok = ok && hipMemsetAsync(mem, 0, bytes, s) == hipSuccess;
    ok = ok && hipStreamSynchronize(s) == hipSuccess;
    if (s) (void)hipStreamDestroy(s);
    if (!ok) {
        (void)hipFree(mem);
        return b;
    }
    b.words = static_cast<uint64_t*>(mem);
    b.vals = reinterpret_cast<float*>(b.words + kPubColWords);
    b.ticket = reinterpret_cast<uint32_t*>(static_cast<char*>(mem) + vals_end);
    b.scratch = reinterpret_cast<float*>(static_cast<char*>(mem) + ticket_end);
    b.scratch_mu = std::make_shared<std::mutex>();
    return b;
}

// RD_OK when `stream` is not being captured into a graph, RD_ERR_CAPTURE
// when it is, RD_ERR_HIP when its state cannot be read.  A call whose plan
// needs a workspace is refused while capturing: a replay of a captured
// stream-ordered workspace faulted in the second kernel that reads it, and
// the cause is not established.
rd_status capture_check(hipStream_t stream) {
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    const hipError_t e = hipStreamIsCapturing(stream, &cap);
    if (e != hipSuccess) {
        t_last_hip = static_cast<int>(e);
        return RD_ERR_HIP;
    }
    return cap == hipStreamCaptureStatusNone ? RD_OK : RD_ERR_CAPTURE;
}

// The single-launch combine's buffer of `stream` and a new epoch for one
// launch on it (the stream is not being captured: such calls are refused
// before this), or false for the two-kernel combine: every buffer taken, none
// to be had, or the per-thread default stream, whose one handle stands for a
// different stream in each host thread -- calls from two threads could run
// at once and share the buffer.
// The buffer of `stream` (created on its first use), or null: see stream_pub.
// Call with d.pub_mu held; entries are never removed, so the pointer stays
// valid.
StreamPub* stream_buffer(Device& d, hipStream_t stream) {
    if (stream == hipStreamPerThread) return nullptr;
    auto it = d.pub_of.find(stream);
    if (it == d.pub_of.end()) {
        if (static_cast<int>(d.pub_of.size()) >= kPubStreams) return nullptr;
        StreamPub b = make_pub();
        if (!b.words) return nullptr;
        it = d.pub_of.emplace(stream, b).first;
    }
    return &it->second;
}

// The scratch of `stream`'s buffer for a workspace of `bytes`, with *hold
// locking the stream's scratch mutex until the caller has enqueued its last
// kernel, or null (too large, or no buffer: the workspace then comes from the
// pool).
float* stream_scratch(Device& d, hipStream_t stream, int64_t bytes,
                      std::unique_lock<std::mutex>* hold) {
    if (bytes <= 0 || size_t(bytes) > kStreamScratchBytes) return nullptr;
    std::shared_ptr<std::mutex> mu;
    float* scratch = nullptr;
    {
        std::lock_guard<std::mutex> lock(d.pub_mu);
        StreamPub* b = stream_buffer(d, stream);
        if (!b) return nullptr;
        mu = b->scratch_mu;
        scratch = b->scratch;
    }
    *hold = std::unique_lock<std::mutex>(*mu);  // the buffer outlives the call
    return scratch;
}

bool stream_pub(Device& d, hipStream_t stream, rd::Published* pub, hipError_t* err) {
    *err = hipSuccess;
    std::lock_guard<std::mutex> lock(d.pub_mu);
    StreamPub* bp = stream_buffer(d, stream);
    if (!bp) return false;
    StreamPub& b = *bp;
    if (++b.epoch == 0) {  // every epoch used: clear the words, start again
        *err = hipMemsetAsync(b.words, 0, size_t(kPubColWords) * sizeof(uint64_t), stream);
        if (*err != hipSuccess) return false;
        b.epoch = 1;
    }
    pub->words = b.words;
    pub->vals = b.vals;
    pub->ticket = b.ticket;
    pub->epoch = b.epoch;
    return true;
}

std::mutex g_tune_mu;
rd_tune g_tune;
bool g_tune_on = false;

rd_status hip_fail(hipError_t e, rd_status st) {
    t_last_hip = static_cast<int>(e);
    return st;
}

bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// [a, a + na) and [b, b + nb) in floats
bool overlap(const float* a, int64_t na, const float* b, int64_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    const uintptr_t a1 = a0 + uintptr_t(na) * 4u, b1 = b0 + uintptr_t(nb) * 4u;
    return a0 < b1 && b0 < a1;
}

// The calling thread's current device (its index in *index), its CU count
// read on its first use.  The first use of a device may load the library's
// code objects onto it, which must not happen inside a graph being
// captured, so a first call on a capturing `stream` is refused with
// RD_ERR_CAPTURE before any of it.
rd_status current_device(Device** out, int* index, hipStream_t stream) {
    int count = 0;
    hipError_t e = hipGetDeviceCount(&count);
    if (e != hipSuccess || count < 1) {
        t_last_hip = static_cast<int>(e);
        return RD_ERR_NO_DEVICE;
    }
    int dev = -1;
    e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, RD_ERR_NO_DEVICE);
    if (dev < 0 || dev >= rd::kMaxDevices) return RD_ERR_NO_DEVICE;
    Device& d = g_devices[dev];
    if (!d.ready.load(std::memory_order_acquire)) {
        const rd_status cs = capture_check(stream);
        if (cs != RD_OK) return cs;
    }
    std::call_once(d.once, [&d, dev] {
        int cu = 0;
        const hipError_t err =
            hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev);
        if (err != hipSuccess || cu < 1) {
            d.err = err != hipSuccess ? err : hipErrorInvalidDevice;
            return;
        }
        d.cu = cu;
        d.ready.store(true, std::memory_order_release);
    });
    if (d.err != hipSuccess) return hip_fail(d.err, RD_ERR_HIP);
    *out = &d;
    if (index) *index = dev;
    return RD_OK;
}

// The device's workspace pool, created by the first call that needs a
// workspace (never while capturing: such calls are refused first).  The
// calling thread's current device is d's.
rd_status device_memory(Device& d) {
    std::call_once(d.mem_once, [&d] {
        int dev = -1;
        hipError_t err = hipGetDevice(&dev);
        if (err != hipSuccess) {
            d.mem_err = err;
            return;
        }
        hipMemPoolProps props;
        memset(&props, 0, sizeof(props));
        props.allocType = hipMemAllocationTypePinned;
        props.handleTypes = hipMemHandleTypeNone;
        props.location.type = hipMemLocationTypeDevice;
        props.location.id = dev;
        err = hipMemPoolCreate(&d.pool, &props);
        if (err != hipSuccess) {
            d.mem_err = err;
            return;
        }
        uint64_t keep = UINT64_MAX;  // hold freed workspace for the next call
        err = hipMemPoolSetAttribute(d.pool, hipMemPoolAttrReleaseThreshold, &keep);
        if (err != hipSuccess) {
            d.mem_err = err;
            return;
        }
    });
    if (d.mem_err != hipSuccess) return hip_fail(d.mem_err, RD_ERR_HIP);
    return RD_OK;
}

// Failure injection for tests of the error paths, read from the environment
// once per process (at the first call that looks): RD_TEST_FAIL_ALLOC makes
// the workspace allocation fail, RD_TEST_FAIL_LAUNCH makes the first launch
// fail; neither enqueues any work.  RD_TEST_SPIN_LIMIT=n caps the polls of a
// look-back wait at n (the kernel still runs to its end; a piece whose wait
// gives up writes NaN).
bool env_on(const char* name) {
    const char* v = getenv(name);
    return v && v[0] && v[0] != '0';
}

struct Injected {
    bool alloc, launch;
    uint32_t spin_limit;  // polls of a look-back wait before it gives up
};

uint32_t env_spin_limit() {
    const char* v = getenv("RD_TEST_SPIN_LIMIT");
    if (!v || !*v) return rd::kLookSpinLimit;
    const unsigned long n = strtoul(v, nullptr, 10);
    return n < rd::kLookSpinLimit ? uint32_t(n) : rd::kLookSpinLimit;
}

const Injected& injected() {
    static const Injected f{env_on("RD_TEST_FAIL_ALLOC"), env_on("RD_TEST_FAIL_LAUNCH"),
                            env_spin_limit()};
    return f;
}

// Runs plan p.  fixed == nullptr: a reduce whose plan takes the
// single-launch combine publishes its results in the stream's buffer (one
// kernel); otherwise the workspace (if any) is the scratch of the stream's
// buffer when it fits, else allocated stream-ordered from the device's pool
// and freed after the last kernel.  All of these are refused while `s` is
// being captured.  fixed != nullptr: it is the workspace, at
// least p.workspace_bytes long, and nothing is allocated (the partial
// results are combined by the second kernel).
rd_status execute(const rd_plan& p, int op, Device& dev, const float* x, const rd::Strides& v,
                  rd::Results out, hipStream_t s, float* fixed) {
    if (p.path == RD_PATH_NONE) return RD_OK;
    if (injected().launch) return hip_fail(hipErrorLaunchFailure, RD_ERR_LAUNCH);
    float* ws = nullptr;
    bool pooled = false;
    std::unique_lock<std::mutex> scratch_hold;
    rd::Published pub;
    bool published = false;
    if (p.workspace_bytes > 0 && !fixed) {
        rd_status st = capture_check(s);
        if (st != RD_OK) return st;
        if (injected().alloc) return hip_fail(hipErrorOutOfMemory, RD_ERR_ALLOC);
        const int64_t words = (op == RD_OP_SOFTMAX_DENOM ? 2 : 1) * v.outer * v.inner * p.split;
        const bool rows_one = p.path == RD_PATH_ROWS && words <= kPubWords;
        // the slab results a column reduce publishes: all but the last slab's
        const bool cols_one = p.path == RD_PATH_COLS && op != RD_OP_SOFTMAX_DENOM &&
                              v.outer * v.inner * (p.split - 1) <= kPubColWords;
        if (p.combine == RD_COMBINE_LAST_BLOCK && (rows_one || cols_one)) {
            hipError_t pe = hipSuccess;
            published = stream_pub(dev, s, &pub, &pe);
            if (pe != hipSuccess) return hip_fail(pe, RD_ERR_HIP);
            pub.spin_limit = injected().spin_limit;
        }
    }
    if (p.workspace_bytes > 0 && fixed) {
        ws = fixed;
    } else if (p.workspace_bytes > 0 && !published) {
        ws = stream_scratch(dev, s, p.workspace_bytes, &scratch_hold);
        if (!ws) {
            rd_status st = device_memory(dev);
            if (st != RD_OK) return st;
            hipError_t e = hipMallocFromPoolAsync(reinterpret_cast<void**>(&ws),
                                                  size_t(p.workspace_bytes), dev.pool, s);
            if (e != hipSuccess) return hip_fail(e, RD_ERR_ALLOC);
            pooled = true;
        }
    }
    // partial results: one array, or the two halves of the pairs
    rd::Results part{ws, nullptr};
    if (ws && op == RD_OP_SOFTMAX_DENOM)
        part.b = ws + p.workspace_bytes / int64_t(2 * sizeof(float));
    const int64_t nout = v.outer * v.inner;
    hipError_t e = hipSuccess;
    switch (p.path) {
        case RD_PATH_ZERO:
            e = rd::launch_fill_start(op, out, nout, s);
            break;
        case RD_PATH_ROWS_SHORT:
            e = rd::launch_rows_short(op, x, v, out, s);
            break;
        case RD_PATH_ROWS:
            if (p.split == 1) {
                e = rd::launch_rows(op, p, x, v, out, nullptr, rd::Results{}, s);
            } else if (published) {
                e = rd::launch_rows(op, p, x, v, rd::Results{}, &pub, out, s);
            } else {
                e = rd::launch_rows(op, p, x, v, part, nullptr, out, s);
                if (e == hipSuccess) e = rd::launch_rows_combine(op, part, nout, p.split, out, s);
            }
            break;
        case RD_PATH_COLS:
        case RD_PATH_COLS_SMALL: {
            if (published) {  // the last slab's blocks join the slabs in one launch
                e = rd::launch_cols(op, p, x, v, rd::Results{}, &pub, out, s);
                break;
            }
            const rd::Results dst = p.split == 1 ? out : part;
            e = p.path == RD_PATH_COLS ? rd::launch_cols(op, p, x, v, dst, nullptr, rd::Results{}, s)
                                       : rd::launch_cols_small(op, p, x, v, dst, s);
            if (e == hipSuccess && p.split > 1)
                e = rd::launch_slab_combine(op, part, p.split, nout, out, s);
            break;
        }
        case RD_PATH_STRIDED:
            e = rd::launch_strided(op, p, x, v, p.split == 1 ? out : part, s);
            if (e == hipSuccess && p.split > 1)
                e = rd::launch_slab_combine(op, part, p.split, nout, out, s);
            break;
        default:
            e = hipErrorInvalidValue;
    }
    if (pooled) {
        hipError_t f = hipFreeAsync(ws, s);
        if (e == hipSuccess && f != hipSuccess) return hip_fail(f, RD_ERR_HIP);
    }
    if (e != hipSuccess) return hip_fail(e, RD_ERR_LAUNCH);
    return RD_OK;
}

// Plans and runs a reduction of the view v (sizes already validated).
rd_status reduce_checked(const float* x, rd::Strides v, int op, rd::Results out,
                         hipStream_t stream) {
    Device* dev = nullptr;
    rd_status st = current_device(&dev, nullptr, stream);
    if (st != RD_OK) return st;
    rd_plan plan;
    {
        std::lock_guard<std::mutex> lock(g_tune_mu);
        st = rd::plan_view(dev->cu, &v, op, g_tune_on ? &g_tune : nullptr, &plan);
    }
    if (st != RD_OK) return st;
    return execute(plan, op, *dev, x, v, out, stream, nullptr);
}

rd::Strides contiguous(int64_t outer, int64_t R, int64_t inner) {
    return rd::Strides{outer, R, inner, R * inner, inner, 1};
}

// Floats from x to one past the furthest element of the view (0 if empty).
int64_t view_extent(const rd::Strides& v) {
    if (v.outer == 0 || v.R == 0 || v.inner == 0) return 0;
    return (v.outer - 1) * v.so + (v.R - 1) * v.sr + (v.inner - 1) * v.si + 1;
}

// The cumulative sum of the view v (sizes and pointers already checked, at
// least one element): plan, workspace, one or three launches.
rd_status cumsum_checked(const float* x, rd::Strides v, bool rev, float* out,
                         hipStream_t stream) {
    Device* dev = nullptr;
    rd_status st = current_device(&dev, nullptr, stream);
    if (st != RD_OK) return st;
    rd_plan p;
    {
        std::lock_guard<std::mutex> lock(g_tune_mu);
        st = rd::plan_cumsum_view(dev->cu, &v, g_tune_on ? &g_tune : nullptr, &p);
    }
    if (st != RD_OK) return st;
    if (p.path == RD_PATH_NONE) return RD_OK;
    if (injected().launch) return hip_fail(hipErrorLaunchFailure, RD_ERR_LAUNCH);
    // A look-back plan of one piece per row waits for nothing (its ticket
    // only orders the rows): on a capturing stream the workgroup-per-row
    // kernel with the same chunk runs instead, with the same bits and no
    // workspace.
    if (p.path == RD_PATH_SCAN_ROWS && p.combine == RD_COMBINE_LOOKBACK && p.split == 1) {
        st = capture_check(stream);
        if (st == RD_ERR_CAPTURE) {
            p.combine = RD_COMBINE_NONE;
            p.workspace_bytes = 0;
        } else if (st != RD_OK) {
            return st;
        }
    }
    float* ws = nullptr;
    rd::Published pub;
    bool published = false;
    if (p.workspace_bytes > 0) {
        st = capture_check(stream);
        if (st != RD_OK) return st;
        if (injected().alloc) return hip_fail(hipErrorOutOfMemory, RD_ERR_ALLOC);
        // a look-back whose totals fit the stream's buffer takes it: its
        // words are tagged with the launch's epoch and its ticket is 0
        // between launches, so nothing is zeroed before the launch
        if (p.path == RD_PATH_SCAN_ROWS && p.combine == RD_COMBINE_LOOKBACK &&
            rd::lookback_words(v.outer * v.inner, p.split) <= kPubColWords) {
            hipError_t pe = hipSuccess;
            published = stream_pub(*dev, stream, &pub, &pe);
            if (pe != hipSuccess) return hip_fail(pe, RD_ERR_HIP);
        }
    }
    bool pooled = false;
    std::unique_lock<std::mutex> scratch_hold;
    if (p.workspace_bytes > 0 && !published) {
        ws = stream_scratch(*dev, stream, p.workspace_bytes, &scratch_hold);
        if (!ws) {
            st = device_memory(*dev);
            if (st != RD_OK) return st;
            hipError_t e = hipMallocFromPoolAsync(reinterpret_cast<void**>(&ws),
                                                  size_t(p.workspace_bytes), dev->pool, stream);
            if (e != hipSuccess) return hip_fail(e, RD_ERR_ALLOC);
            pooled = true;
        }
    }
    const int64_t nrow = v.outer * v.inner;
    // The totals pass of a split scan reads x without the streaming hint when
    // x fits in the last-level cache, so that the scan pass re-reads it from
    // there (measured: 5-11% faster up to 256 MB, 1% slower at 2 GB).
    rd_plan pt = p;
    if (uint64_t(nrow * v.R) * sizeof(float) <= rd::kScanCachedTotalsBytes) pt.nontemporal = 0;
    hipError_t e = hipSuccess;
    if (p.path == RD_PATH_SCAN_ROWS && p.combine == RD_COMBINE_LOOKBACK) {
        e = rd::launch_scan_rows_lookback(p, rev, x, out, v, ws, published ? &pub : nullptr,
                                          injected().spin_limit, stream);
    } else if (p.path == RD_PATH_SCAN_ROWS) {
        if (p.split == 1) {
            e = rd::launch_scan_rows(p, rev, x, out, v, nullptr, nullptr, stream);
        } else {
            const int64_t m = v.outer * p.split;
            float* totals = ws;
            float* carries = ws + m;
            e = rd::launch_scan_rows(pt, rev, x, out, v, nullptr, totals, stream);
            if (e == hipSuccess)
                e = rd::launch_scan_carries(totals, carries, v.outer, p.split, stream);
            if (e == hipSuccess) e = rd::launch_scan_rows(p, rev, x, out, v, carries, nullptr, stream);
        }
    } else {
        auto cols = [&](const rd_plan& q, const float* carry_in, float* totals) {
            if (p.path == RD_PATH_SCAN_COLS_SMALL)
                return rd::launch_scan_small(q, rev, x, out, v, carry_in, totals, stream);
            if (p.path == RD_PATH_SCAN_COLS)
                return rd::launch_scan_cols(q, rev, x, out, v, carry_in, totals, stream);
            return rd::launch_scan_strided(q, rev, x, out, v, carry_in, totals, stream);
        };
        if (p.split == 1) {
            e = cols(p, nullptr, nullptr);
        } else {
            const int64_t m = p.split * nrow;
            float* totals = ws;
            float* carries = ws + m;
            e = cols(pt, nullptr, totals);
            if (e == hipSuccess)
                e = rd::launch_scan_slab_carries(rev, totals, carries, p.split, nrow, stream);
            if (e == hipSuccess) e = cols(p, carries, nullptr);
        }
    }
    if (pooled) {
        hipError_t f = hipFreeAsync(ws, stream);
        if (e == hipSuccess && f != hipSuccess) return hip_fail(f, RD_ERR_HIP);
    }
    if (e != hipSuccess) return hip_fail(e, RD_ERR_LAUNCH);
    return RD_OK;
}

// The arguments of an axis reduce of a contiguous [outer, R, inner] array:
// RD_OK with *empty set when there is nothing to write (outer*inner == 0).
rd_status dim_args(const float* x, int64_t outer, int64_t R, int64_t inner, const float* out,
                   bool* empty) {
    *empty = false;
    if (outer < 0 || R < 0 || inner < 0) return RD_ERR_INVALID_ARG;
    const int64_t lim = INT64_MAX / 4;
    if (outer && inner && inner > lim / outer) return RD_ERR_INVALID_ARG;
    const int64_t nout = outer * inner;
    if (nout && R && R > lim / nout) return RD_ERR_INVALID_ARG;
    const int64_t nin = nout * R;
    if (nout == 0) {
        *empty = true;
        return RD_OK;
    }
    if (!out || !aligned4(out)) return RD_ERR_INVALID_ARG;
    if (nin > 0 && (!x || !aligned4(x))) return RD_ERR_INVALID_ARG;
    if (overlap(x, nin, out, nout)) return RD_ERR_INVALID_ARG;
    return RD_OK;
}

bool op_valid(int32_t op) { return op >= RD_OP_SUM && op <= RD_OP_MIN; }

}  // namespace

namespace rd {

rd_status sum_dim_fixed(const float* x, int64_t outer, int64_t R, int64_t inner, float* out,
                        ScratchFn scratch, int64_t scratch_bytes, hipStream_t stream) {
    bool empty = false;
    rd_status st = dim_args(x, outer, R, inner, out, &empty);
    if (st != RD_OK || empty) return st;  // empty: nothing to write, no HIP call
    Device* dev = nullptr;
    int index = -1;
    st = current_device(&dev, &index, stream);
    if (st != RD_OK) return st;
    float* ws = nullptr;
    st = scratch(index, &ws);
    if (st != RD_OK) return st;
    Strides v = contiguous(outer, R, inner);
    rd_plan plan;
    {
        std::lock_guard<std::mutex> lock(g_tune_mu);
        st = plan_view(dev->cu, &v, RD_OP_SUM, g_tune_on ? &g_tune : nullptr, &plan);
    }
    if (st != RD_OK) return st;
    if (plan.workspace_bytes > scratch_bytes) return RD_ERR_WORKSPACE;
    return execute(plan, RD_OP_SUM, *dev, x, v, Results{out, nullptr}, stream, ws);
}

void set_last_hip_error(hipError_t e) { t_last_hip = static_cast<int>(e); }

}  // namespace rd

extern "C" {

rd_status rd_reduce_1d(const float* x, int64_t n, int32_t op, float* out,
                       hipStream_t stream) {
    if (!op_valid(op)) return RD_ERR_INVALID_ARG;
    if (n < 0 || n > INT64_MAX / 4 || !out || !aligned4(out)) return RD_ERR_INVALID_ARG;
    if (n > 0 && (!x || !aligned4(x))) return RD_ERR_INVALID_ARG;
    if (overlap(x, n, out, 1)) return RD_ERR_INVALID_ARG;
    return reduce_checked(x, contiguous(1, n, 1), op, rd::Results{out, nullptr}, stream);
}

rd_status rd_reduce_dim(const float* x, int64_t outer, int64_t R, int64_t inner, int32_t op,
                        float* out, hipStream_t stream) {
    if (!op_valid(op)) return RD_ERR_INVALID_ARG;
    bool empty = false;
    const rd_status st = dim_args(x, outer, R, inner, out, &empty);
    if (st != RD_OK || empty) return st;  // empty: nothing to write, no HIP call
    return reduce_checked(x, contiguous(outer, R, inner), op, rd::Results{out, nullptr},
                          stream);
}

rd_status rd_reduce_strided(const float* x, int64_t outer, int64_t R, int64_t inner,
                            int64_t stride_outer, int64_t stride_r, int64_t stride_inner,
                            int32_t op, float* out, hipStream_t stream) {
    if (!op_valid(op)) return RD_ERR_INVALID_ARG;
    const rd::Strides v{outer, R, inner, stride_outer, stride_r, stride_inner};
    if (!rd::view_sizes_ok(v)) return RD_ERR_INVALID_ARG;
    const int64_t nout = outer * inner;
    if (nout == 0) return RD_OK;  // nothing to write, no HIP call
    const int64_t span = view_extent(v);
    if (!out || !aligned4(out)) return RD_ERR_INVALID_ARG;
    if (span > 0 && (!x || !aligned4(x))) return RD_ERR_INVALID_ARG;
    if (overlap(x, span, out, nout)) return RD_ERR_INVALID_ARG;
    return reduce_checked(x, v, op, rd::Results{out, nullptr}, stream);
}

rd_status rd_plan_strided(int cu_count, int64_t outer, int64_t R, int64_t inner,
                          int64_t stride_outer, int64_t stride_r, int64_t stride_inner,
                          rd_plan* plan) {
    rd::Strides v{outer, R, inner, stride_outer, stride_r, stride_inner};
    std::lock_guard<std::mutex> lock(g_tune_mu);
    return rd::plan_view(cu_count, &v, RD_OP_SUM, g_tune_on ? &g_tune : nullptr, plan);
}

rd_status rd_softmax_denom_dim(const float* x, int64_t outer, int64_t R, int64_t inner,
                               float* out_max, float* out_sum, hipStream_t stream) {
    if (outer < 0 || R < 0 || inner < 0) return RD_ERR_INVALID_ARG;
    const int64_t lim = INT64_MAX / 8;
    if (outer && inner && inner > lim / outer) return RD_ERR_INVALID_ARG;
    const int64_t nout = outer * inner;
    if (nout && R && R > lim / nout) return RD_ERR_INVALID_ARG;
    const int64_t nin = nout * R;
    if (nout == 0) return RD_OK;  // nothing to write, no HIP call
    if (!out_max || !out_sum || !aligned4(out_max) || !aligned4(out_sum))
        return RD_ERR_INVALID_ARG;
    if (nin > 0 && (!x || !aligned4(x))) return RD_ERR_INVALID_ARG;
    if (overlap(x, nin, out_max, nout) || overlap(x, nin, out_sum, nout) ||
        overlap(out_max, nout, out_sum, nout))
        return RD_ERR_INVALID_ARG;
    return reduce_checked(x, contiguous(outer, R, inner), RD_OP_SOFTMAX_DENOM,
                          rd::Results{out_max, out_sum}, stream);
}

rd_status rd_softmax_denom_strided(const float* x, int64_t outer, int64_t R, int64_t inner,
                                   int64_t stride_outer, int64_t stride_r,
                                   int64_t stride_inner, float* out_max, float* out_sum,
                                   hipStream_t stream) {
    const rd::Strides v{outer, R, inner, stride_outer, stride_r, stride_inner};
    if (!rd::view_sizes_ok(v)) return RD_ERR_INVALID_ARG;
    const int64_t nout = outer * inner;
    if (nout == 0) return RD_OK;  // nothing to write, no HIP call
    if (nout > INT64_MAX / 8) return RD_ERR_INVALID_ARG;
    const int64_t span = view_extent(v);
    if (!out_max || !out_sum || !aligned4(out_max) || !aligned4(out_sum))
        return RD_ERR_INVALID_ARG;
    if (span > 0 && (!x || !aligned4(x))) return RD_ERR_INVALID_ARG;
    if (overlap(x, span, out_max, nout) || overlap(x, span, out_sum, nout) ||
        overlap(out_max, nout, out_sum, nout))
        return RD_ERR_INVALID_ARG;
    return reduce_checked(x, v, RD_OP_SOFTMAX_DENOM, rd::Results{out_max, out_sum}, stream);
}

rd_status rd_softmax_denom_1d(const float* x, int64_t n, float* out_max, float* out_sum,
                              hipStream_t stream) {
    if (n < 0 || n > INT64_MAX / 8) return RD_ERR_INVALID_ARG;
    return rd_softmax_denom_dim(x, 1, n, 1, out_max, out_sum, stream);
}

rd_status rd_cumsum_dim(const float* x, int64_t outer, int64_t R, int64_t inner,
                        int32_t reverse, float* out, hipStream_t stream) {
    if (outer < 0 || R < 0 || inner < 0) return RD_ERR_INVALID_ARG;
    const int64_t lim = INT64_MAX / 4;
    if (outer && inner && inner > lim / outer) return RD_ERR_INVALID_ARG;
    const int64_t nrow = outer * inner;
    if (nrow && R && R > lim / nrow) return RD_ERR_INVALID_ARG;
    const int64_t n = nrow * R;
    if (n == 0) return RD_OK;  // nothing to write, no HIP call
    if (!x || !out || !aligned4(x) || !aligned4(out)) return RD_ERR_INVALID_ARG;
    if (out != x && overlap(x, n, out, n)) return RD_ERR_INVALID_ARG;
    return cumsum_checked(x, contiguous(outer, R, inner), reverse != 0, out, stream);
}

rd_status rd_cumsum_strided(const float* x, int64_t outer, int64_t R, int64_t inner,
                            int64_t stride_outer, int64_t stride_r, int64_t stride_inner,
                            int32_t reverse, float* out, hipStream_t stream) {
    const rd::Strides v{outer, R, inner, stride_outer, stride_r, stride_inner};
    if (!rd::view_sizes_ok(v)) return RD_ERR_INVALID_ARG;
    const int64_t n = outer * R * inner;
    if (n == 0) return RD_OK;  // nothing to write, no HIP call
    if (!x || !out || !aligned4(x) || !aligned4(out)) return RD_ERR_INVALID_ARG;
    // in place only where the view is the output's own layout
    const bool same_layout = (inner == 1 || stride_inner == 1) &&
                             (R == 1 || stride_r == inner) &&
                             (outer == 1 || stride_outer == R * inner);
    if (!(out == x && same_layout) && overlap(x, view_extent(v), out, n))
        return RD_ERR_INVALID_ARG;
    return cumsum_checked(x, v, reverse != 0, out, stream);
}

rd_status rd_plan_cumsum(int cu_count, int64_t outer, int64_t R, int64_t inner, rd_plan* plan) {
    std::lock_guard<std::mutex> lock(g_tune_mu);
    return rd::plan_cumsum(cu_count, outer, R, inner, g_tune_on ? &g_tune : nullptr, plan);
}

rd_status rd_plan_cumsum_strided(int cu_count, int64_t outer, int64_t R, int64_t inner,
                                 int64_t stride_outer, int64_t stride_r, int64_t stride_inner,
                                 rd_plan* plan) {
    rd::Strides v{outer, R, inner, stride_outer, stride_r, stride_inner};
    std::lock_guard<std::mutex> lock(g_tune_mu);
    return rd::plan_cumsum_view(cu_count, &v, g_tune_on ? &g_tune : nullptr, plan);
}

rd_status rd_sum_1d(const float* x, int64_t n, float* out, hipStream_t stream) {
    return rd_reduce_1d(x, n, RD_OP_SUM, out, stream);
}

rd_status rd_sum_dim(const float* x, int64_t outer, int64_t R, int64_t inner, float* out,
                     hipStream_t stream) {
    return rd_reduce_dim(x, outer, R, inner, RD_OP_SUM, out, stream);
}

const char* rd_status_string(rd_status status) {
    switch (status) {
        case RD_OK: return "RD_OK";
        case RD_ERR_INVALID_ARG: return "RD_ERR_INVALID_ARG";
        case RD_ERR_NO_DEVICE: return "RD_ERR_NO_DEVICE";
        case RD_ERR_ALLOC: return "RD_ERR_ALLOC";
        case RD_ERR_LAUNCH: return "RD_ERR_LAUNCH";
        case RD_ERR_HIP: return "RD_ERR_HIP";
        case RD_ERR_CAPTURE: return "RD_ERR_CAPTURE";
        case RD_ERR_WORKSPACE: return "RD_ERR_WORKSPACE";
    }
    return "RD_ERR_UNKNOWN";
}

int rd_last_hip_error(void) { return t_last_hip; }

int rd_version(void) {
    return RD_VERSION_MAJOR * 10000 + RD_VERSION_MINOR * 100 + RD_VERSION_PATCH;
}

rd_status rd_plan_dim(int cu_count, int64_t outer, int64_t R, int64_t inner,
                      rd_plan* plan) {
    std::lock_guard<std::mutex> lock(g_tune_mu);
    return rd::plan_dim(cu_count, outer, R, inner, RD_OP_SUM, g_tune_on ? &g_tune : nullptr,
                        plan);
}

rd_status rd_plan_reduce(int cu_count, int64_t outer, int64_t R, int64_t inner, int32_t op,
                         rd_plan* plan) {
    if (op < RD_OP_SUM || op > RD_OP_SOFTMAX_DENOM) return RD_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lock(g_tune_mu);
    return rd::plan_dim(cu_count, outer, R, inner, op, g_tune_on ? &g_tune : nullptr, plan);
}

rd_status rd_plan_1d(int cu_count, int64_t n, rd_plan* plan) {
    return rd_plan_dim(cu_count, 1, n, 1, plan);
}

rd_status rd_tune_set(const rd_tune* tune) {
    std::lock_guard<std::mutex> lock(g_tune_mu);
    if (!tune) {
        g_tune_on = false;
        memset(&g_tune, 0, sizeof(g_tune));
        return RD_OK;
    }
    if (tune->group < 0 || tune->col_waves < 0 || tune->row_waves < 0 || tune->unroll < 0 ||
        tune->order < 0 || tune->nontemporal < 0 || tune->combine < 0 || tune->path < 0 ||
        tune->split < 0)
        return RD_ERR_INVALID_ARG;
    g_tune = *tune;
    g_tune_on = true;
    return RD_OK;
}

int rd_tune_supported(int32_t op, int32_t path, int32_t group_or_col_waves,
                      int32_t row_waves, int32_t unroll) {
    if (path == RD_PATH_ROWS) return rd::rows_shape_supported(op, group_or_col_waves, unroll);
    if (path == RD_PATH_COLS)
        return rd::cols_shape_supported(op, group_or_col_waves, row_waves, unroll);
    if (path == RD_PATH_COLS_SMALL) return rd::small_shape_supported(op, unroll);
    return 0;
}

}  // extern "C"
